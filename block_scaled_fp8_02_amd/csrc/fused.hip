// fused.hip -- producers of the 1x128 activation quantizer, fused with it.
//
// The Jet-RL notes (section 3.4, the quantization kernels list, and the
// per-block walk-through of the attention and MLP blocks) fuse the 1x128
// activation quantizer into the operator that produces the activation, so
// the bf16 activation never makes a round trip through HBM:
//
//   k_rmsnorm_quant    RMSNorm of a row, rounded to bf16, then 1x128 groups
//   k_silu_mul_quant   bf16(bf16(silu(gate)) * up), then 1x128 groups
//
// Arithmetic (the pages leave it open; the same definitions as the CPU
// oracle of these producers):
//   RMSNorm  ss = sum x_j^2, exact and rounded once to binary64 (double-double
//            accumulation of the exact binary64 squares); r = fl32(1/sqrt(ss/C
//            + eps)) with each step in binary64; y_j = bf16(fl32(fl32(x_j r) w_j))
//   SiLU     s = bf16(silu(g)) rounded once from the exact value; a =
//            bf16(fl32(s u)); the estimate is binary32 and every case where it
//            might round differently goes through binary64 (see silu_bf16)
// Both then quantize exactly as the 1x128 row quantizer: S = fl32(amax/448)
// per group, codes E4M3(fl32(y/S)), padded columns written as code 0.
#include "device_common.hpp"
#include "kernels.hpp"

namespace fp8blk {

// ---------------------------------------------------------------------
// double-double accumulation: (hi, lo) with hi = fl64(hi + lo)
// ---------------------------------------------------------------------
struct DD {
    double hi, lo;
};

// Knuth's TwoSum: s + e == a + b exactly.
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
    s = a + b;
    const double bp = s - a;
    e = (a - (s - bp)) + (b - bp);
}

__device__ __forceinline__ void dd_add(DD& x, double p) {
    double s, e;
    two_sum(x.hi, p, s, e);
    x.hi = s;
    x.lo += e;
}

__device__ __forceinline__ DD dd_merge(DD a, DD b) {
    double s, e;
    two_sum(a.hi, b.hi, s, e);
    e += a.lo + b.lo;
    DD r;
    r.hi = s + e;                      // Fast2Sum (|s| >= |e| for sums of squares)
    r.lo = e - (r.hi - s);
    return r;
}

__device__ __forceinline__ DD dd_shfl_xor(DD x, int m) {
    DD y;
    y.hi = __shfl_xor(x.hi, m);
    y.lo = __shfl_xor(x.lo, m);
    return y;
}

// Quantize 8 values of one 16-lane group slot and store the codes (and,
// from lane 0 of the slot, the scale): the 1x128 rule of k_quant_rows.
__device__ __forceinline__ void quant_group8(const float y[8], int lane16, uint8_t* qdst, float* sdst) {
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(y[i]));
    amax = max16(amax);
    const float S = block_scale<false>(amax);
    const float P = prescale(S);
    const float Sp = S * P, r = recip32(Sp);
    float z[8];
    if (__all(P == 1.0f)) {
#pragma unroll
        for (int i = 0; i < 8; ++i) z[i] = quotient32(y[i], Sp, r);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) z[i] = quotient32(y[i] * P, Sp, r);
    }
    uint2 out;
    out.x = e4m3_pack4_q(z[0], z[1], z[2], z[3]);
    out.y = e4m3_pack4_q(z[4], z[5], z[6], z[7]);
    *reinterpret_cast<uint2*>(qdst) = out;
    if (lane16 == 0) *sdst = S;
}

// Store 8 bf16 values (bits in the low halves of b[]), `valid` of them.
__device__ __forceinline__ void store_bf16x8(uint16_t* p, int valid, const uint32_t b[8]) {
    if (valid == 8) {
        *reinterpret_cast<uint4*>(p) = make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16),
                                                  b[4] | (b[5] << 16), b[6] | (b[7] << 16));
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < valid) p[i] = (uint16_t)b[i];
    }
}

// ---------------------------------------------------------------------
// RMSNorm + 1x128.  One 256-thread block per row; chunk c (8 columns at
// 8c) belongs to thread c % 256, pass k = c / 256.  A 128-column group is
// 16 consecutive chunks, so a 16-lane slot of one pass owns one group.
// Rows up to 2048 * KREG columns keep their values in registers between
// the two passes (KREG, the passes held, is chosen per launch so that the
// register file holds no unused stash); wider rows read them again (L2).
// ---------------------------------------------------------------------
template <typename T, typename WT, int KREG>
__global__ __launch_bounds__(256) void k_rmsnorm_quant(const T* __restrict__ x, int64_t cols, int64_t ldx,
                                                       const WT* __restrict__ w, float eps,
                                                       uint8_t* __restrict__ q, int64_t ldq,
                                                       float* __restrict__ s, int64_t lds,
                                                       float* __restrict__ rstd,
                                                       uint16_t* __restrict__ y, int64_t ldy) {
    __shared__ double red[2][4];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6, lane16 = t & 15;
    const int64_t row = blockIdx.x;
    const T* xr = x + row * ldx;
    const int64_t nchunk = (cols + 127) / 128 * 16;
    const int K = (int)((nchunk + 255) / 256);

    // pass 1: sum of squares (exact binary64 squares, double-double sum)
    float v[KREG][8];
    DD acc{0.0, 0.0};
#pragma unroll
    for (int k = 0; k < KREG; ++k) {
        const int64_t c = (int64_t)k * 256 + t;
        if (k < K && c < nchunk) {
            load8(xr + 8 * c, clamp_valid(cols - 8 * c), v[k]);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const double d = (double)v[k][i];
                dd_add(acc, d * d);
            }
        }
    }
    for (int k = KREG; k < K; ++k) {
        const int64_t c = (int64_t)k * 256 + t;
        if (c < nchunk) {
            float u[8];
            load8(xr + 8 * c, clamp_valid(cols - 8 * c), u);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const double d = (double)u[i];
                dd_add(acc, d * d);
            }
        }
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) acc = dd_merge(acc, dd_shfl_xor(acc, m));
    if (lane == 0) { red[0][wave] = acc.hi; red[1][wave] = acc.lo; }
    __syncthreads();
    DD tot{red[0][0], red[1][0]};
#pragma unroll
    for (int i = 1; i < 4; ++i) tot = dd_merge(tot, DD{red[0][i], red[1][i]});
    const double ss = tot.hi + tot.lo;
    double tq = ss / (double)cols;
    tq = tq + (double)eps;
    tq = __builtin_sqrt(tq);
    tq = 1.0 / tq;
    const float r = (float)tq;
    if (rstd != nullptr && t == 0) rstd[row] = r;

    // pass 2: y = bf16((x r) w), then the 1x128 quantizer
    auto emit = [&](const float xv[8], int64_t c) {
        const int valid = clamp_valid(cols - 8 * c);
        float wv[8];
        load8(w + 8 * c, valid, wv);
        uint32_t b[8];
        float yv[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float xr_ = xv[i] * r;
            b[i] = f32_to_bf16(xr_ * wv[i]);
            yv[i] = bf16_to_f32(b[i]);
        }
        quant_group8(yv, lane16, q + row * ldq + 8 * c, s + row * lds + c / 16);
        if (y != nullptr && valid > 0) store_bf16x8(y + row * ldy + 8 * c, valid, b);
    };
#pragma unroll
    for (int k = 0; k < KREG; ++k) {
        const int64_t c = (int64_t)k * 256 + t;
        if (k < K && c < nchunk) emit(v[k], c);
    }
    for (int k = KREG; k < K; ++k) {
        const int64_t c = (int64_t)k * 256 + t;
        if (c < nchunk) {
            float u[8];
            load8(xr + 8 * c, clamp_valid(cols - 8 * c), u);
            emit(u, c);
        }
    }
}

// ---------------------------------------------------------------------
// SiLU, rounded once to bf16.
//
// Fast path: binary32 with e = e^-|g| (exp_neg64), s = g/(1+e) (g >= 0) or
// g e/(1+e) (g < 0), the quotient by the hardware reciprocal.  Its error is
// a few binary32 ulps, far below the 2^15-ulp gap between bf16 rounding
// boundaries, so its bf16 rounding is the exact one unless the estimate
// lies within SILU_GUARD ulps of a bf16 midpoint.  Those elements, tiny
// gates (|g| < 2^-60, where g/2 may itself be a midpoint) and gates below
// -64 (e^g nears the binary32 subnormal range) take the slow path:
// binary64 with the same formula (g/2 plus a positive residual for |g| <
// 2^-100), rounded to binary32 with round-to-odd and then to bf16 with
// nearest-even, which equals one rounding since binary32 keeps two bits
// more than bf16 (Boldo and Melquiond, IEEE Trans. Computers 57(4), 2008).
// The gate is bf16, so every possible input is checked on the device.
// ---------------------------------------------------------------------
constexpr int SILU_GUARD = 16;

// e^x for x in [-64, 0]: x log2(e) split into an integer n and a fraction f
// with the product carried in two parts (Cody-Waite style), 2^f from the
// hardware exp2, then scaled by 2^n.  No overflow or underflow is possible
// on this range (the result is at least 2^-93).
__device__ __forceinline__ float exp_neg64(float x) {
    const float L_hi = 1.44269502162933349609375f;          // log2(e) rounded to binary32
    const float L_lo = 1.9259629891e-8f;                     // log2(e) - L_hi
    const float t = x * L_hi;
    const float t_lo = __builtin_fmaf(x, L_hi, -t) + x * L_lo;
    const float n = __builtin_rintf(t);
    const float f = (t - n) + t_lo;
    return __builtin_ldexpf(__builtin_amdgcn_exp2f(f), (int)n);
}

__device__ __forceinline__ uint32_t silu_bf16_slow(float gf) {
    const double G = (double)gf;
    double v;
    int rs = 0;                                       // sign of (exact - v)
    if (G == 0.0) {
        v = G;
    } else if (fabs(G) < 0x1p-100) {
        v = G * 0.5;
        rs = 1;                                       // silu(g) = g/2 + g^2/4 - ...
    } else {
        const double E = exp(-fabs(G));
        v = G >= 0.0 ? G / (1.0 + E) : (G * E) / (1.0 + E);
    }
    const float f = (float)v;
    const double back = (double)f;
    const bool neg = __builtin_signbit(v);
    const double av = fabs(v), ab = fabs(back);
    int side = av > ab ? 1 : (av < ab ? -1 : (neg ? -rs : rs));
    uint32_t mag = __float_as_uint(f) & 0x7FFFFFFFu;
    if (side != 0 && (mag & 1u) == 0u) mag = (uint32_t)((int32_t)mag + side);
    const float ro = __uint_as_float(mag | (neg ? 0x80000000u : 0u));
    return f32_to_bf16(ro);
}

__device__ __forceinline__ bool silu_fast(float gf, uint32_t& bits16) {
    const float ag = fabsf(gf);
    const float e = exp_neg64(-fminf(ag, 64.0f));           // gates past -64 take the slow path
    const float d = 1.0f + e;
    const float num = gf >= 0.0f ? gf : gf * e;
    const float est = num * __builtin_amdgcn_rcpf(d);
    const uint32_t u = __float_as_uint(est);
    const int low = (int)(u & 0xFFFFu) - 0x8000;
    bits16 = f32_to_bf16(est);
    return !(ag < 0x1p-60f || gf < -64.0f || (low <= SILU_GUARD && low >= -SILU_GUARD));
}

// ---------------------------------------------------------------------
// SiLU(gate) * up + 1x128: one 16-lane slot per 128-column group, 8
// columns per lane, 16 groups per 256-thread block (as k_quant_rows).
// ---------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_silu_mul_quant(const uint16_t* __restrict__ gate, int64_t ldg,
                                                        const uint16_t* __restrict__ up, int64_t ldu,
                                                        int64_t cols, uint8_t* __restrict__ q, int64_t ldq,
                                                        float* __restrict__ s, int64_t lds,
                                                        uint16_t* __restrict__ a, int64_t lda,
                                                        uint32_t groups_per_row, uint32_t total_groups) {
    const uint32_t grp = blockIdx.x * 16u + (threadIdx.x >> 4);
    if (grp >= total_groups) return;                 // whole 16-lane slots exit together
    const uint32_t row = grp / groups_per_row;
    const uint32_t g = grp - row * groups_per_row;
    const int lane16 = threadIdx.x & 15;
    const int64_t col0 = (int64_t)g * 128 + lane16 * 8;
    const int valid = clamp_valid(cols - col0);
    float gv[8], uv[8];
    load8(gate + (int64_t)row * ldg + col0, valid, gv);
    load8(up + (int64_t)row * ldu + col0, valid, uv);
    uint32_t sb[8];
    bool slow = false;
    bool need[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        need[i] = !silu_fast(gv[i], sb[i]);
        slow |= need[i];
    }
    if (slow) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (need[i]) sb[i] = silu_bf16_slow(gv[i]);
    }
    uint32_t ab[8];
    float av[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        ab[i] = f32_to_bf16(bf16_to_f32(sb[i]) * uv[i]);
        av[i] = bf16_to_f32(ab[i]);
    }
    quant_group8(av, lane16, q + (int64_t)row * ldq + col0, s + (int64_t)row * lds + g);
    if (a != nullptr && valid > 0) store_bf16x8(a + (int64_t)row * lda + col0, valid, ab);
}

// ---------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------
hipError_t launch_rmsnorm_quant(const void* x, bool x_bf16, int64_t rows, int64_t cols, int64_t ldx,
                                const void* w, bool w_bf16, float eps,
                                uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                float* rstd, uint16_t* y, int64_t ldy, hipStream_t st) {
    if (rows == 0 || cols == 0) return hipSuccess;
    if (rows > 0x7FFFFFFFll) return hipErrorInvalidValue;
    const dim3 grid((unsigned)rows);
    const int64_t K = ((cols + 127) / 128 * 16 + 255) / 256;      // passes of 256 chunks
#define FP8B_RN3(T_, W_, KR_)                                                                        \
    k_rmsnorm_quant<T_, W_, KR_><<<grid, 256, 0, st>>>(static_cast<const T_*>(x), cols, ldx,         \
                                                       static_cast<const W_*>(w), eps, q, ldq, s,    \
                                                       lds, rstd, y, ldy)
#define FP8B_RN(T_, W_)                                                                              \
    do {                                                                                             \
        if (K <= 1) FP8B_RN3(T_, W_, 1);                                                             \
        else if (K <= 2) FP8B_RN3(T_, W_, 2);                                                        \
        else if (K <= 4) FP8B_RN3(T_, W_, 4);                                                        \
        else FP8B_RN3(T_, W_, 8);                                                                    \
    } while (0)
    if (x_bf16) {
        if (w_bf16) FP8B_RN(uint16_t, uint16_t); else FP8B_RN(uint16_t, float);
    } else {
        if (w_bf16) FP8B_RN(float, uint16_t); else FP8B_RN(float, float);
    }
#undef FP8B_RN
#undef FP8B_RN3
    return hipGetLastError();
}

hipError_t launch_silu_mul_quant(const uint16_t* gate, int64_t ldg, const uint16_t* up, int64_t ldu,
                                 int64_t rows, int64_t cols, uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                 uint16_t* a, int64_t lda, hipStream_t st) {
    const int64_t gpr = (cols + 127) / 128;
    const int64_t total = rows * gpr;
    if (total == 0) return hipSuccess;
    if (total > 0xFFFFFFF0ll) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((total + 15) / 16));
    k_silu_mul_quant<<<grid, 256, 0, st>>>(gate, ldg, up, ldu, cols, q, ldq, s, lds, a, lda,
                                           (uint32_t)gpr, (uint32_t)total);
    return hipGetLastError();
}

}  // namespace fp8blk
