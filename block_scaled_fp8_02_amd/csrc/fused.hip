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
//   RMSNorm  ss = sum x_j^2, exact and rounded once to binary64 (a plain
//            binary64 sum where that is provably exact, else double-double
//            accumulation of the exact binary64 squares); r = fl32(1/sqrt(ss/C
//            + eps)) with each step in binary64; y_j = bf16(fl32(fl32(x_j r) w_j))
//   SiLU     s = bf16(silu(g)) rounded once from the exact value (a table
//            of the correctly rounded values, built at compile time, for the
//            common gates; closed forms or a binary32 estimate checked
//            against the rounding boundaries, else binary64, for the rest);
//            a = bf16(fl32(s u))
//
// Both work in 8-lane slots, 16 values a lane, one 128-column group a slot:
// the SiLU table lookups and the plain sums leave the quantizer's own
// arithmetic as the main cost, so each lane amortises the per-group scale
// over 16 values rather than 8.
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

// ---------------------------------------------------------------------
// 8-lane slots.  Both producers give each 128-column group an aligned slot
// of 8 lanes; lane j of the slot holds the group's columns 8j..8j+7 and
// 64+8j..64+8j+7, so each of its two 16-byte loads of bf16 covers one
// whole 128-byte half of the group, and the group's amax is a 3-step DPP
// reduction inside the slot (no LDS round trip).
// ---------------------------------------------------------------------

// Max over the aligned 8-lane slot of non-negative, non-NaN values (their
// bit patterns order as the values): swap neighbours, swap pairs, mirror
// the two quads.  Every lane of the slot must be active (bound_ctrl reads
// 0 from an inactive lane, harmless for a maximum of magnitudes).
__device__ __forceinline__ float max8_slot(float v) {
    uint32_t u = __float_as_uint(v);
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0xB1, 0xF, 0xF, true));
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x4E, 0xF, 0xF, true));
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x141, 0xF, 0xF, true));
    return __uint_as_float(u);
}

// 8 bf16 values as 4 little-endian words; `valid` (0..8) are in bounds,
// the rest read as +0.  A full run is one 16-byte load.
__device__ __forceinline__ void load_bf16x8_words(const uint16_t* p, int valid, uint32_t w[4]) {
    if (valid == 8) {
        const uint4 v = *reinterpret_cast<const uint4*>(p);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t lo = 2 * i < valid ? p[2 * i] : 0u;
            const uint32_t hi = 2 * i + 1 < valid ? p[2 * i + 1] : 0u;
            w[i] = lo | (hi << 16);
        }
    }
}

// 8 fp32 values as their bit patterns, as load_bf16x8_words.
__device__ __forceinline__ void load_f32x8_words(const float* p, int valid, uint32_t w[8]) {
    if (valid == 8) {
        const uint4 a = *reinterpret_cast<const uint4*>(p);
        const uint4 b = *reinterpret_cast<const uint4*>(p + 4);
        w[0] = a.x; w[1] = a.y; w[2] = a.z; w[3] = a.w;
        w[4] = b.x; w[5] = b.y; w[6] = b.z; w[7] = b.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = i < valid ? __float_as_uint(p[i]) : 0u;
    }
}

// bf16 number i (0..7) of a word array as fp32.
__device__ __forceinline__ float word_bf16(const uint32_t* w, int i) {
    return __uint_as_float((i & 1) ? (w[i >> 1] & 0xFFFF0000u) : (w[i >> 1] << 16));
}
__device__ __forceinline__ uint32_t word_bits(const uint32_t* w, int i) {
    return (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
}

// Packed unsigned 16-bit max, min and decrement on the two halves of a word.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_max_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ uint32_t pk_min_u16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_min(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}
__device__ __forceinline__ uint32_t pk_dec_u16(uint32_t a) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(u16x2, a) - (u16x2){1, 1});
}

// Two fp32 values rounded to bf16 (nearest even) as one word, the first in
// the low half: the gfx950 packed conversion, which the device test suite
// checks against the integer rounding of f32_to_bf16 on every finite fp32
// bit pattern.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// Quantize the 16 bf16 values (8 words) of a lane in its slot -- the 1x128
// rule of k_quant_rows -- and store its two 8-code runs (and, from lane 0
// of the slot, the scale).  The amax of bf16 values is the largest
// magnitude bit pattern (packed maxima), exact.
__device__ __forceinline__ void quant_slot16(const uint32_t yw[8], int j, uint8_t* q0, uint8_t* q1, float* sdst) {
    uint32_t m = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) m = pk_max_u16(m, yw[i] & 0x7FFF7FFFu);
    float amax = bf16_to_f32(max(m & 0xFFFFu, m >> 16));
    amax = max8_slot(amax);
    const float S = block_scale<false>(amax);
    const float P = prescale(S);
    const float Sp = S * P, r = recip32(Sp);
    float z[16];
    if (__all(P == 1.0f)) {
#pragma unroll
        for (int i = 0; i < 16; ++i) z[i] = quotient32(word_bf16(yw, i), Sp, r);
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) z[i] = quotient32(word_bf16(yw, i) * P, Sp, r);
    }
    *reinterpret_cast<uint2*>(q0) = make_uint2(e4m3_pack4_q(z[0], z[1], z[2], z[3]),
                                               e4m3_pack4_q(z[4], z[5], z[6], z[7]));
    *reinterpret_cast<uint2*>(q1) = make_uint2(e4m3_pack4_q(z[8], z[9], z[10], z[11]),
                                               e4m3_pack4_q(z[12], z[13], z[14], z[15]));
    if (j == 0) *sdst = S;
}

// Store 8 bf16 values (4 words), `valid` of them.
__device__ __forceinline__ void store_bf16x8_words(uint16_t* p, int valid, const uint32_t b[4]) {
    if (valid == 8) {
        *reinterpret_cast<uint4*>(p) = make_uint4(b[0], b[1], b[2], b[3]);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (i < valid) p[i] = (uint16_t)((i & 1) ? (b[i >> 1] >> 16) : (b[i >> 1] & 0xFFFFu));
    }
}

// ---------------------------------------------------------------------
// RMSNorm + 1x128.  One wavefront per row (4 rows per 256-thread block):
// 8 slots of 8 lanes, so one pass covers 1024 columns; pass k gives slot
// lane/8 the group 8k + lane/8.  Rows of up to 1024 * KREG columns keep
// their values in registers (raw words: 8 per pass for bf16, 16 for fp32)
// between the two passes; wider rows read the rest again (from L2).
//
// The sum of squares is a double-double sum over the lanes and passes, as
// the exactness argument needs (see the API), but its terms are the sums
// of a lane's 16 squares per pass where those are exact in plain binary64:
// write a bf16 x as m 2^f (integer m < 2^8, f the exponent of its last
// significand bit); x^2 = m^2 2^(2f) has 16 bits, and when 16 values span
// D = f_max - f_min <= 16 exponents every partial sum of their squares is
// an integer multiple of 2^(2 f_min) below 16 * 2^(16 + 2D) <= 2^53, so
// exactly representable.  D comes from the largest and the smallest
// nonzero magnitude, kept as packed 16-bit maxima and minima of the raw
// words (two elements per operation).  Other runs, and fp32 rows (48-bit
// squares), add each square to the double-double sum.
// ---------------------------------------------------------------------
template <typename T>
struct RowWords {
    static constexpr int N = sizeof(T) == 2 ? 8 : 16;     // words per 16 values
};

template <typename T>
__device__ __forceinline__ void load_row16(const T* p, int v0, int v1, uint32_t (&w)[RowWords<T>::N]) {
    if constexpr (sizeof(T) == 2) {
        load_bf16x8_words(reinterpret_cast<const uint16_t*>(p), v0, w);
        load_bf16x8_words(reinterpret_cast<const uint16_t*>(p) + 64, v1, w + 4);
    } else {
        load_f32x8_words(reinterpret_cast<const float*>(p), v0, w);
        load_f32x8_words(reinterpret_cast<const float*>(p) + 64, v1, w + 8);
    }
}

template <typename T>
__device__ __forceinline__ float row_value(const uint32_t* w, int i) {
    if constexpr (sizeof(T) == 2) return word_bf16(w, i);
    else return __uint_as_float(w[i]);
}

template <typename T, int KREG>
struct RowRegs {
    uint32_t v[KREG][RowWords<T>::N];
};

// Raw words of pass k of a row (zeros past the row).
template <typename T>
__device__ __forceinline__ void load_pass(const T* xr, int64_t cols, int64_t c, uint32_t (&wv)[RowWords<T>::N]) {
    if (c < cols) {
        load_row16<T>(xr + c, clamp_valid(cols - c), clamp_valid(cols - c - 64), wv);
    } else {
#pragma unroll
        for (int i = 0; i < RowWords<T>::N; ++i) wv[i] = 0u;
    }
}

template <typename T, int KREG>
__device__ __forceinline__ void load_row(const T* xr, int64_t cols, int K, int lane, RowRegs<T, KREG>& R) {
#pragma unroll
    for (int k = 0; k < KREG; ++k)
        if (k < K) load_pass<T>(xr, cols, ((int64_t)k * 8 + (lane >> 3)) * 128 + 8 * (lane & 7), R.v[k]);
}

// One row, its first KREG passes in registers (the rest are read again).
template <typename T, typename WT, int KREG>
__device__ __forceinline__ void rmsnorm_row(const T* __restrict__ xr, int64_t row, int64_t cols, int64_t G, int K,
                                            int lane, const RowRegs<T, KREG>& R,
                                            const WT* __restrict__ w, float eps,
                                            uint8_t* __restrict__ q, int64_t ldq,
                                            float* __restrict__ s, int64_t lds, float* __restrict__ rstd,
                                            uint16_t* __restrict__ y, int64_t ldy) {
    constexpr int NW = RowWords<T>::N;
    const int j = lane & 7;
    const WT* wr = w;
    // group of slot lane/8 in pass k, and the first column of lane j in it
    auto grp_of = [&](int k) { return (int64_t)k * 8 + (lane >> 3); };
    auto col_of = [&](int k) { return grp_of(k) * 128 + 8 * j; };

    // pass 1: sum of squares
    DD acc{0.0, 0.0};
    auto add_pass = [&](const uint32_t (&wv)[NW]) {
        bool plain = false;
        if constexpr (sizeof(T) == 2) {
            uint32_t mx = 0u, mn = 0xFFFFFFFFu;
            double p = 0.0;
#pragma unroll
            for (int i = 0; i < NW; ++i) {
                const uint32_t m = wv[i] & 0x7FFF7FFFu;
                mx = pk_max_u16(mx, m);
                mn = pk_min_u16(mn, pk_dec_u16(m));              // zeros wrap to 0xFFFF
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const double d = (double)word_bf16(wv, i);
                p = __builtin_fma(d, d, p);
            }
            const uint32_t mx1 = max(mx & 0xFFFFu, mx >> 16), mn1 = min(mn & 0xFFFFu, mn >> 16);
            const int fmax = max((int)(mx1 >> 7), 1), fmin = max((int)((mn1 + 1u) >> 7), 1);
            plain = mn1 == 0xFFFFu || fmax - fmin <= 16;
            if (plain) dd_add(acc, p);
        }
        if (!plain) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const double d = (double)row_value<T>(wv, i);
                dd_add(acc, d * d);
            }
        }
    };
#pragma unroll
    for (int k = 0; k < KREG; ++k)
        if (k < K) add_pass(R.v[k]);
    for (int k = KREG; k < K; ++k) {
        uint32_t u[NW];
        load_pass<T>(xr, cols, col_of(k), u);
        add_pass(u);
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) acc = dd_merge(acc, dd_shfl_xor(acc, m));
    const double ss = acc.hi + acc.lo;
    double tq = ss / (double)cols;
    tq = tq + (double)eps;
    tq = __builtin_sqrt(tq);
    tq = 1.0 / tq;
    const float r = (float)tq;
    if (rstd != nullptr && lane == 0) rstd[row] = r;

    // pass 2: y = bf16((x r) w), then the 1x128 quantizer
    auto emit = [&](const uint32_t (&wv)[NW], int k) {
        if (grp_of(k) >= G) return;                           // slot past the row (whole slot)
        const int64_t c = col_of(k);
        const int v0 = clamp_valid(cols - c), v1 = clamp_valid(cols - c - 64);
        uint32_t ww[RowWords<WT>::N];
        load_row16<WT>(wr + c, v0, v1, ww);
        uint32_t yw[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float a0 = row_value<T>(wv, 2 * i) * r, a1 = row_value<T>(wv, 2 * i + 1) * r;
            yw[i] = pack_bf16x2(a0 * row_value<WT>(ww, 2 * i), a1 * row_value<WT>(ww, 2 * i + 1));
        }
        uint8_t* qr = q + row * ldq + c;
        quant_slot16(yw, j, qr, qr + 64, s + row * lds + c / 128);
        if (y != nullptr) {
            uint16_t* yr = y + row * ldy + c;
            if (v0 > 0) store_bf16x8_words(yr, v0, yw);
            if (v1 > 0) store_bf16x8_words(yr + 64, v1, yw + 4);
        }
    };
#pragma unroll
    for (int k = 0; k < KREG; ++k)
        if (k < K) emit(R.v[k], k);
    for (int k = KREG; k < K; ++k) {
        uint32_t u[NW];
        load_pass<T>(xr, cols, col_of(k), u);
        emit(u, k);
    }
}

// One row per wavefront.  (A persistent variant that prefetched each
// wavefront's next row into registers measured slower: the two rows'
// registers cut the occupancy to two wavefronts per SIMD.)
template <typename T, typename WT, int KREG>
__global__ __launch_bounds__(256) void k_rmsnorm_quant(const T* __restrict__ x, int64_t rows, int64_t cols,
                                                       int64_t ldx, const WT* __restrict__ w, float eps,
                                                       uint8_t* __restrict__ q, int64_t ldq,
                                                       float* __restrict__ s, int64_t lds,
                                                       float* __restrict__ rstd,
                                                       uint16_t* __restrict__ y, int64_t ldy) {
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (row >= rows) return;                                    // the whole wavefront
    const int64_t G = (cols + 127) / 128;
    const int K = (int)((G + 7) / 8);
    RowRegs<T, KREG> A;
    load_row<T, KREG>(x + row * ldx, cols, K, lane, A);
    rmsnorm_row<T, WT, KREG>(x + row * ldx, row, cols, G, K, lane, A, w, eps, q, ldq, s, lds, rstd, y, ldy);
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
// SiLU table.  The gate is bf16, so silu is a function of 2^16 inputs.
// For 2^-16 <= |g| < 128 (exponent fields 111..133, both signs: 5888
// gates) the correctly rounded bf16 value is tabulated at compile time
// below; outside that range it has a closed form or is rare:
//   2^-120 <= |g| < 2^-16   silu(g) = g/2 + g^2/4 - ..., within far less
//                           than half a bf16 ulp of g/2, which is a bf16
//                           number: the result is g/2 (exponent field - 1)
//   g >= 128                g (1 - e^-g) differs from g by less than half
//                           an ulp: the result is g
//   g <= -128               |silu(g)| < 2^-170, below half the least bf16
//                           subnormal: the result is -0
//   zeros                   +-0
//   the rest                (|g| < 2^-120, infinities, NaN) the checked
//                           binary32 estimate of silu_fast, else
//                           silu_bf16_slow
// ---------------------------------------------------------------------
namespace silu_lut {

constexpr int kE0 = 111;                   // first tabulated exponent field
constexpr int kNE = 23;                    // tabulated exponent fields
constexpr int kHalf = kNE * 128;           // entries per sign
constexpr int kN = 2 * kHalf;              // entry i: sign i / kHalf, magnitude bits (kE0 << 7) + i % kHalf

constexpr double pow2(int n) {             // 2^n, -1022 <= n <= 1023
    return __builtin_bit_cast(double, (uint64_t)(n + 1023) << 52);
}

// e^x for x in [-128, 0] in binary64 arithmetic: x = n ln2 + r with the
// product n ln2 carried in two parts (n ln2_hi exact), |r| <= ln2/2, e^r
// by its Taylor series to degree 22 (truncation below 2^-90), times 2^n.
// Its relative error is a few binary64 ulps.
constexpr double exp_neg(double x) {
    constexpr double inv_ln2 = 1.4426950408889634;
    constexpr double ln2_hi = 0x1.62e42fee00000p-1;          // ln 2 to 32 bits
    constexpr double ln2_lo = 0x1.a39ef35793c76p-33;         // ln 2 - ln2_hi
    const double tn = x * inv_ln2;
    const int n = (int)(tn < 0 ? tn - 0.5 : tn + 0.5);
    const double r = (x - n * ln2_hi) - n * ln2_lo;
    double p = 1.0;
    for (int k = 22; k >= 1; --k) p = 1.0 + p * r / k;
    return p * pow2(n);
}

// bf16 bits of the nearest (ties to even) bf16 number to v, whose relative
// error is below 2^-50.  Sets `ambiguous` when v lies within 2^-41 of a
// rounding boundary in units of the bf16 ulp -- that is, when the error
// could change the rounding.
constexpr uint32_t bf16_nearest(double v, bool& ambiguous) {
    const uint32_t sgn = v < 0 ? 0x8000u : 0u;
    const double a = v < 0 ? -v : v;
    if (a == 0.0) return sgn;
    const int e = (int)((__builtin_bit_cast(uint64_t, a) >> 52) & 0x7FF) - 1023;
    const int qe = (e < -126 ? -126 : e) - 7;                  // exponent of the bf16 ulp
    const double t = a / pow2(qe);                             // exact
    const uint64_t k = (uint64_t)t;
    const double f = t - (double)k;                            // exact
    if (f - 0.5 < 0x1p-41 && 0.5 - f < 0x1p-41) ambiguous = true;
    const uint64_t kr = k + (f > 0.5 ? 1 : 0);
    const float rv = (float)((double)kr * pow2(qe));           // exact: kr <= 256
    return sgn | (__builtin_bit_cast(uint32_t, rv) >> 16);
}

struct alignas(16) Table {
    uint16_t v[kN];
    bool ambiguous;
};

constexpr Table make_table() {
    Table T{};
    for (int i = 0; i < kN; ++i) {
        const uint32_t neg = i >= kHalf ? 1u : 0u;
        const uint32_t bits = (neg << 15) | ((uint32_t)(kE0 << 7) + (uint32_t)(i - (int)neg * kHalf));
        const double g = (double)__builtin_bit_cast(float, bits << 16);
        const double E = exp_neg(neg ? g : -g);                 // e^-|g|
        const double sv = neg ? (g * E) / (1.0 + E) : g / (1.0 + E);
        T.v[i] = (uint16_t)bf16_nearest(sv, T.ambiguous);
    }
    return T;
}

}  // namespace silu_lut

__device__ constexpr silu_lut::Table k_silu_table = silu_lut::make_table();
static_assert(!k_silu_table.ambiguous, "a tabulated SiLU value lies too near a bf16 rounding boundary");
static_assert(sizeof(k_silu_table.v) % 16 == 0, "the table is copied in 16-byte pieces");

// silu of a gate outside the table.
__device__ __noinline__ uint32_t silu_bf16_outside(uint32_t gb) {
    const uint32_t mag = gb & 0x7FFFu, e = mag >> 7;
    if (mag == 0u) return gb;
    if (e >= 7u && e < (uint32_t)silu_lut::kE0) return gb - 0x80u;
    if (e >= (uint32_t)(silu_lut::kE0 + silu_lut::kNE) && e < 255u) return (gb & 0x8000u) ? 0x8000u : gb;
    const float gf = bf16_to_f32(gb);
    uint32_t b;
    return silu_fast(gf, b) ? b : silu_bf16_slow(gf);
}

// ---------------------------------------------------------------------
// SiLU(gate) * up + 1x128.  Each 256-thread block copies the table into
// LDS once, then walks the 128-column groups of the matrix (grid-stride),
// one group per 8-lane slot (16 values a lane); silu is one LDS read.
// ---------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_silu_mul_quant(const uint16_t* __restrict__ gate, int64_t ldg,
                                                        const uint16_t* __restrict__ up, int64_t ldu,
                                                        int64_t cols, uint8_t* __restrict__ q, int64_t ldq,
                                                        float* __restrict__ s, int64_t lds,
                                                        uint16_t* __restrict__ a, int64_t lda,
                                                        uint32_t groups_per_row, uint32_t total_groups) {
    __shared__ __align__(16) uint16_t lut[silu_lut::kN];
    {
        const uint4* src = reinterpret_cast<const uint4*>(k_silu_table.v);
        for (int i = threadIdx.x; i < silu_lut::kN / 8; i += 256) reinterpret_cast<uint4*>(lut)[i] = src[i];
    }
    __syncthreads();
    const int j = threadIdx.x & 7;
    const uint32_t step = gridDim.x * 32u;
    for (uint32_t grp = blockIdx.x * 32u + (threadIdx.x >> 3); grp < total_groups; grp += step) {
        const uint32_t row = grp / groups_per_row;
        const uint32_t g = grp - row * groups_per_row;
        const int64_t c = (int64_t)g * 128 + 8 * j;
        const int v0 = clamp_valid(cols - c), v1 = clamp_valid(cols - c - 64);
        uint32_t gw[8], uw[8];
        const uint16_t* gr = gate + (int64_t)row * ldg + c;
        const uint16_t* ur = up + (int64_t)row * ldu + c;
        load_bf16x8_words(gr, v0, gw);
        load_bf16x8_words(gr + 64, v1, gw + 4);
        load_bf16x8_words(ur, v0, uw);
        load_bf16x8_words(ur + 64, v1, uw + 4);
        uint32_t sb[16];
        bool outside = false;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t gb = word_bits(gw, i);
            const uint32_t m = (gb & 0x7FFFu) - (uint32_t)(silu_lut::kE0 << 7);
            outside |= m >= (uint32_t)silu_lut::kHalf;
            const uint32_t idx = min(m, (uint32_t)silu_lut::kHalf - 1u) + (gb >> 15) * (uint32_t)silu_lut::kHalf;
            sb[i] = lut[idx];
        }
        if (outside) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t gb = word_bits(gw, i);
                if ((gb & 0x7FFFu) - (uint32_t)(silu_lut::kE0 << 7) >= (uint32_t)silu_lut::kHalf)
                    sb[i] = silu_bf16_outside(gb);
            }
        }
        uint32_t aw[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            aw[i] = pack_bf16x2(bf16_to_f32(sb[2 * i]) * word_bf16(uw, 2 * i),
                                bf16_to_f32(sb[2 * i + 1]) * word_bf16(uw, 2 * i + 1));
        uint8_t* qr = q + (int64_t)row * ldq + c;
        quant_slot16(aw, j, qr, qr + 64, s + (int64_t)row * lds + g);
        if (a != nullptr) {
            uint16_t* ar = a + (int64_t)row * lda + c;
            if (v0 > 0) store_bf16x8_words(ar, v0, aw);
            if (v1 > 0) store_bf16x8_words(ar + 64, v1, aw + 4);
        }
    }
}

// The bf16 rounding of the producers, exposed for exhaustive checks.
__global__ __launch_bounds__(256) void k_bf16_round(const float* __restrict__ x, int64_t n,
                                                    uint16_t* __restrict__ out) {
    const int64_t pairs = (n + 1) / 2;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < pairs; i += (int64_t)gridDim.x * 256) {
        const bool two = 2 * i + 1 < n;
        const uint32_t b = pack_bf16x2(x[2 * i], two ? x[2 * i + 1] : 0.0f);
        out[2 * i] = (uint16_t)(b & 0xFFFFu);
        if (two) out[2 * i + 1] = (uint16_t)(b >> 16);
    }
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
    const int64_t K = ((cols + 127) / 128 + 7) / 8;              // passes of 8 groups (1024 columns)
    const dim3 grid((unsigned)((rows + 3) / 4));
#define FP8B_RN3(T_, W_, KR_)                                                                        \
    k_rmsnorm_quant<T_, W_, KR_><<<grid, 256, 0, st>>>(static_cast<const T_*>(x), rows, cols, ldx,   \
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
    const int64_t cap = 8 * (int64_t)device_cu_count();
    const int64_t blocks = (total + 31) / 32;
    const dim3 grid((unsigned)(blocks < cap ? blocks : cap));
    if (total + 32 * (int64_t)grid.x > 0xFFFFFFFFll) return hipErrorInvalidValue;   // 32-bit group walk
    k_silu_mul_quant<<<grid, 256, 0, st>>>(gate, ldg, up, ldu, cols, q, ldq, s, lds, a, lda,
                                           (uint32_t)gpr, (uint32_t)total);
    return hipGetLastError();
}

hipError_t launch_bf16_round(const float* x, int64_t n, uint16_t* out, hipStream_t st) {
    if (n == 0) return hipSuccess;
    int64_t blocks = ((n + 1) / 2 + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    k_bf16_round<<<dim3((unsigned)blocks), 256, 0, st>>>(x, n, out);
    return hipGetLastError();
}

}  // namespace fp8blk
