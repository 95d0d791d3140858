// device_common.hpp -- device helpers shared by the gfx950 kernels:
// bf16 conversion, the exact E4M3 quotient and encoder, wave reductions.
//
// The quantizer Q of the Jet-RL notes (section 2.1) is
//     S = max|X| / 448,   Xhat = E4M3(X / S)
// with the quotient formed in fp32 and rounded to the nearest E4M3 value
// (ties to even, saturating at +-448).  The code below reproduces that
// bit for bit without the long IEEE fp32 division sequence per element.
//
// Lane layout of v_mfma_f32_16x16x128_f8f6f4 (checked on the device): lane
// l supplies row l%16 of an operand; its first 16 bytes are K positions
// 16*(l/16) .. +15 and its last 16 bytes K positions 64 + 16*(l/16) .. +15.
// The scaled form takes the E8M0 scale of row l%16, K block l/16 (32 wide)
// from lane l.  The 4 results of lane l are rows 4*(l/16)+r, column l%16.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8blk {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Nearest-even fp32 -> bf16 (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Group scale S = fl32(amax / 448).  The binary64 quotient rounded to
// binary32 equals the correctly rounded binary32 quotient (double rounding
// through 53 bits is innocuous for a division of 24-bit operands, since
// 53 >= 2*24 + 2).
__device__ __forceinline__ float group_scale(float amax) {
    return (float)((double)amax / 448.0);
}

// Power-of-two exponent of a block: the smallest k with amax <= 448 * 2^k
// (the block maximum never clips), clamped to [-127, 127]; -127 for an
// all-zero block.  With amax = m * 2^e, m in [0.5, 1): 448 = 0.875 * 2^9, so
// k = e - 9 when m <= 0.875 and k = e - 8 otherwise.  It gives the E8M0
// scales of MXFP8 (byte k + 127) and the power-of-two FP32 block scales.
__device__ __forceinline__ int mx_exponent(float amax) {
    if (amax == 0.0f) return -127;
    int e;
    const float m = frexpf(amax, &e);
    const int k = e - 9 + (m > 0.875f ? 1 : 0);
    return k < -127 ? -127 : (k > 127 ? 127 : k);
}

// Block scale of the FP32-scale recipe (P2 = false): fl32(amax / 448); of
// the power-of-two recipe (P2 = true): 2^k with k = mx_exponent(amax).
template <bool P2>
__device__ __forceinline__ float block_scale(float amax) {
    return P2 ? ldexpf(1.0f, mx_exponent(amax)) : group_scale(amax);
}

// E8M0 byte of a power-of-two scale's block, replicated over the four
// 32-wide sub-blocks of one 128-wide group (one little-endian word).
__device__ __forceinline__ uint32_t e8m0_x4(float amax) {
    return (uint32_t)(mx_exponent(amax) + 127) * 0x01010101u;
}

// The quotient fl32(x / S), without the long IEEE division sequence.  With
// r = RN32(1/S), q0 = RN32(x * r) is within one ulp of x/S; the residual
// e = q0*S - x is then exact in one FMA, and one Newton step q0 - e*r
// rounds to RN32(x/S) (Markstein's theorem on FMA-based division): three
// full-rate fp32 operations per element.  The residual is formed as
// q0*S - x and subtracted, so that a zero x keeps its sign (x = -0 gives
// q0 = -0, e = +0, -0 - 0*r = -0).
//
// The theorem needs every intermediate to stay normal.  A group scale S
// outside [2^-60, 2^60] is therefore first moved into range by an exact
// power of two P (prescale): x/S = (x*P)/(S*P), S*P is exact (S*2^64 for a
// tiny or subnormal S; S*2^-64 for a huge one), and so is x*P, except that
// x*P may underflow when S is huge -- then |x/S| < 2^-126 and the code is
// the signed zero of x either way.  S = 0 keeps P = 1 and r = 0: every x of
// such a group is a zero or rounds to one, and q0 - e*r is the signed zero
// of x.  Quotients below 2^-11, whose residuals may underflow, still come
// out below 2^-10 with the sign of x, so their E4M3 code is unaffected.
__device__ __forceinline__ float prescale(float S) {
    return (S < 0x1p-60f && S != 0.0f) ? 0x1p64f : (S > 0x1p60f ? 0x1p-64f : 1.0f);
}

// r = RN32(1/S) (0 when S == 0); double rounding through binary64 is
// innocuous here as for group_scale.
__device__ __forceinline__ float recip32(float S) {
    return S == 0.0f ? 0.0f : (float)(1.0 / (double)S);
}

// RN32(x / S) for S = S_group * P and x = x_in * P (P = prescale(S_group)).
__device__ __forceinline__ float quotient32(float x, float S, float r) {
    const float q0 = x * r;
    const float e = __builtin_fmaf(q0, S, -x);
    return __builtin_fmaf(-e, r, q0);
}

// E4M3 code of a finite fp32 value: nearest, ties to even, |y| >= 448
// saturates to 0x7E/0xFE, the sign of zero is kept.  The value is clamped
// to [-448, 448] (saturation: nothing beyond 448 is representable, and
// values in (448, 464) would round to 448 anyway), then converted by the
// gfx950 OCP-E4M3 conversion, which rounds to nearest-even and keeps
// subnormals; the device test suite checks this conversion against the
// reference encoder on every finite fp32 bit pattern.
__device__ __forceinline__ float sat448(float y) {
    return fminf(fmaxf(y, -448.0f), 448.0f);
}

// Two codes in the low 16 bits (first argument in the low byte).
__device__ __forceinline__ uint32_t e4m3_encode2(float a, float b) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false) & 0xFFFFu;
}

__device__ __forceinline__ uint32_t e4m3_encode(float y) {
    return e4m3_encode2(y, y) & 0xFFu;
}

// Four codes in one little-endian word.
__device__ __forceinline__ uint32_t e4m3_pack4(float a, float b, float c, float d) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(sat448(a), sat448(b), 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(sat448(c), sat448(d), lo, true);
}

// Four codes of quantizer quotients, without the clamp.  A quotient x/S of
// a group member never exceeds amax / fl32(amax/448) <= 448 (1 + 2^-24), so
// its fp32 value is at most one ulp above 448, which the conversion rounds
// to 448 (0x7E) like any value below the next midpoint (464).
__device__ __forceinline__ uint32_t e4m3_pack4_q(float a, float b, float c, float d) {
    const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// Max over the 16 lanes of an aligned 16-lane group.
__device__ __forceinline__ float max16(float v) {
    v = fmaxf(v, __shfl_xor(v, 1));
    v = fmaxf(v, __shfl_xor(v, 2));
    v = fmaxf(v, __shfl_xor(v, 4));
    v = fmaxf(v, __shfl_xor(v, 8));
    return v;
}

// Max over the whole wavefront (64 lanes).
__device__ __forceinline__ float max64(float v) {
    v = max16(v);
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
}

// Load 8 consecutive elements (bf16 or fp32) as fp32; `valid` (0..8) of
// them are in bounds, the rest read as +0.  A full 8-element run is one
// (bf16) or two (fp32) 16-byte loads; 16-byte alignment is a precondition
// checked on the host.
__device__ __forceinline__ void load8(const uint16_t* p, int valid, float v[8]) {
    if (valid == 8) {
        uint4 w = *reinterpret_cast<const uint4*>(p);
        v[0] = bf16_to_f32(w.x & 0xFFFFu); v[1] = bf16_to_f32(w.x >> 16);
        v[2] = bf16_to_f32(w.y & 0xFFFFu); v[3] = bf16_to_f32(w.y >> 16);
        v[4] = bf16_to_f32(w.z & 0xFFFFu); v[5] = bf16_to_f32(w.z >> 16);
        v[6] = bf16_to_f32(w.w & 0xFFFFu); v[7] = bf16_to_f32(w.w >> 16);
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = i < valid ? bf16_to_f32(p[i]) : 0.0f;
    }
}

__device__ __forceinline__ void load8(const float* p, int valid, float v[8]) {
    if (valid == 8) {
        float4 a = *reinterpret_cast<const float4*>(p);
        float4 b = *reinterpret_cast<const float4*>(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = i < valid ? p[i] : 0.0f;
    }
}

__device__ __forceinline__ int clamp_valid(int64_t remaining) {
    return remaining >= 8 ? 8 : (remaining <= 0 ? 0 : (int)remaining);
}

// Grouped (MoE) row segments: expert e owns rows [off[e], off[e+1]); its
// rows are cut into tiles of `bi` rows, and the experts' tiles are numbered
// in expert order.  SegPos is a position in that enumeration: expert e, the
// number of tiles before it, and the number of 128-padded rows before it
// (sum over earlier experts of round_up(n, 128)).
struct SegPos {
    int64_t e, first, P;
};

// Inclusive prefix sum over the 64 lanes of a wavefront.
__device__ __forceinline__ int64_t wave_incl_scan(int64_t v) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const int64_t t = __shfl_up(v, d);
        if (lane >= d) v += t;
    }
    return v;
}

// Wave-cooperative search, from position `from` onwards (from.e <= the
// expert sought), for the expert holding tile number `tile`: 64 experts per
// step, each lane reading one expert's bounds.  Every lane of the wave
// returns the same result; e == E means the tile does not exist.
__device__ __forceinline__ SegPos wave_find_tile(const int32_t* off, int64_t E, int64_t tile, int64_t bi, SegPos from) {
    const int lane = threadIdx.x & 63;
    while (from.e < E) {
        const int64_t e = from.e + lane;
        const bool valid = e < E;
        const int64_t n = valid ? (int64_t)off[e + 1] - off[e] : 0;
        const int64_t nt = (n + bi - 1) / bi, np = (n + 127) / 128 * 128;
        const int64_t it = wave_incl_scan(nt), ip = wave_incl_scan(np);
        const uint64_t hit = __ballot(valid && tile < from.first + it);
        if (hit) {
            const int l = __builtin_ctzll(hit);
            SegPos r;
            r.e = from.e + l;
            r.first = from.first + __shfl(it - nt, l);
            r.P = from.P + __shfl(ip - np, l);
            return r;
        }
        from.e += 64;
        from.first += __shfl(it, 63);
        from.P += __shfl(ip, 63);
    }
    from.e = E;
    return from;
}

// Transpose an 8x8 byte block with byte permutes (32 v_perm_b32): rows
// (lo = bytes 0..3, hi = 4..7) in, columns out.  perm(a, b, sel) picks
// bytes of the 8-byte value {a:b} (b = bytes 0..3, a = bytes 4..7).
__device__ __forceinline__ void transpose8x8_perm(const uint32_t lo[8], const uint32_t hi[8],
                                                  uint32_t tlo[8], uint32_t thi[8]) {
    // stage 1: interleave rows 2i and 2i+1 -> [r0c0 r1c0 r0c1 r1c1] ...
    uint32_t a[4][4];   // [row pair][word]: words 0,1 from lo (cols 0-1, 2-3), 2,3 from hi (cols 4-5, 6-7)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        a[i][0] = __builtin_amdgcn_perm(lo[2 * i + 1], lo[2 * i], 0x05010400u);
        a[i][1] = __builtin_amdgcn_perm(lo[2 * i + 1], lo[2 * i], 0x07030602u);
        a[i][2] = __builtin_amdgcn_perm(hi[2 * i + 1], hi[2 * i], 0x05010400u);
        a[i][3] = __builtin_amdgcn_perm(hi[2 * i + 1], hi[2 * i], 0x07030602u);
    }
    // stage 2: join row pairs (0,1)+(2,3) for tlo and (4,5)+(6,7) for thi
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        tlo[2 * w] = __builtin_amdgcn_perm(a[1][w], a[0][w], 0x05040100u);
        tlo[2 * w + 1] = __builtin_amdgcn_perm(a[1][w], a[0][w], 0x07060302u);
        thi[2 * w] = __builtin_amdgcn_perm(a[3][w], a[2][w], 0x05040100u);
        thi[2 * w + 1] = __builtin_amdgcn_perm(a[3][w], a[2][w], 0x07060302u);
    }
}

// Transpose an 8x8 byte block held as rows (lo = bytes 0..3, hi = 4..7):
// column j of the input becomes row j of the output.
__device__ __forceinline__ void transpose8x8(const uint32_t lo[8], const uint32_t hi[8],
                                             uint32_t tlo[8], uint32_t thi[8]) {
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t* src = j < 4 ? lo : hi;
        const int sh = 8 * (j & 3);
        tlo[j] = ((src[0] >> sh) & 0xFFu) | (((src[1] >> sh) & 0xFFu) << 8) |
                 (((src[2] >> sh) & 0xFFu) << 16) | (((src[3] >> sh) & 0xFFu) << 24);
        thi[j] = ((src[4] >> sh) & 0xFFu) | (((src[5] >> sh) & 0xFFu) << 8) |
                 (((src[6] >> sh) & 0xFFu) << 16) | (((src[7] >> sh) & 0xFFu) << 24);
    }
}

}  // namespace fp8blk
