// peak.hip -- measurement aid, not part of the FP8 path: the matrix-core
// throughput a gfx950 reaches on random operands, the ceiling the GEMMs'
// fractions are read against beside the published one.
//
// Every wave holds four random A fragments, four random B fragments and
// four independent accumulators in registers and issues 16 MFMAs per loop
// step, each with a different (A, B) pair, so the multiplier inputs change
// from one instruction to the next as they do in a GEMM; nothing touches
// memory inside the loop.  The chip's clock under load depends on the data
// it multiplies (it is power limited), which is why the operands are
// random: each byte is a counter hash of (seed, wave, lane, register),
// E4M3 NaN codes replaced by the neighbouring finite code.
#include "device_common.hpp"
#include "kernels.hpp"

namespace fp8blk {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));

// SplitMix64 finaliser (Steele, Lea and Flood, "Fast splittable
// pseudorandom number generators", 2014) of a 64-bit counter.
__device__ __forceinline__ uint64_t mix64(uint64_t z) {
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// Four random E4M3 codes in a word, none of them NaN (0x7F / 0xFF -> 0x7E / 0xFE).
__device__ __forceinline__ int fp8_word(uint64_t ctr) {
    uint32_t w = (uint32_t)mix64(ctr);
    const uint32_t nan = ~(w ^ 0x7F7F7F7Fu) & 0x7F7F7F7Fu;     // 7 low bits of a byte all set
    uint32_t m = nan & (nan >> 1) & (nan >> 2) & (nan >> 3) & (nan >> 4) & (nan >> 5) & (nan >> 6) & 0x01010101u;
    return (int)(w ^ m);                                        // clear bit 0 of every NaN byte
}

// Two random finite bf16 values of magnitude in [2^-8, 2^8) in a word.
__device__ __forceinline__ int bf16_word(uint64_t ctr) {
    uint32_t w = (uint32_t)mix64(ctr);
    // keep sign and mantissa, set the exponent to 119 + (4 random bits)
    const uint32_t keep = w & 0x807F807Fu;
    const uint32_t ex = ((119u + ((w >> 7) & 15u)) << 7) | ((119u + ((w >> 23) & 15u)) << 23);
    return (int)(keep | ex);
}

// The fp8 loop with the per-block promotion of the FP32-scale recipe added,
// pipelined as in the block-scaled GEMM: every MFMA starts from zero (one
// 128-wide K block), and its four results are added into fp32 accumulators
// one step later with one FMA each by a combined scale (ROWSCALE = false,
// the 1x128 x 128x128 GEMMs) or, for per-row scales on both operands (the
// token-axis WGrad), by a product formed per result first (one multiply and
// one FMA each).  Scales are random and opaque to the compiler every step,
// so nothing is hoisted out of the loop.
template <bool ROWSCALE>
__global__ __launch_bounds__(256) void k_mfma_promote_peak(int64_t iters, uint32_t seed, float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const uint64_t wave = (uint64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const uint64_t base = ((uint64_t)seed << 40) ^ (wave << 12) ^ ((uint64_t)lane << 5);
    v8i a[4], b[4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const uint64_t ca = base + (uint64_t)(f * 8 + r), cb = ca + (1ull << 39);
            a[f][r] = fp8_word(ca);
            b[f][r] = fp8_word(cb);
        }
    float sp[4], sq[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        sp[j] = 1.0f + (float)(mix64(base + 100 + j) >> 41) * 0x1p-23f;
        sq[j] = 1.0f + (float)(mix64(base + 200 + j) >> 41) * 0x1p-23f;
    }
    v4f acc[4][4], prev[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        prev[j] = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][r] = v4f{0.f, 0.f, 0.f, 0.f};
    }
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
#pragma unroll
            for (int j = 0; j < 4; ++j) asm volatile("" : "+v"(sp[j]), "+v"(sq[j]));
            v4f cur[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                cur[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[j], b[(j + r) & 3],
                                                                          v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
            const int pr = (r + 3) & 3;                                 // the previous step's sub-tile
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (ROWSCALE) {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        acc[pr][j][e] = __builtin_fmaf(prev[j][e], sp[j] * sq[e], acc[pr][j][e]);
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[pr][j][e] = __builtin_fmaf(prev[j][e], sp[j], acc[pr][j][e]);
                }
                prev[j] = cur[j];
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    v4f s = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) s += acc[j][r];
    const float v = s[0] + s[1] + s[2] + s[3];
    if (lane == 0) out[wave] = v;
}

template <bool BF16>
__global__ __launch_bounds__(256) void k_mfma_peak(int64_t iters, uint32_t seed, float* __restrict__ out) {
    const int lane = threadIdx.x & 63;
    const uint64_t wave = (uint64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const uint64_t base = ((uint64_t)seed << 40) ^ (wave << 12) ^ ((uint64_t)lane << 5);
    v8i a[4], b[4];
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const uint64_t ca = base + (uint64_t)(f * 8 + r), cb = ca + (1ull << 39);
            a[f][r] = BF16 ? bf16_word(ca) : fp8_word(ca);
            b[f][r] = BF16 ? bf16_word(cb) : fp8_word(cb);
        }
    v4f acc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = v4f{0.f, 0.f, 0.f, 0.f};
    for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if constexpr (BF16) {
                    const v8i& x = a[j];
                    const v8i& y = b[(j + r) & 3];
                    // bf16: each 8-word fragment holds two 4-word operands; step r
                    // takes half r&1 of A's and half r>>1 of B's
                    const v4i x4 = v4i{x[0 + 4 * (r & 1)], x[1 + 4 * (r & 1)], x[2 + 4 * (r & 1)], x[3 + 4 * (r & 1)]};
                    const v4i y4 = v4i{y[0 + 4 * (r >> 1)], y[1 + 4 * (r >> 1)], y[2 + 4 * (r >> 1)], y[3 + 4 * (r >> 1)]};
                    acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, x4),
                                                                      __builtin_bit_cast(v8bf, y4), acc[j], 0, 0, 0);
                } else {
                    acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[j], b[(j + r) & 3], acc[j],
                                                                              0, 0, 0, 0, 0, 0);
                }
            }
    }
    const v4f s = acc[0] + acc[1] + acc[2] + acc[3];
    const float v = s[0] + s[1] + s[2] + s[3];
    if (lane == 0) out[wave] = v;                                 // keeps the work alive
}

hipError_t launch_mfma_peak(int kind, int64_t blocks, int64_t iters, uint32_t seed, float* out, hipStream_t st) {
    if (blocks <= 0 || iters <= 0) return hipSuccess;
    if (blocks > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)blocks);
    switch (kind) {
        case 0: k_mfma_peak<false><<<grid, 256, 0, st>>>(iters, seed, out); break;
        case 1: k_mfma_peak<true><<<grid, 256, 0, st>>>(iters, seed, out); break;
        case 2: k_mfma_promote_peak<false><<<grid, 256, 0, st>>>(iters, seed, out); break;
        case 3: k_mfma_promote_peak<true><<<grid, 256, 0, st>>>(iters, seed, out); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace fp8blk
