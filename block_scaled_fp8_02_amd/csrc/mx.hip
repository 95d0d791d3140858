// mx.hip -- MXFP8 quantizer for gfx950 (Miles MXFP8/NVFP4 blog, MXFP8
// paragraphs): 32 consecutive values share one E8M0 power-of-two scale
// 2^k, k the smallest integer with max|block| <= 448 * 2^k (rounded up so
// the block maximum does not clip), and the codes are E4M3(x * 2^-k).  The
// row-wise (1x32) and column-wise (32x1) copies are both quantized from the
// full-precision input, in one pass over a 128x128 tile.
//
// The MX GEMMs themselves run through the generic kernel in gemm.hip with
// the E8M0 scales handed to the scaled MFMA.
#include "device_common.hpp"
#include "kernels.hpp"

namespace fp8blk {

// Codes of four values of a block with exponent k.  No clamp to +-448: k is
// the smallest exponent with max|block| <= 448 * 2^k, or the clamp at -127,
// below which 448 * 2^-127 exceeds every block maximum, or 127, which no
// finite maximum reaches (448 * 2^127 > FLT_MAX); so |x * 2^-k| <= 448.
__device__ __forceinline__ uint32_t mx_encode4(const float* v, int k) {
    return e4m3_pack4_q(ldexpf(v[0], -k), ldexpf(v[1], -k), ldexpf(v[2], -k), ldexpf(v[3], -k));
}

// Lane i of each 16-lane row receives lane i + n of the row (DPP row shift),
// 0 past the row's end.
template <int N>
__device__ __forceinline__ uint32_t row_from_above(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x100 + N, 0xF, 0xF, true);
}

// Max over the 4-lane quad of non-negative, non-NaN values (their bit
// patterns order as the values).
__device__ __forceinline__ float max4_quad(float v) {
    uint32_t u = __float_as_uint(v);
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0xB1, 0xF, 0xF, true));
    u = max(u, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)u, 0x4E, 0xF, 0xF, true));
    return __uint_as_float(u);
}

// Tile 128 rows x 128 cols, one per block, numbered row-tile-major; thread
// t holds rows 8*(t/16)..+7, cols
// 8*(t%16)..+7.  A 32-column row block spans 4 consecutive lanes; a 32-row
// column block spans the 4 row-slices of one wavefront.
template <typename T>
__global__ __launch_bounds__(256) void k_mx_quant(const T* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
                                                  uint8_t* __restrict__ q, int64_t ldq,
                                                  uint8_t* __restrict__ e, int64_t lde,
                                                  uint8_t* __restrict__ qT, int64_t ldqT,
                                                  uint8_t* __restrict__ eT, int64_t ldeT) {
    __shared__ __attribute__((aligned(16))) uint8_t tileT[128 * 128];
    __shared__ uint8_t ebT[4][128];                                   // column E8M0 bytes per 32-row block
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    // E8M0 bytes leave four at a time (one 128-wide tile's four 32-blocks)
    // where the buffers allow 4-byte stores
    const bool e_words = e != nullptr && reinterpret_cast<uintptr_t>(e) % 4 == 0 && lde % 4 == 0;
    const bool eT_words = eT != nullptr && reinterpret_cast<uintptr_t>(eT) % 4 == 0 && ldeT % 4 == 0;
    const int rg = t >> 4, cg = t & 15;
    // consecutive blocks walk along a row of tiles: the tiles in flight at
    // one time read whole input rows and write whole code rows
    const int64_t nct = (cols + 127) / 128;
    const int64_t rb = ((int64_t)blockIdx.x / nct) * 128, cb = ((int64_t)blockIdx.x % nct) * 128;
    const int64_t r0 = rb + rg * 8, c0 = cb + cg * 8;
    const int cvalid = clamp_valid(cols - c0);

    float v[8][8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int64_t r = r0 + p;
        const bool in = r < rows;
        load8(x + (in ? r : 0) * ldx + c0, in ? cvalid : 0, v[p]);
    }

    if (q != nullptr) {
        // row-wise 1x32: lanes 4n..4n+3 of a 16-lane row slice share a block
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            float m = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[p][j]));
            m = max4_quad(m);
            const int k = mx_exponent(m);
            const int64_t r = r0 + p;
            // the row's four E8M0 bytes of this tile (lanes cg = 0, 4, 8, 12)
            // go out as one word from lane cg = 0
            const uint32_t b = (uint32_t)(c0 < cols ? k + 127 : 127);
            const uint32_t b1 = row_from_above<4>(b), b2 = row_from_above<8>(b), b3 = row_from_above<12>(b);
            if (r < rows) {
                *reinterpret_cast<uint2*>(q + r * ldq + c0) = make_uint2(mx_encode4(&v[p][0], k), mx_encode4(&v[p][4], k));
                if (e_words) {
                    if (cg == 0)
                        *reinterpret_cast<uint32_t*>(e + r * lde + cb / 32) = b | (b1 << 8) | (b2 << 16) | (b3 << 24);
                } else if ((cg & 3) == 0) {
                    e[r * lde + c0 / 32] = (uint8_t)b;
                }
            }
        }
    }
    if (qT == nullptr) return;                                       // uniform

    // column-wise 32x1: reduce 8 rows in-thread, then lanes l, l^16, l^32, l^48
    int kc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float m = 0.0f;
#pragma unroll
        for (int p = 0; p < 8; ++p) m = fmaxf(m, fabsf(v[p][j]));
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        kc[j] = mx_exponent(m);
    }
    if (lane < 16) {                                                  // one writer per (column, wave)
        const int64_t rblk = rb / 32 + wave;
        const bool padblk = rb + 32 * wave >= rows;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const uint8_t bt = (uint8_t)(padblk ? 127 : kc[j] + 127);
            if (eT_words) {
                ebT[wave][cg * 8 + j] = bt;                           // the column's word leaves after the barrier
            } else {
                const int64_t c = c0 + j;
                if (c < cols) eT[c * ldeT + rblk] = bt;
            }
        }
    }
    uint32_t lo[8], hi[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        lo[p] = e4m3_pack4_q(ldexpf(v[p][0], -kc[0]), ldexpf(v[p][1], -kc[1]), ldexpf(v[p][2], -kc[2]),
                             ldexpf(v[p][3], -kc[3]));
        hi[p] = e4m3_pack4_q(ldexpf(v[p][4], -kc[4]), ldexpf(v[p][5], -kc[5]), ldexpf(v[p][6], -kc[6]),
                             ldexpf(v[p][7], -kc[7]));
    }
    uint32_t tlo[8], thi[8];
    transpose8x8(lo, hi, tlo, thi);
#pragma unroll
    for (int j = 0; j < 8; ++j)
        *reinterpret_cast<uint2*>(tileT + (cg * 8 + j) * 128 + ((rg ^ cg) << 3)) = make_uint2(tlo[j], thi[j]);
    __syncthreads();
    if (eT_words && t < 128 && cb + t < cols)
        *reinterpret_cast<uint32_t*>(eT + (cb + t) * ldeT + rb / 32) =
            (uint32_t)ebT[0][t] | ((uint32_t)ebT[1][t] << 8) | ((uint32_t)ebT[2][t] << 16) | ((uint32_t)ebT[3][t] << 24);
    // 8 lanes per code row, so that every store instruction writes 8 whole
    // 128-byte rows: lane chunk ch holds logical 8-byte chunks 2ch and 2ch+1,
    // stored at physical (2ch)^s and (2ch+1)^s, s = crow/8 (one aligned
    // 16-byte pair, its halves swapped when s is odd).
    const int ch = t & 7;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int crow = (t >> 3) + 32 * i;
        const int s8 = crow >> 3;
        const uint4 u = *reinterpret_cast<const uint4*>(tileT + crow * 128 + ((((2 * ch) ^ s8) & ~1) << 3));
        const uint4 w = (s8 & 1) ? make_uint4(u.z, u.w, u.x, u.y) : u;
        const int64_t c = cb + crow;
        if (c < cols) *reinterpret_cast<uint4*>(qT + c * ldqT + rb + 16 * ch) = w;
    }
}

// Row-wise copy only (no transposed codes requested): no tile, no LDS.  One
// 16-lane slot per (row, 128-column group), 8 columns a lane, so a 32-wide
// block is one lane quad -- the rollout's few-row activations spread over
// rows x groups slots instead of a handful of 128-row tiles.  The same
// arithmetic per block as the tile kernel's row-wise pass.
template <typename T>
__global__ __launch_bounds__(256) void k_mx_quant_rows(const T* __restrict__ x, int64_t cols, int64_t ldx,
                                                       uint8_t* __restrict__ q, int64_t ldq,
                                                       uint8_t* __restrict__ e, int64_t lde,
                                                       uint32_t groups_per_row, uint32_t total) {
    const uint32_t slot = blockIdx.x * 16u + (threadIdx.x >> 4);
    if (slot >= total) return;                       // whole 16-lane slots exit together
    const bool e_words = e != nullptr && reinterpret_cast<uintptr_t>(e) % 4 == 0 && lde % 4 == 0;
    const uint32_t row = slot / groups_per_row;
    const uint32_t g = slot - row * groups_per_row;
    const int l16 = threadIdx.x & 15;
    const int64_t c0 = (int64_t)g * 128 + 8 * l16;
    float v[8];
    load8(x + (int64_t)row * ldx + c0, clamp_valid(cols - c0), v);
    float m = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
    m = max4_quad(m);
    const int k = mx_exponent(m);
    const uint32_t b = (uint32_t)(c0 < cols ? k + 127 : 127);
    const uint32_t b1 = row_from_above<4>(b), b2 = row_from_above<8>(b), b3 = row_from_above<12>(b);
    *reinterpret_cast<uint2*>(q + (int64_t)row * ldq + c0) = make_uint2(mx_encode4(&v[0], k), mx_encode4(&v[4], k));
    if (e == nullptr) return;
    if (e_words) {
        if (l16 == 0)
            *reinterpret_cast<uint32_t*>(e + (int64_t)row * lde + 4 * (int64_t)g) = b | (b1 << 8) | (b2 << 16) | (b3 << 24);
    } else if ((l16 & 3) == 0) {
        e[(int64_t)row * lde + c0 / 32] = (uint8_t)b;
    }
}

hipError_t launch_mx_quant(const void* x, bool in_bf16, int64_t rows, int64_t cols, int64_t ldx,
                           uint8_t* q, int64_t ldq, uint8_t* e, int64_t lde,
                           uint8_t* qT, int64_t ldqT, uint8_t* eT, int64_t ldeT, hipStream_t st) {
    if (rows == 0 || cols == 0) return hipSuccess;
    if (qT == nullptr) {
        if (q == nullptr) return hipSuccess;
        const int64_t gpr = (cols + 127) / 128, total = rows * gpr;
        if (total > 0xFFFFFFF0ll) return hipErrorInvalidValue;
        const dim3 grid((unsigned)((total + 15) / 16));
        if (in_bf16)
            k_mx_quant_rows<uint16_t><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(x), cols, ldx, q, ldq, e, lde,
                                                            (uint32_t)gpr, (uint32_t)total);
        else
            k_mx_quant_rows<float><<<grid, 256, 0, st>>>(static_cast<const float*>(x), cols, ldx, q, ldq, e, lde,
                                                         (uint32_t)gpr, (uint32_t)total);
        return hipGetLastError();
    }
    const int64_t rt = (rows + 127) / 128, ct = (cols + 127) / 128;
    if (rt * ct > 0x7FFFFFFF) return hipErrorInvalidValue;
    const dim3 grid((unsigned)(rt * ct));
    if (in_bf16)
        k_mx_quant<uint16_t><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(x), rows, cols, ldx, q, ldq, e, lde, qT, ldqT, eT, ldeT);
    else
        k_mx_quant<float><<<grid, 256, 0, st>>>(static_cast<const float*>(x), rows, cols, ldx, q, ldq, e, lde, qT, ldqT, eT, ldeT);
    return hipGetLastError();
}

}  // namespace fp8blk
