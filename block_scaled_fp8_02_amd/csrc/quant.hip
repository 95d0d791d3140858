// quant.hip -- gfx950 quantizer kernels for the block-scaled FP8 path.
//
// All three kernels apply the quantizer Q of the Jet-RL notes (section
// 2.1): S = max|x| / 448 per group, code = E4M3(fl32(x / S)), nearest-even,
// saturating.  They differ only in the grouping (section 4.2 of the notes;
// the summary page's weight and activation quantization paragraphs):
//   k_quant_rows    1x128 along the contiguous axis (X for FProp, dY for DGrad)
//   k_quant_weight  128x128 blocks of W, optionally also the transposed codes
//   k_quant_cols    1x128 along the token axis, written transposed (the
//                   WGrad operands), optionally also the row-wise copy from
//                   the same read of the input
//
// Data movement: every input element is read from HBM exactly once with
// 16-byte vector loads; codes leave as 8- or 16-byte stores.  The
// transposed copies go through a 16 KB LDS tile whose 8-byte chunks are
// XOR-swizzled so that neither the writes nor the row reads conflict.
#include "device_common.hpp"
#include "kernels.hpp"

namespace fp8blk {

// ---------------------------------------------------------------------
// 1x128 row-wise.  A 16-lane slot owns one group of 128 elements, 8 per
// lane; a 256-thread block owns 16 consecutive groups (row-major order).
// ---------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_quant_rows(const T* __restrict__ x, int64_t cols, int64_t ldx,
                                                    uint8_t* __restrict__ q, int64_t ldq,
                                                    float* __restrict__ s, int64_t lds,
                                                    uint32_t groups_per_row, uint32_t total_groups) {
    const uint32_t grp = blockIdx.x * 16u + (threadIdx.x >> 4);
    if (grp >= total_groups) return;                 // whole 16-lane slots exit together
    const uint32_t row = grp / groups_per_row;
    const uint32_t g = grp - row * groups_per_row;
    const int lane16 = threadIdx.x & 15;
    const int64_t col0 = (int64_t)g * 128 + lane16 * 8;
    const int valid = clamp_valid(cols - col0);
    float v[8];
    load8(x + (int64_t)row * ldx + col0, valid, v);
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) amax = fmaxf(amax, fabsf(v[i]));
    amax = max16(amax);
    const float S = group_scale(amax);
    const double R = quotient_recip(S);
    uint2 out;
    out.x = encode4(v[0], v[1], v[2], v[3], R);
    out.y = encode4(v[4], v[5], v[6], v[7], R);
    *reinterpret_cast<uint2*>(q + (int64_t)row * ldq + col0) = out;
    if (lane16 == 0) s[(int64_t)row * lds + g] = S;
}

// ---------------------------------------------------------------------
// 128x128 weight tile per block.  Thread t holds rows 8*(t/16)..+7 and
// columns 8*(t%16)..+7 of the tile (64 values); one scale per tile.
// ---------------------------------------------------------------------
template <typename T>
__global__ __launch_bounds__(256) void k_quant_weight(const T* __restrict__ w, int64_t D, int64_t C, int64_t ldw,
                                                      uint8_t* __restrict__ q, int64_t ldq,
                                                      float* __restrict__ s, int64_t lds,
                                                      uint8_t* __restrict__ qT, int64_t ldqT) {
    __shared__ float red[4];
    __shared__ __attribute__((aligned(16))) uint8_t tileT[128 * 128];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int rg = t >> 4, cg = t & 15;
    const int64_t bi = blockIdx.x, bj = blockIdx.y;
    const int64_t r0 = bi * 128 + rg * 8;
    const int64_t c0 = bj * 128 + cg * 8;
    const int cvalid = clamp_valid(C - c0);

    float v[8][8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int64_t r = r0 + p;
        const bool in = r < D;
        load8(w + (in ? r : 0) * ldw + c0, in ? cvalid : 0, v[p]);
    }
    float amax = 0.0f;
#pragma unroll
    for (int p = 0; p < 8; ++p)
#pragma unroll
        for (int j = 0; j < 8; ++j) amax = fmaxf(amax, fabsf(v[p][j]));
    amax = max64(amax);
    if (lane == 0) red[wave] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float S = group_scale(amax);
    const double R = quotient_recip(S);
    if (t == 0) s[bi * lds + bj] = S;

    uint32_t lo[8], hi[8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        lo[p] = encode4(v[p][0], v[p][1], v[p][2], v[p][3], R);
        hi[p] = encode4(v[p][4], v[p][5], v[p][6], v[p][7], R);
        if (r0 + p < D) *reinterpret_cast<uint2*>(q + (r0 + p) * ldq + c0) = make_uint2(lo[p], hi[p]);
    }
    if (qT == nullptr) return;                       // uniform across the block

    uint32_t tlo[8], thi[8];
    transpose8x8(lo, hi, tlo, thi);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int crow = cg * 8 + j;                 // row of the transposed tile
        *reinterpret_cast<uint2*>(tileT + crow * 128 + ((rg ^ cg) << 3)) = make_uint2(tlo[j], thi[j]);
    }
    __syncthreads();
    const int crow = t >> 1, h = t & 1;
    const int64_t c = bj * 128 + crow;
    if (c < C) {
        uint32_t wv[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int phys = (8 * h + i) ^ (crow >> 3);
            const uint2 u = *reinterpret_cast<const uint2*>(tileT + crow * 128 + (phys << 3));
            wv[2 * i] = u.x;
            wv[2 * i + 1] = u.y;
        }
        uint8_t* dst = qT + c * ldqT + bi * 128 + 64 * h;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<uint4*>(dst + 16 * i) = make_uint4(wv[4 * i], wv[4 * i + 1], wv[4 * i + 2], wv[4 * i + 3]);
    }
}

// ---------------------------------------------------------------------
// Token-axis 1x128 groups, written transposed; optional row-wise copy.
// Tile: 128 rows (one token group) x 128 columns, thread layout as in
// k_quant_weight.  In grouped mode the row tiles follow the experts'
// segments and block row-index y enumerates them expert by expert.
// ---------------------------------------------------------------------
struct SegInfo {
    int64_t a, b, pos;   // rows [a, b) of this tile; first output column pos
};

__device__ __forceinline__ SegInfo find_segment_tile(const int32_t* offsets, int64_t E, int64_t tile) {
    // Linear scan over experts: tile index -> (expert, group within expert).
    int64_t acc = 0, P = 0;
    for (int64_t e = 0; e < E; ++e) {
        const int64_t a = offsets[e], b = offsets[e + 1];
        const int64_t n = b - a;
        const int64_t tiles = (n + 127) / 128;
        if (tile < acc + tiles) {
            const int64_t g = tile - acc;
            const int64_t ra = a + 128 * g;
            return SegInfo{ra, ra + 128 < b ? ra + 128 : b, P + 128 * g};
        }
        acc += tiles;
        P += 128 * tiles;
    }
    return SegInfo{0, 0, -1};
}

template <typename T, bool ROWS>
__global__ __launch_bounds__(256) void k_quant_cols(const T* __restrict__ x, int64_t rows, int64_t cols, int64_t ldx,
                                                    const int32_t* __restrict__ offsets, int64_t E,
                                                    uint8_t* __restrict__ qT, int64_t ldqT,
                                                    float* __restrict__ sT, int64_t ldsT,
                                                    uint8_t* __restrict__ q, int64_t ldq,
                                                    float* __restrict__ s, int64_t lds) {
    __shared__ float colmax[4][128];
    __shared__ double colR[128];
    __shared__ double rowR[128];
    __shared__ int64_t seg[3];
    __shared__ __attribute__((aligned(16))) uint8_t tileT[128 * 128];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int rg = t >> 4, cg = t & 15;

    int64_t a, b, pos;
    if (offsets == nullptr) {
        a = (int64_t)blockIdx.x * 128;
        b = a + 128 < rows ? a + 128 : rows;
        pos = a;
    } else {
        if (t == 0) {
            const SegInfo si = find_segment_tile(offsets, E, blockIdx.x);
            seg[0] = si.a; seg[1] = si.b; seg[2] = si.pos;
        }
        __syncthreads();
        a = seg[0]; b = seg[1]; pos = seg[2];
        if (pos < 0) return;                         // beyond the last tile: whole block
    }
    const int64_t cb = (int64_t)blockIdx.y * 128;
    const int64_t c0 = cb + cg * 8;
    const int cvalid = clamp_valid(cols - c0);

    float v[8][8];
#pragma unroll
    for (int p = 0; p < 8; ++p) {
        const int64_t r = a + rg * 8 + p;
        const bool in = r < b;
        load8(x + (in ? r : 0) * ldx + c0, in ? cvalid : 0, v[p]);
    }

    // column maxima: 8 rows in-thread, 4 row-slices in-wave, 4 waves via LDS
    float cm[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float m = 0.0f;
#pragma unroll
        for (int p = 0; p < 8; ++p) m = fmaxf(m, fabsf(v[p][j]));
        m = fmaxf(m, __shfl_xor(m, 16));
        m = fmaxf(m, __shfl_xor(m, 32));
        cm[j] = m;
    }
    if (lane < 16) {
#pragma unroll
        for (int j = 0; j < 8; ++j) colmax[wave][cg * 8 + j] = cm[j];
    }
    if (ROWS) {
        float rm[8];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            float m = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[p][j]));
            rm[p] = max16(m);
        }
        if (cg < 8) {
            float m = rm[0];
#pragma unroll
            for (int p = 1; p < 8; ++p) m = cg == p ? rm[p] : m;
            const float S = group_scale(m);
            rowR[rg * 8 + cg] = quotient_recip(S);
            const int64_t r = a + rg * 8 + cg;
            if (r < b) s[r * lds + blockIdx.y] = S;
        }
    }
    __syncthreads();
    if (t < 128) {
        const float m = fmaxf(fmaxf(colmax[0][t], colmax[1][t]), fmaxf(colmax[2][t], colmax[3][t]));
        const float S = group_scale(m);
        colR[t] = quotient_recip(S);
        if (cb + t < cols) sT[(cb + t) * ldsT + pos / 128] = S;
    }
    __syncthreads();

    if (ROWS) {
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            const double R = rowR[rg * 8 + p];
            const int64_t r = a + rg * 8 + p;
            const uint32_t lo = encode4(v[p][0], v[p][1], v[p][2], v[p][3], R);
            const uint32_t hi = encode4(v[p][4], v[p][5], v[p][6], v[p][7], R);
            if (r < b) *reinterpret_cast<uint2*>(q + r * ldq + c0) = make_uint2(lo, hi);
        }
    }

    uint32_t lo[8], hi[8];
    {
        double Rc[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) Rc[j] = colR[cg * 8 + j];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
            lo[p] = e4m3_pack4(exact_quotient(v[p][0], Rc[0]), exact_quotient(v[p][1], Rc[1]),
                               exact_quotient(v[p][2], Rc[2]), exact_quotient(v[p][3], Rc[3]));
            hi[p] = e4m3_pack4(exact_quotient(v[p][4], Rc[4]), exact_quotient(v[p][5], Rc[5]),
                               exact_quotient(v[p][6], Rc[6]), exact_quotient(v[p][7], Rc[7]));
        }
    }
    uint32_t tlo[8], thi[8];
    transpose8x8(lo, hi, tlo, thi);
#pragma unroll
    for (int j = 0; j < 8; ++j)
        *reinterpret_cast<uint2*>(tileT + (cg * 8 + j) * 128 + ((rg ^ cg) << 3)) = make_uint2(tlo[j], thi[j]);
    __syncthreads();
    const int crow = t >> 1, h = t & 1;
    const int64_t c = cb + crow;
    if (c < cols) {
        uint32_t wv[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int phys = (8 * h + i) ^ (crow >> 3);
            const uint2 u = *reinterpret_cast<const uint2*>(tileT + crow * 128 + (phys << 3));
            wv[2 * i] = u.x;
            wv[2 * i + 1] = u.y;
        }
        uint8_t* dst = qT + c * ldqT + pos + 64 * h;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *reinterpret_cast<uint4*>(dst + 16 * i) = make_uint4(wv[4 * i], wv[4 * i + 1], wv[4 * i + 2], wv[4 * i + 3]);
    }
}

// ---------------------------------------------------------------------
// Elementwise access to the codec (exhaustive device checks).
// ---------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_encode(const float* __restrict__ x, const float* __restrict__ s,
                                                int64_t n, uint8_t* __restrict__ out) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
        const double R = s ? quotient_recip(s[i]) : 1.0;
        out[i] = (uint8_t)e4m3_encode(exact_quotient(x[i], R));
    }
}

// ---------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------
hipError_t launch_quant_rows(const void* x, bool in_bf16, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t* q, int64_t ldq, float* s, int64_t lds, hipStream_t st) {
    const int64_t gpr = (cols + 127) / 128;
    const int64_t total = rows * gpr;
    if (total == 0) return hipSuccess;
    if (total > 0xFFFFFFF0ll) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((total + 15) / 16));
    if (in_bf16)
        k_quant_rows<uint16_t><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(x), cols, ldx, q, ldq, s, lds,
                                                      (uint32_t)gpr, (uint32_t)total);
    else
        k_quant_rows<float><<<grid, 256, 0, st>>>(static_cast<const float*>(x), cols, ldx, q, ldq, s, lds,
                                                   (uint32_t)gpr, (uint32_t)total);
    return hipGetLastError();
}

hipError_t launch_quant_weight(const void* w, bool in_bf16, int64_t D, int64_t C, int64_t ldw,
                               uint8_t* q, int64_t ldq, float* s, int64_t lds,
                               uint8_t* qT, int64_t ldqT, hipStream_t st) {
    if (D == 0 || C == 0) return hipSuccess;
    const int64_t bd = (D + 127) / 128, bc = (C + 127) / 128;
    if (bd > 0x7FFFFFFF || bc > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)bd, (unsigned)bc);
    if (in_bf16)
        k_quant_weight<uint16_t><<<grid, 256, 0, st>>>(static_cast<const uint16_t*>(w), D, C, ldw, q, ldq, s, lds, qT, ldqT);
    else
        k_quant_weight<float><<<grid, 256, 0, st>>>(static_cast<const float*>(w), D, C, ldw, q, ldq, s, lds, qT, ldqT);
    return hipGetLastError();
}

hipError_t launch_quant_cols(const void* x, bool in_bf16, int64_t rows, int64_t cols, int64_t ldx,
                             const int32_t* offsets, int64_t E,
                             uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT,
                             uint8_t* q, int64_t ldq, float* s, int64_t lds, hipStream_t st) {
    if (rows == 0 || cols == 0) return hipSuccess;
    const int64_t row_tiles = (rows + 127) / 128 + (offsets ? E : 0);
    const int64_t col_tiles = (cols + 127) / 128;
    if (row_tiles > 0x7FFFFFFF || col_tiles > 65535) return hipErrorInvalidValue;
    const dim3 grid((unsigned)row_tiles, (unsigned)col_tiles);
    const bool rowsout = q != nullptr;
    if (in_bf16) {
        auto xp = static_cast<const uint16_t*>(x);
        if (rowsout)
            k_quant_cols<uint16_t, true><<<grid, 256, 0, st>>>(xp, rows, cols, ldx, offsets, E, qT, ldqT, sT, ldsT, q, ldq, s, lds);
        else
            k_quant_cols<uint16_t, false><<<grid, 256, 0, st>>>(xp, rows, cols, ldx, offsets, E, qT, ldqT, sT, ldsT, q, ldq, s, lds);
    } else {
        auto xp = static_cast<const float*>(x);
        if (rowsout)
            k_quant_cols<float, true><<<grid, 256, 0, st>>>(xp, rows, cols, ldx, offsets, E, qT, ldqT, sT, ldsT, q, ldq, s, lds);
        else
            k_quant_cols<float, false><<<grid, 256, 0, st>>>(xp, rows, cols, ldx, offsets, E, qT, ldqT, sT, ldsT, q, ldq, s, lds);
    }
    return hipGetLastError();
}

hipError_t launch_encode(const float* x, const float* s, int64_t n, uint8_t* out, hipStream_t st) {
    if (n == 0) return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    k_encode<<<dim3((unsigned)blocks), 256, 0, st>>>(x, s, n, out);
    return hipGetLastError();
}

}  // namespace fp8blk
