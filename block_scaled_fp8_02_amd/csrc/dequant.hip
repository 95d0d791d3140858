// dequant.hip -- bf16 dequantization of FP8 operands, for the
// dequantized-backward mode (the Miles MXFP8/NVFP4 blog's backward-mode
// section: the backward GEMMs run in bf16 on bf16 dequantizations of the
// exact FP8 operands the forward pass produced, W for DGrad and X for WGrad,
// with dY in bf16 and no column-wise FP8 copy).
//
//   k_dequant_bf16   codes + scales -> bf16(fl32(E4M3(q) * s)); the scale
//                    layouts are the 1x128 row groups, the 128x128 weight
//                    blocks and the MX 1x32 E8M0 groups
//   k_zero_2d        the output of an empty contraction
// The GEMMs themselves and the transposing dequantization that feeds them
// are in bf16gemm.hip.
#include <hip/hip_runtime.h>

#include "device_common.hpp"
#include "kernels.hpp"

namespace fp8blk {

// One thread per 8 consecutive codes of a row; grid-stride over rows x
// ceil(cols/8) chunks.  KIND: 0 = 1x128 row groups (fp32 s[row][c/128]),
// 1 = 128x128 blocks (fp32 s[row/128][c/128]), 2 = MX 1x32 (E8M0
// e[row][c/32], scale 2^(e-127)).  8 consecutive columns never straddle a
// group of any kind (8 divides 32 and 128).
template <int KIND>
__global__ __launch_bounds__(256) void k_dequant_bf16(const uint8_t* __restrict__ q, int64_t ldq,
                                                      const void* __restrict__ sp, int64_t lds,
                                                      int64_t rows, int64_t cols,
                                                      uint16_t* __restrict__ out, int64_t ldo) {
    const int64_t cpr = (cols + 7) / 8;
    const int64_t total = rows * cpr;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t r = i / cpr;
        const int64_t c0 = (i - r * cpr) * 8;
        const int valid = clamp_valid(cols - c0);
        float sc;
        if (KIND == 2) {
            const int e = static_cast<const uint8_t*>(sp)[r * lds + c0 / 32];
            sc = __builtin_ldexpf(1.0f, e - 127);
        } else {
            const int64_t sr = KIND == 1 ? r / 128 : r;
            sc = static_cast<const float*>(sp)[sr * lds + c0 / 128];
        }
        // the code row is padded to a multiple of 128, so 8 bytes are in bounds
        const uint2 w = *reinterpret_cast<const uint2*>(q + r * ldq + c0);
        const auto a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, false);
        const auto b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.x, true);
        const auto c = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, false);
        const auto d = __builtin_amdgcn_cvt_pk_f32_fp8((int)w.y, true);
        const float v[8] = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
        uint32_t h[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) h[k] = f32_to_bf16(v[k] * sc);
        uint16_t* o = out + r * ldo + c0;
        if (valid == 8) {
            *reinterpret_cast<uint4*>(o) = make_uint4(h[0] | (h[1] << 16), h[2] | (h[3] << 16),
                                                      h[4] | (h[5] << 16), h[6] | (h[7] << 16));
        } else {
            for (int k = 0; k < valid; ++k) o[k] = (uint16_t)h[k];
        }
    }
}

hipError_t launch_dequant_bf16(const uint8_t* q, int64_t ldq, const void* s, int64_t lds, int kind,
                               int64_t rows, int64_t cols, uint16_t* out, int64_t ldo, hipStream_t st) {
    const int64_t total = rows * ((cols + 7) / 8);
    if (total == 0) return hipSuccess;
    int64_t blocks = (total + 255) / 256;
    const int64_t cap = 8 * (int64_t)device_cu_count();
    if (blocks > cap) blocks = cap;
    const dim3 grid((unsigned)blocks);
    if (kind == 0) k_dequant_bf16<0><<<grid, 256, 0, st>>>(q, ldq, s, lds, rows, cols, out, ldo);
    else if (kind == 1) k_dequant_bf16<1><<<grid, 256, 0, st>>>(q, ldq, s, lds, rows, cols, out, ldo);
    else k_dequant_bf16<2><<<grid, 256, 0, st>>>(q, ldq, s, lds, rows, cols, out, ldo);
    return hipGetLastError();
}

// Zero rows x row_bytes bytes with row stride ld_bytes (a GEMM output whose
// contraction is empty).  A kernel rather than a memset, so that a caller
// capturing the stream into a graph records no memset node.
__global__ __launch_bounds__(256) void k_zero_2d(uint8_t* __restrict__ p, int64_t ld_bytes, int64_t row_bytes,
                                                 int64_t rows) {
    const int64_t total = rows * row_bytes;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
        const int64_t r = i / row_bytes;
        p[r * ld_bytes + (i - r * row_bytes)] = 0;
    }
}

hipError_t launch_zero_2d(void* p, int64_t ld_bytes, int64_t row_bytes, int64_t rows, hipStream_t st) {
    const int64_t total = rows * row_bytes;
    if (total == 0) return hipSuccess;
    int64_t blocks = (total + 255) / 256;
    const int64_t cap = 8 * (int64_t)device_cu_count();
    if (blocks > cap) blocks = cap;
    k_zero_2d<<<dim3((unsigned)blocks), 256, 0, st>>>(static_cast<uint8_t*>(p), ld_bytes, row_bytes, rows);
    return hipGetLastError();
}

}  // namespace fp8blk
