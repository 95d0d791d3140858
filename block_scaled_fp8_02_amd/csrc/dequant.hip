// dequant.hip -- the dequantized-backward mode: bf16 GEMMs on bf16
// dequantizations of the exact FP8 operands the forward pass produced.
//
// The Miles MXFP8/NVFP4 blog offers it as a selectable backward mode: the
// backward GEMMs run in bf16, their FP8-side operands are the forward's
// codes dequantized to bf16 (W for DGrad, X for WGrad), dY stays bf16, and
// no column-wise FP8 copy is needed.  Here:
//
//   k_dequant_bf16   codes + scales -> bf16(fl32(E4M3(q) * s)); the scale
//                    layouts are the 1x128 row groups, the 128x128 weight
//                    blocks and the MX 1x32 E8M0 groups
//   lt_gemm          the plain bf16 GEMM (fp32 accumulation) through
//                    hipBLASLt, the library GEMM for bf16 operands
#include <hip/hip_runtime.h>
#include <hipblaslt/hipblaslt.h>

#include <map>
#include <mutex>
#include <tuple>

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

// ---------------------------------------------------------------------
// hipBLASLt bf16 GEMM, column-major: D[m x n] = op(A)[m x k] op(B)[k x n]
// (+ beta D).  One handle per device, created on first use; the chosen
// algorithm is cached per problem (no workspace: only algorithms that need
// none are considered, so no memory is allocated per call).
// ---------------------------------------------------------------------
namespace {

struct LtKey {
    int dev, ta, tb, out_f32, beta;
    int64_t m, n, k, lda, ldb, ldd;
    bool operator<(const LtKey& o) const {
        return std::tie(dev, ta, tb, out_f32, beta, m, n, k, lda, ldb, ldd) <
               std::tie(o.dev, o.ta, o.tb, o.out_f32, o.beta, o.m, o.n, o.k, o.lda, o.ldb, o.ldd);
    }
};

std::mutex g_lt_mutex;
hipblasLtHandle_t g_lt_handle[64] = {};
std::map<LtKey, hipblasLtMatmulAlgo_t> g_lt_algos;

}  // namespace

hipError_t lt_gemm(bool ta, bool tb, int64_t m, int64_t n, int64_t k,
                   const uint16_t* A, int64_t lda, const uint16_t* B, int64_t ldb,
                   void* D, int64_t ldd, bool out_f32, float beta, hipStream_t st, int* lt_status) {
    *lt_status = 0;
    if (m == 0 || n == 0) return hipSuccess;
    int dev = 0;
    hipError_t he = hipGetDevice(&dev);
    if (he != hipSuccess) return he;
    if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;

    hipblasLtMatmulDesc_t desc = nullptr;
    hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
    hipblasStatus_t s = HIPBLAS_STATUS_SUCCESS;
    const hipblasOperation_t opa = ta ? HIPBLAS_OP_T : HIPBLAS_OP_N, opb = tb ? HIPBLAS_OP_T : HIPBLAS_OP_N;
    const hipDataType dt = out_f32 ? HIP_R_32F : HIP_R_16BF;
    hipblasLtMatmulAlgo_t algo;
    std::lock_guard<std::mutex> lock(g_lt_mutex);
    if (g_lt_handle[dev] == nullptr) {
        s = hipblasLtCreate(&g_lt_handle[dev]);
        if (s != HIPBLAS_STATUS_SUCCESS) { *lt_status = (int)s; g_lt_handle[dev] = nullptr; return hipErrorUnknown; }
    }
    hipblasLtHandle_t h = g_lt_handle[dev];
#define FP8B_LT(call)                                  \
    do {                                               \
        s = (call);                                    \
        if (s != HIPBLAS_STATUS_SUCCESS) goto done;    \
    } while (0)
    {
        FP8B_LT(hipblasLtMatmulDescCreate(&desc, HIPBLAS_COMPUTE_32F, HIP_R_32F));
        FP8B_LT(hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSA, &opa, sizeof(opa)));
        FP8B_LT(hipblasLtMatmulDescSetAttribute(desc, HIPBLASLT_MATMUL_DESC_TRANSB, &opb, sizeof(opb)));
        FP8B_LT(hipblasLtMatrixLayoutCreate(&la, HIP_R_16BF, ta ? k : m, ta ? m : k, lda));
        FP8B_LT(hipblasLtMatrixLayoutCreate(&lb, HIP_R_16BF, tb ? n : k, tb ? k : n, ldb));
        FP8B_LT(hipblasLtMatrixLayoutCreate(&ld, dt, m, n, ldd));
        const LtKey key{dev, (int)ta, (int)tb, (int)out_f32, beta != 0.0f, m, n, k, lda, ldb, ldd};
        auto it = g_lt_algos.find(key);
        if (it != g_lt_algos.end()) {
            algo = it->second;
        } else {
            hipblasLtMatmulPreference_t pref = nullptr;
            FP8B_LT(hipblasLtMatmulPreferenceCreate(&pref));
            uint64_t wsz = 0;
            s = hipblasLtMatmulPreferenceSetAttribute(pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsz, sizeof(wsz));
            hipblasLtMatmulHeuristicResult_t res[1];
            int found = 0;
            if (s == HIPBLAS_STATUS_SUCCESS)
                s = hipblasLtMatmulAlgoGetHeuristic(h, desc, la, lb, ld, ld, pref, 1, res, &found);
            hipblasLtMatmulPreferenceDestroy(pref);
            if (s != HIPBLAS_STATUS_SUCCESS) goto done;
            if (found < 1) { s = HIPBLAS_STATUS_NOT_SUPPORTED; goto done; }
            algo = res[0].algo;
            g_lt_algos.emplace(key, algo);
        }
        const float alpha = 1.0f;
        FP8B_LT(hipblasLtMatmul(h, desc, &alpha, A, la, B, lb, &beta, D, ld, D, ld, &algo, nullptr, 0, st));
    }
done:
#undef FP8B_LT
    if (ld) hipblasLtMatrixLayoutDestroy(ld);
    if (lb) hipblasLtMatrixLayoutDestroy(lb);
    if (la) hipblasLtMatrixLayoutDestroy(la);
    if (desc) hipblasLtMatmulDescDestroy(desc);
    if (s != HIPBLAS_STATUS_SUCCESS) { *lt_status = (int)s; return hipErrorUnknown; }
    return hipGetLastError();
}

}  // namespace fp8blk
