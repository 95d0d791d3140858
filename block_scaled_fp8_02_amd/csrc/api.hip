// api.hip -- the C ABI declared in include/fp8blk.h: host-side argument
// validation, then one stream-ordered launch per call.  No allocation, no
// synchronization, no exceptions across the boundary.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "../../include/fp8blk.h"
#include "kernels.hpp"

using namespace fp8blk;

namespace {

thread_local int g_last_hip_error = 0;

inline int64_t rup128(int64_t n) { return (n + 127) / 128 * 128; }
inline int64_t cdiv(int64_t n, int64_t m) { return (n + m - 1) / m; }
inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
inline int esize(int dt) { return dt == FP8B_BF16 ? 2 : 4; }
inline bool dtype_ok(int dt) { return dt == FP8B_F32 || dt == FP8B_BF16; }

inline int hip_status(hipError_t e) {
    if (e == hipSuccess) return FP8B_OK;
    g_last_hip_error = (int)e;
    return FP8B_EHIP;
}

// Input tensor: rows x cols of dtype dt with row stride ld (elements).
int check_input(const void* x, int dt, int64_t rows, int64_t cols, int64_t ld) {
    if (!dtype_ok(dt)) return FP8B_EINVAL;
    if (rows < 0 || cols < 0 || ld < cols) return FP8B_ESHAPE;
    if (rows == 0 || cols == 0) return FP8B_OK;          // nothing is read
    if (x == nullptr) return FP8B_EINVAL;
    if (!aligned(x, 16) || (ld * esize(dt)) % 16 != 0) return FP8B_EALIGN;
    return FP8B_OK;
}

// FP8 code buffer: rows x ld bytes holding a padded contraction axis K.
int check_codes(const void* q, int64_t rows, int64_t K, int64_t ld) {
    if (rows < 0 || K < 0 || ld < rup128(K)) return FP8B_ESHAPE;
    if (rows == 0 || K == 0) return FP8B_OK;             // nothing is touched
    if (q == nullptr) return FP8B_EINVAL;
    if (!aligned(q, 16) || ld % 16 != 0) return FP8B_EALIGN;
    return FP8B_OK;
}

int check_scales(const void* s, int64_t rows, int64_t ncols, int64_t ld, uintptr_t align) {
    if (rows < 0 || ncols < 0 || ld < ncols) return FP8B_ESHAPE;
    if (rows == 0 || ncols == 0) return FP8B_OK;
    if (s == nullptr) return FP8B_EINVAL;
    if (!aligned(s, align)) return FP8B_EALIGN;
    return FP8B_OK;
}

int check_output(const void* o, int dt, int64_t rows, int64_t cols, int64_t ld, int beta) {
    if (!dtype_ok(dt)) return FP8B_EINVAL;
    if (beta != 0 && beta != 1) return FP8B_EINVAL;
    if (beta == 1 && dt != FP8B_F32) return FP8B_EUNSUPPORTED;
    if (rows < 0 || cols < 0 || ld < cols) return FP8B_ESHAPE;
    if (rows == 0 || cols == 0) return FP8B_OK;
    if (o == nullptr) return FP8B_EINVAL;
    if (!aligned(o, 16) || (ld * esize(dt)) % 16 != 0) return FP8B_EALIGN;
    return FP8B_OK;
}

// Largest leading dimensions the GEMMs take: FP8 code rows in bytes, scale
// rows in elements.
constexpr int64_t kMaxGemmCodeLd = (int64_t)1 << 24;
constexpr int64_t kMaxGemmScaleLd = (int64_t)1 << 22;

#define FP8B_TRY(expr)                  \
    do {                                \
        const int _st = (expr);         \
        if (_st != FP8B_OK) return _st; \
    } while (0)

// Shared validation of the dense GEMM family.
//   op 0 FProp: a = xq [N x C], b = wq [D x C], sb = ws [D/128 x C/128]  -> [N x D]
//   op 1 DGrad: a = gq [N x D], b = wqT [C x D], sb = ws [D/128 x C/128] -> [N x C]
//   op 2 WGrad: a = gqT [D x N], b = xqT [C x N], per-row scales          -> [D x C]
//   op 3..5: the MX forms of the same, with E8M0 scales per 32.
int validate_gemm(int op, const void* a, int64_t lda, const void* sa, int64_t ldsa,
                  const void* b, int64_t ldb, const void* sb, int64_t ldsb,
                  const void* out, int odt, int64_t ldo, int beta, int64_t N, int64_t D, int64_t C) {
    if (op < 0 || op > 5) return FP8B_EINVAL;
    if (N < 0 || D < 0 || C < 0) return FP8B_ESHAPE;
    const bool mx = op >= 3;
    const int base = op % 3;
    int64_t M, Nn, K;
    if (base == 0) { M = N; Nn = D; K = C; }
    else if (base == 1) { M = N; Nn = C; K = D; }
    else { M = D; Nn = C; K = N; }
    if (base != 2 && beta != 0) return FP8B_EINVAL;
    // the kernels address a tile's 256 rows (codes and scale rows) with
    // 32-bit offsets from a per-tile base
    if (lda > kMaxGemmCodeLd || ldb > kMaxGemmCodeLd || ldsa > kMaxGemmScaleLd || ldsb > kMaxGemmScaleLd)
        return FP8B_EUNSUPPORTED;
    FP8B_TRY(check_codes(a, M, K, lda));
    FP8B_TRY(check_codes(b, Nn, K, ldb));
    const int64_t kb = mx ? rup128(K) / 32 : cdiv(K, 128);
    const uintptr_t sal = 4;                             // fp32 words, or E8M0 bytes read as words
    FP8B_TRY(check_scales(sa, M, kb, ldsa, sal));
    if (!mx && base != 2) {
        // 128x128 weight scale grid [ceil(D/128) x ceil(C/128)], row stride ldsb
        FP8B_TRY(check_scales(sb, cdiv(D, 128), cdiv(C, 128), ldsb, 4));
    } else {
        FP8B_TRY(check_scales(sb, Nn, kb, ldsb, sal));
    }
    // E8M0 rows are fetched four bytes (one K block) at a time
    if (mx && K > 0 && ((M > 0 && ldsa % 4 != 0) || (Nn > 0 && ldsb % 4 != 0))) return FP8B_EALIGN;
    FP8B_TRY(check_output(out, odt, M, Nn, ldo, beta));
    return FP8B_OK;
}

GemmArgs dense_args(int op, const void* a, int64_t lda, const void* sa, int64_t ldsa,
                    const void* b, int64_t ldb, const void* sb, int64_t ldsb,
                    void* out, int odt, int64_t ldo, int beta, int64_t N, int64_t D, int64_t C) {
    GemmArgs g{};
    const int base = op % 3;
    g.P = static_cast<const uint8_t*>(a); g.ldp = lda;
    g.sP = sa; g.ldsp = ldsa;
    g.Q = static_cast<const uint8_t*>(b); g.ldq = ldb;
    g.sQ = sb;
    g.O = out; g.ldo = ldo; g.out_f32 = odt == FP8B_F32; g.beta = beta;
    if (base == 0) { g.M = N; g.Nn = D; g.K = C; }
    else if (base == 1) { g.M = N; g.Nn = C; g.K = D; }
    else { g.M = D; g.Nn = C; g.K = N; }
    if (op >= 3) {
        g.scale_mode = SCALE_MX; g.sq_rs = ldsb; g.sq_ks = 1;
    } else if (base == 0) {
        g.scale_mode = SCALE_Q_BLOCK; g.sq_rs = ldsb; g.sq_ks = 1;       // ws[d/128][kb]
    } else if (base == 1) {
        g.scale_mode = SCALE_Q_BLOCK; g.sq_rs = 1; g.sq_ks = ldsb;       // ws[kb][c/128]
    } else {
        g.scale_mode = SCALE_Q_ROW; g.sq_rs = ldsb; g.sq_ks = 1;         // xsT[c][kb]
    }
    g.group_mode = GROUP_NONE;
    return g;
}

int check_offsets(const int32_t* offsets, int64_t E) {
    if (E < 1 || E > 65535) return FP8B_ESHAPE;
    if (offsets == nullptr) return FP8B_EINVAL;
    if (!aligned(offsets, 4)) return FP8B_EALIGN;
    return FP8B_OK;
}

}  // namespace

extern "C" {

int fp8b_abi_version(void) { return 4; }

const char* fp8b_status_string(int status) {
    switch (status) {
        case FP8B_OK: return "ok";
        case FP8B_EINVAL: return "invalid argument (null pointer or bad enum)";
        case FP8B_ESHAPE: return "invalid shape or leading dimension";
        case FP8B_EALIGN: return "pointer or leading dimension not 16-byte aligned";
        case FP8B_EUNSUPPORTED: return "unsupported combination";
        case FP8B_EHIP: return "HIP launch error";
        default: return "unknown status";
    }
}

int fp8b_last_hip_error(void) { return g_last_hip_error; }

// E8M0 bytes of power-of-two groups (nullable): rows x round_up(K,128)/32,
// written as 4-byte words, so the pointer and the row stride are multiples of 4.
static int check_e8(const uint8_t* e, int64_t rows, int64_t K, int64_t ld) {
    if (e == nullptr) return FP8B_OK;
    FP8B_TRY(check_scales(e, rows, rup128(K) / 32, ld, 4));
    if (rows > 0 && K > 0 && ld % 4 != 0) return FP8B_EALIGN;
    return FP8B_OK;
}

static int quantize_act_impl(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t* q, int64_t ldq, float* s, int64_t lds,
                             bool pow2, uint8_t* e8, int64_t lde, void* stream) {
    FP8B_TRY(check_input(x, xt, rows, cols, ldx));
    FP8B_TRY(check_codes(q, rows, cols, ldq));
    FP8B_TRY(check_scales(s, rows, cdiv(cols, 128), lds, 4));
    FP8B_TRY(check_e8(e8, rows, cols, lde));
    return hip_status(launch_quant_rows(x, xt == FP8B_BF16, rows, cols, ldx, q, ldq, s, lds, pow2, e8, lde,
                                        static_cast<hipStream_t>(stream)));
}

int fp8_quantize_act_1x128(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                           uint8_t* q, int64_t ldq, float* s, int64_t lds, void* stream) {
    return quantize_act_impl(x, xt, rows, cols, ldx, q, ldq, s, lds, false, nullptr, 0, stream);
}

int fp8_quantize_act_1x128_pow2(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                                uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                uint8_t* e8, int64_t lde, void* stream) {
    return quantize_act_impl(x, xt, rows, cols, ldx, q, ldq, s, lds, true, e8, lde, stream);
}

static int quantize_weight_impl(const void* w, int wt, int64_t D, int64_t C, int64_t ldw,
                                uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                uint8_t* qT, int64_t ldqT,
                                bool pow2, uint8_t* e8, int64_t lde, uint8_t* e8T, int64_t ldeT, void* stream) {
    FP8B_TRY(check_input(w, wt, D, C, ldw));
    FP8B_TRY(check_codes(q, D, C, ldq));
    FP8B_TRY(check_scales(s, cdiv(D, 128), cdiv(C, 128), lds, 4));
    if (qT != nullptr) FP8B_TRY(check_codes(qT, C, D, ldqT));
    FP8B_TRY(check_e8(e8, D, C, lde));
    FP8B_TRY(check_e8(e8T, C, D, ldeT));
    return hip_status(launch_quant_weight(w, wt == FP8B_BF16, D, C, ldw, q, ldq, s, lds, qT, ldqT,
                                          pow2, e8, lde, e8T, ldeT, static_cast<hipStream_t>(stream)));
}

int fp8_quantize_weight_128x128(const void* w, int wt, int64_t D, int64_t C, int64_t ldw,
                                uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                uint8_t* qT, int64_t ldqT, void* stream) {
    return quantize_weight_impl(w, wt, D, C, ldw, q, ldq, s, lds, qT, ldqT, false, nullptr, 0, nullptr, 0, stream);
}

int fp8_quantize_weight_128x128_pow2(const void* w, int wt, int64_t D, int64_t C, int64_t ldw,
                                     uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                     uint8_t* qT, int64_t ldqT,
                                     uint8_t* e8, int64_t lde, uint8_t* e8T, int64_t ldeT, void* stream) {
    return quantize_weight_impl(w, wt, D, C, ldw, q, ldq, s, lds, qT, ldqT, true, e8, lde, e8T, ldeT, stream);
}

static int quantize_transposed_impl(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                                    const int32_t* offsets, int64_t E,
                                    uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT,
                                    uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                    bool pow2, uint8_t* e8T, int64_t ldeT, uint8_t* e8, int64_t lde,
                                    void* stream) {
    FP8B_TRY(check_input(x, xt, rows, cols, ldx));
    const int64_t P = offsets ? rows + 128 * E : rows;    // upper bound of the padded token axis
    FP8B_TRY(check_codes(qT, cols, P, ldqT));
    FP8B_TRY(check_scales(sT, cols, cdiv(P, 128), ldsT, 4));
    if ((q == nullptr) != (s == nullptr)) return FP8B_EINVAL;
    if (q != nullptr) {
        FP8B_TRY(check_codes(q, rows, cols, ldq));
        FP8B_TRY(check_scales(s, rows, cdiv(cols, 128), lds, 4));
    }
    if (e8 != nullptr && q == nullptr) return FP8B_EINVAL;
    FP8B_TRY(check_e8(e8T, cols, P, ldeT));
    FP8B_TRY(check_e8(e8, rows, cols, lde));
    return hip_status(launch_quant_cols(x, xt == FP8B_BF16, rows, cols, ldx, offsets, E, qT, ldqT, sT, ldsT,
                                        q, ldq, s, lds, pow2, e8T, ldeT, e8, lde, static_cast<hipStream_t>(stream)));
}

int fp8_quantize_transposed(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                            uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT,
                            uint8_t* q, int64_t ldq, float* s, int64_t lds, void* stream) {
    return quantize_transposed_impl(x, xt, rows, cols, ldx, nullptr, 0, qT, ldqT, sT, ldsT, q, ldq, s, lds,
                                    false, nullptr, 0, nullptr, 0, stream);
}

int fp8_quantize_transposed_pow2(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                                 uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT, uint8_t* e8T, int64_t ldeT,
                                 uint8_t* q, int64_t ldq, float* s, int64_t lds, uint8_t* e8, int64_t lde,
                                 void* stream) {
    return quantize_transposed_impl(x, xt, rows, cols, ldx, nullptr, 0, qT, ldqT, sT, ldsT, q, ldq, s, lds,
                                    true, e8T, ldeT, e8, lde, stream);
}

int fp8_quantize_transposed_grouped(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                                    const int32_t* offsets, int64_t E,
                                    uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT,
                                    uint8_t* q, int64_t ldq, float* s, int64_t lds, void* stream) {
    FP8B_TRY(check_offsets(offsets, E));
    return quantize_transposed_impl(x, xt, rows, cols, ldx, offsets, E, qT, ldqT, sT, ldsT, q, ldq, s, lds,
                                    false, nullptr, 0, nullptr, 0, stream);
}

static int requantize_impl(const uint8_t* q, int64_t ldq, const float* s, int64_t lds,
                           int64_t rows, int64_t cols, const int32_t* offsets, int64_t E,
                           uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT, void* stream) {
    FP8B_TRY(check_codes(q, rows, cols, ldq));
    FP8B_TRY(check_scales(s, rows, cdiv(cols, 128), lds, 4));
    const int64_t P = offsets ? rows + 128 * E : rows;
    FP8B_TRY(check_codes(qT, cols, P, ldqT));
    FP8B_TRY(check_scales(sT, cols, cdiv(P, 128), ldsT, 4));
    return hip_status(launch_requant_cols(q, ldq, s, lds, rows, cols, offsets, E, qT, ldqT, sT, ldsT,
                                          static_cast<hipStream_t>(stream)));
}

int fp8_requantize_transposed(const uint8_t* q, int64_t ldq, const float* s, int64_t lds,
                              int64_t rows, int64_t cols,
                              uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT, void* stream) {
    return requantize_impl(q, ldq, s, lds, rows, cols, nullptr, 0, qT, ldqT, sT, ldsT, stream);
}

int fp8_requantize_transposed_grouped(const uint8_t* q, int64_t ldq, const float* s, int64_t lds,
                                      int64_t rows, int64_t cols, const int32_t* offsets, int64_t E,
                                      uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT, void* stream) {
    FP8B_TRY(check_offsets(offsets, E));
    return requantize_impl(q, ldq, s, lds, rows, cols, offsets, E, qT, ldqT, sT, ldsT, stream);
}

int fp8_rmsnorm_quantize_1x128(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                               const void* w, int wt, float eps,
                               uint8_t* q, int64_t ldq, float* s, int64_t lds,
                               float* rstd, uint16_t* y, int64_t ldy, void* stream) {
    FP8B_TRY(check_input(x, xt, rows, cols, ldx));
    if (!(eps > 0.0f) || !(eps < __builtin_inff())) return FP8B_EINVAL;
    FP8B_TRY(check_input(w, wt, cols > 0 && rows > 0 ? 1 : 0, cols, (cols + 7) / 8 * 8));   // one row: only w's alignment
    FP8B_TRY(check_codes(q, rows, cols, ldq));
    FP8B_TRY(check_scales(s, rows, cdiv(cols, 128), lds, 4));
    if (y != nullptr) FP8B_TRY(check_input(y, FP8B_BF16, rows, cols, ldy));
    return hip_status(launch_rmsnorm_quant(x, xt == FP8B_BF16, rows, cols, ldx, w, wt == FP8B_BF16, eps,
                                           q, ldq, s, lds, rstd, y, ldy, static_cast<hipStream_t>(stream)));
}

int fp8_silu_mul_quantize_1x128(const uint16_t* gate, int64_t ldg, const uint16_t* up, int64_t ldu,
                                int64_t rows, int64_t cols, uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                uint16_t* a, int64_t lda, void* stream) {
    FP8B_TRY(check_input(gate, FP8B_BF16, rows, cols, ldg));
    FP8B_TRY(check_input(up, FP8B_BF16, rows, cols, ldu));
    FP8B_TRY(check_codes(q, rows, cols, ldq));
    FP8B_TRY(check_scales(s, rows, cdiv(cols, 128), lds, 4));
    if (a != nullptr) FP8B_TRY(check_input(a, FP8B_BF16, rows, cols, lda));
    return hip_status(launch_silu_mul_quant(gate, ldg, up, ldu, rows, cols, q, ldq, s, lds, a, lda,
                                            static_cast<hipStream_t>(stream)));
}

static int check_fp8_operand(const uint8_t* q, int64_t ldq, const void* sc, int64_t lds, int kind,
                             int64_t rows, int64_t cols) {
    if (kind < FP8B_SCALE_ROWS_1X128 || kind > FP8B_SCALE_MX_1X32) return FP8B_EINVAL;
    FP8B_TRY(check_codes(q, rows, cols, ldq));
    if (kind == FP8B_SCALE_ROWS_1X128) return check_scales(sc, rows, cdiv(cols, 128), lds, 4);
    if (kind == FP8B_SCALE_BLOCKS_128X128) return check_scales(sc, cdiv(rows, 128), cdiv(cols, 128), lds, 4);
    return check_scales(sc, rows, rup128(cols) / 32, lds, 1);
}

// Largest row stride (elements) of a bf16 GEMM operand: a tile's 256 rows
// are addressed with 32-bit byte offsets, as in the FP8 GEMMs.
constexpr int64_t kMaxBf16Ld = (int64_t)1 << 23;

// Source kind of launch_transpose_bf16 for an FP8 operand of scale kind `kind`.
static inline int transpose_src(int kind) { return kind + 1; }

int fp8_dequantize_bf16(const uint8_t* q, int64_t ldq, const void* sc, int64_t lds, int kind,
                        int64_t rows, int64_t cols, uint16_t* out, int64_t ldo, void* stream) {
    FP8B_TRY(check_fp8_operand(q, ldq, sc, lds, kind, rows, cols));
    FP8B_TRY(check_input(out, FP8B_BF16, rows, cols, ldo));
    return hip_status(launch_dequant_bf16(q, ldq, sc, lds, kind, rows, cols, out, ldo,
                                          static_cast<hipStream_t>(stream)));
}

int fp8_dequant_gemm_dgrad(const uint16_t* dy, int64_t lddy, const uint8_t* wq, int64_t ldwq,
                           const void* ws, int64_t ldws, int wkind, int64_t N, int64_t D, int64_t C,
                           uint16_t* dx, int64_t lddx, uint16_t* work, int64_t ldwork, void* stream) {
    if (wkind != FP8B_SCALE_BLOCKS_128X128 && wkind != FP8B_SCALE_MX_1X32) return FP8B_EINVAL;
    FP8B_TRY(check_input(dy, FP8B_BF16, N, D, lddy));
    FP8B_TRY(check_fp8_operand(wq, ldwq, ws, ldws, wkind, D, C));
    FP8B_TRY(check_input(work, FP8B_BF16, C, D, ldwork));          // receives W^T [C x D]
    FP8B_TRY(check_output(dx, FP8B_BF16, N, C, lddx, 0));
    if (lddy > kMaxBf16Ld || ldwork > kMaxBf16Ld) return FP8B_EUNSUPPORTED;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (N == 0 || C == 0) return FP8B_OK;
    if (D == 0) return hip_status(launch_zero_2d(dx, lddx * 2, C * 2, N, st));
    FP8B_TRY(hip_status(launch_transpose_bf16(transpose_src(wkind), wq, ldwq, ws, ldws, D, C, work, ldwork, st)));
    Bf16GemmArgs g{};
    g.P = dy; g.ldp = lddy;
    g.Q = work; g.ldq = ldwork;
    g.O = dx; g.ldo = lddx; g.out_f32 = false; g.beta = 0;
    g.M = N; g.Nn = C; g.K = D;
    return hip_status(launch_gemm_bf16(g, st));
}

int fp8_dequant_gemm_wgrad(const uint16_t* dy, int64_t lddy, const uint8_t* xq, int64_t ldxq,
                           const void* xs, int64_t ldxs, int xkind, int64_t N, int64_t D, int64_t C,
                           void* dw, int dwt, int64_t lddw, int beta,
                           uint16_t* work, int64_t ldwork, void* stream) {
    if (xkind != FP8B_SCALE_ROWS_1X128 && xkind != FP8B_SCALE_MX_1X32) return FP8B_EINVAL;
    FP8B_TRY(check_input(dy, FP8B_BF16, N, D, lddy));
    FP8B_TRY(check_fp8_operand(xq, ldxq, xs, ldxs, xkind, N, C));
    FP8B_TRY(check_input(work, FP8B_BF16, C + D, N, ldwork));      // X^T [C x N], then dY^T [D x N]
    FP8B_TRY(check_output(dw, dwt, D, C, lddw, beta));
    if (lddy > kMaxBf16Ld || ldwork > kMaxBf16Ld) return FP8B_EUNSUPPORTED;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (D == 0 || C == 0) return FP8B_OK;
    if (N == 0) {
        if (beta) return FP8B_OK;
        return hip_status(launch_zero_2d(dw, lddw * esize(dwt), C * esize(dwt), D, st));
    }
    uint16_t* xT = work;
    uint16_t* gT = work + C * ldwork;
    FP8B_TRY(hip_status(launch_transpose_bf16(transpose_src(xkind), xq, ldxq, xs, ldxs, N, C, xT, ldwork, st)));
    FP8B_TRY(hip_status(launch_transpose_bf16(0, dy, lddy, nullptr, 0, N, D, gT, ldwork, st)));
    Bf16GemmArgs g{};
    g.P = gT; g.ldp = ldwork;
    g.Q = xT; g.ldq = ldwork;
    g.O = dw; g.ldo = lddw; g.out_f32 = dwt == FP8B_F32; g.beta = beta;
    g.M = D; g.Nn = C; g.K = N;
    return hip_status(launch_gemm_bf16(g, st));
}

int fp8b_validate_gemm(int op, const void* a, int64_t lda, const void* sa, int64_t ldsa,
                       const void* b, int64_t ldb, const void* sb, int64_t ldsb,
                       const void* out, int out_dtype, int64_t ldo, int beta,
                       int64_t N, int64_t D, int64_t C) {
    return validate_gemm(op, a, lda, sa, ldsa, b, ldb, sb, ldsb, out, out_dtype, ldo, beta, N, D, C);
}

static int gemm_dense(int op, const void* a, int64_t lda, const void* sa, int64_t ldsa,
                      const void* b, int64_t ldb, const void* sb, int64_t ldsb,
                      void* out, int odt, int64_t ldo, int beta, int64_t N, int64_t D, int64_t C,
                      void* stream) {
    FP8B_TRY(validate_gemm(op, a, lda, sa, ldsa, b, ldb, sb, ldsb, out, odt, ldo, beta, N, D, C));
    const GemmArgs g = dense_args(op, a, lda, sa, ldsa, b, ldb, sb, ldsb, out, odt, ldo, beta, N, D, C);
    return hip_status(launch_gemm(g, static_cast<hipStream_t>(stream)));
}

// K split of a few-row DGrad (op 1 or 4): number of K ranges (1: none) and
// K blocks per range.  About 256 blocks (one per compute unit of an MI355X)
// over the 128-column output tiles, at least 8 K blocks per range.  The plan
// is a fixed function of (N, D, C), never of the device it runs on, so the
// partition, and with it every output bit, is the same on any device or
// compute-unit partition.
constexpr int64_t kSplitBlocks = 256;

static void dgrad_split_plan(int64_t N, int64_t D, int64_t C, int64_t* S, int64_t* kbs) {
    *S = 1;
    *kbs = 0;
    if (N <= 0 || N > 64 || C <= 0 || D <= 0) return;
    const int64_t KB = cdiv(D, 128), nbj = cdiv(C, 128), cus = kSplitBlocks;
    if (KB < 16 || 2 * nbj > cus) return;
    int64_t s = cus / nbj;
    if (s > KB / 8) s = KB / 8;
    if (s < 2) return;
    const int64_t k = cdiv(KB, s);
    *S = cdiv(KB, k);
    *kbs = k;
}

// fp32 partial rows of the split: row stride rounded up to 4 floats (16 bytes).
static inline int64_t split_ld(int64_t C) { return (C + 3) / 4 * 4; }

static int64_t dgrad_split_bytes(int64_t N, int64_t D, int64_t C) {
    int64_t S, kbs;
    dgrad_split_plan(N, D, C, &S, &kbs);
    return S < 2 ? 0 : S * N * split_ld(C) * 4;
}

static int gemm_dgrad_split(int op, const void* a, int64_t lda, const void* sa, int64_t ldsa,
                     const void* b, int64_t ldb, const void* sb, int64_t ldsb,
                     void* out, int odt, int64_t ldo, int64_t N, int64_t D, int64_t C,
                     void* work, int64_t work_bytes, void* stream) {
    FP8B_TRY(validate_gemm(op, a, lda, sa, ldsa, b, ldb, sb, ldsb, out, odt, ldo, 0, N, D, C));
    const hipStream_t st = static_cast<hipStream_t>(stream);
    const GemmArgs g = dense_args(op, a, lda, sa, ldsa, b, ldb, sb, ldsb, out, odt, ldo, 0, N, D, C);
    int64_t S, kbs;
    dgrad_split_plan(N, D, C, &S, &kbs);
    if (S < 2) return hip_status(launch_gemm(g, st));
    if (work == nullptr) return FP8B_EINVAL;
    if (!aligned(work, 16)) return FP8B_EALIGN;
    const int64_t ldp = split_ld(C);
    if (work_bytes < S * N * ldp * 4) return FP8B_ESHAPE;
    GemmArgs p = g;
    p.O = work; p.out_f32 = true; p.ldo = ldp; p.beta = 0;
    p.o_estride = N * ldp;
    p.ksplit = S; p.kb_split = kbs;
    FP8B_TRY(hip_status(launch_gemm(p, st)));
    return hip_status(launch_split_sum(static_cast<const float*>(work), S, N * ldp, ldp, N, C,
                                       out, odt == FP8B_F32, ldo, st));
}

int fp8_gemm_fprop(const uint8_t* xq, int64_t ldxq, const float* xs, int64_t ldxs,
                   const uint8_t* wq, int64_t ldwq, const float* ws, int64_t ldws,
                   void* y, int yt, int64_t ldy, int64_t N, int64_t D, int64_t C, void* stream) {
    return gemm_dense(0, xq, ldxq, xs, ldxs, wq, ldwq, ws, ldws, y, yt, ldy, 0, N, D, C, stream);
}

int fp8_gemm_dgrad(const uint8_t* gq, int64_t ldgq, const float* gs, int64_t ldgs,
                   const uint8_t* wqT, int64_t ldwqT, const float* ws, int64_t ldws,
                   void* dx, int dxt, int64_t lddx, int64_t N, int64_t D, int64_t C, void* stream) {
    return gemm_dense(1, gq, ldgq, gs, ldgs, wqT, ldwqT, ws, ldws, dx, dxt, lddx, 0, N, D, C, stream);
}

int64_t fp8_gemm_dgrad_split_bytes(int64_t N, int64_t D, int64_t C) { return dgrad_split_bytes(N, D, C); }

int fp8_gemm_dgrad_split(const uint8_t* gq, int64_t ldgq, const float* gs, int64_t ldgs,
                         const uint8_t* wqT, int64_t ldwqT, const float* ws, int64_t ldws,
                         void* dx, int dxt, int64_t lddx, int64_t N, int64_t D, int64_t C,
                         void* work, int64_t work_bytes, void* stream) {
    return gemm_dgrad_split(1, gq, ldgq, gs, ldgs, wqT, ldwqT, ws, ldws, dx, dxt, lddx, N, D, C,
                            work, work_bytes, stream);
}

}  // extern "C"

// Scratch of fp8_gemm_dgrad_split_noalloc: the largest fp32 partial-sum
// workspace the split plan can ask for (256 blocks of 64 rows x 128 columns).
// Each device holds its own copy from the library's load until the process
// ends.  In host code `scratch` is only the host-side stand-in of the device
// array: its device address is looked up per device (scratch_for_stream)
// and only that address is passed to kernels.
constexpr int64_t kNoAllocScratchBytes = 256 * 64 * 128 * 4;
static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxScratchDevices];                   // per device, once looked up

// Device address of `scratch` on the device that `stream` belongs to.  The
// first call for a device makes that device current, asks the runtime for
// the symbol's address there and restores the caller's device; later calls
// reuse the address.  Allocates nothing.
int scratch_for_stream(void* stream, void** out) {
    int dev = 0;
    hipError_t e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev);
    if (e != hipSuccess) return hip_status(e);
    if (dev < 0 || dev >= kMaxScratchDevices) return FP8B_EUNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_addr[dev] == nullptr) {
        int cur = 0;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return hip_status(e);
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_status(e);
        void* p = nullptr;
        const hipError_t eg = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev && (e = hipSetDevice(cur)) != hipSuccess) return hip_status(e);
        if (eg != hipSuccess) return hip_status(eg);
        if (p == nullptr) return hip_status(hipErrorInvalidSymbol);
        g_scratch_addr[dev] = p;
    }
    *out = g_scratch_addr[dev];
    return FP8B_OK;
}

}  // namespace

extern "C" {

int fp8_gemm_dgrad_split_noalloc(const uint8_t* gq, int64_t ldgq, const float* gs, int64_t ldgs,
                                 const uint8_t* wqT, int64_t ldwqT, const float* ws, int64_t ldws,
                                 void* dx, int dxt, int64_t lddx, int64_t N, int64_t D, int64_t C,
                                 void* stream) {
    FP8B_TRY(validate_gemm(1, gq, ldgq, gs, ldgs, wqT, ldwqT, ws, ldws, dx, dxt, lddx, 0, N, D, C));
    const int64_t need = dgrad_split_bytes(N, D, C);
    if (need > kNoAllocScratchBytes) return FP8B_EUNSUPPORTED;
    void* work = nullptr;
    if (need > 0) FP8B_TRY(scratch_for_stream(stream, &work));
    return gemm_dgrad_split(1, gq, ldgq, gs, ldgs, wqT, ldwqT, ws, ldws, dx, dxt, lddx, N, D, C,
                            work, kNoAllocScratchBytes, stream);
}

int fp8_gemm_wgrad(const uint8_t* gqT, int64_t ldgqT, const float* gsT, int64_t ldgsT,
                   const uint8_t* xqT, int64_t ldxqT, const float* xsT, int64_t ldxsT,
                   void* dw, int dwt, int64_t lddw, int beta,
                   int64_t N, int64_t D, int64_t C, void* stream) {
    return gemm_dense(2, gqT, ldgqT, gsT, ldgsT, xqT, ldxqT, xsT, ldxsT, dw, dwt, lddw, beta, N, D, C, stream);
}

// Grouped FProp / DGrad: per-expert weights; rows follow the offsets.
static int gemm_grouped_rows(int op, const uint8_t* a, int64_t lda, const float* sa, int64_t ldsa,
                             const uint8_t* b, int64_t ldb, int64_t b_estride,
                             const float* sb, int64_t ldsb, int64_t sb_estride,
                             void* out, int odt, int64_t ldo,
                             const int32_t* offsets, int64_t E, int64_t N, int64_t D, int64_t C, void* stream) {
    FP8B_TRY(check_offsets(offsets, E));
    if (b_estride < 0 || sb_estride < 0) return FP8B_ESHAPE;
    // per-expert validation with the expert's D x C weight
    FP8B_TRY(validate_gemm(op, a, lda, sa, ldsa, b, ldb, sb, ldsb, out, odt, ldo, 0, N, D, C));
    if (b_estride % 16 != 0) return FP8B_EALIGN;
    GemmArgs g = dense_args(op, a, lda, sa, ldsa, b, ldb, sb, ldsb, out, odt, ldo, 0, N, D, C);
    g.group_mode = GROUP_ROWS;
    g.offsets = offsets; g.E = E;
    g.q_estride = b_estride; g.sq_estride = sb_estride;
    return hip_status(launch_gemm(g, static_cast<hipStream_t>(stream)));
}

int fp8_gemm_fprop_grouped(const uint8_t* xq, int64_t ldxq, const float* xs, int64_t ldxs,
                           const uint8_t* wq, int64_t ldwq, int64_t wq_estride,
                           const float* ws, int64_t ldws, int64_t ws_estride,
                           void* y, int yt, int64_t ldy,
                           const int32_t* offsets, int64_t E, int64_t N, int64_t D, int64_t C,
                           void* stream) {
    return gemm_grouped_rows(0, xq, ldxq, xs, ldxs, wq, ldwq, wq_estride, ws, ldws, ws_estride, y, yt, ldy,
                             offsets, E, N, D, C, stream);
}

int fp8_gemm_dgrad_grouped(const uint8_t* gq, int64_t ldgq, const float* gs, int64_t ldgs,
                           const uint8_t* wqT, int64_t ldwqT, int64_t wqT_estride,
                           const float* ws, int64_t ldws, int64_t ws_estride,
                           void* dx, int dxt, int64_t lddx,
                           const int32_t* offsets, int64_t E, int64_t N, int64_t D, int64_t C,
                           void* stream) {
    return gemm_grouped_rows(1, gq, ldgq, gs, ldgs, wqT, ldwqT, wqT_estride, ws, ldws, ws_estride, dx, dxt, lddx,
                             offsets, E, N, D, C, stream);
}

int fp8_gemm_wgrad_grouped(const uint8_t* gqT, int64_t ldgqT, const float* gsT, int64_t ldgsT,
                           const uint8_t* xqT, int64_t ldxqT, const float* xsT, int64_t ldxsT,
                           void* dw, int dwt, int64_t lddw, int64_t dw_estride, int beta,
                           const int32_t* offsets, int64_t E, int64_t N, int64_t D, int64_t C,
                           void* stream) {
    FP8B_TRY(check_offsets(offsets, E));
    // the padded token axis is bounded by N + 128*E
    const int64_t P = N + 128 * E;
    FP8B_TRY(validate_gemm(2, gqT, ldgqT, gsT, ldgsT, xqT, ldxqT, xsT, ldxsT, dw, dwt, lddw, beta, P, D, C));
    if (dw_estride < (int64_t)D * lddw) return FP8B_ESHAPE;
    if ((dw_estride * esize(dwt)) % 16 != 0) return FP8B_EALIGN;
    GemmArgs g = dense_args(2, gqT, ldgqT, gsT, ldgsT, xqT, ldxqT, xsT, ldxsT, dw, dwt, lddw, beta, P, D, C);
    g.group_mode = GROUP_K;
    g.offsets = offsets; g.E = E;
    g.o_estride = dw_estride;
    return hip_status(launch_gemm(g, static_cast<hipStream_t>(stream)));
}

int fp8_mx_quantize_1x32(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                         uint8_t* q, int64_t ldq, uint8_t* e, int64_t lde,
                         uint8_t* qT, int64_t ldqT, uint8_t* eT, int64_t ldeT, void* stream) {
    FP8B_TRY(check_input(x, xt, rows, cols, ldx));
    if ((q == nullptr) != (e == nullptr) || (qT == nullptr) != (eT == nullptr)) return FP8B_EINVAL;
    if (q == nullptr && qT == nullptr) return FP8B_EINVAL;
    if (q != nullptr) {
        FP8B_TRY(check_codes(q, rows, cols, ldq));
        FP8B_TRY(check_scales(e, rows, rup128(cols) / 32, lde, 1));
    }
    if (qT != nullptr) {
        FP8B_TRY(check_codes(qT, cols, rows, ldqT));
        FP8B_TRY(check_scales(eT, cols, rup128(rows) / 32, ldeT, 1));
    }
    return hip_status(launch_mx_quant(x, xt == FP8B_BF16, rows, cols, ldx, q, ldq, e, lde, qT, ldqT, eT, ldeT,
                                      static_cast<hipStream_t>(stream)));
}

int fp8_mx_gemm_fprop(const uint8_t* xq, int64_t ldxq, const uint8_t* xe, int64_t ldxe,
                      const uint8_t* wq, int64_t ldwq, const uint8_t* we, int64_t ldwe,
                      void* y, int yt, int64_t ldy, int64_t N, int64_t D, int64_t C, void* stream) {
    return gemm_dense(3, xq, ldxq, xe, ldxe, wq, ldwq, we, ldwe, y, yt, ldy, 0, N, D, C, stream);
}

int fp8_mx_gemm_dgrad(const uint8_t* gq, int64_t ldgq, const uint8_t* ge, int64_t ldge,
                      const uint8_t* wqT, int64_t ldwqT, const uint8_t* weT, int64_t ldweT,
                      void* dx, int dxt, int64_t lddx, int64_t N, int64_t D, int64_t C, void* stream) {
    return gemm_dense(4, gq, ldgq, ge, ldge, wqT, ldwqT, weT, ldweT, dx, dxt, lddx, 0, N, D, C, stream);
}

int fp8_mx_gemm_dgrad_split(const uint8_t* gq, int64_t ldgq, const uint8_t* ge, int64_t ldge,
                            const uint8_t* wqT, int64_t ldwqT, const uint8_t* weT, int64_t ldweT,
                            void* dx, int dxt, int64_t lddx, int64_t N, int64_t D, int64_t C,
                            void* work, int64_t work_bytes, void* stream) {
    return gemm_dgrad_split(4, gq, ldgq, ge, ldge, wqT, ldwqT, weT, ldweT, dx, dxt, lddx, N, D, C,
                            work, work_bytes, stream);
}

int fp8_mx_gemm_wgrad(const uint8_t* gqT, int64_t ldgqT, const uint8_t* geT, int64_t ldgeT,
                      const uint8_t* xqT, int64_t ldxqT, const uint8_t* xeT, int64_t ldxeT,
                      void* dw, int dwt, int64_t lddw, int beta,
                      int64_t N, int64_t D, int64_t C, void* stream) {
    return gemm_dense(5, gqT, ldgqT, geT, ldgeT, xqT, ldxqT, xeT, ldxeT, dw, dwt, lddw, beta, N, D, C, stream);
}

int64_t fp8_decode_pack_bytes(int64_t D, int64_t C, int part) {
    if (D < 0 || C < 0) return 0;
    const int64_t rows = cdiv(D, 16) * 16;
    if (part == 0) return rows * rup128(C);
    if (part == 1) return rows * cdiv(C, 128) * 4;
    return 0;
}

int fp8_pack_decode_weight(const uint8_t* wq, int64_t ldwq, const uint8_t* we, int64_t ldwe,
                           int64_t D, int64_t C, uint8_t* wp, uint32_t* wep, void* stream) {
    if (D < 0 || C < 0) return FP8B_ESHAPE;
    FP8B_TRY(check_codes(wq, D, C, ldwq));
    if (we != nullptr) {
        FP8B_TRY(check_scales(we, D, rup128(C) / 32, ldwe, 4));
        if (ldwe % 4 != 0) return FP8B_EALIGN;
    }
    if (D == 0 || C == 0) return FP8B_OK;
    if (wp == nullptr || (we != nullptr && wep == nullptr)) return FP8B_EINVAL;
    if (!aligned(wp, 16) || (we != nullptr && !aligned(wep, 4))) return FP8B_EALIGN;
    return hip_status(launch_pack_decode(wq, ldwq, we, ldwe, D, cdiv(C, 128), wp, we != nullptr ? wep : nullptr,
                                         static_cast<hipStream_t>(stream)));
}

// Decode FProp on a packed weight (op 0 block-scaled, op 3 MX).  The packed
// codes are validated as a code operand with rows of round_up(C,128) bytes,
// the packed MX words as scale rows of round_up(C,128)/32 bytes.
static int gemm_decode(int op, const uint8_t* xq, int64_t ldxq, const void* xs, int64_t ldxs,
                       const uint8_t* wp, const void* ws, int64_t ldws,
                       void* y, int yt, int64_t ldy, int64_t N, int64_t D, int64_t C, void* stream) {
    if (N > 64) return FP8B_EUNSUPPORTED;
    const int64_t ldp = rup128(C), ldsw = op == 3 ? rup128(C) / 32 : ldws;
    FP8B_TRY(validate_gemm(op, xq, ldxq, xs, ldxs, wp, ldp, ws, ldsw, y, yt, ldy, 0, N, D, C));
    const hipStream_t st = static_cast<hipStream_t>(stream);
    if (N == 0 || D == 0) return FP8B_OK;
    if (C == 0) return hip_status(launch_zero_2d(y, ldy * esize(yt), D * esize(yt), N, st));
    const GemmArgs g = dense_args(op, xq, ldxq, xs, ldxs, wp, ldp, ws, ldsw, y, yt, ldy, 0, N, D, C);
    return hip_status(launch_gemm_decode_packed(g, st));
}

int fp8_gemm_fprop_decode(const uint8_t* xq, int64_t ldxq, const float* xs, int64_t ldxs,
                          const uint8_t* wp, const float* ws, int64_t ldws,
                          void* y, int yt, int64_t ldy, int64_t N, int64_t D, int64_t C, void* stream) {
    return gemm_decode(0, xq, ldxq, xs, ldxs, wp, ws, ldws, y, yt, ldy, N, D, C, stream);
}

int fp8_mx_gemm_fprop_decode(const uint8_t* xq, int64_t ldxq, const uint8_t* xe, int64_t ldxe,
                             const uint8_t* wp, const uint32_t* wep,
                             void* y, int yt, int64_t ldy, int64_t N, int64_t D, int64_t C, void* stream) {
    return gemm_decode(3, xq, ldxq, xe, ldxe, wp, wep, 0, y, yt, ldy, N, D, C, stream);
}

int fp8b_mfma_peak(int kind, int64_t blocks, int64_t iters, uint32_t seed, float* out, double* flops,
                   void* stream) {
    if (kind < 0 || kind > 3) return FP8B_EINVAL;
    if (blocks < 0 || iters < 0 || blocks > 0x7FFFFFFF) return FP8B_ESHAPE;
    if (blocks > 0 && iters > 0 && out == nullptr) return FP8B_EINVAL;
    if (flops != nullptr) *flops = (double)blocks * 4.0 * 16.0 * (double)iters * (kind == 1 ? 16384.0 : 65536.0);
    return hip_status(launch_mfma_peak(kind, blocks, iters, seed, out, static_cast<hipStream_t>(stream)));
}

int fp8b_e4m3_encode(const float* x, const float* s, int64_t n, uint8_t* out, void* stream) {
    if (n < 0) return FP8B_ESHAPE;
    if (n > 0 && (x == nullptr || out == nullptr)) return FP8B_EINVAL;
    return hip_status(launch_encode(x, s, n, out, static_cast<hipStream_t>(stream)));
}

int fp8b_bf16_round(const float* x, int64_t n, uint16_t* out, void* stream) {
    if (n < 0) return FP8B_ESHAPE;
    if (n > 0 && (x == nullptr || out == nullptr)) return FP8B_EINVAL;
    return hip_status(launch_bf16_round(x, n, out, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
