/*
 * fp8blk.h -- C ABI of the block-scaled FP8 linear-layer library for
 * AMD Instinct MI355X (gfx950).
 *
 * The library implements the unified FP8 precision flow for linear layers
 * described on the Jet-RL pages:
 *   - quantizer Q: S = max|X| / 448, Xhat = X / S rounded to the nearest
 *     OCP E4M3 value (Jet-RL notes, section 2.1, definition of Q);
 *   - activations and gradients quantized per 1x128 group along the
 *     contraction axis, weights per 128x128 block (Jet-RL notes, section
 *     4.2; summary page, "Weight quantization" and "Activation and gradient
 *     quantization");
 *   - FProp Y = X W^T, DGrad dX = dY W, WGrad dW = dY^T X as block-scaled
 *     FP8 GEMMs with fp32 accumulation (Jet-RL notes, section 2.2 and 4.2);
 *   - an MXFP8 variant with 1x32 E4M3 blocks sharing an E8M0 power-of-two
 *     scale rounded up so nothing clips (Miles MXFP8/NVFP4 blog, MXFP8
 *     paragraphs).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All pointers are DEVICE pointers (except where stated) owned by the
 *   caller.  The library allocates and frees no device memory and calls no
 *   other GPU library; it keeps no state between calls apart from lazily
 *   loaded code objects and, for fp8_gemm_dgrad_split_noalloc, the device
 *   address of its scratch array on each device.
 * - Every call is asynchronous on `stream` (a hipStream_t passed as void*;
 *   NULL is the default stream).  Buffers must stay valid until the stream
 *   reaches the operation.
 * - Layouts are row-major with explicit leading dimensions counted in
 *   ELEMENTS of the buffer's type (bytes for FP8/E8M0 buffers).
 * - FP8 code buffers pad the contraction axis to a multiple of 128: the
 *   quantizers write 0x00 into the padding, and the GEMMs read the whole
 *   padded length.  The pad therefore contributes exactly zero.
 * - Return value: 0 (FP8B_OK) on success.  Argument errors are detected on
 *   the host before anything is launched and return a nonzero status; a
 *   failed launch returns FP8B_EHIP with the HIP error code retrievable by
 *   fp8b_last_hip_error() (thread-local).  Nothing aborts the process and
 *   no C++ exception crosses this boundary.
 * - Inputs must be finite; this is not checked on the device.
 * - Results are deterministic and the same on every device.  Every FProp
 *   and WGrad output row depends only on its own input row: the reduction
 *   order of an output element does not depend on the number of rows in
 *   the call (unified rollout/training forward).  DGrad with at most 64 rows
 *   and a long contraction runs the K-split order of fp8_gemm_dgrad_split
 *   (fixed by N, D and C alone); DGrad rows are otherwise row-local too.
 */
#ifndef FP8BLK_H
#define FP8BLK_H

#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define FP8B_API __attribute__((visibility("default")))
#else
#define FP8B_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum fp8b_status_code {
    FP8B_OK = 0,
    FP8B_EINVAL = 1,       /* null pointer where one is required, bad enum value */
    FP8B_ESHAPE = 2,       /* dimension < 0, leading dimension too small, bad group count */
    FP8B_EALIGN = 3,       /* pointer or leading dimension not 16-byte aligned */
    FP8B_EUNSUPPORTED = 4, /* valid request the library does not implement */
    FP8B_EHIP = 5          /* HIP launch error; see fp8b_last_hip_error() */
};

enum fp8b_dtype {
    FP8B_F32 = 0,          /* IEEE binary32 */
    FP8B_BF16 = 1          /* bfloat16 (upper half of binary32), stored as uint16 */
};

enum fp8b_scale_kind {     /* scale layout of an FP8 operand (codes rows x ldq, K padded to 128) */
    FP8B_SCALE_ROWS_1X128 = 0,     /* fp32 s[row][k/128] (fp8_quantize_act_1x128) */
    FP8B_SCALE_BLOCKS_128X128 = 1, /* fp32 s[row/128][k/128] (fp8_quantize_weight_128x128) */
    FP8B_SCALE_MX_1X32 = 2         /* E8M0 byte e[row][k/32], scale 2^(e-127), row stride >= round_up(K,128)/32 */
};

/* Version of this ABI (incremented on any incompatible change). */
FP8B_API int fp8b_abi_version(void);

/* Static, human-readable text for a status code. */
FP8B_API const char* fp8b_status_string(int status);

/* HIP error code of the last FP8B_EHIP returned on the calling thread. */
FP8B_API int fp8b_last_hip_error(void);

/* ------------------------------------------------------------------ */
/* Quantizers                                                          */
/* ------------------------------------------------------------------ */

/* 1x128 per-group quantization along the contiguous axis
 * (Jet-RL summary, "Activation and gradient quantization: 1x128 per-group";
 * used for X in FProp and for dY along D in DGrad).
 *   x  : rows x cols of dtype xt, row stride ldx >= cols.
 *   q  : rows x ldq bytes, ldq >= round_up(cols,128), ldq % 16 == 0;
 *        columns [cols, round_up(cols,128)) are written 0x00.
 *   s  : rows x lds fp32, lds >= ceil(cols/128); s[r][g] = max|x[r][128g..]|/448.
 * Codes are E4M3(fl32(x / s)), nearest-even, saturating at +-448; a group
 * with s == 0 stores the signed zero of each input. */
FP8B_API int fp8_quantize_act_1x128(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                           uint8_t* q, int64_t ldq, float* s, int64_t lds, void* stream);

/* 128x128 per-block weight quantization (Jet-RL summary, "Weight
 * quantization: 128x128 per-block"; redone after every optimizer step).
 *   w  : D x C of dtype wt, row stride ldw >= C.
 *   q  : D x ldq bytes, ldq >= round_up(C,128), ldq % 16 == 0; pad 0x00.
 *   s  : ceil(D/128) x lds fp32, lds >= ceil(C/128).
 *   qT : optional (NULL to skip): the same codes transposed, C x ldqT bytes,
 *        ldqT >= round_up(D,128), ldqT % 16 == 0; columns [D, round_up(D,128))
 *        written 0x00.  DGrad reads W through this copy with the same scale
 *        grid read transposed (the block scales are symmetric in D and C).
 * Several weights of equal C may be stacked along D (e.g. the E experts of a
 * MoE layer as one (E*D) x C matrix) when D is a multiple of 128. */
FP8B_API int fp8_quantize_weight_128x128(const void* w, int wt, int64_t D, int64_t C, int64_t ldw,
                                uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                uint8_t* qT, int64_t ldqT, void* stream);

/* 1x128 groups along the token (row) axis, written transposed: the
 * WGrad operands dY^T and X^T (Jet-RL notes, section 4.2: WGrad groups its
 * operands along the token axis).  Reads x once and can also emit the
 * row-wise 1x128 quantization of the same tensor from the same read.
 *   x   : rows x cols of dtype xt, row stride ldx.
 *   qT  : cols x ldqT bytes, ldqT >= round_up(rows,128), ldqT % 16 == 0;
 *         qT[c][r] is the code of x[r][c]; pad positions 0x00.
 *   sT  : cols x ldsT fp32, ldsT >= ceil(rows/128).
 *   q, s: optional (both NULL or both set) output of fp8_quantize_act_1x128,
 *        with ldq/lds as there. */
FP8B_API int fp8_quantize_transposed(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                            uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT,
                            uint8_t* q, int64_t ldq, float* s, int64_t lds, void* stream);

/* Token-axis quantization, grouped (MoE).  offsets: DEVICE int32[E+1], non-decreasing, offsets[0]
 * = 0, offsets[E] = rows; rows [offsets[e], offsets[e+1]) belong to expert
 * e and token groups restart at every offsets[e].  Expert e occupies qT
 * columns [P_e, P_e + round_up(n_e,128)) with n_e = offsets[e+1]-offsets[e]
 * and P_e = sum_{e'<e} round_up(n_e',128), and sT columns [P_e/128,
 * P_e/128 + ceil(n_e/128)).  The caller sizes ldqT >= round_up(rows +
 * 128*E, 128) (a bound of P_E) and ldsT >= ldqT/128.  The optional row-wise
 * output does not depend on the grouping.  offsets are read on the device
 * and are not validated there: they must describe a partition of the rows. */
FP8B_API int fp8_quantize_transposed_grouped(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                                    const int32_t* offsets, int64_t E,
                                    uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT,
                                    uint8_t* q, int64_t ldq, float* s, int64_t lds, void* stream);

/* Fused producers of the 1x128 activation quantizer.  The Jet-RL notes
 * (section 3.4, the quantization kernels and the per-block walk-through of
 * the attention and MLP blocks) fuse the activation quantizer into the
 * operator that produces the activation, so the bf16 activation is not
 * written to HBM and read back.  Both calls produce exactly the codes and
 * scales that fp8_quantize_act_1x128 gives for the bf16 activation of the
 * unfused operator, with that operator's arithmetic defined as follows (the
 * pages leave it open).  Outputs q, s as fp8_quantize_act_1x128. */

/* RMSNorm + 1x128.  x: rows x ldx of dtype xt; w: cols weights of dtype wt
 * (16-byte aligned); eps > 0 and finite.  Per row: ss = sum of x_j^2, exact
 * and rounded once to binary64; r = fl32(1 / sqrt(ss / cols + eps)), each
 * step a binary64 operation; y_j = bf16(fl32(fl32(x_j * r) * w_j)) (round to
 * nearest even); then the 1x128 quantizer on y.  ss is the exact sum rounded
 * once whenever the row's nonzero magnitudes lie within a factor 2^30 of
 * each other (double-double sum); otherwise it is within 2^-100 relative.  Optional outputs (NULL to skip): rstd
 * [rows] fp32 = r (what the backward pass needs), y rows x ldy bf16 (16-byte
 * aligned, ldy * 2 a multiple of 16).  The caller keeps |w| * sqrt(cols)
 * below the bf16 maximum.  Errors: FP8B_EINVAL (NULL, bad dtype, eps <= 0
 * or not finite), FP8B_ESHAPE, FP8B_EALIGN, FP8B_EHIP. */
FP8B_API int fp8_rmsnorm_quantize_1x128(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                               const void* w, int wt, float eps,
                               uint8_t* q, int64_t ldq, float* s, int64_t lds,
                               float* rstd, uint16_t* y, int64_t ldy, void* stream);

/* SiLU(gate) * up + 1x128 (the gated MLP's down-projection input).  gate and
 * up: rows x cols bf16 with strides ldg, ldu (for a fused gate+up GEMM
 * output H [rows x 2I]: gate = H, up = H + I, both strides 2I).  Per
 * element: s = bf16(silu(g)), silu(g) = g / (1 + e^-g) rounded once from its
 * exact value; a = bf16(fl32(s * u)); then the 1x128 quantizer on a.
 * Optional output a (NULL to skip): rows x lda bf16, the activation the
 * backward pass of the down projection may keep.  Errors as above. */
FP8B_API int fp8_silu_mul_quantize_1x128(const uint16_t* gate, int64_t ldg, const uint16_t* up, int64_t ldu,
                                int64_t rows, int64_t cols, uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                uint16_t* a, int64_t lda, void* stream);

/* Token-axis requantization of saved FP8 activations (the flow the Jet-RL
 * pages attribute to DeepSeek-V3, which keeps only the FP8 copy of X and
 * forms WGrad's X^T from it).  Input: the output of fp8_quantize_act_1x128,
 * codes q (rows x ldq bytes,
 * 1x128 groups along the contiguous axis, cols real columns; bytes past
 * cols are ignored) and scales s (rows x lds fp32).  Each element is
 * dequantized as fl32(E4M3(q) * s) (one binary32 multiply; the pages leave
 * the precision open) and the result is quantized exactly as by
 * fp8_quantize_transposed: qT cols x ldqT, sT cols x ldsT, same rules.  The
 * read is 1 byte (+ 4/128) per element instead of the 2 of a bf16 source;
 * the price is a second rounding. */
FP8B_API int fp8_requantize_transposed(const uint8_t* q, int64_t ldq, const float* s, int64_t lds,
                              int64_t rows, int64_t cols,
                              uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT, void* stream);

/* The same with the MoE grouping of fp8_quantize_transposed_grouped (device
 * offsets, token groups restart at every expert). */
FP8B_API int fp8_requantize_transposed_grouped(const uint8_t* q, int64_t ldq, const float* s, int64_t lds,
                                      int64_t rows, int64_t cols, const int32_t* offsets, int64_t E,
                                      uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT, void* stream);

/* Dequantized-backward mode (the Miles MXFP8/NVFP4 blog's backward-mode
 * section): the backward GEMMs run in bf16 on bf16 dequantizations of the
 * exact FP8 operands the forward pass produced (W for DGrad, X for WGrad);
 * dY stays bf16 and no column-wise FP8 copy is needed.  Dequantization:
 * out = bf16(fl32(E4M3(q) * scale)), nearest-even at both steps. */

/* Codes q (rows x ldq, K = cols padded to 128) with scales of the given
 * layout -> out rows x ldo bf16 (16-byte aligned, ldo * 2 a multiple of 16). */
FP8B_API int fp8_dequantize_bf16(const uint8_t* q, int64_t ldq, const void* s, int64_t lds, int kind,
                        int64_t rows, int64_t cols, uint16_t* out, int64_t ldo, void* stream);

/* Both GEMMs below run on the library's bf16 MFMA kernel (gfx950
 * v_mfma_f32_16x16x32_bf16, fp32 accumulation, bf16 output rounded to
 * nearest-even), which reads both operands contiguous along the contraction
 * axis.  The caller-owned bf16 workspace `work` receives those operand
 * copies (each row a contiguous run of the contraction axis, ldwork a
 * multiple of 8 elements, 16-byte aligned), written by the call before its
 * GEMM: the dequantized FP8 operand transposed, and for WGrad dY transposed.
 * bf16 inputs and outputs follow the 16-byte rules of the FP8 kernels
 * (pointer and ld * element size multiples of 16); rows are read in whole
 * 16-byte chunks up to round_up(K, 8) elements (K the contraction length),
 * and the elements past K are ignored.  Row strides of dy and work are at
 * most 2^23 elements (FP8B_EUNSUPPORTED beyond). */

/* dX [N x C] bf16 = dY [N x D] bf16 * W^ [D x C], W^ the dequantized forward
 * weight codes (kind FP8B_SCALE_BLOCKS_128X128 or FP8B_SCALE_MX_1X32, codes
 * D x ldwq, K = C).  work: C x ldwork bf16, ldwork >= D; receives W^T. */
FP8B_API int fp8_dequant_gemm_dgrad(const uint16_t* dy, int64_t lddy, const uint8_t* wq, int64_t ldwq,
                           const void* ws, int64_t ldws, int wkind, int64_t N, int64_t D, int64_t C,
                           uint16_t* dx, int64_t lddx, uint16_t* work, int64_t ldwork, void* stream);

/* dW [D x C] = dY^T X^ (+ dW when beta = 1; dwt FP8B_F32 required then), X^
 * the dequantized forward activation codes (kind FP8B_SCALE_ROWS_1X128 or
 * FP8B_SCALE_MX_1X32, rows N, K = C).  work: (C + D) x ldwork bf16, ldwork
 * >= N; rows [0, C) receive X^T and rows [C, C + D) receive dY^T (columns
 * [N, round_up(N, 8)) are written zero).  An empty contraction (N = 0) writes
 * zeros (beta = 0) or leaves dW unchanged (beta = 1). */
FP8B_API int fp8_dequant_gemm_wgrad(const uint16_t* dy, int64_t lddy, const uint8_t* xq, int64_t ldxq,
                           const void* xs, int64_t ldxs, int xkind, int64_t N, int64_t D, int64_t C,
                           void* dw, int dwt, int64_t lddw, int beta,
                           uint16_t* work, int64_t ldwork, void* stream);

/* Power-of-two block scales (the SkyRL section "FP8 quantization with FP32
 * and power-of-two block scales": FP32 scales constrained to powers of two,
 * an exponent-only representation, the only kind Blackwell tensor cores
 * take).  Same groupings, layouts and codes rule as the three quantizers above, with the scale of
 * a group S = 2^k, k the smallest integer with max|x| <= 448 * 2^k (rounded
 * up so the group maximum does not clip; the pages do not state the rounding,
 * this is the rule they give for E8M0 scales), clamped to [-127, 127]; an
 * all-zero group has S = 2^-127.  The fp32 scales feed the block-scaled GEMMs
 * unchanged.  Each call can also write the E8M0 byte k + 127 of every group,
 * repeated over its four 32-wide sub-blocks, in the layout of the MXFP8
 * scales (rows x ld bytes, ld >= round_up(K,128)/32, K the codes' padded
 * contraction axis; pointer and ld multiples of 4; NULL to skip): with those
 * bytes the MXFP8 GEMMs below compute the same products on the gfx950
 * scaled MFMA, with no per-block promotion in software. */

/* fp8_quantize_act_1x128 with power-of-two scales; e8: rows x lde E8M0 bytes (nullable). */
FP8B_API int fp8_quantize_act_1x128_pow2(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                                uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                uint8_t* e8, int64_t lde, void* stream);

/* fp8_quantize_weight_128x128 with power-of-two scales; e8: D x lde E8M0 bytes of q's rows (the
 * block's byte repeated for its 128 rows), e8T: C x ldeT bytes of qT's rows
 * (nullable each; e8T is the scale input of fp8_mx_gemm_dgrad). */
FP8B_API int fp8_quantize_weight_128x128_pow2(const void* w, int wt, int64_t D, int64_t C, int64_t ldw,
                                     uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                     uint8_t* qT, int64_t ldqT,
                                     uint8_t* e8, int64_t lde, uint8_t* e8T, int64_t ldeT, void* stream);

/* fp8_quantize_transposed with power-of-two scales; e8T: cols x ldeT bytes of qT's groups, e8:
 * rows x lde bytes of the row-wise copy (requires q; nullable each). */
FP8B_API int fp8_quantize_transposed_pow2(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                                 uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT, uint8_t* e8T, int64_t ldeT,
                                 uint8_t* q, int64_t ldq, float* s, int64_t lds, uint8_t* e8, int64_t lde,
                                 void* stream);

/* ------------------------------------------------------------------ */
/* Block-scaled FP8 GEMMs (fp32 accumulation; each 128-wide K block's    */
/* partial product is scaled by s_a * s_b before it is added)           */
/* ------------------------------------------------------------------ */

/* Limits shared by every GEMM below (block-scaled and MX, dense and grouped):
 * the leading dimensions of the FP8 code operands are at most 2^24 bytes and
 * those of their scale operands at most 2^22 elements; larger ones return
 * FP8B_EUNSUPPORTED (the kernels address a tile's rows with 32-bit offsets). */

/* FProp Y[N x D] = X W^T (Jet-RL notes, section 2.2 FProp; 4.2: the
 * activation 1x128 and the weight 128x128).
 *   xq [N x ldxq] codes, xs [N x ldxs] fp32 (fp8_quantize_act_1x128 of X [N x C]);
 *   wq [D x ldwq] codes, ws [ceil(D/128) x ldws] fp32 (fp8_quantize_weight_128x128);
 *   y  [N x ldy] of dtype yt (FP8B_BF16: round-to-nearest-even; FP8B_F32). */
FP8B_API int fp8_gemm_fprop(const uint8_t* xq, int64_t ldxq, const float* xs, int64_t ldxs,
                   const uint8_t* wq, int64_t ldwq, const float* ws, int64_t ldws,
                   void* y, int yt, int64_t ldy, int64_t N, int64_t D, int64_t C, void* stream);

/* DGrad dX[N x C] = dY W (Jet-RL notes, section 2.2 DGrad; 4.2: same
 * kernel configuration as FProp, the weight only transposed).
 *   gq [N x ldgq] codes, gs [N x ldgs] fp32 (fp8_quantize_act_1x128 of dY [N x D], groups along D);
 *   wqT [C x ldwqT] codes (the transposed copy written by fp8_quantize_weight_128x128), ws [ceil(D/128) x ldws]. */
FP8B_API int fp8_gemm_dgrad(const uint8_t* gq, int64_t ldgq, const float* gs, int64_t ldgs,
                   const uint8_t* wqT, int64_t ldwqT, const float* ws, int64_t ldws,
                   void* dx, int dxt, int64_t lddx, int64_t N, int64_t D, int64_t C, void* stream);

/* DGrad dX = dY W (Jet-RL notes, section 2.2 DGrad; 4.2: dY grouped 1x128
 * along D, W in 128x128 blocks), for few token rows (N <= 64), with the
 * contraction D split into consecutive ranges of 128-wide K blocks.  Such an output has too few
 * 128-column tiles to occupy every compute unit, and each tile would re-read
 * all of dY; here block row y of the grid runs the K blocks of range y in
 * ascending order into fp32 partial sums in `work`, and a second kernel adds
 * the ranges in ascending order and rounds once.  Every output element is
 * still a fixed, deterministic sum: per range as in fp8_gemm_dgrad, then the
 * ranges in order (the summation order differs from fp8_gemm_dgrad's, so the
 * two agree to the GEMM tolerance, not bit for bit).
 *   fp8_gemm_dgrad_split_bytes: bytes of `work` the split needs for this
 *   shape; 0 when no split applies (N > 64, fewer than 16 K blocks, or more
 *   than 128 output tiles of 128 columns), and then fp8_gemm_dgrad_split is
 *   fp8_gemm_dgrad (work may be NULL).  The partition (about 256 blocks of at
 *   least 8 K blocks each) and this size depend on N, D and C only, never on
 *   the device, so the output bits are the same on every device.  At most
 *   256 * 64 * 128 * 4 bytes = 8 MiB.  Negative sizes return 0.
 *   work: DEVICE buffer of at least that many bytes, 16-byte aligned, owned
 *   by the caller, not read before it is written; it must not be used by
 *   other work until the call's kernels have finished on `stream`.
 *   Errors as fp8_gemm_dgrad, plus FP8B_EINVAL (work NULL), FP8B_EALIGN,
 *   FP8B_ESHAPE (work_bytes too small) when a split applies.
 * fp8_mx_gemm_dgrad_split is the same for fp8_mx_gemm_dgrad's operands. */
FP8B_API int64_t fp8_gemm_dgrad_split_bytes(int64_t N, int64_t D, int64_t C);
FP8B_API int fp8_gemm_dgrad_split(const uint8_t* gq, int64_t ldgq, const float* gs, int64_t ldgs,
                         const uint8_t* wqT, int64_t ldwqT, const float* ws, int64_t ldws,
                         void* dx, int dxt, int64_t lddx, int64_t N, int64_t D, int64_t C,
                         void* work, int64_t work_bytes, void* stream);

/* fp8_gemm_dgrad_split without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The fp32 partial sums go to a scratch
 * array of 8 MiB (the largest workspace fp8_gemm_dgrad_split_bytes can
 * return) that the library holds in each device's memory from its load
 * until the process ends; the call allocates and frees nothing.  Output
 * bit for bit equal to fp8_gemm_dgrad_split's (same kernels, same
 * partition).  The scratch array is shared by every call on one device and
 * keeps the last call's partial sums (nothing in it needs clearing: each
 * call writes every partial sum it reads): calls on one device must not
 * overlap in time (same stream, or streams ordered by events), or they race
 * on it.  The device is the one `stream` belongs to; its first call there
 * looks the array's address up once (the current device is restored).
 * Errors as fp8_gemm_dgrad, FP8B_EUNSUPPORTED if a split would need more
 * than 8 MiB (no shape does) or the device index is 64 or more, FP8B_EHIP if
 * the runtime cannot locate the array. */
FP8B_API int fp8_gemm_dgrad_split_noalloc(const uint8_t* gq, int64_t ldgq, const float* gs, int64_t ldgs,
                                 const uint8_t* wqT, int64_t ldwqT, const float* ws, int64_t ldws,
                                 void* dx, int dxt, int64_t lddx, int64_t N, int64_t D, int64_t C,
                                 void* stream);

/* WGrad dW[D x C] = dY^T X (Jet-RL notes, section 2.2 WGrad; 4.2: both
 * operands grouped along the token axis).
 *   gqT [D x ldgqT], gsT [D x ldgsT] (fp8_quantize_transposed of dY); xqT [C x ldxqT], xsT [C x ldxsT]
 *   (fp8_quantize_transposed of X); contraction length N (tokens).
 *   beta = 0: dw = result; beta = 1: dw += result (dwt must be FP8B_F32). */
FP8B_API int fp8_gemm_wgrad(const uint8_t* gqT, int64_t ldgqT, const float* gsT, int64_t ldgsT,
                   const uint8_t* xqT, int64_t ldxqT, const float* xsT, int64_t ldxsT,
                   void* dw, int dwt, int64_t lddw, int beta,
                   int64_t N, int64_t D, int64_t C, void* stream);

/* Grouped (MoE) forms.  offsets: DEVICE int32[E+1] as for the grouped
 * quantizer.  Expert e's weight codes start at w + e*w_estride (bytes) and
 * its scales at ws + e*ws_estride (floats); stacking the experts as one
 * (E*D) x C matrix quantized by fp8_quantize_weight_128x128 gives w_estride = D*ldwq and
 * ws_estride = (D/128)*ldws, and for the transposed copy qT [C x E*D]
 * w_estride = D.
 * FProp: rows of expert e of xq times W_e^T -> rows of y.
 * DGrad: rows of expert e of gq times W_e   -> rows of dx. */
FP8B_API int fp8_gemm_fprop_grouped(const uint8_t* xq, int64_t ldxq, const float* xs, int64_t ldxs,
                           const uint8_t* wq, int64_t ldwq, int64_t wq_estride,
                           const float* ws, int64_t ldws, int64_t ws_estride,
                           void* y, int yt, int64_t ldy,
                           const int32_t* offsets, int64_t E, int64_t N, int64_t D, int64_t C,
                           void* stream);
FP8B_API int fp8_gemm_dgrad_grouped(const uint8_t* gq, int64_t ldgq, const float* gs, int64_t ldgs,
                           const uint8_t* wqT, int64_t ldwqT, int64_t wqT_estride,
                           const float* ws, int64_t ldws, int64_t ws_estride,
                           void* dx, int dxt, int64_t lddx,
                           const int32_t* offsets, int64_t E, int64_t N, int64_t D, int64_t C,
                           void* stream);
/* WGrad per expert: dW_e = dY_e^T X_e from the grouped transposed operands
 * (fp8_quantize_transposed_grouped); dW_e is written at dw + e*dw_estride (elements).  An expert
 * with no rows gets dW_e = 0 (beta = 0) or is left unchanged (beta = 1). */
FP8B_API int fp8_gemm_wgrad_grouped(const uint8_t* gqT, int64_t ldgqT, const float* gsT, int64_t ldgsT,
                           const uint8_t* xqT, int64_t ldxqT, const float* xsT, int64_t ldxsT,
                           void* dw, int dwt, int64_t lddw, int64_t dw_estride, int beta,
                           const int32_t* offsets, int64_t E, int64_t N, int64_t D, int64_t C,
                           void* stream);

/* ------------------------------------------------------------------ */
/* MXFP8 (Miles MXFP8/NVFP4 blog, MXFP8 paragraphs)                    */
/* ------------------------------------------------------------------ */

/* MXFP8: 1x32 blocks, scale 2^k stored as the E8M0 byte k+127, k the smallest
 * integer with max|block| <= 448*2^k, clamped to [-127,127] (all-zero block:
 * k = -127); codes E4M3(x * 2^-k).  Either output pair may be NULL:
 *   q  [rows x ldq], e [rows x lde]: row-wise (blocks along cols);
 *   qT [cols x ldqT], eT [cols x ldeT]: column-wise (blocks along rows),
 *   each quantized from x itself (never from the other copy).
 * Code buffers pad the block axis to a multiple of 128 with 0x00
 * (ldq >= round_up(cols,128), ldqT >= round_up(rows,128), multiples of 16);
 * E8M0 buffers hold round_up(K,128)/32 entries per row, pad entries 127. */
FP8B_API int fp8_mx_quantize_1x32(const void* x, int xt, int64_t rows, int64_t cols, int64_t ldx,
                         uint8_t* q, int64_t ldq, uint8_t* e, int64_t lde,
                         uint8_t* qT, int64_t ldqT, uint8_t* eT, int64_t ldeT, void* stream);

/* MX GEMMs on gfx950 scaled MFMA.  All three are
 *   out[i][j] = sum_k (a[i][k] 2^(ea[i][k/32]-127)) (b[j][k] 2^(eb[j][k/32]-127))
 * with both operands K-contiguous:
 *   FProp: a = X row-wise [N x C], b = W row-wise [D x C]          -> y [N x D]
 *   DGrad: a = dY row-wise [N x D], b = W column-wise [C x D]      -> dx [N x C]
 *   WGrad: a = dY column-wise [D x N], b = X column-wise [C x N]   -> dw [D x C]
 * E8M0 operands: pointers and row strides multiples of 4 (FP8B_EALIGN
 * otherwise; each K block's four bytes are fetched as one word). */
FP8B_API int fp8_mx_gemm_fprop(const uint8_t* xq, int64_t ldxq, const uint8_t* xe, int64_t ldxe,
                      const uint8_t* wq, int64_t ldwq, const uint8_t* we, int64_t ldwe,
                      void* y, int yt, int64_t ldy, int64_t N, int64_t D, int64_t C, void* stream);
FP8B_API int fp8_mx_gemm_dgrad(const uint8_t* gq, int64_t ldgq, const uint8_t* ge, int64_t ldge,
                      const uint8_t* wqT, int64_t ldwqT, const uint8_t* weT, int64_t ldweT,
                      void* dx, int dxt, int64_t lddx, int64_t N, int64_t D, int64_t C, void* stream);
FP8B_API int fp8_mx_gemm_dgrad_split(const uint8_t* gq, int64_t ldgq, const uint8_t* ge, int64_t ldge,
                            const uint8_t* wqT, int64_t ldwqT, const uint8_t* weT, int64_t ldweT,
                            void* dx, int dxt, int64_t lddx, int64_t N, int64_t D, int64_t C,
                            void* work, int64_t work_bytes, void* stream);
FP8B_API int fp8_mx_gemm_wgrad(const uint8_t* gqT, int64_t ldgqT, const uint8_t* geT, int64_t ldgeT,
                      const uint8_t* xqT, int64_t ldxqT, const uint8_t* xeT, int64_t ldxeT,
                      void* dw, int dwt, int64_t lddw, int beta,
                      int64_t N, int64_t D, int64_t C, void* stream);

/* ------------------------------------------------------------------ */
/* Rollout decode: FProp of at most 64 tokens on a packed weight        */
/* ------------------------------------------------------------------ */

/* Rollout runs the training forward's FP8 FProp (Jet-RL notes, section 2.2
 * FProp, and the unified precision flow of the Jet-RL summary: rollout uses
 * the same quantized weights and GEMM as the training forward) on few
 * tokens, where reading the weight is the whole cost.  The decode layout
 * holds the same codes in the order the decode kernel's loads consume them,
 * so each load reads 1 KB of consecutive bytes; it is written once per
 * weight update and read by every decode step.  The results are bit for bit
 * those of fp8_gemm_fprop / fp8_mx_gemm_fprop on the row-major weight (same
 * products, same per-output reduction order).
 *
 * fp8_decode_pack_bytes: bytes of the decode-layout codes (part 0:
 * 16 ceil(D/16) round_up(C,128)) or of the packed MX scale words (part 1:
 * 16 ceil(D/16) ceil(C/128) 4); 0 for negative sizes or another part.
 *
 * fp8_pack_decode_weight: decode layout of wq [D x ldwq] codes (as written by
 * fp8_quantize_weight_128x128 or fp8_mx_quantize_1x32; ldwq >= round_up(C,128),
 * pointer and ldwq multiples of 16) into wp (DEVICE, part-0 bytes, 16-byte
 * aligned; rows past D in the last group of 16 are zero codes); when we is
 * not NULL, also the E8M0 bytes we [D x ldwe] (pointer and ldwe multiples of
 * 4, ldwe >= round_up(C,128)/32) into the words wep (DEVICE, part-1 bytes,
 * 4-byte aligned; required then).  The layout, for g < ceil(D/16), K block
 * k < ceil(C/128), h in {0,1}, lane l < 64: wp bytes
 * [((g ceil(C/128) + k) 2 + h) 1024 + 16 l, +16) hold row 16 g + l % 16,
 * bytes [128 k + 16 (l/16 + 4 h), +16) of the row-major codes; word
 * wep[(g ceil(C/128) + k) 16 + r] holds the four E8M0 bytes of row 16 g + r
 * for K block k (0x7F7F7F7F past D).  wp and wep are owned by the caller;
 * D == 0 or C == 0 writes nothing. */
FP8B_API int64_t fp8_decode_pack_bytes(int64_t D, int64_t C, int part);
FP8B_API int fp8_pack_decode_weight(const uint8_t* wq, int64_t ldwq, const uint8_t* we, int64_t ldwe,
                                    int64_t D, int64_t C, uint8_t* wp, uint32_t* wep, void* stream);

/* FProp y[N x D] = X W^T with N <= 64 (N > 64: FP8B_EUNSUPPORTED) on the
 * decode layout wp of W's codes; xq/xs and ws as for fp8_gemm_fprop
 * (1x128 tokens, 128x128 weight scales), y [N x ldy] of dtype yt.
 * C == 0 writes zeros. */
FP8B_API int fp8_gemm_fprop_decode(const uint8_t* xq, int64_t ldxq, const float* xs, int64_t ldxs,
                                   const uint8_t* wp, const float* ws, int64_t ldws,
                                   void* y, int yt, int64_t ldy, int64_t N, int64_t D, int64_t C, void* stream);

/* The MXFP8 form: xq/xe as for fp8_mx_gemm_fprop, the weight as wp and wep
 * from fp8_pack_decode_weight of its codes and E8M0 bytes. */
FP8B_API int fp8_mx_gemm_fprop_decode(const uint8_t* xq, int64_t ldxq, const uint8_t* xe, int64_t ldxe,
                                      const uint8_t* wp, const uint32_t* wep,
                                      void* y, int yt, int64_t ldy, int64_t N, int64_t D, int64_t C,
                                      void* stream);

/* ------------------------------------------------------------------ */
/* Codec access (for exhaustive checks of the device codec)            */
/* ------------------------------------------------------------------ */

/* out[i] = E4M3 code of x[i] / s[i] exactly as the quantizers compute it:
 * fp32 quotient, nearest-even E4M3, saturating; s[i] == 0 gives the signed
 * zero of x[i].  If s is NULL the divisor is 1 (plain encode of x). */
FP8B_API int fp8b_e4m3_encode(const float* x, const float* s, int64_t n, uint8_t* out, void* stream);

/* out[i] = bf16 bits of x[i] rounded to nearest, ties to even, by the
 * conversion the fused producers use for their bf16 activations (elements
 * taken in pairs, as the kernels pack them).  x: DEVICE fp32[n]; out: DEVICE
 * uint16[n].  Errors: FP8B_ESHAPE (n < 0), FP8B_EINVAL (NULL), FP8B_EHIP. */
FP8B_API int fp8b_bf16_round(const float* x, int64_t n, uint16_t* out, void* stream);

/* ------------------------------------------------------------------ */
/* Measurement aid (not part of the FP8 path)                          */
/* ------------------------------------------------------------------ */

/* Matrix-core throughput on random operands: the ceiling the GEMMs are
 * compared with beside the published peak (the chip is power limited, and
 * its clock under load depends on the data the matrix cores multiply).
 * kind 0: v_mfma_f32_16x16x128_f8f6f4 on E4M3 codes (NaN codes excluded);
 * kind 1: v_mfma_f32_16x16x32_bf16 on bf16 values of magnitude in [2^-8, 2^8);
 * kind 2: kind 0 with the FP32-scale promotion of the 1x128 x 128x128 GEMMs
 *         (each MFMA's four results added into fp32 accumulators one step
 *         later with one FMA each by a combined scale);
 * kind 3: kind 0 with the promotion of the token-axis WGrad (per-row scales
 *         on both operands: one multiply and one FMA per result).
 * Launches `blocks` blocks of 4 waves; each wave keeps four random A and
 * four random B fragments and four accumulators in registers (bytes from a
 * SplitMix64 hash of seed, wave, lane and register) and issues 16 MFMAs per
 * iteration, `iters` iterations, with no memory traffic in the loop.
 * out: DEVICE fp32[4 * blocks], one value per wave (keeps the work live).
 * flops (host, nullable): receives the floating-point operations launched,
 * blocks * 4 * 16 * iters * (16384 for kind 1, else 65536); the promotion
 * work of kinds 2 and 3 is not counted, as in the GEMMs' own figures.
 * Errors: FP8B_EINVAL (bad kind, NULL out), FP8B_ESHAPE, FP8B_EHIP. */
FP8B_API int fp8b_mfma_peak(int kind, int64_t blocks, int64_t iters, uint32_t seed, float* out, double* flops,
                   void* stream);

/* Host-only argument check of the GEMM entry points: runs exactly the
 * validation the launch would run and returns its status, launching
 * nothing.  op: 0 FProp, 1 DGrad, 2 WGrad, 3 MX FProp, 4 MX DGrad,
 * 5 MX WGrad.  Pointers are only tested for NULL and alignment. */
FP8B_API int fp8b_validate_gemm(int op, const void* a, int64_t lda, const void* sa, int64_t ldsa,
                       const void* b, int64_t ldb, const void* sb, int64_t ldsb,
                       const void* out, int out_dtype, int64_t ldo, int beta,
                       int64_t N, int64_t D, int64_t C);

#ifdef __cplusplus
}
#endif

#endif /* FP8BLK_H */
