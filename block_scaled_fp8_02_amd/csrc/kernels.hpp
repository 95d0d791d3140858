// kernels.hpp -- internal launch interface between the C ABI layer
// (api.hip) and the kernel translation units.  Arguments are validated by
// the caller; these functions only launch and report hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8blk {

// Quantizers.  pow2 selects power-of-two block scales (2^k, k the smallest
// exponent with amax <= 448 * 2^k) and lets the kernels also write the E8M0
// bytes of every group, replicated over its four 32-wide sub-blocks (e8 for
// the row-wise codes, e8T for the transposed ones; nullable).

// Row-wise 1x128 quantization (in_bf16: bf16 input, else fp32).
hipError_t launch_quant_rows(const void* x, bool in_bf16, int64_t rows, int64_t cols, int64_t ldx,
                             uint8_t* q, int64_t ldq, float* s, int64_t lds,
                             bool pow2, uint8_t* e8, int64_t lde, hipStream_t st);

// 128x128 weight quantization with optional transposed copy.
hipError_t launch_quant_weight(const void* w, bool in_bf16, int64_t D, int64_t C, int64_t ldw,
                               uint8_t* q, int64_t ldq, float* s, int64_t lds,
                               uint8_t* qT, int64_t ldqT,
                               bool pow2, uint8_t* e8, int64_t lde, uint8_t* e8T, int64_t ldeT, hipStream_t st);

// Token-axis 1x128 quantization written transposed, optionally also the
// row-wise copy; offsets == nullptr means one segment of all rows.
hipError_t launch_quant_cols(const void* x, bool in_bf16, int64_t rows, int64_t cols, int64_t ldx,
                             const int32_t* offsets, int64_t E,
                             uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT,
                             uint8_t* q, int64_t ldq, float* s, int64_t lds,
                             bool pow2, uint8_t* e8T, int64_t ldeT, uint8_t* e8, int64_t lde, hipStream_t st);

// Token-axis quantization of saved 1x128 FP8 data (codes q, scales s):
// each element dequantized as fl32(E4M3(q) * s), then as launch_quant_cols.
hipError_t launch_requant_cols(const uint8_t* q, int64_t ldq, const float* s, int64_t lds,
                               int64_t rows, int64_t cols, const int32_t* offsets, int64_t E,
                               uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT, hipStream_t st);

// Fused producers of the 1x128 activation quantizer (fused.hip).
hipError_t launch_rmsnorm_quant(const void* x, bool x_bf16, int64_t rows, int64_t cols, int64_t ldx,
                                const void* w, bool w_bf16, float eps,
                                uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                float* rstd, uint16_t* y, int64_t ldy, hipStream_t st);
hipError_t launch_silu_mul_quant(const uint16_t* gate, int64_t ldg, const uint16_t* up, int64_t ldu,
                                 int64_t rows, int64_t cols, uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                 uint16_t* a, int64_t lda, hipStream_t st);

// Dequantized-backward mode.  dequant.hip: bf16 dequantization of FP8 codes
// (kind 0: 1x128 row groups, 1: 128x128 blocks, 2: MX 1x32 E8M0).
// Zero a rows x row_bytes region with row stride ld_bytes (a kernel, not a memset).
hipError_t launch_zero_2d(void* p, int64_t ld_bytes, int64_t row_bytes, int64_t rows, hipStream_t st);
hipError_t launch_dequant_bf16(const uint8_t* q, int64_t ldq, const void* s, int64_t lds, int kind,
                               int64_t rows, int64_t cols, uint16_t* out, int64_t ldo, hipStream_t st);

// bf16gemm.hip: O[i][j] (+)= sum_k P[i][k] Q[j][k], P (M x K) and Q (Nn x K)
// bf16 contiguous along K (row strides ldp, ldq in elements, multiples of 8;
// elements up to round_up(K, 8) of a row are read, those past K ignored),
// fp32 accumulation, bf16 (nearest-even) or fp32 output (beta = 1: added to
// the fp32 output).
struct Bf16GemmArgs {
    const uint16_t* P; int64_t ldp;
    const uint16_t* Q; int64_t ldq;
    void* O; int64_t ldo; bool out_f32; int beta;
    int64_t M, Nn, K;
};
hipError_t launch_gemm_bf16(const Bf16GemmArgs& a, hipStream_t st);
// out[c][r] = in[r][c] as bf16 (out row stride ldo, a multiple of 8 >= rows):
// src 0 bf16 input (row stride ldi, a multiple of 8); 1, 2, 3 FP8 codes
// (rows padded to 128) dequantized with the scale layouts of kind 0, 1, 2
// above, bf16(fl32(E4M3(q) * scale)).
hipError_t launch_transpose_bf16(int src, const void* in, int64_t ldi, const void* s, int64_t lds,
                                 int64_t rows, int64_t cols, uint16_t* out, int64_t ldo, hipStream_t st);

// Elementwise codec access.
hipError_t launch_encode(const float* x, const float* s, int64_t n, uint8_t* out, hipStream_t st);
hipError_t launch_bf16_round(const float* x, int64_t n, uint16_t* out, hipStream_t st);

// Matrix-core throughput on random register operands (peak.hip): kind 0 the
// fp8 16x16x128 MFMA, kind 1 the bf16 16x16x32 MFMA; blocks of 256 threads,
// 16 * iters MFMAs per wave, one fp32 per wave into out.
hipError_t launch_mfma_peak(int kind, int64_t blocks, int64_t iters, uint32_t seed, float* out, hipStream_t st);

// Compute units of the current device (cached per device).
int device_cu_count();


// Generic block-scaled / MX GEMM:
//   O[i][j] (+)= sum_k P[i][k] Q[j][k] * scales
// P: M x K codes (row stride ldp), Q: Nn x K codes (row stride ldq), both
// padded with zero codes to a multiple of 128 along K.
enum ScaleMode {
    SCALE_Q_BLOCK = 0,   // sQ per 128-row block of Q: sQ[(j/128)*sq_rs + kb*sq_ks]
    SCALE_Q_ROW = 1,     // sQ per row of Q:           sQ[j*sq_rs + kb*sq_ks]
    SCALE_MX = 2         // E8M0 bytes per 32-block:   eP[i*ldsp + k/32], eQ[j*sq_rs + k/32]
};
enum GroupMode {
    GROUP_NONE = 0,
    GROUP_ROWS = 1,      // expert e owns P/O rows [off[e], off[e+1]) and Q_e = Q + e*q_estride
    GROUP_K = 2          // expert e owns K range [P_e, P_e + round_up(n_e,128)), O_e = O + e*o_estride
};

struct GemmArgs {
    const uint8_t* P; int64_t ldp;
    const void* sP; int64_t ldsp;
    const uint8_t* Q; int64_t ldq;
    const void* sQ; int64_t sq_rs; int64_t sq_ks;
    void* O; int64_t ldo; bool out_f32; int beta;
    int64_t M, Nn, K;
    int scale_mode;
    int group_mode;
    const int32_t* offsets; int64_t E;
    int64_t q_estride, sq_estride, o_estride;
    int64_t epb;          // GROUP_K: experts per block (set by the launcher)
    int64_t ksplit;       // GROUP_NONE, M <= 64: K ranges run by block rows (0 or 1: none)
    int64_t kb_split;     // K blocks per range; range y writes fp32 O + y * o_estride
};

hipError_t launch_gemm(const GemmArgs& a, hipStream_t st);

// Few-token GEMM with the weight streamed through registers (decode.hip):
// whether it takes a launch (at most 64 rows of P, a long Q, no K split, no
// grouping, 128x128 or MX scales), and the launch.  Per-output arithmetic
// identical to launch_gemm's.
bool rows96_applies(const GemmArgs& a);
hipError_t launch_gemm_rows96(const GemmArgs& a, hipStream_t st);
// The same kernel on a weight in the decode layout (Q and, for MX, sQ as
// written by launch_pack_decode; 128x128 scales as for launch_gemm): any
// Nn, 1 <= M <= 64, beta 0.
hipError_t launch_gemm_decode_packed(const GemmArgs& a, hipStream_t st);
// Decode layout of row-major codes wq [D x ldwq] (KB K blocks per row) and,
// when we != nullptr, of their E8M0 bytes we [D x ldwe]: wp gets
// 16 ceil(D/16) KB 128 bytes, wep 16 ceil(D/16) KB words.
hipError_t launch_pack_decode(const uint8_t* wq, int64_t ldwq, const uint8_t* we, int64_t ldwe,
                              int64_t D, int64_t KB, uint8_t* wp, uint32_t* wep, hipStream_t st);

// out[i][j] = sum over s = 0 .. S-1, in that order, of part[s * slice + i * ldp + j]
// (fp32), stored as bf16 (nearest-even) or fp32 at row stride ldo.
hipError_t launch_split_sum(const float* part, int64_t S, int64_t slice, int64_t ldp, int64_t M, int64_t Nn,
                            void* out, bool out_f32, int64_t ldo, hipStream_t st);

// MXFP8 1x32 quantization (row-wise and/or column-wise).
hipError_t launch_mx_quant(const void* x, bool in_bf16, int64_t rows, int64_t cols, int64_t ldx,
                           uint8_t* q, int64_t ldq, uint8_t* e, int64_t lde,
                           uint8_t* qT, int64_t ldqT, uint8_t* eT, int64_t ldeT, hipStream_t st);

}  // namespace fp8blk
