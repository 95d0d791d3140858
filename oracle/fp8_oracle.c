/*
 * fp8_oracle.c -- CPU oracle for the block-scaled FP8 linear-layer path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file; only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or constant
 * with the HIP library: the codec here is a table search over the E4M3
 * value set, the library's codec is independent bit arithmetic.
 *
 * Plain C11, host only.  Build with -O2 -fno-fast-math -ffp-contract=off on
 * x86-64 (SSE, FLT_EVAL_METHOD == 0) so that every `float` operation below is
 * exactly one IEEE-754 binary32 operation rounded to nearest-even.  OpenMP
 * only splits independent rows across threads; it never reorders the
 * arithmetic that produces one output value.
 *
 * What is computed, and where the method pages define it:
 *
 *   Quantizer Q (Jet-RL, "Background: quantization basics", the equation for
 *   Q): S = max|X| / Delta_max with Delta_max = 448 for E4M3, and
 *   Xhat = X / S taken to the nearest E4M3 value.  The page prints floor
 *   brackets around X/S; the companion summary page ("Technical Approach",
 *   weight and activation quantization) says the quotient is rounded to the
 *   nearest representable FP8 value.  Reading used here: fp32 quotient, then
 *   round-to-nearest-even into E4M3 with saturation at +-448.
 *
 *   Granularities (Jet-RL "GEMM quantization granularity" section; summary
 *   page "Weight quantization: 128x128 per-block" and "Activation and
 *   gradient quantization: 1x128 per-group"): weights per 128x128 tile,
 *   activations and gradients per 1x128 group along the contraction axis,
 *   WGrad operands grouped along the token axis.
 *
 *   MXFP8 (Miles MXFP8/NVFP4 blog, MXFP8 format paragraph): 32 consecutive
 *   E4M3 values share one E8M0 power-of-two scale, rounded up so that the
 *   block maximum does not clip; row-wise and column-wise copies are each
 *   quantized from the full-precision data.
 *
 *   GEMMs (Jet-RL "Quantization of linear layers": FProp Y = X W^T,
 *   WGrad dW = dY^T X, DGrad dX = dY W): dequantize every operand exactly
 *   into fp64 and accumulate in fp64 in ascending contraction index.
 *
 * Parity pins for every function here live in tests/ (marker "not gpu").
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_API __attribute__((visibility("default")))

/* ------------------------------------------------------------------ */
/* E4M3 value set (OCP 8-bit floating point, as cited by the Jet-RL     */
/* page for Delta_max = 448): 1 sign bit, 4 exponent bits with bias 7,  */
/* 3 mantissa bits, no infinities, S.1111.111 is NaN.                   */
/* ------------------------------------------------------------------ */

static double E4M3[256];
static int e4m3_ready = 0;

static void e4m3_build(void)
{
    if (e4m3_ready) return;
    for (int c = 0; c < 256; ++c) {
        int sign = c >> 7;
        int e = (c >> 3) & 15;
        int m = c & 7;
        double v;
        if (e == 15 && m == 7)
            v = NAN;
        else if (e == 0)
            v = ldexp((double)m, -9);            /* subnormal: m/8 * 2^(1-7) */
        else
            v = ldexp(1.0 + m / 8.0, e - 7);     /* normal */
        E4M3[c] = sign ? -v : v;
    }
    e4m3_ready = 1;
}

ORACLE_API double ora_e4m3_decode(int code)
{
    e4m3_build();
    return E4M3[code & 255];
}

/* Nearest E4M3 value to v, ties to the even code, |v| >= 448 saturates.
 * The magnitudes E4M3[0x00..0x7E] increase strictly with the code, so the
 * largest code whose value does not exceed |v| is found by bisection and
 * |v| is then compared with the exact midpoint to the next code.  Every
 * midpoint has at most 5 significant bits, so the comparison is exact. */
ORACLE_API uint8_t ora_e4m3_encode_f64(double v)
{
    e4m3_build();
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs(v);
    if (a >= 448.0) return (uint8_t)(0x7E | sign);
    int lo = 0x00, hi = 0x7E;                    /* E4M3[lo] <= a < E4M3[hi] */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (E4M3[mid] <= a) lo = mid; else hi = mid;
    }
    double midpoint = 0.5 * (E4M3[lo] + E4M3[hi]);
    int c;
    if (a < midpoint) c = lo;
    else if (a > midpoint) c = hi;
    else c = (lo % 2 == 0) ? lo : hi;            /* tie: even code */
    return (uint8_t)(c | sign);
}

ORACLE_API uint8_t ora_e4m3_encode(float v)
{
    return ora_e4m3_encode_f64((double)v);
}

ORACLE_API void ora_e4m3_encode_array(const float* v, int64_t n, uint8_t* out)
{
    e4m3_build();
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = ora_e4m3_encode(v[i]);
}

/* ------------------------------------------------------------------ */
/* Quantizer Q on one group: S = max|x| / 448 (one fp32 division), then  */
/* q = E4M3(x / S) (one fp32 division, then the E4M3 rounding).  An      */
/* all-zero group, or one whose S underflows to zero, stores S = 0 and   */
/* the signed zero of each input.                                        */
/* ------------------------------------------------------------------ */

/* The power-of-two exponent of a block with maximum magnitude amax: the
 * smallest integer k with amax <= 448 * 2^k (so the block maximum never
 * clips), clamped to [-127, 127]; an all-zero block takes k = -127.  Used
 * for the E8M0 scales of MXFP8 and for the power-of-two FP32 scales. */
static int mx_exponent(float amax)
{
    if (amax == 0.0f) return -127;
    int lo = -127, hi = 127;                     /* predicate monotone in k */
    if ((double)amax > ldexp(448.0, hi)) return 127;
    while (lo < hi) {
        int mid = lo + (hi - lo) / 2;
        if ((double)amax <= ldexp(448.0, mid)) hi = mid; else lo = mid + 1;
    }
    return lo;
}

static float group_scale(float amax)
{
    return amax / 448.0f;
}

/* Power-of-two FP32 block scale (the SkyRL section "FP8 quantization with
 * FP32 and power-of-two block scales": scales constrained to powers of two,
 * an exponent-only representation).  The pages do not say how the exponent
 * is chosen; reading used here, as for the MXFP8 scales: rounded up so the
 * block maximum does not clip, S = 2^k with k = mx_exponent(amax). */
static float group_scale_p2(float amax)
{
    return ldexpf(1.0f, mx_exponent(amax));
}

static float scale_rule(float amax, int pow2)
{
    return pow2 ? group_scale_p2(amax) : group_scale(amax);
}

static uint8_t quant_elem(float x, float S)
{
    if (S == 0.0f) return signbit(x) ? 0x80 : 0x00;
    float y = x / S;
    return ora_e4m3_encode(y);
}

/* 1x128 per-group quantization along the contiguous axis (activations X
 * for FProp, gradients dY for DGrad).  q: rows x ldq bytes, the columns
 * [cols, round_up(cols,128)) are written 0x00.  s: rows x ceil(cols/128). */
static void quant_1x128(const float* x, int64_t rows, int64_t cols, int64_t ldx,
                        uint8_t* q, int64_t ldq, float* s, int64_t lds, int pow2)
{
    e4m3_build();
    int64_t groups = (cols + 127) / 128;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t g = 0; g < groups; ++g) {
            int64_t k0 = 128 * g;
            int64_t k1 = k0 + 128 < cols ? k0 + 128 : cols;
            float amax = 0.0f;
            for (int64_t k = k0; k < k1; ++k) {
                float a = fabsf(x[r * ldx + k]);
                if (a > amax) amax = a;
            }
            float S = scale_rule(amax, pow2);
            s[r * lds + g] = S;
            for (int64_t k = k0; k < k1; ++k) q[r * ldq + k] = quant_elem(x[r * ldx + k], S);
            for (int64_t k = k1; k < k0 + 128; ++k) q[r * ldq + k] = 0x00;
        }
    }
}

/* 128x128 per-block weight quantization.  W is D x C (output channels x
 * input channels).  s: ceil(D/128) x ceil(C/128).  qT (optional) holds the
 * same codes transposed, C x ldqT; its columns [D, round_up(D,128)) are
 * written 0x00, as are q's columns [C, round_up(C,128)). */
static void quant_128x128(const float* w, int64_t D, int64_t C, int64_t ldw,
                          uint8_t* q, int64_t ldq, float* s, int64_t lds,
                          uint8_t* qT, int64_t ldqT, int pow2)
{
    e4m3_build();
    int64_t bd = (D + 127) / 128, bc = (C + 127) / 128;
    #pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < bd * bc; ++t) {
        int64_t i = t / bc, j = t % bc;
        int64_t d0 = 128 * i, d1 = d0 + 128 < D ? d0 + 128 : D;
        int64_t c0 = 128 * j, c1 = c0 + 128 < C ? c0 + 128 : C;
        float amax = 0.0f;
        for (int64_t d = d0; d < d1; ++d)
            for (int64_t c = c0; c < c1; ++c) {
                float a = fabsf(w[d * ldw + c]);
                if (a > amax) amax = a;
            }
        float S = scale_rule(amax, pow2);
        s[i * lds + j] = S;
        for (int64_t d = d0; d < d1; ++d)
            for (int64_t c = c0; c < c1; ++c) {
                uint8_t code = quant_elem(w[d * ldw + c], S);
                q[d * ldq + c] = code;
                if (qT) qT[c * ldqT + d] = code;
            }
    }
    int64_t Cp = bc * 128, Dp = bd * 128;
    for (int64_t d = 0; d < D; ++d)
        for (int64_t c = C; c < Cp; ++c) q[d * ldq + c] = 0x00;
    if (qT)
        for (int64_t c = 0; c < C; ++c)
            for (int64_t d = D; d < Dp; ++d) qT[c * ldqT + d] = 0x00;
}

/* 1x128 groups along the token axis, written transposed (the WGrad
 * operands dY^T and X^T).  x is rows x cols; the output qT is cols x ldqT,
 * column r of x becoming position r of each output row.  With offsets
 * (E+1 non-decreasing row indices) the rows form E segments and groups
 * restart at each segment start; segment e occupies output positions
 * [P_e, P_e + round_up(n_e,128)) with P_e = sum_{e'<e} round_up(n_e',128),
 * and its scales occupy sT columns [P_e/128, P_e/128 + ceil(n_e/128)).
 * Without offsets there is one segment covering all rows.  Positions past
 * a segment's last row inside its last group are written 0x00. */
static void quant_colwise(const float* x, int64_t rows, int64_t cols, int64_t ldx,
                          const int32_t* offsets, int64_t E,
                          uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT, int pow2)
{
    e4m3_build();
    int64_t nseg = offsets ? E : 1;
    int64_t pos = 0;
    for (int64_t e = 0; e < nseg; ++e) {
        int64_t a = offsets ? offsets[e] : 0;
        int64_t b = offsets ? offsets[e + 1] : rows;
        int64_t n = b - a;
        int64_t ng = (n + 127) / 128;
        #pragma omp parallel for schedule(static)
        for (int64_t c = 0; c < cols; ++c) {
            for (int64_t g = 0; g < ng; ++g) {
                int64_t r0 = a + 128 * g;
                int64_t r1 = r0 + 128 < b ? r0 + 128 : b;
                float amax = 0.0f;
                for (int64_t r = r0; r < r1; ++r) {
                    float v = fabsf(x[r * ldx + c]);
                    if (v > amax) amax = v;
                }
                float S = scale_rule(amax, pow2);
                sT[c * ldsT + pos / 128 + g] = S;
                for (int64_t r = r0; r < r1; ++r)
                    qT[c * ldqT + pos + (r - a)] = quant_elem(x[r * ldx + c], S);
                for (int64_t r = r1; r < r0 + 128; ++r)
                    qT[c * ldqT + pos + (r - a)] = 0x00;
            }
        }
        pos += 128 * ng;
    }
}

/* Exported forms: FP32 scales (the pages' default recipe) and the
 * power-of-two FP32 scales (_p2), same groupings and layouts. */
ORACLE_API void ora_quant_1x128(const float* x, int64_t rows, int64_t cols, int64_t ldx,
                                uint8_t* q, int64_t ldq, float* s, int64_t lds)
{ quant_1x128(x, rows, cols, ldx, q, ldq, s, lds, 0); }

ORACLE_API void ora_quant_1x128_p2(const float* x, int64_t rows, int64_t cols, int64_t ldx,
                                   uint8_t* q, int64_t ldq, float* s, int64_t lds)
{ quant_1x128(x, rows, cols, ldx, q, ldq, s, lds, 1); }

ORACLE_API void ora_quant_128x128(const float* w, int64_t D, int64_t C, int64_t ldw,
                                  uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                  uint8_t* qT, int64_t ldqT)
{ quant_128x128(w, D, C, ldw, q, ldq, s, lds, qT, ldqT, 0); }

ORACLE_API void ora_quant_128x128_p2(const float* w, int64_t D, int64_t C, int64_t ldw,
                                     uint8_t* q, int64_t ldq, float* s, int64_t lds,
                                     uint8_t* qT, int64_t ldqT)
{ quant_128x128(w, D, C, ldw, q, ldq, s, lds, qT, ldqT, 1); }

ORACLE_API void ora_quant_colwise(const float* x, int64_t rows, int64_t cols, int64_t ldx,
                                  const int32_t* offsets, int64_t E,
                                  uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT)
{ quant_colwise(x, rows, cols, ldx, offsets, E, qT, ldqT, sT, ldsT, 0); }

ORACLE_API void ora_quant_colwise_p2(const float* x, int64_t rows, int64_t cols, int64_t ldx,
                                     const int32_t* offsets, int64_t E,
                                     uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT)
{ quant_colwise(x, rows, cols, ldx, offsets, E, qT, ldqT, sT, ldsT, 1); }

/* ------------------------------------------------------------------ */
/* MXFP8: 1x32 blocks with a shared power-of-two scale 2^k stored as the  */
/* E8M0 byte k + 127.  k is the smallest integer with amax <= 448 * 2^k,  */
/* so the block maximum never clips, clamped to [-127, 127]; an all-zero  */
/* block takes k = -127.  Codes are E4M3(x * 2^-k): the product is exact */
/* in double and the E4M3 rounding is the only rounding.                 */
/* ------------------------------------------------------------------ */

/* Requantization of saved 1x128 FP8 data along the token axis (the
 * DeepSeek-V3-style flow the Jet-RL pages describe for WGrad's X^T, which
 * keeps only the FP8 activations): each element is dequantized to fp32 with
 * one binary32 multiply, fl32(E4M3(q) * s), and the result goes through the
 * token-axis quantizer above.  The pages do not fix the dequantization
 * precision; reading used: fp32, the precision the quantizer works in.
 * q: rows x ldq codes of cols columns, s: rows x lds scales (1x128). */
ORACLE_API void ora_requant_colwise(const uint8_t* q, int64_t ldq, const float* s, int64_t lds,
                                    int64_t rows, int64_t cols, const int32_t* offsets, int64_t E,
                                    uint8_t* qT, int64_t ldqT, float* sT, int64_t ldsT)
{
    e4m3_build();
    float* x = (float*)malloc((size_t)(rows > 0 ? rows : 1) * (size_t)(cols > 0 ? cols : 1) * sizeof(float));
    if (!x) return;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c)
            x[r * cols + c] = (float)E4M3[q[r * ldq + c]] * s[r * lds + c / 128];
    quant_colwise(x, rows, cols, cols, offsets, E, qT, ldqT, sT, ldsT, 0);
    free(x);
}

ORACLE_API int ora_mx_exponent(float amax) { return mx_exponent(amax); }

/* Row-wise MX: blocks of 32 along the contiguous axis.  q: rows x ldq with
 * columns [cols, round_up(cols,128)) written 0x00; e: rows x lde with the
 * E8M0 bytes of blocks [ceil(cols/32), round_up(cols,128)/32) written 127
 * (scale 1.0, multiplying only zero codes). */
ORACLE_API void ora_mx_quant_rows(const float* x, int64_t rows, int64_t cols, int64_t ldx,
                                  uint8_t* q, int64_t ldq, uint8_t* e, int64_t lde)
{
    e4m3_build();
    int64_t nb = (cols + 31) / 32;
    int64_t kp = (cols + 127) / 128 * 128;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            int64_t k0 = 32 * b, k1 = k0 + 32 < cols ? k0 + 32 : cols;
            float amax = 0.0f;
            for (int64_t k = k0; k < k1; ++k) {
                float a = fabsf(x[r * ldx + k]);
                if (a > amax) amax = a;
            }
            int k = mx_exponent(amax);
            e[r * lde + b] = (uint8_t)(k + 127);
            double inv = ldexp(1.0, -k);
            for (int64_t c = k0; c < k1; ++c)
                q[r * ldq + c] = ora_e4m3_encode_f64((double)x[r * ldx + c] * inv);
        }
        for (int64_t c = cols; c < kp; ++c) q[r * ldq + c] = 0x00;
        for (int64_t b = nb; b < kp / 32; ++b) e[r * lde + b] = 127;
    }
}

/* Column-wise MX: blocks of 32 along the row axis, written transposed:
 * qT is cols x ldqT, eT is cols x ldeT, padding as for the row-wise copy. */
ORACLE_API void ora_mx_quant_cols(const float* x, int64_t rows, int64_t cols, int64_t ldx,
                                  uint8_t* qT, int64_t ldqT, uint8_t* eT, int64_t ldeT)
{
    e4m3_build();
    int64_t nb = (rows + 31) / 32;
    int64_t kp = (rows + 127) / 128 * 128;
    #pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; ++c) {
        for (int64_t b = 0; b < nb; ++b) {
            int64_t r0 = 32 * b, r1 = r0 + 32 < rows ? r0 + 32 : rows;
            float amax = 0.0f;
            for (int64_t r = r0; r < r1; ++r) {
                float a = fabsf(x[r * ldx + c]);
                if (a > amax) amax = a;
            }
            int k = mx_exponent(amax);
            eT[c * ldeT + b] = (uint8_t)(k + 127);
            double inv = ldexp(1.0, -k);
            for (int64_t r = r0; r < r1; ++r)
                qT[c * ldqT + r] = ora_e4m3_encode_f64((double)x[r * ldx + c] * inv);
        }
        for (int64_t r = rows; r < kp; ++r) qT[c * ldqT + r] = 0x00;
        for (int64_t b = nb; b < kp / 32; ++b) eT[c * ldeT + b] = 127;
    }
}

/* ------------------------------------------------------------------ */
/* Exact dequantization into fp64.  An E4M3 value has 4 significant bits */
/* and an fp32 scale 24, so each product is exact in binary64.           */
/* ------------------------------------------------------------------ */

/* Per-row groups of `group` along the contiguous axis (1x128: group=128). */
ORACLE_API void ora_deq_rowgroups(const uint8_t* q, int64_t ldq, const float* s, int64_t lds,
                                  int64_t rows, int64_t K, int64_t group, double* out, int64_t ldo)
{
    e4m3_build();
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k)
            out[r * ldo + k] = E4M3[q[r * ldq + k]] * (double)s[r * lds + k / group];
}

/* 128x128 blocks. */
ORACLE_API void ora_deq_128x128(const uint8_t* q, int64_t ldq, const float* s, int64_t lds,
                                int64_t D, int64_t C, double* out, int64_t ldo)
{
    e4m3_build();
    #pragma omp parallel for schedule(static)
    for (int64_t d = 0; d < D; ++d)
        for (int64_t c = 0; c < C; ++c)
            out[d * ldo + c] = E4M3[q[d * ldq + c]] * (double)s[(d / 128) * lds + c / 128];
}

/* MX blocks of 32 along the contiguous axis with E8M0 scales 2^(e-127). */
ORACLE_API void ora_deq_mx(const uint8_t* q, int64_t ldq, const uint8_t* e, int64_t lde,
                           int64_t rows, int64_t K, double* out, int64_t ldo)
{
    e4m3_build();
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t k = 0; k < K; ++k)
            out[r * ldo + k] = E4M3[q[r * ldq + k]] * ldexp(1.0, (int)e[r * lde + k / 32] - 127);
}

/* out[i][j] = sum_k A[i][k] * B[k][j] in fp64, each sum taken in ascending
 * k (the loop order i-k-j adds one product to every out[i][j] per k, so it
 * vectorises across j without reassociating any single sum). */
ORACLE_API void ora_matmul_f64(const double* A, int64_t lda, const double* B, int64_t ldb,
                               int64_t M, int64_t N, int64_t K, double* out, int64_t ldo)
{
    #pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < M; ++i) {
        double* o = out + i * ldo;
        for (int64_t j = 0; j < N; ++j) o[j] = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = A[i * lda + k];
            const double* b = B + k * ldb;
            for (int64_t j = 0; j < N; ++j) o[j] += a * b[j];
        }
    }
}

ORACLE_API int ora_version(void) { return 1; }
