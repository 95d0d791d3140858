/* sanitize_check.c -- TEST INFRASTRUCTURE: runs every function of the CPU
 * oracle (fp8_oracle.c, included below) on small ragged inputs held in
 * buffers of exactly the documented sizes, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (gcc -fsanitize=address,
 * undefined).  An out-of-bounds access, use of freed memory, signed overflow,
 * bad shift or misaligned access aborts the run with a report; the checks
 * below only assert a few results so that the calls are not dead code.  Run
 * by tests/test_oracle_sanitized.py. */
#include "fp8_oracle.c"

#include <assert.h>
#include <stdio.h>

static float* fbuf(int64_t n, uint64_t* st) {
    float* p = (float*)malloc((size_t)(n > 0 ? n : 1) * sizeof(float));
    for (int64_t i = 0; i < n; ++i) {          /* xorshift64: deterministic values of varied magnitude */
        *st ^= *st << 13; *st ^= *st >> 7; *st ^= *st << 17;
        const double u = (double)(*st >> 11) / 9007199254740992.0 - 0.5;
        p[i] = (float)(u * ldexp(1.0, (int)(*st % 40) - 20));
    }
    return p;
}

static uint8_t* bbuf(int64_t n) { return (uint8_t*)malloc((size_t)(n > 0 ? n : 1)); }
static int64_t rup(int64_t n, int64_t m) { return (n + m - 1) / m * m; }
static int64_t cdv(int64_t n, int64_t m) { return (n + m - 1) / m; }

static void one_shape(int64_t rows, int64_t cols, uint64_t* st) {
    const int64_t kp = rup(cols, 128), kr = rup(rows, 128);
    float* x = fbuf(rows * cols, st);
    if (rows > 2 && cols > 0) { x[0] = 0.0f; x[1] = -0.0f; x[cols] = 3.4e38f; x[2 * cols] = 1e-45f; }

    uint8_t* q = bbuf(rows * kp);
    float* s = (float*)malloc((size_t)(rows * cdv(cols, 128) > 0 ? rows * cdv(cols, 128) : 1) * sizeof(float));
    ora_quant_1x128(x, rows, cols, cols, q, kp, s, cdv(cols, 128));
    ora_quant_1x128_p2(x, rows, cols, cols, q, kp, s, cdv(cols, 128));

    uint8_t* wq = bbuf(rows * kp);
    uint8_t* wqT = bbuf(cols * kr);
    float* ws = (float*)malloc((size_t)(cdv(rows, 128) * cdv(cols, 128) > 0 ? cdv(rows, 128) * cdv(cols, 128) : 1) * sizeof(float));
    ora_quant_128x128(x, rows, cols, cols, wq, kp, ws, cdv(cols, 128), wqT, kr);
    ora_quant_128x128_p2(x, rows, cols, cols, wq, kp, ws, cdv(cols, 128), NULL, 0);

    uint8_t* qT = bbuf(cols * kr);
    float* sT = (float*)malloc((size_t)(cols * cdv(rows, 128) > 0 ? cols * cdv(rows, 128) : 1) * sizeof(float));
    ora_quant_colwise(x, rows, cols, cols, NULL, 0, qT, kr, sT, cdv(rows, 128));
    ora_quant_colwise_p2(x, rows, cols, cols, NULL, 0, qT, kr, sT, cdv(rows, 128));
    ora_requant_colwise(q, kp, s, cdv(cols, 128), rows, cols, NULL, 0, qT, kr, sT, cdv(rows, 128));

    /* grouped: segments of 0, 1, rest (and an empty last one); padded extent */
    if (rows >= 1) {
        int32_t offs[5] = {0, 0, 1, (int32_t)rows, (int32_t)rows};
        int64_t P = 0;
        for (int e = 0; e < 4; ++e) P += rup(offs[e + 1] - offs[e], 128);
        uint8_t* gT = bbuf(cols * P);
        float* gsT = (float*)malloc((size_t)(cols * (P / 128) > 0 ? cols * (P / 128) : 1) * sizeof(float));
        ora_quant_colwise(x, rows, cols, cols, offs, 4, gT, P, gsT, P / 128);
        ora_requant_colwise(q, kp, s, cdv(cols, 128), rows, cols, offs, 4, gT, P, gsT, P / 128);
        free(gT); free(gsT);
    }

    uint8_t* mq = bbuf(rows * kp);
    uint8_t* me = bbuf(rows * (kp / 32));
    ora_mx_quant_rows(x, rows, cols, cols, mq, kp, me, kp / 32);
    uint8_t* mqT = bbuf(cols * kr);
    uint8_t* meT = bbuf(cols * (kr / 32));
    ora_mx_quant_cols(x, rows, cols, cols, mqT, kr, meT, kr / 32);

    double* d = (double*)malloc((size_t)(rows * cols > 0 ? rows * cols : 1) * sizeof(double));
    ora_deq_rowgroups(q, kp, s, cdv(cols, 128), rows, cols, 128, d, cols);
    ora_deq_128x128(wq, kp, ws, cdv(cols, 128), rows, cols, d, cols);
    ora_deq_mx(mq, kp, me, kp / 32, rows, cols, d, cols);

    double* out = (double*)malloc((size_t)(rows * rows > 0 ? rows * rows : 1) * sizeof(double));
    double* dT = (double*)malloc((size_t)(rows * cols > 0 ? rows * cols : 1) * sizeof(double));
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) dT[c * rows + r] = d[r * cols + c];
    ora_matmul_f64(d, cols, dT, rows, rows, rows, cols, out, rows);

    free(x); free(q); free(s); free(wq); free(wqT); free(ws); free(qT); free(sT);
    free(mq); free(me); free(mqT); free(meT); free(d); free(out); free(dT);
}

int main(void) {
    uint64_t st = 0x9E3779B97F4A7C15ull;
    for (int c = 0; c < 256; ++c) {
        const double v = ora_e4m3_decode(c);
        if (c != 0x7F && c != 0xFF) assert(ora_e4m3_encode((float)v) == (c == 0x80 ? 0x80 : c));
    }
    float xs[6] = {448.0f, 464.0f, 1e30f, -1e-10f, 0.0f, 1.5f * 0.001953125f};
    uint8_t codes[6];
    ora_e4m3_encode_array(xs, 6, codes);
    assert(codes[0] == 0x7E && codes[1] == 0x7E && codes[2] == 0x7E && codes[3] == 0x80 && codes[5] == 0x02);
    assert(ora_mx_exponent(448.0f) == 0 && ora_mx_exponent(0.0f) == -127);
    const int64_t shapes[][2] = {{0, 0}, {1, 1}, {3, 130}, {129, 257}, {300, 5}, {256, 384}, {5, 0}, {0, 7}};
    for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i) one_shape(shapes[i][0], shapes[i][1], &st);
    printf("oracle sanitizer run: ok\n");
    return 0;
}
