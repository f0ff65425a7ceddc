/*
 * Driver for the sanitizer run of the CPU oracle: builds the oracle source into
 * this program (one translation unit) and calls every exported function on
 * small inputs that reach its edge cases -- zeros and negative zeros, bf16
 * subnormals, saturating outliers, all-zero blocks, a static global scale, both
 * element formats, row subsets and all three epilogues.  Compiled with
 * -fsanitize=address,undefined by tests/test_oracle_sanitize.py; any report
 * aborts with a non-zero status.  Prints "sanitize ok" at the end.
 */
#include "../oracle/mxq_oracle.c"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;

static uint64_t next_u64(void) {
    /* SplitMix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

/* A bf16 tensor with every kind of value the quantizers treat specially. */
static void fill(uint16_t* x, int64_t n) {
    for (int64_t i = 0; i < n; ++i) {
        uint16_t b = (uint16_t)(next_u64() & 0xFFFF);
        if (((b >> 7) & 0xFF) == 0xFF) b &= 0x807F;          /* no Inf / NaN */
        switch (i % 97) {
            case 0: b = 0x0000; break;                           /* +0 */
            case 1: b = 0x8000; break;                           /* -0 */
            case 2: b = 0x0001; break;                           /* smallest subnormal */
            case 3: b = 0x7F7F; break;                           /* largest finite */
            default: b = (uint16_t)((b & 0x807F) | (((b >> 7) % 24 + 112) << 7)); /* moderate */
        }
        x[i] = b;
    }
    for (int64_t i = 64; i < 96 && i < n; ++i) x[i] = (i & 1) ? 0x8000 : 0x0000;   /* an all-zero block */
}

int main(void) {
    const int64_t rows = 6, cols = 128, n = rows * cols, N = 4;
    uint16_t* x = malloc(n * sizeof *x);
    uint8_t* q8 = malloc(n);
    uint8_t* s8 = malloc(n / 32);
    uint8_t* q4 = malloc(n / 2);
    uint8_t* s4 = malloc(n / 16);
    uint8_t* qw = malloc(n);
    double* deq = malloc(n * sizeof *deq);
    double* w = malloc(N * cols * sizeof *w);
    double* out = malloc(rows * N * sizeof *out);
    uint16_t bias[4] = {0x3F80, 0xBF80, 0x0000, 0x4000};
    int64_t idx[3] = {5, 0, 3};
    double num[5] = {0.0, 0.25, 17.6, 1e6, 3.5};
    uint8_t codes[5];
    float g = 0.0f, gin = 0.0625f, s = 0.0f;
    fill(x, n);

    for (int fmt = ORC_E4M3; fmt <= ORC_E5M2; ++fmt) {
        if (orc_quantize_mxfp8(x, rows, cols, fmt, q8, s8) != 0) return 2;
        orc_dequant_mxfp8(q8, s8, cols, fmt, NULL, rows, deq);
        orc_dequant_mxfp8(q8, s8, cols, fmt, idx, 3, deq);
    }
    if (orc_quantize_nvfp4(x, rows, cols, NULL, q4, s4, &g) != 0) return 3;
    orc_dequant_nvfp4(q4, s4, g, cols, NULL, rows, deq);
    if (orc_quantize_nvfp4(x, rows, cols, &gin, q4, s4, &g) != 0) return 4;
    orc_dequant_nvfp4(q4, s4, g, cols, idx, 3, deq);
    if (orc_quantize_fp8_tensor(x, rows, cols, NULL, qw, &s) != 0) return 5;
    if (orc_quantize_fp8_tensor(x, rows, cols, &gin, qw, &s) != 0) return 6;
    (void)orc_nvfp4_calibrate(x, n, 0.0f);
    (void)orc_nvfp4_global_scale(x, n);
    (void)orc_fp8_tensor_scale(x, n);
    for (int64_t i = 0; i < N * cols; ++i) w[i] = orc_code_value(ORC_E2M1, (int)(i % 16)) * 0.125;
    for (int epi = ORC_EPI_NONE; epi <= ORC_EPI_BIAS_GELU_TANH; ++epi)
        orc_linear(deq, w, 0.5, bias, epi, 3, N, cols, out);
    orc_round_quotient_array(ORC_E4M3, num, 0.125, 5, codes);
    (void)orc_round_quotient(ORC_E2M1, 5.0, 2.0);
    (void)orc_rn_fp32_div(1.0, 2688.0);
    for (int c = 0; c < 256; ++c) {
        (void)orc_code_value(ORC_E4M3, c);
        (void)orc_code_value(ORC_E5M2, c);
        (void)orc_e8m0_value(c);
        (void)orc_bf16_value((uint16_t)(c << 8));
    }
    orc_set_threads(orc_max_threads());
    free(x); free(q8); free(s8); free(q4); free(s4); free(qw); free(deq); free(w); free(out);
    printf("sanitize ok\n");
    return 0;
}
