/*
 * mxq_oracle.c -- plain, slow CPU oracle for microscaling quantization and the
 * block-scaled linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the bench's
 * CPU-baseline leg may load this library.  It shares no code, header, table or
 * constant with the HIP path and must never be called by the product path.
 *
 * What it follows (pages, by title and section):
 *  - "NVIDIA量化推理：5步极速优化显存+成功率翻倍", section "MXFP8和NVFP4技术背景解析":
 *    microscaling groups small blocks of values (16 or 32) that share a scale;
 *    MXFP8 is the OCP 8-bit format with E4M3 / E5M2 elements; NVFP4 uses E2M1
 *    elements in blocks of 16 with an FP8 block scale.
 *  - "NVIDIA Blackwell平台FP4量化技术解析与图像生成优化", section 3.1: the runtime
 *    quantizer returns FP4 data, FP8 block scales and an FP32 global scale; the
 *    global scale is FP32, block scales are FP8.
 *  - "FP8量化技术提升SD3.5在低带宽环境下的响应速度", step 2 (quantization mapping):
 *    q = round(x / scale) and x_dequant = q * scale.
 *  - "麦橘超然性能实战分析：float8量化如何提升GPU利用率", section 2.2: E4M3 is
 *    1 sign + 4 exponent + 3 mantissa bits, E5M2 is 1 + 5 + 2.
 *
 * Readings where the pages are silent (each one is listed in the design notes):
 *  - every stored quantity is ONE round-to-nearest-even of its exact real value,
 *    ties to the even code, saturating at the largest finite magnitude;
 *  - the sign bit of every element code is the sign bit of the input;
 *  - MXFP8: E = floor(log2(amax_block)) - emax (emax 8 for E4M3, 15 for E5M2),
 *    clamped to [-127, 127], E = -127 for an all-zero block; scale byte E + 127;
 *  - NVFP4: s_g = RN_fp32(amax_tensor / (6 * 448)) (1 for an all-zero tensor),
 *    S_b = RN_E4M3(amax_block / (6 s_g)), q = RN_E2M1(x / (S_b s_g)),
 *    magnitude 0 when S_b is 0;
 *  - packing: NVFP4 element 2j in the low nibble of byte j; scales row-major.
 *
 * Arithmetic: every quotient is compared, never computed: "num/den >= v" is
 * evaluated as "num >= v*den" with v*den formed in fp64 and checked to be exact
 * (fma residual zero) -- a failed check aborts, it never silently rounds.
 * The GEMM reference sums exact fp64 products in fp64.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_E4M3 = 0, ORC_E5M2 = 1, ORC_E2M1 = 2 };
enum { ORC_EPI_NONE = 0, ORC_EPI_BIAS = 1, ORC_EPI_BIAS_GELU_TANH = 2 };

static void orc_fail(const char* what) {
    fprintf(stderr, "oracle: %s\n", what);
    abort();
}

/* ---------------------------------------------------------------- decoding */

/* bf16: 1 sign, 8 exponent bits (bias 127), 7 mantissa bits; subnormals kept. */
double orc_bf16_value(uint16_t b) {
    int s = (b >> 15) & 1, e = (b >> 7) & 0xFF, m = b & 0x7F;
    double v;
    if (e == 0xFF) return m ? NAN : (s ? -INFINITY : INFINITY);
    if (e == 0) v = ldexp((double)m, -126 - 7);
    else v = ldexp(128.0 + m, e - 127 - 7);
    return s ? -v : v;
}

/* Element formats, decoded from their bit layouts.
 * E4M3 ("fn"): bias 7, exponent field 0 subnormal, magnitude 0x7F is NaN, no Inf.
 * E5M2: bias 15, exponent field 31 is Inf (mantissa 0) / NaN.
 * E2M1: bias 1, exponent field 0 subnormal (step 0.5); no special codes. */
double orc_code_value(int fmt, int code) {
    int ebits, mbits, bias, sbit;
    switch (fmt) {
        case ORC_E4M3: ebits = 4; mbits = 3; bias = 7; break;
        case ORC_E5M2: ebits = 5; mbits = 2; bias = 15; break;
        case ORC_E2M1: ebits = 2; mbits = 1; bias = 1; break;
        default: orc_fail("bad format"); return 0;
    }
    sbit = 1 + ebits + mbits - 1;
    int s = (code >> sbit) & 1;
    int e = (code >> mbits) & ((1 << ebits) - 1);
    int m = code & ((1 << mbits) - 1);
    double v;
    if (fmt == ORC_E4M3 && e == 15 && m == 7) return NAN;
    if (fmt == ORC_E5M2 && e == 31) return m ? NAN : (s ? -INFINITY : INFINITY);
    if (e == 0) v = ldexp((double)m, 1 - bias - mbits);
    else v = ldexp((double)((1 << mbits) + m), e - bias - mbits);
    return s ? -v : v;
}

/* E8M0: 2^(c - 127); c = 255 is NaN. */
double orc_e8m0_value(int c) {
    if (c == 255) return NAN;
    return ldexp(1.0, c - 127);
}

static int fmt_magnitude_bits(int fmt) {
    return fmt == ORC_E2M1 ? 3 : 7;
}

/* ------------------------------------------------ exact comparisons, rounding */

/* a*b in fp64, aborting unless it is exact. */
static double exact_mul(double a, double b) {
    double p = a * b;
    if (!isfinite(p) || fma(a, b, -p) != 0.0 || (p == 0.0 && a != 0.0 && b != 0.0))
        orc_fail("product not exact in fp64");
    return p;
}

/* Finite non-negative values of a format in code order (magnitude codes are
 * monotone in value for these layouts; checked). */
static int finite_table(int fmt, double* vals) {
    int n = 0, nb = fmt_magnitude_bits(fmt);
    for (int c = 0; c < (1 << nb); ++c) {
        double v = orc_code_value(fmt, c);
        if (!isfinite(v)) continue;
        if (n > 0 && !(v > vals[n - 1])) orc_fail("table not increasing");
        if (c != n) orc_fail("finite codes not contiguous from 0");
        vals[n++] = v;
    }
    return n;
}

/* Magnitude code of RNE_sat(num / den), num >= 0, den > 0, both exact fp64,
 * for the value table vals[0..n).  Find v_i <= q < v_{i+1} by bisection,
 * then compare q with the midpoint; a tie goes to the even code.  q at or
 * above the largest value saturates. */
static int round_in_table(const double* vals, int n, double num, double den) {
    if (!(num >= 0.0) || !(den > 0.0)) orc_fail("round_quotient domain");
    if (num >= exact_mul(vals[n - 1], den)) return n - 1;
    /* bisection keeping vals[i] * den <= num < vals[j] * den (vals[0] = 0) */
    int i = 0, j = n - 1;
    while (j - i > 1) {
        int k = (i + j) / 2;
        if (num >= exact_mul(vals[k], den)) i = k; else j = k;
    }
    double mid = 0.5 * (vals[i] + vals[i + 1]);       /* exact: one more bit */
    double mden = exact_mul(mid, den);
    if (num < mden) return i;
    if (num > mden) return i + 1;
    return (i % 2 == 0) ? i : i + 1;
}

int orc_round_quotient(int fmt, double num, double den) {
    double vals[128];
    int n = finite_table(fmt, vals);
    return round_in_table(vals, n, num, den);
}

void orc_round_quotient_array(int fmt, const double* num, double den, int64_t n, uint8_t* out) {
    double vals[128];
    int nv = finite_table(fmt, vals);
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)round_in_table(vals, nv, num[i], den);
}

/* a - b, aborting unless it is exact (TwoSum error term zero). */
static double exact_sub(double a, double b) {
    double s = a - b;
    double bv = s - a;
    double err = (a - (s - bv)) + (-b - bv);
    if (err != 0.0) orc_fail("difference not exact in fp64");
    return s;
}

/* RN_fp32(a / d) for a >= 0, d > 0 exact: among the fp32 neighbours of an fp64
 * estimate, take the one whose multiple of d lies closest to a (distances are
 * exact fp64), ties to the even fp32 encoding. */
float orc_rn_fp32_div(double a, double d) {
    float f = (float)(a / d);
    float cand[3] = {nextafterf(f, 0.0f), f, nextafterf(f, INFINITY)};
    float best = cand[0];
    double bestd = -1.0;
    for (int k = 0; k < 3; ++k) {
        double dist = fabs(exact_sub(a, exact_mul(d, (double)cand[k])));
        uint32_t bits;
        memcpy(&bits, &cand[k], 4);
        if (bestd < 0.0 || dist < bestd || (dist == bestd && (bits & 1u) == 0)) {
            best = cand[k];
            bestd = dist;
        }
    }
    return best;
}

/* ------------------------------------------------------------------ MXFP8 */

/* Quantize bf16 x[rows, cols] (row-major, blocks of 32 along cols) into codes
 * q[rows, cols] and E8M0 scales[rows, cols/32].  fmt: ORC_E4M3 or ORC_E5M2. */
int orc_quantize_mxfp8(const uint16_t* x, int64_t rows, int64_t cols, int fmt,
                       uint8_t* q, uint8_t* scales) {
    if (cols % 32 != 0 || (fmt != ORC_E4M3 && fmt != ORC_E5M2)) return -1;
    const int emax = (fmt == ORC_E4M3) ? 8 : 15;   /* exponent of the largest finite value */
    const int64_t nb = cols / 32;
    double vals[128];
    const int nv = finite_table(fmt, vals);
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint16_t* xb = x + r * cols + b * 32;
            double amax = 0.0;
            for (int i = 0; i < 32; ++i) amax = fmax(amax, fabs(orc_bf16_value(xb[i])));
            int E;
            if (amax == 0.0) E = -127;
            else {
                int e2;
                frexp(amax, &e2);                  /* amax = f * 2^e2, f in [0.5, 1) */
                E = (e2 - 1) - emax;               /* floor(log2 amax) - emax */
                if (E < -127) E = -127;
                if (E > 127) E = 127;
            }
            scales[r * nb + b] = (uint8_t)(E + 127);
            double den = ldexp(1.0, E);
            for (int i = 0; i < 32; ++i) {
                double v = orc_bf16_value(xb[i]);
                int mag = round_in_table(vals, nv, fabs(v), den);
                int sign = (xb[i] >> 15) & 1;
                q[r * cols + b * 32 + i] = (uint8_t)(mag | (sign << 7));
            }
        }
    }
    return 0;
}

/* ------------------------------------------------------------------ NVFP4 */

/* The dynamic per-tensor decode scale: RN_fp32(amax / 2688), 1 for all-zero. */
float orc_nvfp4_global_scale(const uint16_t* x, int64_t n) {
    double amax = 0.0;
    for (int64_t i = 0; i < n; ++i) amax = fmax(amax, fabs(orc_bf16_value(x[i])));
    if (amax == 0.0) return 1.0f;
    return orc_rn_fp32_div(amax, 6.0 * 448.0);
}

/* Weight-only FP8 (page "麦橘超然性能实战分析：float8量化如何提升GPU利用率",
 * section 3.2: the DiT weights are loaded as float8_e4m3fn while activations stay
 * bf16, and section 4 / page "FP8量化技术提升SD3.5在低带宽环境下的响应速度", step 2:
 * q = round(w / scale), dequantized as q * scale; the product runs in bf16).
 * Per-tensor decode scale s = RN_fp32(amax / 448) (1 for an all-zero tensor) or
 * the given one; q = RN_E4M3,sat(w / s), sign copied. */
float orc_fp8_tensor_scale(const uint16_t* x, int64_t n) {
    double amax = 0.0;
    for (int64_t i = 0; i < n; ++i) amax = fmax(amax, fabs(orc_bf16_value(x[i])));
    if (amax == 0.0) return 1.0f;
    return orc_rn_fp32_div(amax, 448.0);
}

int orc_quantize_fp8_tensor(const uint16_t* x, int64_t rows, int64_t cols, const float* scale_in,
                            uint8_t* q, float* scale_out) {
    const float s = scale_in ? *scale_in : orc_fp8_tensor_scale(x, rows * cols);
    if (!(s > 0.0f) || !isfinite(s)) return -2;
    *scale_out = s;
    double v43[128];
    const int n43 = finite_table(ORC_E4M3, v43);
    const double sd = (double)s;
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t c = 0; c < cols; ++c) {
            const uint16_t b = x[r * cols + c];
            const int mag = round_in_table(v43, n43, fabs(orc_bf16_value(b)), sd);
            q[r * cols + c] = (uint8_t)(mag | (((b >> 15) & 1) << 7));
        }
    }
    return 0;
}

/* Static-scale calibration (page "FP8量化技术提升SD3.5在低带宽环境下的响应速度",
 * step 1: record each layer's maximum over a calibration batch and set the scale
 * so that nothing is truncated).  Folds one calibration tensor into the running
 * decode scale: max(running, RN_fp32(amax / 2688)); an all-zero tensor adds 0. */
float orc_nvfp4_calibrate(const uint16_t* x, int64_t n, float running) {
    double amax = 0.0;
    for (int64_t i = 0; i < n; ++i) amax = fmax(amax, fabs(orc_bf16_value(x[i])));
    const float s = amax == 0.0 ? 0.0f : orc_rn_fp32_div(amax, 6.0 * 448.0);
    return s > running ? s : running;
}

/* Quantize bf16 x[rows, cols] (blocks of 16 along cols) into packed E2M1 codes
 * q[rows, cols/2] (element 2j low nibble), E4M3 block scales[rows, cols/16] and
 * the fp32 global decode scale.  global_in: NULL for the dynamic scale, else
 * the static scale to use (must be positive and finite). */
int orc_quantize_nvfp4(const uint16_t* x, int64_t rows, int64_t cols, const float* global_in,
                       uint8_t* q, uint8_t* scales, float* global_out) {
    if (cols % 16 != 0) return -1;
    float sg = global_in ? *global_in : orc_nvfp4_global_scale(x, rows * cols);
    if (!(sg > 0.0f) || !isfinite(sg)) return -2;
    *global_out = sg;
    const double sgd = (double)sg;
    const double six_sg = exact_mul(6.0, sgd);
    const int64_t nb = cols / 16;
    double v43[128], v21[16];
    const int n43 = finite_table(ORC_E4M3, v43), n21 = finite_table(ORC_E2M1, v21);
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < nb; ++b) {
            const uint16_t* xb = x + r * cols + b * 16;
            double amax = 0.0;
            for (int i = 0; i < 16; ++i) amax = fmax(amax, fabs(orc_bf16_value(xb[i])));
            int sb = round_in_table(v43, n43, amax, six_sg);
            scales[r * nb + b] = (uint8_t)sb;
            double S = orc_code_value(ORC_E4M3, sb);
            uint8_t nib[16];
            for (int i = 0; i < 16; ++i) {
                int sign = (xb[i] >> 15) & 1;
                int mag = 0;
                if (S > 0.0) mag = round_in_table(v21, n21, fabs(orc_bf16_value(xb[i])), exact_mul(S, sgd));
                nib[i] = (uint8_t)(mag | (sign << 3));
            }
            for (int j = 0; j < 8; ++j)
                q[r * (cols / 2) + b * 8 + j] = (uint8_t)(nib[2 * j] | (nib[2 * j + 1] << 4));
        }
    }
    return 0;
}

/* -------------------------------------------------------------- dequantize */

/* Rows row_idx[0..n_rows) (all rows when row_idx is NULL) of an MXFP8 operand
 * [*, cols] to fp64: val(q) * 2^(scale - 127). */
void orc_dequant_mxfp8(const uint8_t* q, const uint8_t* scales, int64_t cols, int fmt,
                       const int64_t* row_idx, int64_t n_rows, double* out) {
    const int64_t nb = cols / 32;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t r = row_idx ? row_idx[i] : i;
        for (int64_t k = 0; k < cols; ++k)
            out[i * cols + k] = orc_code_value(fmt, q[r * cols + k]) * orc_e8m0_value(scales[r * nb + k / 32]);
    }
}

/* Rows of an NVFP4 operand to fp64: val(q) * val_E4M3(S_b) * s_g. */
void orc_dequant_nvfp4(const uint8_t* q, const uint8_t* scales, float global_scale, int64_t cols,
                       const int64_t* row_idx, int64_t n_rows, double* out) {
    const int64_t nb = cols / 16;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n_rows; ++i) {
        int64_t r = row_idx ? row_idx[i] : i;
        for (int64_t k = 0; k < cols; ++k) {
            uint8_t byte = q[r * (cols / 2) + k / 2];
            int code = (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);
            double S = orc_code_value(ORC_E4M3, scales[r * nb + k / 16]);
            out[i * cols + k] = orc_code_value(ORC_E2M1, code) * S * (double)global_scale;
        }
    }
}

/* --------------------------------------------------------------- the linear */

static double gelu_tanh(double x) {
    const double c = sqrt(2.0 / M_PI);
    return 0.5 * x * (1.0 + tanh(c * (x + 0.044715 * x * x * x)));
}

/* out[m, n] = epi(alpha * sum_k a[m, k] * w[n, k] + bias[n]) in fp64, with
 * a [n_rows, K] and w [N, K] dequantized operands (nn.Linear orientation).
 * bias: bf16 [N] or NULL.  epi: 0 none, 1 bias, 2 bias then GELU (tanh form). */
void orc_linear(const double* a, const double* w, double alpha, const uint16_t* bias, int epi,
                int64_t n_rows, int64_t N, int64_t K, double* out) {
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < n_rows; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k) acc += a[m * K + k] * w[n * K + k];
            double y = alpha * acc;
            if (epi >= ORC_EPI_BIAS) y += orc_bf16_value(bias[n]);
            if (epi == ORC_EPI_BIAS_GELU_TANH) y = gelu_tanh(y);
            out[m * N + n] = y;
        }
    }
}

int orc_max_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void orc_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
