/*
 * hif4_oracle.c -- plain, slow CPU oracle for the HiF4 W4A4 hot path.
 *
 * TEST INFRASTRUCTURE. Only the test suite, the smoke entry point and the
 * cpu_baseline leg of the benchmark may load this code. The product path
 * (the HIP library) never calls it and shares no source with it.
 *
 * Sources (cited by page title and section throughout):
 *  [HiF4-fmt]  HiFloat4 calibration article (hwcomputing.csdn.net),
 *              section "一：HiFloat4 (HiF4) 格式": the 64-element unit, the
 *              E6M2 level-1 scale, the E1 level-2 (per 8) and level-3
 *              (per 4) micro-exponents, the S1P2 element and its value set,
 *              and the 32-bit metadata budget.
 *  [HiGPTQ]    same article, section 3.1 "HiGPTQ": exponents named 1-0,
 *              2-(0..7), 3-(0..15) in column order, each fixed from
 *              statistics of the data it covers.
 *  [HiFlat]    same article, section 3.3 "HiFlatQuant": HiF4's range is wide
 *              enough that no clipping thresholds are needed.
 *  [HiAR]      same article, section 3.2 "HiAutoRound": learnable offsets K
 *              (16 per unit, added to the level-3 exponents, E' = E + RZ(K))
 *              and M (mantissa compensation, shifted M' = M >> RZ(K) before
 *              it is added), and the quantize step of its training loop.
 *  [TA-method] "Tail-Aware HiFloat4: W4A4 PTQ calibration for Wan2.2"
 *              (agents-report.net), sections "方法概述" and
 *              "尾部百分位統計的動機": per-channel tail percentile statistics
 *              of the activations build a channel-protection mask.
 *  [TA-abs]    arXiv 2605.26628 record, abstract: W4A4 HiFloat4 fake
 *              quantization of the main linear layers.
 *  GPTQ        Frantar et al., "GPTQ: Accurate Post-Training Quantization
 *              for Generative Pre-trained Transformers" (2022): the
 *              published error-compensation update HiGPTQ adapts.
 *
 * The element formula of [HiF4-fmt] is an image that did not survive; the
 * readings this file takes where the pages are silent are marked READING.
 *
 * Build: gcc -O2 -ffp-contract=off -fopenmp -fPIC -shared (oracle/build.py).
 * Floating point is IEEE double; every comparison below is between values
 * that are exact in double, so the encoder decisions are exact on reals.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define HIF4O_OK 0
#define HIF4O_ERR_ARG 1
#define HIF4O_ERR_NONFINITE 2

#define UNIT 64 /* [HiF4-fmt]: one HiF4 unit groups 64 elements */

/* ---------------------------------------------------------------- formats */

/* bf16 bit pattern -> its exact value as a double. */
static double bf16_value(uint16_t bits)
{
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* Level-1 scale, E6M2 ([HiF4-fmt]: 6 exponent bits, 2 mantissa bits).
 * READING: unsigned code c in 0..255, exponent field c>>2 with bias 31,
 * every code normal (no zero / Inf / NaN): v(c) = 2^(c>>2 - 31) * (1 + (c&3)/4). */
double hif4o_e6m2_value(int c)
{
    return ldexp(1.0 + (double)(c & 3) / 4.0, (c >> 2) - 31);
}

/* E1 micro-exponent ([HiF4-fmt]: power-of-two scaling inside the unit).
 * READING: bit b multiplies by 2^b. */
static double e1_factor(int b) { return b ? 2.0 : 1.0; }

/* READING (code layout). Unit u of a row owns bytes [32u, 32u+32) of the row's
 * codes. Element j of the unit lives in byte 4*(j/8) + (j%4); it is the low
 * nibble when (j%8) < 4 and the high nibble otherwise. So the 32-bit word w of
 * the unit holds level-2 group w ([HiGPTQ] order along K): its low nibbles are
 * level-3 group 2w, its high nibbles level-3 group 2w+1.
 * meta = c | e2bits << 8 | e3bits << 16, bit g of e2bits for elements 8g..8g+7,
 * bit q of e3bits for elements 4q..4q+3: 8 + 8 + 16 = 32 bits ([HiF4-fmt]). */
static int code_byte(int j) { return 4 * (j / 8) + (j % 4); }
static int code_shift(int j) { return (j % 8) < 4 ? 0 : 4; }

/* S1P2 nibble ([HiF4-fmt]): sign bit, one integer bit, two fraction bits.
 * READING: sign = bit 3, magnitude k/4 with k = nibble & 7 (integer bit k>>2,
 * fraction bits k&3), so |value| is one of 0, 0.25, ..., 1.75. */
static double s1p2_value(int nib)
{
    double mag = (double)(nib & 7) / 4.0;
    return (nib & 8) ? -mag : mag;
}

/* ------------------------------------------------------------ quantize */

/* Encode one 64-element unit. x[] are exact reals (bf16 values read as
 * doubles; masked entries already replaced by 0).
 * READING (the encoding rule; [HiGPTQ] fixes each exponent from the data it
 * covers, [HiFlat] says no clipping is needed): choose every scale as small
 * as it can be without any element exceeding its grid maximum, then round
 * each element to the nearest grid point, ties to even. */
/* Steps 1-4 of the unit encoding: the level-1 code c and the level-2 and
 * level-3 bits, each from the maxima of the values it covers. */
static void unit_scales(const double x[UNIT], int *c_out, int e2[8], int e3[16])
{
    /* step 1: the maxima of |x| over the unit, each level-2 group (8) and
     * each level-3 group (4). */
    double A = 0.0, M8[8], M4[16];
    for (int g = 0; g < 8; ++g) M8[g] = 0.0;
    for (int q = 0; q < 16; ++q) M4[q] = 0.0;
    for (int j = 0; j < UNIT; ++j) {
        double a = fabs(x[j]);
        if (a > A) A = a;
        if (a > M8[j / 8]) M8[j / 8] = a;
        if (a > M4[j / 4]) M4[j / 4] = a;
    }

    /* step 2: level-1 code = the smallest c whose largest representable
     * magnitude, 1.75 * 2 * 2 * v(c) = 7 v(c), is at least A. If no code
     * reaches A the range saturates at c = 255. */
    int c = 255;
    for (int cc = 0; cc < 256; ++cc) {
        if (7.0 * hif4o_e6m2_value(cc) >= A) {
            c = cc;
            break;
        }
    }
    double s = hif4o_e6m2_value(c);

    /* step 3: level-2 bit of group g is set iff the group does not fit
     * under 1.75 * 2 * s (its largest magnitude with e2 = 0). */
    for (int g = 0; g < 8; ++g) e2[g] = M8[g] > 1.75 * 2.0 * s;

    /* step 4: level-3 bit of group q is set iff the group does not fit
     * under 1.75 * 2^e2 * s (its largest magnitude with e3 = 0). */
    for (int q = 0; q < 16; ++q) e3[q] = M4[q] > 1.75 * e1_factor(e2[q / 2]) * s;
    *c_out = c;
}

static void quantize_unit(const double x[UNIT], uint8_t codes[32], uint32_t *meta)
{
    int c, e2[8], e3[16];
    unit_scales(x, &c, e2, e3);
    double s = hif4o_e6m2_value(c);

    /* step 5: round |x| onto the grid {k D / 4 : k = 0..7}, D = s 2^e2 2^e3,
     * to nearest with ties to even k. The grid midpoints are (2m+1) D / 8;
     * k counts the midpoints strictly below |x|; at a midpoint the even
     * neighbour wins. Beyond the last midpoint k stays 7 (saturation). */
    memset(codes, 0, 32);
    for (int j = 0; j < UNIT; ++j) {
        double D = s * e1_factor(e2[j / 8]) * e1_factor(e3[j / 4]);
        double a = fabs(x[j]);
        int k = 0;
        for (int m = 0; m < 7; ++m) {
            double mid = (double)(2 * m + 1) * D / 8.0;
            if (a > mid) {
                k = m + 1;
            } else {
                if (a == mid) k = (m % 2 == 0) ? m : m + 1;
                break;
            }
        }
        /* READING: zero is always +0 (no sign on a zero element). */
        int sign = (x[j] < 0.0) && (k != 0);
        int nib = k | (sign << 3);
        codes[code_byte(j)] |= (uint8_t)(nib << code_shift(j));
    }

    uint32_t m = (uint32_t)c;
    for (int g = 0; g < 8; ++g) m |= (uint32_t)e2[g] << (8 + g);
    for (int q = 0; q < 16; ++q) m |= (uint32_t)e3[q] << (16 + q);
    *meta = m;
}

/* x: bf16 bits [rows][ld], k % 64 == 0. codes: [rows][k/2], meta: [rows][k/64].
 * mask: NULL or u8 [k]; nonzero = protected channel. Protected entries are
 * encoded as 0 and their bf16 bits copied, in ascending channel order, to
 * kept [rows][n_mask] ([TA-method]: protected channels stay high precision).
 * Returns HIF4O_ERR_NONFINITE if any (unprotected) input is Inf or NaN. */
int hif4o_quantize(const uint16_t *x, int64_t rows, int64_t k, int64_t ld,
                   const uint8_t *mask, int64_t n_mask, uint16_t *kept,
                   uint8_t *codes, uint32_t *meta)
{
    if (rows < 0 || k < 0 || k % UNIT != 0 || ld < k) return HIF4O_ERR_ARG;
    if (mask) {
        int64_t cnt = 0;
        for (int64_t i = 0; i < k; ++i) cnt += mask[i] != 0;
        if (cnt != n_mask || (n_mask > 0 && !kept)) return HIF4O_ERR_ARG;
    }
    int64_t units = k / UNIT;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < rows; ++r) {
        const uint16_t *xr = x + r * ld;
        int64_t kp = 0;
        for (int64_t u = 0; u < units; ++u) {
            double v[UNIT];
            for (int j = 0; j < UNIT; ++j) {
                int64_t ch = u * UNIT + j;
                double val = bf16_value(xr[ch]);
                if (mask && mask[ch]) {
                    kept[r * n_mask + kp++] = xr[ch];
                    val = 0.0;
                } else if (!isfinite(val)) {
                    bad = 1;
                    val = 0.0;
                }
                v[j] = val;
            }
            quantize_unit(v, codes + r * (k / 2) + u * 32, meta + r * units + u);
        }
    }
    return bad ? HIF4O_ERR_NONFINITE : HIF4O_OK;
}

/* ------------------------------------------------- HiAutoRound offsets */

/* The quantize step of [HiAR] with given offsets (the training loop that
 * learns them is out of scope). Per unit: c and the level-2 bits as in
 * hif4o_quantize; each level-3 bit e3 of the 16 groups, then its offset.
 * READINGS ([HiAR] gives the two formulas only):
 *  - K and M are real-valued. K has one entry per level-3 group, K [rows][k/4];
 *    M one per element ("independent mantissa" in the section's comparison),
 *    M [rows][k].
 *  - RZ is rounding toward zero. The level-3 exponent is a 1-bit field, so
 *    e3' = e3 + RZ(K) is held to {0, 1}.
 *  - "M >> RZ(K)" on a real M is M * 2^-d with d = e3' - e3, the change of
 *    the exponent actually applied: that is what keeps M' on the scale of
 *    the element's new step, the continuity the section asks for.
 *  - M' is added to the element's magnitude in units of its step (as
 *    AutoRound adds its rounding offset to W / s), then rounded to the
 *    nearest k, ties to even, held to 0..7; the sign is kept; a zero element
 *    has no sign.
 *  - Precision: the decision is taken in IEEE binary32, as the kernel takes
 *    it: t = fl(|x| / (D / 4)) with D = s 2^(e2 + e3') (exact in binary32),
 *    u = fl(t + M'), k = rint(u). For bf16 x, fl(t) never crosses a
 *    rounding tie (t has at most 8 significant bits over a divisor of
 *    4 + m), so with K = 0 and M = 0 this is exactly hif4o_quantize. */
static int offset_e3(int e3, float K)
{
    float t = (float)e3 + truncf(K);
    return t >= 1.0f ? 1 : 0; /* t is a whole number; NaN gives 0 */
}

int hif4o_quantize_offsets(const uint16_t *x, int64_t rows, int64_t k, int64_t ld,
                           const float *koff, const float *moff, uint8_t *codes,
                           uint32_t *meta)
{
    if (rows < 0 || k < 0 || k % UNIT != 0 || ld < k) return HIF4O_ERR_ARG;
    int64_t units = k / UNIT;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t u = 0; u < units; ++u) {
            double v[UNIT];
            for (int j = 0; j < UNIT; ++j) {
                double val = bf16_value(x[r * ld + u * UNIT + j]);
                if (!isfinite(val)) {
                    bad = 1;
                    val = 0.0;
                }
                v[j] = val;
            }
            int c, e2[8], e3[16];
            unit_scales(v, &c, e2, e3);
            const float *ku = koff + r * (k / 4) + u * 16;
            const float *mu = moff + r * k + u * UNIT;
            int e3n[16];
            for (int q = 0; q < 16; ++q) e3n[q] = offset_e3(e3[q], ku[q]);
            float s = (float)hif4o_e6m2_value(c); /* exact in binary32 */
            uint8_t *uc = codes + r * (k / 2) + u * 32;
            memset(uc, 0, 32);
            for (int j = 0; j < UNIT; ++j) {
                int q = j / 4;
                float D = ldexpf(s, e2[j / 8] + e3n[q]);
                float ax = (float)fabs(v[j]); /* exact: v is a bf16 value */
                int d = e3n[q] - e3[q];
                float mp = d > 0 ? mu[j] * 0.5f : (d < 0 ? mu[j] * 2.0f : mu[j]);
                float t = ax / (D * 0.25f);
                float uu = t + mp;
                int kk = 0;
                if (uu > 0.0f) {
                    float rr = rintf(uu);
                    kk = rr >= 7.0f ? 7 : (int)rr;
                }
                int sign = (v[j] < 0.0) && (kk != 0);
                uc[code_byte(j)] |= (uint8_t)((kk | (sign << 3)) << code_shift(j));
            }
            uint32_t m = (uint32_t)c;
            for (int g = 0; g < 8; ++g) m |= (uint32_t)e2[g] << (8 + g);
            for (int q = 0; q < 16; ++q) m |= (uint32_t)e3n[q] << (16 + q);
            meta[r * units + u] = m;
        }
    }
    return bad ? HIF4O_ERR_NONFINITE : HIF4O_OK;
}

/* ---------------------------------------------------------- dequantize */

/* The value of element j of a unit (READING of the lost element formula):
 * x = S1P2(nibble) * 2^e2[j/8] * 2^e3[j/4] * v(c). */
static double unit_element(const uint8_t *ucodes, uint32_t m, int j)
{
    int nib = (ucodes[code_byte(j)] >> code_shift(j)) & 15;
    int c = (int)(m & 255u);
    int e2 = (int)((m >> (8 + j / 8)) & 1u);
    int e3 = (int)((m >> (16 + j / 4)) & 1u);
    return s1p2_value(nib) * e1_factor(e2) * e1_factor(e3) * hif4o_e6m2_value(c);
}

/* codes [rows][k/2], meta [rows][k/64] -> out [rows][k] as doubles. */
int hif4o_dequantize(const uint8_t *codes, const uint32_t *meta, int64_t rows, int64_t k,
                     double *out)
{
    if (rows < 0 || k < 0 || k % UNIT != 0) return HIF4O_ERR_ARG;
    int64_t units = k / UNIT;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t u = 0; u < units; ++u)
            for (int j = 0; j < UNIT; ++j)
                out[r * k + u * UNIT + j] =
                    unit_element(codes + r * (k / 2) + u * 32, meta[r * units + u], j);
    return HIF4O_OK;
}

/* -------------------------------------------------------------- linear */

/* Fake-quantized linear ([TA-abs]; the form Y = X W^T of the same article's
 * FlatQuant section): Y[i][j] = sum_t a[i][t] b[j][t] with a = deq(Q(X)),
 * b = deq(Q(W)), summed in double in t order. S[i][j] = sum_t |a||b| sizes
 * the error bound of a float32 accumulation. Operands are given as codes. */
int hif4o_linear(const uint8_t *xc, const uint32_t *xm, const uint8_t *wc, const uint32_t *wm,
                 int64_t m, int64_t n, int64_t k, double *y, double *s)
{
    if (m < 0 || n < 0 || k < 0 || k % UNIT != 0) return HIF4O_ERR_ARG;
    double *a = (double *)malloc(sizeof(double) * (size_t)(m * k + 1));
    double *b = (double *)malloc(sizeof(double) * (size_t)(n * k + 1));
    if (!a || !b) {
        free(a);
        free(b);
        return HIF4O_ERR_ARG;
    }
    hif4o_dequantize(xc, xm, m, k, a);
    hif4o_dequantize(wc, wm, n, k, b);
#pragma omp parallel for schedule(dynamic)
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0, mag = 0.0;
            for (int64_t t = 0; t < k; ++t) {
                double p = a[i * k + t] * b[j * k + t];
                acc += p;
                mag += fabs(p);
            }
            y[i * n + j] = acc;
            if (s) s[i * n + j] = mag;
        }
    }
    free(a);
    free(b);
    return HIF4O_OK;
}

/* ---------------------------------------------------------- percentile */

static int cmp_double(const void *pa, const void *pb)
{
    double a = *(const double *)pa, b = *(const double *)pb;
    return (a > b) - (a < b);
}

/* W4A4 linear with protected channels ([TA-method], section "方法概述":
 * the channels the mask protects stay in high precision; layer form
 * Y = X W^T from the article's FlatQuant section). The HiF4 streams hold +0
 * at the protected channels (the mask removes them before quantization,
 * see hif4o_quantize), and their original bf16 values come separately as
 * xk [m][nk] and wk [n][nk], channels in the same (ascending) order on both
 * sides. In double:
 *   Y = deq(Q(X)) deq(Q(W))^T + xk wk^T,
 * and S = the sum of |product| over both parts. */
int hif4o_linear_protected(const uint8_t *xc, const uint32_t *xm, const uint16_t *xk,
                           const uint8_t *wc, const uint32_t *wm, const uint16_t *wk,
                           int64_t m, int64_t n, int64_t k, int64_t nk, double *y, double *s)
{
    if (nk < 0 || nk > k) return HIF4O_ERR_ARG;
    int rc = hif4o_linear(xc, xm, wc, wm, m, n, k, y, s);
    if (rc != HIF4O_OK) return rc;
#pragma omp parallel for schedule(dynamic)
    for (int64_t i = 0; i < m; ++i) {
        for (int64_t j = 0; j < n; ++j) {
            double acc = 0.0, mag = 0.0;
            for (int64_t t = 0; t < nk; ++t) {
                double p = bf16_value(xk[i * nk + t]) * bf16_value(wk[j * nk + t]);
                acc += p;
                mag += fabs(p);
            }
            y[i * n + j] += acc;
            if (s) s[i * n + j] += mag;
        }
    }
    return HIF4O_OK;
}

/* Per-channel tail statistic ([TA-method]: a percentile of the activation
 * magnitudes per channel, used in place of the maximum).
 * READING: the type-7 (linear interpolation) quantile at level q of |x[:, ch]|
 * over all rows: sort ascending into v, h = q (n-1), lo = floor(h),
 * hi = min(lo+1, n-1), stat = v[lo] + (h - lo) (v[hi] - v[lo]), each double
 * operation rounded on its own, then rounded to float. */
int hif4o_percentile(const uint16_t *x, int64_t rows, int64_t c, int64_t ld, double q,
                     float *stats)
{
    if (rows < 1 || c < 0 || ld < c || !(q >= 0.0 && q <= 1.0)) return HIF4O_ERR_ARG;
    int bad = 0;
#pragma omp parallel for schedule(dynamic) reduction(| : bad)
    for (int64_t ch = 0; ch < c; ++ch) {
        double *v = (double *)malloc(sizeof(double) * (size_t)rows);
        if (!v) {
            bad = 1;
            continue;
        }
        for (int64_t r = 0; r < rows; ++r) {
            v[r] = fabs(bf16_value(x[r * ld + ch]));
            if (!isfinite(v[r])) bad = 1;
        }
        qsort(v, (size_t)rows, sizeof(double), cmp_double);
        double h = q * (double)(rows - 1);
        double lo_f = floor(h);
        int64_t lo = (int64_t)lo_f;
        int64_t hi = lo + 1 < rows ? lo + 1 : rows - 1;
        double f = h - lo_f;
        double d = v[hi] - v[lo];
        double t = f * d;
        double r = v[lo] + t;
        stats[ch] = (float)r;
        free(v);
    }
    return bad ? HIF4O_ERR_NONFINITE : HIF4O_OK;
}

/* ----------------------------------------------------------------- mask */

static const float *g_sort_stats; /* used only inside hif4o_topn_mask */

static int cmp_rank(const void *pa, const void *pb)
{
    int64_t a = *(const int64_t *)pa, b = *(const int64_t *)pb;
    float sa = g_sort_stats[a], sb = g_sort_stats[b];
    if (sa > sb) return -1;
    if (sa < sb) return 1;
    return (a > b) - (a < b);
}

/* Channel-protection mask ([TA-method]: the channels with the largest tail
 * statistics are protected). READING: order channels by (stat descending,
 * index ascending); the first n_protect get mask 1. Not thread-safe (qsort
 * comparator state); the tests call it from one thread. */
int hif4o_topn_mask(const float *stats, int64_t c, int64_t n_protect, uint8_t *mask)
{
    if (c < 0 || n_protect < 0 || n_protect > c) return HIF4O_ERR_ARG;
    int64_t *idx = (int64_t *)malloc(sizeof(int64_t) * (size_t)(c + 1));
    if (!idx) return HIF4O_ERR_ARG;
    for (int64_t i = 0; i < c; ++i) idx[i] = i;
    g_sort_stats = stats;
    qsort(idx, (size_t)c, sizeof(int64_t), cmp_rank);
    for (int64_t i = 0; i < c; ++i) mask[i] = 0;
    for (int64_t i = 0; i < n_protect; ++i) mask[idx[i]] = 1;
    free(idx);
    return HIF4O_OK;
}

/* -------------------------------------------------------------- HiGPTQ */

/* fp32 rows [rows][ld] -> codes [rows][k/2], meta [rows][k/64]: the same
 * encoding rule as hif4o_quantize, applied to the exact values of floats
 * (HiGPTQ's working weights are real numbers, not bf16). */
int hif4o_quantize_f32(const float *x, int64_t rows, int64_t k, int64_t ld, uint8_t *codes,
                       uint32_t *meta)
{
    if (rows < 0 || k < 0 || k % UNIT != 0 || ld < k) return HIF4O_ERR_ARG;
    int64_t units = k / UNIT;
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t u = 0; u < units; ++u) {
            double v[UNIT];
            for (int j = 0; j < UNIT; ++j) {
                v[j] = (double)x[r * ld + u * UNIT + j];
                if (!isfinite(v[j])) {
                    bad = 1;
                    v[j] = 0.0;
                }
            }
            quantize_unit(v, codes + r * (k / 2) + u * 32, meta + r * units + u);
        }
    }
    return bad ? HIF4O_ERR_NONFINITE : HIF4O_OK;
}

/* HiGPTQ ([HiGPTQ], section 3.1): one group of 64 columns (one HiF4 unit)
 * per call, under one of the article's three schemes.
 *
 *  scheme 1  the 64 columns are quantized at once, with the level-1,
 *            level-2 and level-3 exponents all fixed from them;
 *  scheme 2  the level-1 exponent (1-0) is fixed from the group first; then
 *            8 columns at a time: their level-2 and level-3 exponents are
 *            fixed from their current values, they are quantized, and the
 *            weights not yet quantized are updated before the next 8;
 *  scheme 3  the level-1 exponent is fixed first; for each level-2 group,
 *            its level-2 exponent is fixed from its 8 current values, its
 *            first 4 columns are quantized (level-3 fixed from them), the
 *            weights not yet quantized are updated, and the second 4
 *            columns re-estimate their level-3 exponent and are quantized.
 *
 * The update is the one of GPTQ (Frantar et al., "GPTQ: Accurate
 * Post-Training Quantization for Generative Pre-trained Transformers", 2022),
 * restated for a set T of columns fixed together: with H the layer's Hessian
 * over the input channels and H^-1 = U^T U (U upper triangular, the caller's
 * factor), fixing T to Q_T moves the columns after T by
 *     W_R -= F U_TR,   F = E U_TT^-1,   E = W_T - deq(Q_T),
 * the optimal compensation of the quadratic loss once the earlier columns are
 * fixed (for a trailing block, (H_{>=t})^-1 = U_{>=t}^T U_{>=t}). F is formed
 * by forward substitution (F U_TT = E, U_TT upper triangular), in double.
 * Schemes 2 and 3 apply it per 8 or per 4 columns; the columns after the
 * group receive the sum of those updates, F U_SR with F the group's 64 F
 * values side by side.
 *
 *  w      double [n][k], the working weights; the group's columns end holding
 *         the values they were quantized from, the columns after it are
 *         updated in place.
 *  u      double [k][k], row-major, upper triangular (nonzero diagonal).
 *  unit   the group index (columns 64 unit .. 64 unit + 63).
 *  codes  [n][k/2], meta [n][k/64]: unit `unit` of every row is written. */

/* Level-2 / level-3 bits and element rounding (steps 3-5 of the rule) for
 * elements j0 .. j0 + len - 1 of a unit under level-1 scale s; e2 of their
 * level-2 group is the given one when e2_fixed >= 0. Writes the nibbles, the
 * meta bits and the dequantized values.
 *
 * Decision margins (diagnostic output; no effect on the result): when
 * `margin` is not NULL, each decision that reads a value some update has
 * moved (moved[j] != 0) lowers *margin to its distance from the boundary it
 * was decided against -- |M8 - 3.5 s| for a
 * level-2 bit, |M4 - 1.75 2^e2 s| for a level-3 bit, the distance of |x| to
 * the nearest rounding midpoint for an element -- divided by sc[] (the
 * largest sc[j] of the values the decision reads), the size of the sums
 * that produced those values. A run in other precision that starts from the
 * same weights can only decide differently where this ratio is within its
 * rounding error. */
static void encode_span(const double x[UNIT], int j0, int len, double s, int e2_fixed,
                        uint8_t codes[32], uint32_t *meta, double deq[UNIT],
                        const double *sc, const int *moved, double *margin)
{
    int g = j0 / 8;
    double m8 = 0.0, sc8 = 0.0;
    int mv8 = 0;
    for (int j = 8 * g; j < 8 * g + 8; ++j) {
        m8 = fabs(x[j]) > m8 ? fabs(x[j]) : m8;
        if (margin) {
            sc8 = sc[j] > sc8 ? sc[j] : sc8;
            mv8 |= moved[j];
        }
    }
    int e2 = e2_fixed >= 0 ? e2_fixed : (m8 > 1.75 * 2.0 * s);
    if (margin && mv8 && e2_fixed < 0) {
        double r = fabs(m8 - 1.75 * 2.0 * s) / sc8;
        if (r < *margin) *margin = r;
    }
    for (int q = j0 / 4; q < (j0 + len) / 4; ++q) {
        double m4 = 0.0, sc4 = 0.0;
        int mv4 = 0;
        for (int j = 4 * q; j < 4 * q + 4; ++j) {
            m4 = fabs(x[j]) > m4 ? fabs(x[j]) : m4;
            if (margin) {
                sc4 = sc[j] > sc4 ? sc[j] : sc4;
                mv4 |= moved[j];
            }
        }
        int e3 = m4 > 1.75 * e1_factor(e2) * s;
        if (margin && mv4) {
            double r = fabs(m4 - 1.75 * e1_factor(e2) * s) / sc4;
            if (r < *margin) *margin = r;
        }
        *meta |= (uint32_t)e3 << (16 + q);
        double D = s * e1_factor(e2) * e1_factor(e3);
        for (int j = 4 * q; j < 4 * q + 4; ++j) {
            double a = fabs(x[j]);
            int k = 0;
            for (int m = 0; m < 7; ++m) {
                double mid = (double)(2 * m + 1) * D / 8.0;
                if (a > mid) {
                    k = m + 1;
                } else {
                    if (a == mid) k = (m % 2 == 0) ? m : m + 1;
                    break;
                }
            }
            if (margin && moved[j]) {
                for (int m = 0; m < 7; ++m) {
                    double r = fabs(a - (double)(2 * m + 1) * D / 8.0) / sc[j];
                    if (r < *margin) *margin = r;
                }
            }
            int sign = (x[j] < 0.0) && (k != 0);
            codes[code_byte(j)] |= (uint8_t)((k | (sign << 3)) << code_shift(j));
            deq[j] = (sign ? -1.0 : 1.0) * (double)k * D / 4.0;
        }
    }
    *meta |= (uint32_t)e2 << (8 + g);
}

/* Level-1 code of a unit whose largest magnitude is amax: the smallest c with
 * 7 v(c) >= amax (255 when none). */
static int level1_of(double amax)
{
    for (int cc = 0; cc < 256; ++cc)
        if (7.0 * hif4o_e6m2_value(cc) >= amax) return cc;
    return 255;
}

/* One group step; see hif4o_higptq_unit_scheme_margin and hif4o_higptq_run_margin
 * for margin and accmag. With accmag, a value counts as moved from the start
 * of the step when accmag of its entry is nonzero, and then the level-1 code
 * and scheme 1's decisions read moved values too. */
static int higptq_step(double *w, int64_t n, int64_t k, const double *u, int64_t unit,
                       int scheme, uint8_t *codes, uint32_t *meta, double *margin,
                       double *accmag)
{
    if (n < 0 || k <= 0 || k % UNIT != 0 || unit < 0 || unit >= k / UNIT) return HIF4O_ERR_ARG;
    if (scheme < 1 || scheme > 3) return HIF4O_ERR_ARG;
    const int64_t s0 = unit * UNIT, r0 = s0 + UNIT, units = k / UNIT;
    for (int j = 0; j < UNIT; ++j)
        if (!(u[(s0 + j) * k + (s0 + j)] != 0.0)) return HIF4O_ERR_ARG;
    const int span = scheme == 1 ? 64 : (scheme == 2 ? 8 : 4);
    int bad = 0;
#pragma omp parallel for schedule(static) reduction(| : bad)
    for (int64_t r = 0; r < n; ++r) {
        double *wr = w + r * k;
        double v[UNIT], deq[UNIT], f[UNIT], sc[UNIT];
        int moved[UNIT];
        double mg = INFINITY;
        double *am = accmag ? accmag + r * k : NULL;
        int any_moved = 0;
        for (int j = 0; j < UNIT; ++j) {
            v[j] = wr[s0 + j];
            sc[j] = fabs(v[j]) + (am ? am[s0 + j] : 0.0);
            moved[j] = am && am[s0 + j] != 0.0;
            any_moved |= moved[j];
            if (!isfinite(v[j])) bad = 1;
        }
        uint8_t *uc = codes + r * (k / 2) + unit * 32;
        uint32_t *um = meta + r * units + unit;
        double amax = 0.0, scmax = 0.0;
        for (int j = 0; j < UNIT; ++j) {
            amax = fabs(v[j]) > amax ? fabs(v[j]) : amax;
            scmax = sc[j] > scmax ? sc[j] : scmax;
        }
        const int c1 = level1_of(amax);
        if (margin && any_moved) {
            /* level-1: amax against 7 v(c) and 7 v(c - 1) */
            double r1 = fabs(7.0 * hif4o_e6m2_value(c1) - amax);
            if (c1 > 0) {
                double r0 = fabs(amax - 7.0 * hif4o_e6m2_value(c1 - 1));
                r1 = r0 < r1 ? r0 : r1;
            }
            r1 /= scmax;
            if (r1 < mg) mg = r1;
        }
        if (scheme == 1) {
            quantize_unit(v, uc, um); /* all exponents from the group at once */
            for (int j = 0; j < UNIT; ++j) deq[j] = unit_element(uc, *um, j);
            if (margin && any_moved) {
                /* the same decisions again, for their margins only */
                uint8_t cs[32] = {0};
                uint32_t ms = (uint32_t)c1;
                double ds[UNIT];
                for (int t0 = 0; t0 < UNIT; t0 += 8)
                    encode_span(v, t0, 8, hif4o_e6m2_value(c1), -1, cs, &ms, ds, sc, moved, &mg);
            }
        } else {
            /* level-1 from the group as it stands before any update */
            memset(uc, 0, 32);
            *um = (uint32_t)c1;
        }
        for (int t0 = 0; t0 < UNIT; t0 += span) {
            if (scheme == 2) {
                encode_span(v, t0, 8, hif4o_e6m2_value((int)(*um & 255u)), -1, uc, um, deq, sc,
                            moved, margin ? &mg : NULL);
            } else if (scheme == 3) {
                int e2 = -1;
                if (t0 % 8 == 4) e2 = (int)((*um >> (8 + t0 / 8)) & 1u); /* fixed before the group's first 4 */
                encode_span(v, t0, 4, hif4o_e6m2_value((int)(*um & 255u)), e2, uc, um, deq, sc,
                            moved, margin ? &mg : NULL);
            }
            /* forward substitution over the span: f_j = (e_j - sum f_i U_ij) / U_jj */
            for (int j = t0; j < t0 + span; ++j) {
                double acc = v[j] - deq[j];
                for (int i = t0; i < j; ++i) acc -= f[i] * u[(s0 + i) * k + (s0 + j)];
                f[j] = acc / u[(s0 + j) * k + (s0 + j)];
            }
            /* update the group's columns after the span */
            for (int j = t0 + span; j < UNIT; ++j) {
                double acc = 0.0, mag = 0.0;
                for (int i = t0; i < t0 + span; ++i) {
                    acc += f[i] * u[(s0 + i) * k + (s0 + j)];
                    mag += fabs(f[i]) * fabs(u[(s0 + i) * k + (s0 + j)]);
                }
                v[j] -= acc;
                sc[j] += mag;
                if (mag != 0.0) moved[j] = 1;
            }
        }
        if (margin) margin[r] = accmag ? (mg < margin[r] ? mg : margin[r]) : mg;
        for (int j = 0; j < UNIT; ++j) wr[s0 + j] = v[j];
        for (int64_t c = r0; c < k; ++c) {
            double acc = 0.0, mag = 0.0;
            for (int i = 0; i < UNIT; ++i) {
                acc += f[i] * u[(s0 + i) * k + c];
                mag += fabs(f[i]) * fabs(u[(s0 + i) * k + c]);
            }
            wr[c] -= acc;
            if (am) am[c] += mag;
        }
    }
    return bad ? HIF4O_ERR_NONFINITE : HIF4O_OK;
}

/* margin: NULL, or double [n]. Row r receives the smallest decision margin
 * (see encode_span) over the decisions of schemes 2 and 3 that read updated
 * values, with sc[j] = |w[j]| + sum over the updates of column j of
 * sum_i |f_i| |U_ij|; +inf under scheme 1 and for decisions on the weights as
 * given (scheme 1's, and every level-1 code), which any run starting from the
 * same weights takes identically. */
int hif4o_higptq_unit_scheme_margin(double *w, int64_t n, int64_t k, const double *u,
                                    int64_t unit, int scheme, uint8_t *codes, uint32_t *meta,
                                    double *margin)
{
    return higptq_step(w, n, k, u, unit, scheme, codes, meta, margin, NULL);
}

/* HiGPTQ over groups unit0 .. unit0 + units - 1 in order, each exactly
 * hif4o_higptq_unit_scheme's step (same arithmetic, same results). Margins
 * over the whole run: accmag (double [n][k], in/out, zero for a run from
 * weights as given) holds per entry the sum over the updates applied so far
 * of sum_i |f_i| |U_ic|; a decision reads a moved value when an update of this
 * run or an earlier one (accmag != 0) or of its own group has moved it, and
 * then lowers margin[r] (in/out: start it at +inf) to its distance from its
 * boundary over sc = |value| + accmag + the group's own update sizes. The
 * level-1 code (amax against 7 v(c) and 7 v(c - 1)) and scheme 1's decisions
 * count too once the group holds a moved value. A run in other precision from
 * the same weights can decide differently from this one only on a row whose
 * margin lies within its rounding error. */
int hif4o_higptq_run_margin(double *w, int64_t n, int64_t k, const double *u, int64_t unit0,
                            int64_t units, int scheme, uint8_t *codes, uint32_t *meta,
                            double *margin, double *accmag)
{
    if (!margin || !accmag || units < 0 || unit0 < 0) return HIF4O_ERR_ARG;
    for (int64_t t = 0; t < units; ++t) {
        int st = higptq_step(w, n, k, u, unit0 + t, scheme, codes, meta, margin, accmag);
        if (st != HIF4O_OK) return st;
    }
    return HIF4O_OK;
}

int hif4o_higptq_unit_scheme(double *w, int64_t n, int64_t k, const double *u, int64_t unit,
                             int scheme, uint8_t *codes, uint32_t *meta)
{
    return hif4o_higptq_unit_scheme_margin(w, n, k, u, unit, scheme, codes, meta, NULL);
}

/* Scheme 1 (kept as its own entry). */
int hif4o_higptq_unit(double *w, int64_t n, int64_t k, const double *u, int64_t unit,
                      uint8_t *codes, uint32_t *meta)
{
    return hif4o_higptq_unit_scheme(w, n, k, u, unit, 1, codes, meta);
}
