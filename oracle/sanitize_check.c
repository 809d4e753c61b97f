/*
 * sanitize_check.c -- drives every entry point of the C oracle over small,
 * strided and degenerate inputs, for a build under AddressSanitizer and
 * UndefinedBehaviorSanitizer (tests/test_oracle_sanitize.py compiles it
 * together with hif4_oracle.c and runs it).
 *
 * TEST INFRASTRUCTURE, like the oracle itself. It checks memory safety and
 * defined behaviour (every buffer sized exactly, strided rows, empty and
 * non-finite inputs, argument errors) and the documented status codes; the
 * values themselves are pinned by the oracle's other tests.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int hif4o_quantize(const uint16_t *x, int64_t rows, int64_t k, int64_t ld, const uint8_t *mask,
                   int64_t n_mask, uint16_t *kept, uint8_t *codes, uint32_t *meta);
int hif4o_quantize_offsets(const uint16_t *x, int64_t rows, int64_t k, int64_t ld,
                           const float *koff, const float *moff, uint8_t *codes, uint32_t *meta);
int hif4o_dequantize(const uint8_t *codes, const uint32_t *meta, int64_t rows, int64_t k,
                     double *out);
int hif4o_linear(const uint8_t *xc, const uint32_t *xm, const uint8_t *wc, const uint32_t *wm,
                 int64_t m, int64_t n, int64_t k, double *y, double *s);
int hif4o_linear_protected(const uint8_t *xc, const uint32_t *xm, const uint16_t *xk,
                           const uint8_t *wc, const uint32_t *wm, const uint16_t *wk, int64_t m,
                           int64_t n, int64_t k, int64_t nk, double *y, double *s);
int hif4o_percentile(const uint16_t *x, int64_t rows, int64_t c, int64_t ld, double q,
                     float *stats);
int hif4o_topn_mask(const float *stats, int64_t c, int64_t n_protect, uint8_t *mask);
int hif4o_quantize_f32(const float *x, int64_t rows, int64_t k, int64_t ld, uint8_t *codes,
                       uint32_t *meta);
int hif4o_higptq_unit(double *w, int64_t n, int64_t k, const double *u, int64_t unit,
                      uint8_t *codes, uint32_t *meta);
int hif4o_higptq_unit_scheme(double *w, int64_t n, int64_t k, const double *u, int64_t unit,
                             int scheme, uint8_t *codes, uint32_t *meta);
int hif4o_higptq_unit_scheme_margin(double *w, int64_t n, int64_t k, const double *u,
                                    int64_t unit, int scheme, uint8_t *codes, uint32_t *meta,
                                    double *margin);
int hif4o_higptq_run_margin(double *w, int64_t n, int64_t k, const double *u, int64_t unit0,
                            int64_t units, int scheme, uint8_t *codes, uint32_t *meta,
                            double *margin, double *accmag);
double hif4o_e6m2_value(int c);

enum { OK = 0, ERR_ARG = 1, ERR_NONFINITE = 2 };

static int failures = 0;

static void expect(int got, int want, const char *what)
{
    if (got != want) {
        fprintf(stderr, "FAIL %s: status %d, expected %d\n", what, got, want);
        ++failures;
    }
}

/* xorshift64* (Vigna, "An experimental exploration of Marsaglia's xorshift
 * generators, scrambled", 2016) */
static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t rnd(void)
{
    rng_state ^= rng_state >> 12;
    rng_state ^= rng_state << 25;
    rng_state ^= rng_state >> 27;
    return rng_state * 0x2545F4914F6CDD1Dull;
}

static double unif(void) { return (double)(rnd() >> 11) * 0x1.0p-53; }

static uint16_t bf16_of(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    return (uint16_t)(u >> 16); /* truncation: any bf16 pattern will do here */
}

/* exact-size heap buffers, so that any overrun reaches a redzone */
static void *buf(size_t bytes) { return malloc(bytes ? bytes : 1); }

static void check_quantize(void)
{
    const int64_t rows = 5, k = 128, ld = 160;
    uint16_t *x = buf(sizeof(uint16_t) * (size_t)((rows - 1) * ld + k));
    for (int64_t i = 0; i < (rows - 1) * ld + k; ++i)
        x[i] = bf16_of((float)((unif() - 0.5) * ldexp(1.0, (int)(rnd() % 40) - 20)));
    x[3] = 0x0000;  /* +0 */
    x[4] = 0x8000;  /* -0 */
    x[5] = 0x0001;  /* subnormal */
    uint8_t *codes = buf((size_t)(rows * k / 2));
    uint32_t *meta = buf(sizeof(uint32_t) * (size_t)(rows * k / 64));
    expect(hif4o_quantize(x, rows, k, ld, NULL, 0, NULL, codes, meta), OK, "quantize");

    uint8_t *mask = buf((size_t)k);
    memset(mask, 0, (size_t)k);
    mask[0] = 1;
    mask[63] = 7;
    mask[127] = 1;
    uint16_t *kept = buf(sizeof(uint16_t) * (size_t)(rows * 3));
    expect(hif4o_quantize(x, rows, k, ld, mask, 3, kept, codes, meta), OK, "quantize masked");
    memset(mask, 1, (size_t)k);  /* every channel protected */
    uint16_t *kept_all = buf(sizeof(uint16_t) * (size_t)(rows * k));
    expect(hif4o_quantize(x, rows, k, ld, mask, k, kept_all, codes, meta), OK,
           "quantize fully masked");

    expect(hif4o_quantize(x, 0, k, ld, NULL, 0, NULL, codes, meta), OK, "quantize empty");
    expect(hif4o_quantize(x, rows, 100, ld, NULL, 0, NULL, codes, meta), ERR_ARG,
           "quantize k % 64");
    expect(hif4o_quantize(x, rows, k, k - 1, NULL, 0, NULL, codes, meta), ERR_ARG,
           "quantize ld < k");
    x[ld + 7] = 0x7F80;  /* +inf in row 1 */
    expect(hif4o_quantize(x, rows, k, ld, NULL, 0, NULL, codes, meta), ERR_NONFINITE,
           "quantize inf");
    x[ld + 7] = 0x7FC1;  /* NaN */
    expect(hif4o_quantize(x, rows, k, ld, NULL, 0, NULL, codes, meta), ERR_NONFINITE,
           "quantize NaN");
    free(kept_all);
    free(kept);
    free(mask);
    free(codes);
    free(meta);
    free(x);
}

static void check_offsets(void)
{
    const int64_t rows = 3, k = 192, ld = 200;
    uint16_t *x = buf(sizeof(uint16_t) * (size_t)((rows - 1) * ld + k));
    for (int64_t i = 0; i < (rows - 1) * ld + k; ++i)
        x[i] = bf16_of((float)((unif() - 0.5) * 8.0));
    float *koff = buf(sizeof(float) * (size_t)(rows * k / 4));
    float *moff = buf(sizeof(float) * (size_t)(rows * k));
    for (int64_t i = 0; i < rows * k / 4; ++i) koff[i] = (float)(unif() * 5.0 - 2.5);
    for (int64_t i = 0; i < rows * k; ++i) moff[i] = (float)(unif() * 2.0 - 1.0);
    koff[1] = NAN;
    uint8_t *codes = buf((size_t)(rows * k / 2));
    uint32_t *meta = buf(sizeof(uint32_t) * (size_t)(rows * k / 64));
    expect(hif4o_quantize_offsets(x, rows, k, ld, koff, moff, codes, meta), OK,
           "quantize_offsets");
    expect(hif4o_quantize_offsets(x, rows, 65, ld, koff, moff, codes, meta), ERR_ARG,
           "quantize_offsets k % 64");
    free(codes);
    free(meta);
    free(koff);
    free(moff);
    free(x);
}

static void check_dequantize_and_linear(void)
{
    const int64_t m = 3, n = 5, k = 128, nk = 3;
    uint8_t *xc = buf((size_t)(m * k / 2)), *wc = buf((size_t)(n * k / 2));
    uint32_t *xm = buf(sizeof(uint32_t) * (size_t)(m * k / 64));
    uint32_t *wm = buf(sizeof(uint32_t) * (size_t)(n * k / 64));
    /* arbitrary code and meta words: every nibble, level-1 code and exponent bit */
    for (int64_t i = 0; i < m * k / 2; ++i) xc[i] = (uint8_t)rnd();
    for (int64_t i = 0; i < n * k / 2; ++i) wc[i] = (uint8_t)rnd();
    for (int64_t i = 0; i < m * k / 64; ++i) xm[i] = (uint32_t)rnd();
    for (int64_t i = 0; i < n * k / 64; ++i) wm[i] = (uint32_t)rnd();
    xm[0] = 0;    /* level-1 code 0 */
    wm[0] = 255;  /* level-1 code 255 */
    double *out = buf(sizeof(double) * (size_t)(m * k));
    expect(hif4o_dequantize(xc, xm, m, k, out), OK, "dequantize");
    expect(hif4o_dequantize(xc, xm, m, 96, out), ERR_ARG, "dequantize k % 64");

    double *y = buf(sizeof(double) * (size_t)(m * n)), *s = buf(sizeof(double) * (size_t)(m * n));
    expect(hif4o_linear(xc, xm, wc, wm, m, n, k, y, s), OK, "linear");
    expect(hif4o_linear(xc, xm, wc, wm, 1, 1, 64, y, s), OK, "linear 1x1x64");
    uint16_t *xk = buf(sizeof(uint16_t) * (size_t)(m * nk));
    uint16_t *wk = buf(sizeof(uint16_t) * (size_t)(n * nk));
    for (int64_t i = 0; i < m * nk; ++i) xk[i] = bf16_of((float)(unif() * 100.0));
    for (int64_t i = 0; i < n * nk; ++i) wk[i] = bf16_of((float)(unif() - 0.5));
    expect(hif4o_linear_protected(xc, xm, xk, wc, wm, wk, m, n, k, nk, y, s), OK,
           "linear_protected");
    expect(hif4o_linear_protected(xc, xm, NULL, wc, wm, NULL, m, n, k, 0, y, s), OK,
           "linear_protected without kept channels");
    free(xk);
    free(wk);
    free(y);
    free(s);
    free(out);
    free(xc);
    free(wc);
    free(xm);
    free(wm);
}

static void check_percentile_and_mask(void)
{
    const int64_t rows = 37, c = 9, ld = 11;
    uint16_t *x = buf(sizeof(uint16_t) * (size_t)((rows - 1) * ld + c));
    for (int64_t i = 0; i < (rows - 1) * ld + c; ++i)
        x[i] = bf16_of((float)((unif() - 0.5) * ldexp(1.0, (int)(rnd() % 20) - 10)));
    float *stats = buf(sizeof(float) * (size_t)c);
    const double qs[] = {0.0, 0.5, 0.999, 1.0};
    for (int i = 0; i < 4; ++i)
        expect(hif4o_percentile(x, rows, c, ld, qs[i], stats), OK, "percentile");
    expect(hif4o_percentile(x, 1, c, ld, 0.999, stats), OK, "percentile one row");
    expect(hif4o_percentile(x, rows, c, ld, 1.5, stats), ERR_ARG, "percentile q > 1");
    expect(hif4o_percentile(x, 0, c, ld, 0.5, stats), ERR_ARG, "percentile no rows");

    uint8_t *mask = buf((size_t)c);
    for (int64_t n = 0; n <= c; ++n)
        expect(hif4o_topn_mask(stats, c, n, mask), OK, "topn_mask");
    for (int64_t i = 0; i < c; ++i) stats[i] = 1.0f;  /* all tied */
    expect(hif4o_topn_mask(stats, c, 4, mask), OK, "topn_mask ties");
    free(mask);
    free(stats);
    free(x);
}

static void check_quantize_f32(void)
{
    const int64_t rows = 2, k = 64, ld = 70;
    float *x = buf(sizeof(float) * (size_t)((rows - 1) * ld + k));
    for (int64_t i = 0; i < (rows - 1) * ld + k; ++i)
        x[i] = (float)((unif() - 0.5) * 1e3);
    uint8_t *codes = buf((size_t)(rows * k / 2));
    uint32_t *meta = buf(sizeof(uint32_t) * (size_t)(rows * k / 64));
    expect(hif4o_quantize_f32(x, rows, k, ld, codes, meta), OK, "quantize_f32");
    x[5] = INFINITY;
    expect(hif4o_quantize_f32(x, rows, k, ld, codes, meta), ERR_NONFINITE, "quantize_f32 inf");
    free(codes);
    free(meta);
    free(x);
}

static void check_higptq(void)
{
    const int64_t n = 3, k = 128, units = k / 64;
    double *w = buf(sizeof(double) * (size_t)(n * k));
    double *w0 = buf(sizeof(double) * (size_t)(n * k));
    double *u = buf(sizeof(double) * (size_t)(k * k));
    for (int64_t i = 0; i < n * k; ++i) w0[i] = (unif() - 0.5) * 0.1;
    for (int64_t i = 0; i < k; ++i)
        for (int64_t j = 0; j < k; ++j)
            u[i * k + j] = j < i ? 0.0 : (j == i ? 0.5 + unif() : (unif() - 0.5) * 0.2);
    uint8_t *codes = buf((size_t)(n * k / 2));
    uint32_t *meta = buf(sizeof(uint32_t) * (size_t)(n * units));
    double *margin = buf(sizeof(double) * (size_t)n);
    double *accmag = buf(sizeof(double) * (size_t)(n * k));
    for (int scheme = 1; scheme <= 3; ++scheme) {
        memcpy(w, w0, sizeof(double) * (size_t)(n * k));
        for (int64_t t = 0; t < units; ++t)
            expect(hif4o_higptq_unit_scheme(w, n, k, u, t, scheme, codes, meta), OK,
                   "higptq_unit_scheme");
        memcpy(w, w0, sizeof(double) * (size_t)(n * k));
        expect(hif4o_higptq_unit_scheme_margin(w, n, k, u, units - 1, scheme, codes, meta, margin),
               OK, "higptq_unit_scheme_margin");
        memcpy(w, w0, sizeof(double) * (size_t)(n * k));
        memset(accmag, 0, sizeof(double) * (size_t)(n * k));
        for (int64_t r = 0; r < n; ++r) margin[r] = INFINITY;
        expect(hif4o_higptq_run_margin(w, n, k, u, 0, units, scheme, codes, meta, margin, accmag),
               OK, "higptq_run_margin");
    }
    memcpy(w, w0, sizeof(double) * (size_t)(n * k));
    expect(hif4o_higptq_unit(w, n, k, u, 0, codes, meta), OK, "higptq_unit");
    expect(hif4o_higptq_unit(w, n, k, u, units, codes, meta), ERR_ARG, "higptq_unit past K");
    expect(hif4o_higptq_unit_scheme(w, n, k, u, 0, 4, codes, meta), ERR_ARG, "higptq scheme 4");
    u[0] = 0.0;  /* zero pivot */
    expect(hif4o_higptq_unit(w, n, k, u, 0, codes, meta), ERR_ARG, "higptq zero pivot");
    expect(hif4o_higptq_run_margin(w, n, k, u, 0, 1, 1, codes, meta, NULL, accmag), ERR_ARG,
           "higptq_run_margin without margin");
    free(accmag);
    free(margin);
    free(codes);
    free(meta);
    free(u);
    free(w0);
    free(w);
}

int main(void)
{
    for (int c = 0; c < 256; ++c)
        if (!(hif4o_e6m2_value(c) > 0.0)) {
            fprintf(stderr, "FAIL e6m2_value(%d)\n", c);
            ++failures;
        }
    check_quantize();
    check_offsets();
    check_dequantize_and_linear();
    check_percentile_and_mask();
    check_quantize_f32();
    check_higptq();
    if (failures) {
        fprintf(stderr, "%d check(s) failed\n", failures);
        return 1;
    }
    printf("sanitize-check OK\n");
    return 0;
}
