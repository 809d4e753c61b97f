/*
 * hif4.h -- C ABI of libhif4.so: HiFloat4 (HiF4) W4A4 fake-quantized linear
 * layers on AMD Instinct MI355X (gfx950).
 *
 * Sources:
 *  [HiF4-fmt]  HiFloat4 calibration article (hwcomputing.csdn.net), section
 *              "一：HiFloat4 (HiF4) 格式": 64-element units, one E6M2 level-1
 *              scale, 8 E1 level-2 exponents (one per 8 elements), 16 E1
 *              level-3 exponents (one per 4), S1P2 4-bit elements with
 *              magnitudes 0 and 0.25..1.75, 32 metadata bits per unit.
 *  [HiGPTQ]    same article, section 3.1: exponent order along K (1-0,
 *              2-(0..7), 3-(0..15)), each fixed from the data it covers.
 *  [HiFlat]    same article, section 3.3: HiF4 needs no clipping thresholds.
 *  [TA-method] "Tail-Aware HiFloat4: W4A4 PTQ calibration for Wan2.2"
 *              (agents-report.net), sections "方法概述", "校準與緊湊 PTQ 狀態"
 *              and "尾部百分位統計的動機": W4A4 fake quantization of the target
 *              linear layers; per-channel tail-percentile statistics of the
 *              calibration activations build a channel-protection mask;
 *              protected channels stay in high precision.
 *  [TA-abs]    arXiv 2605.26628 record, abstract (same method, English).
 *
 * ENCODING (where the pages are silent this library takes, and its oracle
 * pins, the following readings):
 *  - level-1 code c (u8): v(c) = 2^((c>>2) - 31) * (1 + (c&3)/4), all codes
 *    normal; an E1 bit b scales by 2^b; a nibble is sign<<3 | k, |value| = k/4.
 *  - element j of a unit: x = S1P2(nibble_j) * 2^e2[j/8] * 2^e3[j/4] * v(c).
 *  - quantize: c = smallest code with 7 v(c) >= max|x| (255 if none);
 *    e2[g] = [max over 8 > 3.5 v(c)]; e3[q] = [max over 4 > 1.75 2^e2 v(c)];
 *    k = round-to-nearest-even(4|x| / (v(c) 2^(e2+e3))), at most 7; zero is +0.
 *  - layout: a row of k elements has k/64 units. codes [rows][k/2] bytes: unit
 *    u owns bytes 32u..32u+31; element j of the unit sits in byte
 *    4*(j/8) + j%4, low nibble if j%8 < 4, else high nibble. meta
 *    [rows][k/64] u32: c | e2bits << 8 | e3bits << 16 (bit g of e2bits for
 *    elements 8g..8g+7, bit q of e3bits for elements 4q..4q+3).
 *
 * CONVENTIONS (all entry points):
 *  - Every pointer argument is DEVICE memory owned by the caller; the library
 *    allocates nothing and keeps no state between calls (a per-device
 *    "is this gfx950" flag is cached). Calls are reentrant. The one exception
 *    is hif4_linear_xcodes_wbf16_noalloc, which stages its scratch in a
 *    static device array (see there).
 *  - Work is enqueued asynchronously on `stream` (NULL = the null stream); the
 *    library never synchronizes. Faults inside a kernel surface at the
 *    caller's next synchronization.
 *  - Argument checks happen before any HIP call; on an error nothing is
 *    enqueued and outputs are untouched. No C++ exception crosses the ABI.
 *  - Results are deterministic and identical from run to run (integer
 *    histograms, no floating-point atomics, fixed reduction order).
 *  - Inputs must be finite; Inf/NaN inputs give unspecified (but in-bounds)
 *    results.
 */
#ifndef HIF4_H
#define HIF4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HIF4_API_VERSION 1

#ifndef HIF4_EXPORT
#define HIF4_EXPORT __attribute__((visibility("default")))
#endif

typedef enum hif4_status {
    HIF4_OK = 0,
    HIF4_ERR_NULL = 1,      /* a required pointer is NULL */
    HIF4_ERR_SHAPE = 2,     /* a size is negative, k % 64 != 0, ld < k, n_protect > c, ... */
    HIF4_ERR_ALIGN = 3,     /* a pointer or leading dimension breaks the stated alignment */
    HIF4_ERR_WORKSPACE = 4, /* workspace NULL or smaller than the *_workspace_bytes query */
    HIF4_ERR_DTYPE = 5,     /* unknown hif4_dtype */
    HIF4_ERR_DEVICE = 6,    /* current device is not gfx950, or no device */
    HIF4_ERR_LAUNCH = 7,    /* a kernel failed to enqueue */
    HIF4_ERR_ARG = 8,       /* another argument is out of range (q outside [0,1], ...) */
    HIF4_ERR_SCRATCH = 9    /* the allocation-free entry point's static scratch is too small */
} hif4_status;

typedef enum hif4_dtype { HIF4_F32 = 0, HIF4_BF16 = 1 } hif4_dtype;

/* Static, NUL-terminated description of a status code. Never NULL. */
HIF4_EXPORT const char *hif4_status_string(int status);

/* HIF4_API_VERSION of the built library. */
HIF4_EXPORT int hif4_version(void);

/*
 * hif4_quantize -- HiF4-quantize the rows of a bf16 matrix along k
 * ([HiF4-fmt] unit structure; [HiGPTQ] order and per-group statistics;
 * [HiFlat] no clipping; rule as stated above).
 *
 *  x      bf16 [rows][ld], row-major; 16-byte aligned, ld % 8 == 0, ld >= k.
 *  rows   >= 0 (0 enqueues nothing).   k   >= 0, k % 64 == 0.
 *  mask   NULL, or u8 [k], 16-byte aligned: nonzero = protected input channel
 *         ([TA-method]).
 *         Protected entries are encoded as +0 and do not influence the scales.
 *  n_mask number of nonzero mask bytes (must equal it; kept entries beyond
 *         the true count are left unwritten, none is written out of bounds).
 *  kept   NULL when mask is NULL or n_mask == 0; else bf16 [rows][n_mask]:
 *         row r receives x[r][ch] for every protected ch, ascending ch.
 *  codes  u8 [rows][k/2], 16-byte aligned.    meta  u32 [rows][k/64], 4-byte aligned.
 *  With a mask, k must be <= 65536.
 */
HIF4_EXPORT hif4_status hif4_quantize(const void *x, int64_t rows, int64_t k, int64_t ld,
                          const uint8_t *mask, int64_t n_mask, void *kept,
                          uint8_t *codes, uint32_t *meta, hipStream_t stream);

/*
 * hif4_dequantize -- decode HiF4 codes to real values ([HiF4-fmt]; the
 * quantize-then-dequantize form of fake quantization, [TA-abs]). Every decoded
 * value is exact in both fp32 and bf16.
 *
 *  codes u8 [rows][k/2] (16-byte aligned), meta u32 [rows][k/64].
 *  out   [rows][k] of out_dtype (HIF4_F32 or HIF4_BF16), 16-byte aligned.
 */
HIF4_EXPORT hif4_status hif4_dequantize(const uint8_t *codes, const uint32_t *meta, int64_t rows, int64_t k,
                            void *out, int out_dtype, hipStream_t stream);

/*
 * hif4_linear_workspace_bytes -- bytes of device workspace the linear entry
 * points need for an (m x k) activation, an (n x k) weight and n_kept
 * protected channels: hif4_linear_w4a4 needs (m, n, k, n_kept),
 * hif4_linear_xcodes_wbf16 needs (m, n, 0, n_kept) (0 when n_kept == 0).
 * Returns 0 for sizes no linear entry point accepts: negative, m, n or k of
 * 2^31 or more, or n_kept above 65536.
 */
HIF4_EXPORT size_t hif4_linear_workspace_bytes(int64_t m, int64_t n, int64_t k, int64_t n_kept);

/*
 * hif4_linear_w4a4 -- W4A4 fake-quantized linear layer ([TA-abs]; the layer
 * form Y = X W^T of the calibration article's FlatQuant section), with
 * optional protected channels ([TA-method], "方法概述": the channels the
 * mask protects stay in high precision):
 *     Y[i][j] = sum_t deq(Q(X))[i][t] * deq(Q(W))[j][t]
 *             + sum_{p < n_kept} x_kept[i][p] * w_kept[j][p],
 * accumulated in fp32: one accumulator per output, one rounding per 16-term
 * matrix-core step. The worst case is (k + 64 ceil(n_kept / 64)) / 16 * 2^-24
 * * sum |a||b| over both parts; rounding errors of independent sign keep the
 * error far below that, and within 1e-5 * sum |a||b| on every shape tested
 * (K up to 13,824, same-sign data included).
 *
 *  X is given EITHER as bf16 x [m][k] (row stride k; it is quantized along k
 *  into the workspace first, with `mask` applied when n_kept > 0) OR
 *  pre-quantized (x == NULL; x_codes [m][k/2], x_meta [m][k/64], and
 *  x_kept bf16 [m][n_kept] when n_kept > 0 -- hif4_quantize's outputs).
 *  W is always pre-quantized: w_codes [n][k/2], w_meta [n][k/64] (the
 *  nn.Linear [out][in] layout, quantized along in) and, when n_kept > 0,
 *  w_kept bf16 [n][n_kept] (hif4_quantize with the same mask).
 *  mask     u8 [k], 16-byte aligned, exactly n_kept nonzero entries (used
 *           only when x is given and n_kept > 0; then k <= 65536).
 *  n_kept   0 <= n_kept <= k; 0 = no protected channels (mask, x_kept and
 *           w_kept are then ignored and may be NULL).
 *  y        [m][n] of y_dtype (HIF4_F32, or HIF4_BF16 rounded to nearest even).
 *  workspace device memory of at least hif4_linear_workspace_bytes(m, n, k,
 *            n_kept) bytes, 256-byte aligned; its contents are scratch.
 *  Pointers 16-byte aligned except meta (4-byte) and kept (2-byte).
 *  m, n >= 0; k % 64 == 0.
 */
HIF4_EXPORT hif4_status hif4_linear_w4a4(const void *x, const uint8_t *x_codes, const uint32_t *x_meta,
                             const uint8_t *w_codes, const uint32_t *w_meta,
                             const uint8_t *mask, const void *x_kept, const void *w_kept,
                             int64_t n_kept, int64_t m, int64_t n, int64_t k, void *y,
                             int y_dtype, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * hif4_linear_xcodes_wbf16 -- the contraction step of hif4_linear_w4a4 with
 * the weight already decoded (the serving case: a static weight is decoded
 * once with hif4_dequantize(..., HIF4_BF16) and reused for every batch):
 *     Y[i][j] = sum_t deq(X codes)[i][t] * w[j][t]
 *             + sum_{p < n_kept} x_kept[i][p] * w_kept[j][p],  accumulated in fp32.
 *
 *  x_codes [m][k/2], x_meta [m][k/64]: HiF4 activation (hif4_quantize layout).
 *  w       bf16 [n][k], row stride k. With w = deq(Q(W)) (every value exact
 *          in bf16) the result equals hif4_linear_w4a4's bit for bit; any
 *          other bf16 w gives Y = deq(X) w^T with the same accumulation.
 *  x_kept, w_kept, n_kept: protected channels as in hif4_linear_w4a4.
 *  y       [m][n] of y_dtype (HIF4_F32, or HIF4_BF16 rounded to nearest even).
 *  workspace: needed only when n_kept > 0: at least
 *          hif4_linear_workspace_bytes(m, n, 0, n_kept) bytes, 256-byte aligned.
 *  Pointers 16-byte aligned except x_meta (4-byte) and kept (2-byte);
 *  m, n >= 0; k % 64 == 0. k == 0 writes Y = 0.
 */
HIF4_EXPORT hif4_status hif4_linear_xcodes_wbf16(const uint8_t *x_codes, const uint32_t *x_meta,
                                     const void *w, const void *x_kept, const void *w_kept,
                                     int64_t n_kept, int64_t m, int64_t n, int64_t k, void *y,
                                     int y_dtype, void *workspace, size_t workspace_bytes,
                                     hipStream_t stream);

/*
 * hif4_linear_xcodes_wbf16_noalloc -- hif4_linear_xcodes_wbf16 for callers
 * that cannot allocate device memory: code being captured into a HIP graph,
 * tight serving loops, harnesses that forbid hipMalloc. Same arguments,
 * result and error behaviour as hif4_linear_xcodes_wbf16 (bit for bit the
 * same Y), minus the workspace: the protected-channel operands (Xr, Wr) are
 * staged in a static device array of the library instead.
 *
 *  - That array holds HIF4_NOALLOC_SCRATCH_BYTES (32 MiB) per GPU, for the
 *    life of the process. A call with n_kept > 0 needs m * 2 * kr + n * 2 * kr
 *    bytes of it (kr = n_kept rounded up to 64; each of the two parts rounded
 *    up to 256 bytes), none with n_kept == 0. A larger call returns
 *    HIF4_ERR_SCRATCH and enqueues nothing.
 *  - The call allocates nothing: no hipMalloc, hipFree or allocating library
 *    routine. Its first call on a device looks up that device's copy of the
 *    array once (hipGetSymbolAddress) and caches the address per device.
 *  - Every call on one GPU shares that GPU's array. Calls whose execution
 *    overlaps on one GPU (on different streams, or from several threads
 *    without ordering) race on it and give undefined Y; calls ordered on one
 *    stream are safe. Each call writes all of the array it reads, so the
 *    previous call's contents never leak into a result.
 */
#define HIF4_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

HIF4_EXPORT hif4_status hif4_linear_xcodes_wbf16_noalloc(const uint8_t *x_codes,
                                             const uint32_t *x_meta, const void *w,
                                             const void *x_kept, const void *w_kept,
                                             int64_t n_kept, int64_t m, int64_t n, int64_t k,
                                             void *y, int y_dtype, hipStream_t stream);

/*
 * hif4_percentile_workspace_bytes -- workspace bytes for hif4_percentile_mask
 * over rows x c values (depends on rows from 8192 rows on; no device needed).
 * Returns 0 beyond the entry point's limits: negative sizes, rows of 2^32 or
 * more, c above 65536.
 */
HIF4_EXPORT size_t hif4_percentile_workspace_bytes(int64_t rows, int64_t c);

/*
 * hif4_percentile_mask -- tail-aware channel statistics and protection mask
 * ([TA-method]: a per-channel percentile of the activation magnitudes stands
 * in for the maximum; the channels with the largest statistics are protected).
 *
 *  stats[ch] = type-7 quantile at level q of |x[0..rows-1][ch]|: with the
 *    magnitudes sorted ascending into v, h = q (rows-1), lo = floor(h),
 *    hi = min(lo+1, rows-1), stats = fp32(v[lo] + (h-lo) (v[hi]-v[lo])),
 *    each double operation rounded separately.
 *  mask[ch] = 1 for the n_protect largest stats (ties: lower ch first), else 0.
 *
 *  x         bf16 [rows][ld], 16-byte aligned, ld % 8 == 0, c <= ld <= 2^22,
 *            1 <= rows < 2^32.
 *  c         number of channels, 1 <= c <= 65536.   q in [0, 1].
 *  n_protect 0 <= n_protect <= c (e.g. ceil(p * c) for a top-p mask).
 *  stats     fp32 [c];  mask  u8 [c].
 *  workspace >= hif4_percentile_workspace_bytes(rows, c) bytes, 256-byte
 *            aligned; scratch. Below 8192 rows about 1.6 KiB per channel;
 *            from 8192 rows on it also holds the one-pass path's partial
 *            counts, 133,120 bytes each, about 512 of them per 2^24
 *            (row, 128-channel block) pairs or part thereof: 75 MB for
 *            57,600 x 5120, 213 MB for 921,600 x 5120. On completion the u32 at byte offset
 *            hif4_percentile_workspace_bytes(rows, c) - 256 holds the number
 *            of channels whose statistic came from exact radix passes: c when
 *            the one-pass window path below does not apply; otherwise the
 *            channels for which the window missed rank lo or hi.
 *
 *  Long columns (rows >= 8192 and ld * S <= 2^20, with the sample stride
 *  S = max(8, ceil(rows / 8192))) first take a one-pass path: the coarse
 *  histogram of every S-th row places, per channel, a window of 512
 *  consecutive magnitude keys around the quantile; one pass over all rows
 *  counts the keys below the window and each key inside it. Channels whose
 *  ranks lo and hi both fall inside are final; the rest are recomputed
 *  exactly, each by two radix passes over its own column, inside the same
 *  final kernel (slow per channel, and normally none). Results are identical
 *  either way.
 */
HIF4_EXPORT hif4_status hif4_percentile_mask(const void *x, int64_t rows, int64_t c, int64_t ld, double q,
                                 int64_t n_protect, float *stats, uint8_t *mask,
                                 void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * hif4_quantize_f32 -- HiF4-quantize rows of fp32 values along k, with the
 * same rule as hif4_quantize applied to the exact fp32 values (HiGPTQ's
 * working weights are real numbers, not bf16).
 *
 *  x      fp32 [rows][ld], 16-byte aligned, ld % 4 == 0, ld >= k; finite.
 *  codes  u8 [rows][k/2], 16-byte aligned.    meta  u32 [rows][k/64].
 *  rows >= 0, k % 64 == 0.
 */
HIF4_EXPORT hif4_status hif4_quantize_f32(const float *x, int64_t rows, int64_t k, int64_t ld,
                              uint8_t *codes, uint32_t *meta, hipStream_t stream);

/*
 * hif4_quantize_offsets -- the quantize step of HiAutoRound (the calibration
 * article, section 3.2 "HiAutoRound": learnable offsets K on the level-3
 * exponents, E' = E + RZ(K), 16 per unit, and M on the mantissas, shifted as
 * M' = M >> RZ(K) before being added), with the offsets given; the training
 * loop that learns them is not part of this library.
 * Readings (the section gives the two formulas only):
 *   - the level-1 code and level-2 bits are chosen as in hif4_quantize; each
 *     level-3 bit e3 too, then e3' = clamp(e3 + trunc(K[q]), 0, 1);
 *   - with d = e3' - e3, M' = M * 2^-d (the shift follows the exponent
 *     change actually applied);
 *   - k = clamp(rint(fl(t + M')), 0, 7), t = fl(|x| / (D / 4)),
 *     D = v(c) 2^(e2 + e3'), each operation IEEE binary32 with round to
 *     nearest even; the sign of x is kept, a zero code has no sign.
 * With K = 0 and M = 0 the output equals hif4_quantize's (unmasked).
 *
 *  x      bf16 [rows][ld], 16-byte aligned, ld % 8 == 0, ld >= k; finite.
 *  koff   fp32 [rows][k/4], row stride k/4 (one K per level-3 group, groups
 *         in K order), 16-byte aligned; finite.
 *  moff   fp32 [rows][k], row stride k (one M per element), 16-byte aligned;
 *         finite.
 *  codes  u8 [rows][k/2], 16-byte aligned.    meta  u32 [rows][k/64].
 *  rows >= 0, k % 64 == 0. Non-finite inputs give unspecified codes.
 */
HIF4_EXPORT hif4_status hif4_quantize_offsets(const void *x, int64_t rows, int64_t k, int64_t ld,
                                  const float *koff, const float *moff, uint8_t *codes,
                                  uint32_t *meta, hipStream_t stream);

/* hif4_higptq_workspace_bytes -- workspace of hif4_higptq_unit for n rows
 * (0 for n < 0 or n >= 2^24, which the entry point refuses). */
HIF4_EXPORT size_t hif4_higptq_workspace_bytes(int64_t n);

/*
 * hif4_higptq_unit -- one group step of HiGPTQ (the calibration article,
 * section 3.1 "HiGPTQ": groups of 64 columns, one HiF4 unit each, with three
 * schemes for fixing the exponents):
 *   scheme 1: the group's 64 columns are quantized at once, all exponents
 *             fixed from them;
 *   scheme 2: the level-1 exponent is fixed from the group first; then 8
 *             columns at a time: level-2 and level-3 fixed from their current
 *             values, quantized, and the weights not yet quantized updated;
 *   scheme 3: level-1 fixed first; per level-2 group, its exponent is fixed
 *             from its 8 current values, its first 4 columns are quantized,
 *             the rest updated, and the second 4 columns re-estimate their
 *             level-3 exponent and are quantized.
 * The update after a set T of columns is GPTQ's (Frantar et al., 2022), with
 * H^-1 = U^T U (H the layer's Hessian over the input channels, U upper
 * triangular):  E = W_T - deq(Q_T),  W_after -= E U_TT^-1 U_T,after.
 * Call it for unit = 0, 1, ... in order; codes/meta then hold the result.
 *
 *  w      fp32 [n][ldw] working weights (in: the current values; out: the
 *         columns after the group updated in place; the group's and earlier
 *         columns are not modified), 16-byte aligned, ldw % 4 == 0,
 *         k <= ldw < 2^22 and n < 2^24 (HIF4_ERR_SHAPE otherwise).
 *  u      fp32 [k][ldu], upper triangular factor, 16-byte aligned,
 *         ldu % 4 == 0, k <= ldu < 2^22; its diagonal in the group must be nonzero (a zero
 *         gives non-finite weights, not a fault).
 *  unit   0 <= unit < k/64: the group's columns are 64 unit .. 64 unit + 63.
 *  scheme 1, 2 or 3 (HIF4_ERR_ARG otherwise).
 *  codes  u8 [n][k/2], meta u32 [n][k/64]: unit `unit` of every row written.
 *  workspace >= hif4_higptq_workspace_bytes(n) bytes, 256-byte aligned; on
 *         return it holds F, fp32 [n][64] row-major (the group's
 *         compensation coefficients, E U^-1 per quantized set).
 *  The fp32 compensation is within rounding of the fp64 formula above; under
 *  scheme 1 the group's codes are exactly the quantization of the weights as
 *  given (schemes 2 and 3 quantize values updated within the group).
 */
HIF4_EXPORT hif4_status hif4_higptq_unit(float *w, int64_t n, int64_t k, int64_t ldw, const float *u,
                             int64_t ldu, int64_t unit, int scheme, uint8_t *codes,
                             uint32_t *meta, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/* Largest block of hif4_higptq_block, in units of 64 columns. */
#define HIF4_HIGPTQ_MAX_BLOCK_UNITS 16

/* hif4_higptq_block_workspace_bytes -- workspace of hif4_higptq_block for n
 * rows and a block of `units` groups: 256 units * ceil(n / 64) * 64 bytes
 * (0 for units outside 1..16, n < 0 or n >= 2^24). */
HIF4_EXPORT size_t hif4_higptq_block_workspace_bytes(int64_t n, int64_t units);

/*
 * hif4_higptq_block -- one block step of HiGPTQ with a blocksize of 64 units
 * columns. GPTQ as the calibration article describes it (section 2.1 "GPTQ")
 * splits the columns into blocks: inside a block the columns are quantized in
 * order, each one's error compensated on the block's columns not yet
 * quantized; once the block is done its whole error is carried to the
 * columns after it in one update. Section 3.1 "HiGPTQ" requires the blocksize
 * to be 64 or a multiple of 64, each group of 64 being one HiF4 unit. Here the
 * groups unit0 .. unit0 + units - 1 are each taken as hif4_higptq_unit takes
 * one group (same schemes); inside the block the updates are nested: the
 * first half of the groups (recursively), then the second half's columns
 * updated once with the first half's F, then the second half (recursively);
 * then W_after -= F_B U_B,after once for the block's compensation
 * coefficients F_B. Every column still takes every earlier group's
 * correction before its own group is quantized.
 * The result is that of hif4_higptq_unit called for unit0 .. unit0 + units - 1
 * in order, up to the order of the fp32 roundings; a block carries the update
 * of the later columns over 64 units columns at once, so a pass over W moves
 * it 1/units as often. Call it for unit0 = 0, units, 2 units, ... (the last
 * block may be shorter).
 *
 *  w, n, k, ldw, u, ldu, scheme, codes, meta: as for hif4_higptq_unit
 *         (HIF4_ERR_SHAPE, HIF4_ERR_ARG, HIF4_ERR_ALIGN alike).
 *  unit0, units  1 <= units <= HIF4_HIGPTQ_MAX_BLOCK_UNITS, 0 <= unit0 and
 *         unit0 + units <= k/64 (HIF4_ERR_ARG otherwise): the block's
 *         columns are 64 unit0 .. 64 (unit0 + units) - 1. The columns before
 *         the block and those of its first group are not modified; each later
 *         group's columns end holding the values that group was quantized
 *         from (as after hif4_higptq_unit for the groups before it); the
 *         columns after the block are updated in place.
 *  codes, meta: units unit0 .. unit0 + units - 1 of every row written.
 *  workspace >= hif4_higptq_block_workspace_bytes(n, units), 256-byte
 *         aligned (HIF4_ERR_WORKSPACE / HIF4_ERR_ALIGN); on return it holds
 *         F_B transposed: fp32 [64 units][ldt], ldt = n rounded up to a
 *         multiple of 64, row 64 j + c holding column c of group j's F for
 *         rows 0 .. n - 1 (the padding is scratch).
 */
HIF4_EXPORT hif4_status hif4_higptq_block(float *w, int64_t n, int64_t k, int64_t ldw,
                              const float *u, int64_t ldu, int64_t unit0, int64_t units,
                              int scheme, uint8_t *codes, uint32_t *meta, void *workspace,
                              size_t workspace_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* HIF4_H */
