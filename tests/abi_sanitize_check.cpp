// abi_sanitize_check.cpp -- drives the host-side argument checks and
// workspace queries of the C-ABI (csrc/api.hip) for a build whose host code
// runs under AddressSanitizer and UndefinedBehaviorSanitizer
// (tests/test_oracle_sanitize.py builds and runs it).
//
// Every call here is refused, or is empty, before any device work, so the
// program needs no GPU: it checks that invalid arguments map to the
// documented status codes and that the size queries stay defined (no signed
// overflow, no wrap into a small size) over the whole int64 argument range.
#include <stdint.h>
#include <stdio.h>

#include "hif4.h"

static int failures = 0;

static void expect(long long got, long long want, const char* what) {
  if (got != want) {
    fprintf(stderr, "FAIL %s: got %lld, expected %lld\n", what, got, want);
    ++failures;
  }
}

int main() {
  // a 256-byte-aligned stand-in address: never dereferenced by these calls
  char* const A = reinterpret_cast<char*>(0x100000);
  const int64_t big[] = {INT64_MAX, INT64_MAX - 63, (int64_t)1 << 62, (int64_t)1 << 40,
                         (int64_t)1 << 32, (int64_t)1 << 31};

  // status strings and the version
  for (int s = -1; s < 12; ++s)
    if (!hif4_status_string(s)) {
      fprintf(stderr, "FAIL status string %d\n", s);
      ++failures;
    }
  expect(hif4_version(), 1, "version");

  // workspace queries: 0 for shapes the entry points refuse, never a wrapped
  // small size
  for (int64_t v : big) {
    expect((long long)hif4_linear_workspace_bytes(v, 8, 64, 0), 0, "linear ws, m");
    expect((long long)hif4_linear_workspace_bytes(8, v, 64, 0), 0, "linear ws, n");
    expect((long long)hif4_linear_workspace_bytes(8, 8, v, 0), 0, "linear ws, k");
    expect((long long)hif4_linear_workspace_bytes(8, 8, 64, v), 0, "linear ws, n_kept");
    if (v > 0xFFFFFFFFll)  // rows below 2^32 are accepted
      expect((long long)hif4_percentile_workspace_bytes(v, 5120), 0, "percentile ws, rows");
    expect((long long)hif4_percentile_workspace_bytes(57600, v), 0, "percentile ws, c");
    expect((long long)hif4_higptq_workspace_bytes(v), 0, "higptq ws");
    expect((long long)hif4_higptq_block_workspace_bytes(v, 8), 0, "higptq block ws");
  }
  expect((long long)hif4_linear_workspace_bytes(-1, 8, 64, 0), 0, "linear ws, m < 0");
  expect(hif4_linear_workspace_bytes(57600, 13824, 5120, 52) > 0, 1, "linear ws, FFN-up");
  expect(hif4_percentile_workspace_bytes(57600, 5120) > 0, 1, "percentile ws, FFN-up");
  expect(hif4_percentile_workspace_bytes(0xFFFFFFFFll, 65536) > 0, 1, "percentile ws, limits");
  expect(hif4_higptq_block_workspace_bytes(13824, 16) > 0, 1, "higptq block ws");

  // quantize
  expect(hif4_quantize(A, -1, 64, 64, nullptr, 0, nullptr, (uint8_t*)A, (uint32_t*)A, nullptr),
         HIF4_ERR_SHAPE, "quantize rows < 0");
  expect(hif4_quantize(A, 4, INT64_MAX, INT64_MAX, nullptr, 0, nullptr, (uint8_t*)A,
                       (uint32_t*)A, nullptr),
         HIF4_ERR_SHAPE, "quantize k % 64");
  expect(hif4_quantize(A, INT64_MAX, (int64_t)1 << 40, (int64_t)1 << 40, nullptr, 0, nullptr,
                       (uint8_t*)A, (uint32_t*)A, nullptr) != HIF4_OK,
         1, "quantize huge shape refused");
  expect(hif4_quantize(A, 4, 64, 64, (const uint8_t*)A, INT64_MAX, (void*)A, (uint8_t*)A,
                       (uint32_t*)A, nullptr),
         HIF4_ERR_SHAPE, "quantize n_mask > k");
  expect(hif4_quantize(nullptr, 4, 64, 64, nullptr, 0, nullptr, (uint8_t*)A, (uint32_t*)A,
                       nullptr),
         HIF4_ERR_NULL, "quantize x null");
  expect(hif4_quantize(A + 2, 4, 64, 64, nullptr, 0, nullptr, (uint8_t*)A, (uint32_t*)A,
                       nullptr),
         HIF4_ERR_ALIGN, "quantize x misaligned");
  expect(hif4_quantize(A, 0, 64, 64, nullptr, 0, nullptr, nullptr, nullptr, nullptr), HIF4_OK,
         "quantize empty");

  // dequantize
  expect(hif4_dequantize((const uint8_t*)A, (const uint32_t*)A, 4, 100, A, HIF4_F32, nullptr),
         HIF4_ERR_SHAPE, "dequantize k % 64");
  expect(hif4_dequantize((const uint8_t*)A, (const uint32_t*)A, INT64_MAX, INT64_MAX - 63, A,
                         HIF4_F32, nullptr) != HIF4_OK,
         1, "dequantize huge shape refused");
  expect(hif4_dequantize((const uint8_t*)A, (const uint32_t*)A, 4, 64, A, 7, nullptr),
         HIF4_ERR_DTYPE, "dequantize dtype");

  // linear entry points
  const size_t ws = hif4_linear_workspace_bytes(8, 8, 64, 0);
  expect(hif4_linear_w4a4(A, nullptr, nullptr, (const uint8_t*)A, (const uint32_t*)A, nullptr,
                          nullptr, nullptr, 0, 8, 8, 60, A, HIF4_F32, A, ws, nullptr),
         HIF4_ERR_SHAPE, "linear k % 64");
  expect(hif4_linear_w4a4(A, nullptr, nullptr, (const uint8_t*)A, (const uint32_t*)A, nullptr,
                          nullptr, nullptr, 0, INT64_MAX, INT64_MAX, (int64_t)1 << 62, A,
                          HIF4_F32, A, ws, nullptr),
         HIF4_ERR_SHAPE, "linear huge shape");
  expect(hif4_linear_w4a4(A, nullptr, nullptr, (const uint8_t*)A, (const uint32_t*)A, nullptr,
                          nullptr, nullptr, 0, 8, 8, 64, A, HIF4_F32, A, ws - 1, nullptr),
         HIF4_ERR_WORKSPACE, "linear workspace short");
  expect(hif4_linear_w4a4(A, nullptr, nullptr, (const uint8_t*)A, (const uint32_t*)A,
                          (const uint8_t*)A, nullptr, A, INT64_MAX, 8, 8, 64, A, HIF4_F32, A,
                          ws, nullptr),
         HIF4_ERR_SHAPE, "linear n_kept huge");
  expect(hif4_linear_xcodes_wbf16((const uint8_t*)A, (const uint32_t*)A, A, nullptr, nullptr, 0,
                                  8, 8, 64, A, 2, nullptr, 0, nullptr),
         HIF4_ERR_DTYPE, "xcodes dtype");
  expect(hif4_linear_xcodes_wbf16((const uint8_t*)A, (const uint32_t*)A, A, A, A, 5, 8, 8, 64,
                                  A, HIF4_F32, A, 1, nullptr),
         HIF4_ERR_WORKSPACE, "xcodes workspace short");
  expect(hif4_linear_xcodes_wbf16_noalloc((const uint8_t*)A, (const uint32_t*)A, A, A, A, 64,
                                          ((int64_t)1 << 31) - 1, 8, 64, A, HIF4_F32, nullptr),
         HIF4_ERR_SCRATCH, "noalloc beyond its scratch");

  // percentile and mask
  const size_t pws = hif4_percentile_workspace_bytes(100, 256);
  float* const Af = reinterpret_cast<float*>(A);
  expect(hif4_percentile_mask(A, INT64_MAX, 256, 256, 0.5, 1, Af, (uint8_t*)A, A, pws, nullptr),
         HIF4_ERR_SHAPE, "percentile rows huge");
  expect(hif4_percentile_mask(A, 100, 256, INT64_MAX, 0.5, 1, Af, (uint8_t*)A, A, pws, nullptr),
         HIF4_ERR_SHAPE, "percentile ld huge");
  expect(hif4_percentile_mask(A, 100, 256, 256, -0.0 / 0.0 * 0.0, 1, Af, (uint8_t*)A, A, pws,
                              nullptr),
         HIF4_ERR_ARG, "percentile q NaN");
  expect(hif4_percentile_mask(A, 100, 256, 256, 0.5, 1, Af, (uint8_t*)A, A, pws - 1, nullptr),
         HIF4_ERR_WORKSPACE, "percentile workspace short");

  // HiGPTQ and HiAutoRound
  float* const W = reinterpret_cast<float*>(A);
  const size_t gws = hif4_higptq_workspace_bytes(10);
  expect(hif4_higptq_unit(W, 10, 128, 128, W, 128, 0, 1, (uint8_t*)A, (uint32_t*)A, A, gws - 1,
                          nullptr),
         HIF4_ERR_WORKSPACE, "higptq workspace short");
  expect(hif4_higptq_unit(W, INT64_MAX, 128, 128, W, 128, 0, 1, (uint8_t*)A, (uint32_t*)A, A, gws,
                          nullptr),
         HIF4_ERR_SHAPE, "higptq n huge");
  expect(hif4_higptq_unit(W, 10, 128, 128, W, 128, INT64_MAX, 1, (uint8_t*)A, (uint32_t*)A, A,
                          gws, nullptr),
         HIF4_ERR_ARG, "higptq unit huge");
  const size_t bws = hif4_higptq_block_workspace_bytes(10, 3);
  expect(hif4_higptq_block(W, 10, 256, 256, W, 256, INT64_MAX - 1, 3, 1, (uint8_t*)A,
                           (uint32_t*)A, A, bws, nullptr),
         HIF4_ERR_ARG, "higptq block unit0 huge");
  expect(hif4_quantize_offsets(A, 4, 64, 64, Af, Af, (uint8_t*)A, (uint32_t*)(A + 2), nullptr),
         HIF4_ERR_ALIGN, "quantize_offsets meta misaligned");
  expect(hif4_quantize_offsets(A, INT64_MAX, 64, 64, Af, Af, (uint8_t*)A, (uint32_t*)A, nullptr)
             != HIF4_OK,
         1, "quantize_offsets rows huge refused");
  expect(hif4_quantize_f32(Af, 4, 65, 72, (uint8_t*)A, (uint32_t*)A, nullptr), HIF4_ERR_SHAPE,
         "quantize_f32 k % 64");

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("abi-sanitize-check OK\n");
  return 0;
}
