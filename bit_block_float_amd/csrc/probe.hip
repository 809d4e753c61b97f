// probe.hip -- measurement probes for the rooflines the benchmark reports
// against; not part of the method and not in libhif4.so (built as
// libhif4_probe.so, declared in include/hif4_probe.h).
//
// Probes: HBM streaming rates (copy, read only, and the quantizer's 4 : 1
// read : write mix) and the bf16 matrix-core ceiling under a full-chip load.
// For the latter every wave issues back-to-back v_mfma_f32_32x32x16_bf16 on
// 16 independent accumulator blocks (the W4A4 kernel's 128 x 128 wave tile,
// one wave per SIMD, four waves per workgroup), with register operands only
// -- no memory traffic, no LDS, no other VALU work in the loop. Its rate is
// what the contraction could reach at the clock the chip holds under that
// load.
#include <hip/hip_runtime.h>

#include "../../include/hif4_probe.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void mfma_bf16_peak_kernel(int iters, float* __restrict__ out) {
  // operands derived from the lane (so nothing folds): small values, the
  // sums stay finite for any iteration count used here
  bf16x8_t a, b;
  const float base = (float)((threadIdx.x & 7) + 1) * (1.0f / 1024.0f);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(base * (float)(i + 1));
    b[i] = (__bf16)(base * (float)(8 - i));
  }
  f32x16_t acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[j][r] = 0.0f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[j][r];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// HBM copy ceiling: a grid-stride copy of 16-byte words with four loads in
// flight per lane before the stores (the streaming shape of the quantizer).
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void copy_probe_kernel(const u32x4_t* __restrict__ src,
                                                         u32x4_t* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4_t a = __builtin_nontemporal_load(src + i);
    const u32x4_t b = __builtin_nontemporal_load(src + i + stride);
    const u32x4_t c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4_t d = __builtin_nontemporal_load(src + i + 3 * stride);
    __builtin_nontemporal_store(a, dst + i);
    __builtin_nontemporal_store(b, dst + i + stride);
    __builtin_nontemporal_store(c, dst + i + 2 * stride);
    __builtin_nontemporal_store(d, dst + i + 3 * stride);
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

// HBM read ceiling: the same stream with no stores but one word per thread
// (the shape of the percentile's window pass, which only reads).
__global__ __launch_bounds__(256) void read_probe_kernel(const u32x4_t* __restrict__ src,
                                                         uint32_t* __restrict__ out, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  uint32_t acc = 0u;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4_t a = __builtin_nontemporal_load(src + i);
    const u32x4_t b = __builtin_nontemporal_load(src + i + stride);
    const u32x4_t c = __builtin_nontemporal_load(src + i + 2 * stride);
    const u32x4_t d = __builtin_nontemporal_load(src + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^
           d.z ^ d.w;
  }
  for (; i < n; i += stride) acc ^= src[i].x;
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc;
}

// Streaming ceiling with the quantizer's traffic mix: per lane four 16-byte
// loads and one 16-byte store (4 bytes read for each one written; the
// quantizer reads 2 bytes per element and writes 0.5625), grid-stride. The
// source is read as four contiguous quarters, so that every load
// instruction covers 1 KiB of consecutive words, as the store does.
__global__ __launch_bounds__(256) void read4_write1_probe_kernel(const u32x4_t* __restrict__ src,
                                                                 u32x4_t* __restrict__ dst,
                                                                 size_t n_out) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_out; i += stride) {
    const u32x4_t a = __builtin_nontemporal_load(src + i);
    const u32x4_t b = __builtin_nontemporal_load(src + n_out + i);
    const u32x4_t c = __builtin_nontemporal_load(src + 2 * n_out + i);
    const u32x4_t d = __builtin_nontemporal_load(src + 3 * n_out + i);
    __builtin_nontemporal_store(a ^ b ^ c ^ d, dst + i);
  }
}

}  // namespace

extern "C" int hif4_probe_read4_write1(const void* src, size_t src_bytes, void* dst, int blocks,
                                       hipStream_t stream) {
  if (!src || !dst || src_bytes % 64 != 0 || blocks <= 0) return 1;
  hipLaunchKernelGGL(read4_write1_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const u32x4_t*)src, (u32x4_t*)dst, src_bytes / 64);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

extern "C" int hif4_probe_read(const void* src, size_t bytes, void* out, int blocks,
                               hipStream_t stream) {
  if (!src || !out || bytes % 16 != 0 || blocks <= 0) return 1;
  hipLaunchKernelGGL(read_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const u32x4_t*)src, (uint32_t*)out, bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

extern "C" int hif4_probe_copy(const void* src, void* dst, size_t bytes, int blocks,
                               hipStream_t stream) {
  if (!src || !dst || bytes % 16 != 0 || blocks <= 0) return 1;
  hipLaunchKernelGGL(copy_probe_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                     (const u32x4_t*)src, (u32x4_t*)dst, bytes / 16);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}

extern "C" int hif4_probe_mfma_bf16(int blocks, int iters, float* out, hipStream_t stream) {
  if (blocks <= 0 || iters <= 0 || out == nullptr) return 1;
  hipLaunchKernelGGL(mfma_bf16_peak_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, iters,
                     out);
  return hipGetLastError() == hipSuccess ? 0 : 7;
}
