// gptq.hip -- HiF4 quantize of fp32 values and the HiGPTQ scheme-1 step.
//
// HiGPTQ: HiFloat4 calibration article (hwcomputing.csdn.net), section 3.1
// "HiGPTQ": groups of 64 columns (one HiF4 unit each) quantized under one of
// three schemes (64 columns at once; 8 at a time; 4 at a time, the level-1
// exponent fixed first in the latter two), the weights not yet quantized
// updated to compensate after each quantized set. The update is GPTQ's (Frantar et al., "GPTQ: Accurate
// Post-Training Quantization for Generative Pre-trained Transformers", 2022)
// for a set S of columns fixed together, with H^-1 = U^T U (U upper
// triangular, given by the caller):
//     E = W_S - deq(Q(W_S)),   F = E U_SS^-1,   W_R -= F U_SR
// for R = the columns after S.
//
// The working weights are fp32, so the quantizer here takes fp32 values: the
// rule is the one of quant.hip (hif4.h states it), with the element rounding
// done by counting grid midpoints -- (2m+1) D/8 has at most 7 significant
// bits, exact in fp32, so the comparisons are exact for any fp32 input.
#include "hif4_dev.h"

namespace hif4 {

// One 64-element unit of fp32 values (v, in registers) -> its 8 code words
// and meta word, and the dequantized values (deq, exact in fp32).
__device__ __forceinline__ void quantize_unit_f32(const float (&v)[64], uint32_t (&cw)[8],
                                                  uint32_t& meta, float (&deq)[64]) {
  // step 1: maxima of |x| per level-3 group (4), level-2 group (8), unit
  float m4[16];
#pragma unroll
  for (int q = 0; q < 16; ++q)
    m4[q] = fmaxf(fmaxf(fabsf(v[4 * q]), fabsf(v[4 * q + 1])),
                  fmaxf(fabsf(v[4 * q + 2]), fabsf(v[4 * q + 3])));
  float a = 0.0f;
#pragma unroll
  for (int q = 0; q < 16; ++q) a = fmaxf(a, m4[q]);
  // step 2: level-1 code
  const uint32_t c = level1_code(a);
  const float s = e6m2_f32(c);
  uint32_t mw = c;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    // steps 3-4: level-2 / level-3 bits (exact compares)
    const uint32_t e2 = fmaxf(m4[2 * g], m4[2 * g + 1]) > 3.5f * s;
    const float t3 = (e2 ? 3.5f : 1.75f) * s;
    const uint32_t e3a = m4[2 * g] > t3, e3b = m4[2 * g + 1] > t3;
    mw |= (e2 << (8 + g)) | (e3a << (16 + 2 * g)) | (e3b << (17 + 2 * g));
    uint32_t word = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int j = 8 * g + i;
      const uint32_t e3 = i < 4 ? e3a : e3b;
      const float D = ldexpf(s, (int)(e2 + e3));
      const float ax = fabsf(v[j]);
      // step 5: k = midpoints (2m+1) D/8 below |x|; at a midpoint the even
      // neighbour wins (> for even m, >= for odd m); 7 beyond the last one
      uint32_t k = 0u;
#pragma unroll
      for (int m = 0; m < 7; ++m) {
        const float mid = D * (0.125f * (float)(2 * m + 1));
        k += (m & 1) ? (ax >= mid ? 1u : 0u) : (ax > mid ? 1u : 0u);
      }
      const uint32_t sgn = (v[j] < 0.0f && k != 0u) ? 8u : 0u;
      word |= (k | sgn) << (i < 4 ? 8 * i : 8 * (i - 4) + 4);
      const float mag = D * (0.25f * (float)k);
      deq[j] = sgn ? -mag : mag;
    }
    cw[g] = word;
  }
  meta = mw;
}

// fp32 quantize: one thread per (row, unit); lanes of a wave take
// consecutive units of a row.
__global__ __launch_bounds__(256) void quantize_f32_kernel(const float* __restrict__ x,
                                                           int64_t ld, int64_t rows,
                                                           int64_t units,
                                                           uint32_t* __restrict__ codes32,
                                                           uint32_t* __restrict__ meta) {
  const int64_t total = rows * units;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t r = t / units, u = t - r * units;
    const float4* src = reinterpret_cast<const float4*>(x + r * ld + u * 64);
    float v[64];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float4 q = src[i];
      v[4 * i] = q.x;
      v[4 * i + 1] = q.y;
      v[4 * i + 2] = q.z;
      v[4 * i + 3] = q.w;
    }
    uint32_t cw[8], mw;
    float deq[64];
    quantize_unit_f32(v, cw, mw, deq);
    uint4* dst = reinterpret_cast<uint4*>(codes32 + t * 8);
    dst[0] = make_uint4(cw[0], cw[1], cw[2], cw[3]);
    dst[1] = make_uint4(cw[4], cw[5], cw[6], cw[7]);
    meta[t] = mw;
  }
}

// HiGPTQ group step, part 1: one thread per row, the group's 64 values in
// registers, U_SS in LDS. Writes unit `unit` of the row's codes and meta and
// the row's 64 values of F (the compensation of the columns after the group
// is F U_SR, part 2).
//   scheme 1: quantize the 64 values at once (all exponents from them), then
//             F = E U_SS^-1 by forward substitution;
//   scheme 2: level-1 from the 64 values first; then per 8 columns: level-2
//             and level-3 from their current values, quantize, F over the 8
//             (forward substitution on their diagonal block of U), and update
//             the group's later columns by F U before the next 8;
//   scheme 3: as scheme 2 per 4 columns, with each level-2 exponent fixed
//             from its 8 current values before its first 4 columns.
template <int kScheme>
__global__ __launch_bounds__(256) void higptq_group_kernel(
    const float* __restrict__ w, int64_t ldw, int64_t n, const float* __restrict__ u,
    int64_t ldu, int64_t s0, int64_t units, int64_t unit, uint32_t* __restrict__ codes32,
    uint32_t* __restrict__ meta, float* __restrict__ f) {
  __shared__ float uss[64 * 65];  // U_SS, row i at uss[65 i] (padded)
  for (int t = threadIdx.x; t < 64 * 64; t += blockDim.x) {
    const int i = t >> 6, j = t & 63;
    uss[65 * i + j] = u[(s0 + i) * ldu + s0 + j];
  }
  __syncthreads();
  const int64_t r = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (r >= n) return;
  const float4* src = reinterpret_cast<const float4*>(w + r * ldw + s0);
  float v[64];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float4 q = src[i];
    v[4 * i] = q.x;
    v[4 * i + 1] = q.y;
    v[4 * i + 2] = q.z;
    v[4 * i + 3] = q.w;
  }
  uint32_t cw[8], mw;
  if constexpr (kScheme == 1) {
    float deq[64];
    quantize_unit_f32(v, cw, mw, deq);
    // E = W_S - deq (exact: the two differ by at most half a grid step), then
    // f_j = (e_j - sum_{i<j} f_i U_ij) / U_jj, overwriting v
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      float acc = v[j] - deq[j];
#pragma unroll
      for (int i = 0; i < j; ++i) acc = fmaf(-v[i], uss[65 * i + j], acc);
      v[j] = acc / uss[65 * j + j];
    }
  } else {
    constexpr int kSpan = kScheme == 2 ? 8 : 4;
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 64; ++j) a = fmaxf(a, fabsf(v[j]));
    const uint32_t c = level1_code(a);  // fixed from the group before any update
    const float s = e6m2_f32(c);
    mw = c;
#pragma unroll
    for (int g = 0; g < 8; ++g) cw[g] = 0u;
    uint32_t e2 = 0u;
#pragma unroll
    for (int t0 = 0; t0 < 64; t0 += kSpan) {
      const int g = t0 / 8;
      if (t0 % 8 == 0) {  // level-2 of group g from its 8 current values
        float m8 = 0.0f;
#pragma unroll
        for (int j = 8 * g; j < 8 * g + 8; ++j) m8 = fmaxf(m8, fabsf(v[j]));
        e2 = m8 > 3.5f * s;
        mw |= e2 << (8 + g);
      }
      float e[kSpan];
#pragma unroll
      for (int q = t0 / 4; q < (t0 + kSpan) / 4; ++q) {
        float m4 = 0.0f;
#pragma unroll
        for (int j = 4 * q; j < 4 * q + 4; ++j) m4 = fmaxf(m4, fabsf(v[j]));
        const uint32_t e3 = m4 > (e2 ? 3.5f : 1.75f) * s;
        mw |= e3 << (16 + q);
        const float D = ldexpf(s, (int)(e2 + e3));
#pragma unroll
        for (int j = 4 * q; j < 4 * q + 4; ++j) {
          const float ax = fabsf(v[j]);
          uint32_t k = 0u;
#pragma unroll
          for (int m = 0; m < 7; ++m) {
            const float mid = D * (0.125f * (float)(2 * m + 1));
            k += (m & 1) ? (ax >= mid ? 1u : 0u) : (ax > mid ? 1u : 0u);
          }
          const uint32_t sgn = (v[j] < 0.0f && k != 0u) ? 8u : 0u;
          const int i8 = j % 8;
          cw[g] |= (k | sgn) << (i8 < 4 ? 8 * i8 : 8 * (i8 - 4) + 4);
          const float mag = D * (0.25f * (float)k);
          e[j - t0] = v[j] - (sgn ? -mag : mag);  // exact, as in scheme 1
        }
      }
      // F over the span (forward substitution), stored over the span's values
#pragma unroll
      for (int j = t0; j < t0 + kSpan; ++j) {
        float acc = e[j - t0];
#pragma unroll
        for (int i = t0; i < j; ++i) acc = fmaf(-v[i], uss[65 * i + j], acc);
        v[j] = acc / uss[65 * j + j];
      }
      // the group's later columns, before they are quantized
#pragma unroll
      for (int j = t0 + kSpan; j < 64; ++j) {
        float acc = v[j];
#pragma unroll
        for (int i = t0; i < t0 + kSpan; ++i) acc = fmaf(-v[i], uss[65 * i + j], acc);
        v[j] = acc;
      }
    }
  }
  uint4* dst = reinterpret_cast<uint4*>(codes32 + (r * units + unit) * 8);
  dst[0] = make_uint4(cw[0], cw[1], cw[2], cw[3]);
  dst[1] = make_uint4(cw[4], cw[5], cw[6], cw[7]);
  meta[r * units + unit] = mw;
  float4* fo = reinterpret_cast<float4*>(f + r * 64);
#pragma unroll
  for (int i = 0; i < 16; ++i) fo[i] = make_float4(v[4 * i], v[4 * i + 1], v[4 * i + 2], v[4 * i + 3]);
}

// HiGPTQ group step, part 2: W[:, c0..k) -= F U[s0.., c0..k), a rank-64
// update. Workgroup tile: 64 rows x 128 columns; thread: 8 rows x 4 columns.
// The thread's 8 x 4 block of W is loaded first, so that its latency
// overlaps the staging of F (64 x 64) and of the U panel (64 x 128) in LDS
// and the 64-step product; per step a thread reads one float4 of U and two
// of F for 32 FMAs.
constexpr int kUpdRows = 64, kUpdCols = 128;
__global__ __launch_bounds__(256) void higptq_update_kernel(
    float* __restrict__ w, int64_t ldw, int64_t n, int64_t k, const float* __restrict__ u,
    int64_t ldu, int64_t s0, int64_t c0, const float* __restrict__ f) {
  __shared__ __align__(16) float fs[64][kUpdRows];  // fs[i][row]
  __shared__ __align__(16) float us[64][kUpdCols];  // us[i][col]
  const int64_t row0 = (int64_t)blockIdx.y * kUpdRows;
  const int64_t col0 = c0 + (int64_t)blockIdx.x * kUpdCols;
  const int tc = threadIdx.x & 31, tr = threadIdx.x >> 5;  // 32 column quads x 8 row groups
  const int64_t colq = col0 + 4 * tc;
  const bool vec = colq + 4 <= k;  // a whole float4 of this row segment lies inside W
  float wv[8][4];
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int64_t row = row0 + tr * 8 + a;
    if (row < n && vec) {
      const float4 q = *reinterpret_cast<const float4*>(w + row * ldw + colq);
      wv[a][0] = q.x; wv[a][1] = q.y; wv[a][2] = q.z; wv[a][3] = q.w;
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b)
        wv[a][b] = (row < n && colq + b < k) ? w[row * ldw + colq + b] : 0.0f;
    }
  }
  // staging with 16-byte loads: F rows (64 floats each) transposed into
  // fs[i][row], U panel rows copied as they are
  for (int t = threadIdx.x; t < 16 * kUpdRows; t += blockDim.x) {
    const int rr = t >> 4, i4 = (t & 15) * 4;
    const int64_t row = row0 + rr;
    float4 q = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    if (row < n) q = *reinterpret_cast<const float4*>(f + row * 64 + i4);
    fs[i4][rr] = q.x;
    fs[i4 + 1][rr] = q.y;
    fs[i4 + 2][rr] = q.z;
    fs[i4 + 3][rr] = q.w;
  }
  for (int t = threadIdx.x; t < 64 * (kUpdCols / 4); t += blockDim.x) {
    const int i = t / (kUpdCols / 4), c4 = (t % (kUpdCols / 4)) * 4;
    const int64_t col = col0 + c4;
    const float* src = u + (s0 + i) * ldu + col;
    float4 q;
    if (col + 4 <= k) {
      q = *reinterpret_cast<const float4*>(src);
    } else {
      q.x = col < k ? src[0] : 0.0f;
      q.y = col + 1 < k ? src[1] : 0.0f;
      q.z = col + 2 < k ? src[2] : 0.0f;
      q.w = col + 3 < k ? src[3] : 0.0f;
    }
    *reinterpret_cast<float4*>(&us[i][c4]) = q;
  }
  __syncthreads();
  float acc[8][4];
#pragma unroll
  for (int a = 0; a < 8; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = 0.0f;
#pragma unroll 4
  for (int i = 0; i < 64; ++i) {
    const float4 uq = *reinterpret_cast<const float4*>(&us[i][4 * tc]);
    const float4 f0 = *reinterpret_cast<const float4*>(&fs[i][tr * 8]);
    const float4 f1 = *reinterpret_cast<const float4*>(&fs[i][tr * 8 + 4]);
    const float fv[8] = {f0.x, f0.y, f0.z, f0.w, f1.x, f1.y, f1.z, f1.w};
#pragma unroll
    for (int a = 0; a < 8; ++a) {
      acc[a][0] = fmaf(fv[a], uq.x, acc[a][0]);
      acc[a][1] = fmaf(fv[a], uq.y, acc[a][1]);
      acc[a][2] = fmaf(fv[a], uq.z, acc[a][2]);
      acc[a][3] = fmaf(fv[a], uq.w, acc[a][3]);
    }
  }
#pragma unroll
  for (int a = 0; a < 8; ++a) {
    const int64_t row = row0 + tr * 8 + a;
    if (row >= n) continue;
    if (vec) {
      *reinterpret_cast<float4*>(w + row * ldw + colq) =
          make_float4(wv[a][0] - acc[a][0], wv[a][1] - acc[a][1], wv[a][2] - acc[a][2],
                      wv[a][3] - acc[a][3]);
    } else {
#pragma unroll
      for (int b = 0; b < 4; ++b)
        if (colq + b < k) w[row * ldw + colq + b] = wv[a][b] - acc[a][b];
    }
  }
}

}  // namespace hif4

using namespace hif4;

hipError_t hif4_launch_quantize_f32(const float* x, int64_t rows, int64_t k, int64_t ld,
                                    uint8_t* codes, uint32_t* meta, hipStream_t stream) {
  if (rows == 0 || k == 0) return hipSuccess;
  const int64_t units = k / 64, total = rows * units;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  hipLaunchKernelGGL(quantize_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, ld,
                     rows, units, reinterpret_cast<uint32_t*>(codes), meta);
  return hipGetLastError();
}

hipError_t hif4_launch_higptq_unit(float* w, int64_t n, int64_t k, int64_t ldw, const float* u,
                                   int64_t ldu, int64_t unit, int scheme, uint8_t* codes,
                                   uint32_t* meta, float* f, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t s0 = unit * 64, units = k / 64;
  const dim3 gg((unsigned)((n + 255) / 256)), gb(256);
  uint32_t* c32 = reinterpret_cast<uint32_t*>(codes);
  if (scheme == 1)
    hipLaunchKernelGGL(higptq_group_kernel<1>, gg, gb, 0, stream, w, ldw, n, u, ldu, s0, units,
                       unit, c32, meta, f);
  else if (scheme == 2)
    hipLaunchKernelGGL(higptq_group_kernel<2>, gg, gb, 0, stream, w, ldw, n, u, ldu, s0, units,
                       unit, c32, meta, f);
  else
    hipLaunchKernelGGL(higptq_group_kernel<3>, gg, gb, 0, stream, w, ldw, n, u, ldu, s0, units,
                       unit, c32, meta, f);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t c0 = s0 + 64;
  if (c0 >= k) return hipSuccess;
  const dim3 grid((unsigned)((k - c0 + kUpdCols - 1) / kUpdCols),
                  (unsigned)((n + kUpdRows - 1) / kUpdRows));
  hipLaunchKernelGGL(higptq_update_kernel, grid, dim3(256), 0, stream, w, ldw, n, k, u, ldu, s0,
                     c0, (const float*)f);
  return hipGetLastError();
}
