// gptq.hip -- HiF4 quantize of fp32 values and the HiGPTQ group step.
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

// HiGPTQ group step, part 1: four lanes per row (a quad), lane q owning the
// group's columns j = 4m + q (m = 0..15), so that a level-3 group is one
// column per lane and its maximum a two-step quad reduction; U_SS in LDS.
// Writes unit `unit` of the row's codes and meta and the row's 64 values of F
// (the compensation of the columns after the group is F U_SR, part 2).
//   scheme 1: quantize the 64 values at once (all exponents from them), then
//             F = E U_SS^-1;
//   scheme 2: level-1 from the 64 values first; then per 8 columns: level-2
//             and level-3 from their current values, quantize, F over the 8,
//             and the group's later columns updated by F U before the next 8;
//   scheme 3: as scheme 2 per 4 columns, with each level-2 exponent fixed
//             from its 8 current values before its first 4 columns.
// F is formed right-looking: once f_i = v_i / U_ii is known (v_i broadcast
// from its owner lane), every later column takes v_j -= f_i U_ij. Per column
// that is the order of the forward substitution, i = 0, 1, ...: the same
// operations in the same order as one thread per row would do.
__device__ __forceinline__ float quad_maxf(float x) {
  x = fmaxf(x, __uint_as_float(dpp<kDppQuadXor1>(__float_as_uint(x))));
  return fmaxf(x, __uint_as_float(dpp<kDppQuadXor2>(__float_as_uint(x))));
}
template <int kLane>
__device__ __forceinline__ float quad_bcastf(float x) {
  return __uint_as_float(dpp<kLane * 0x55>(__float_as_uint(x)));  // quad_perm [o,o,o,o]
}

template <int kScheme>
__global__ __launch_bounds__(256) void higptq_group_kernel(
    const float* __restrict__ w, int64_t ldw, int64_t n, const float* __restrict__ u,
    int64_t ldu, int64_t s0, int64_t units, int64_t unit, uint32_t* __restrict__ codes32,
    uint32_t* __restrict__ meta, float* __restrict__ f) {
  // U_SS regrouped by owner lane: U[i][4m + q] at us[64 i + 16 q + m]
  __shared__ __align__(16) float us[64 * 64];
  const int64_t r = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 2;
  const int q = threadIdx.x & 3;
  // the row's values first, so that their latency overlaps the staging
  float v[16];
  if (r < n) {
    const float* wr = w + r * ldw + s0 + q;
#pragma unroll
    for (int m = 0; m < 16; ++m) v[m] = wr[4 * m];
  }
  for (int t = threadIdx.x; t < 64 * 64; t += blockDim.x) {
    const int i = t >> 6, j = t & 63;
    us[64 * i + 16 * (j & 3) + (j >> 2)] = u[(s0 + i) * ldu + s0 + j];
  }
  __syncthreads();
  if (r >= n) return;  // the whole quad
  // level-1 from the 64 values as given (every scheme)
  float a = 0.0f;
#pragma unroll
  for (int m = 0; m < 16; ++m) a = fmaxf(a, fabsf(v[m]));
  a = quad_maxf(a);
  const uint32_t c = level1_code(a);
  const float s = e6m2_f32(c);
  uint32_t mw = c;
  uint32_t cw[8];  // this lane's byte (q) of each code word
#pragma unroll
  for (int g = 0; g < 8; ++g) cw[g] = 0u;
  constexpr int kSpan = kScheme == 1 ? 64 : (kScheme == 2 ? 8 : 4);
  uint32_t e2g[8];
#pragma unroll
  for (int t0 = 0; t0 < 64; t0 += kSpan) {
    // level-2 exponents of the level-2 groups starting in the span, from
    // their 8 current values (columns 8g + q, 8g + 4 + q on this lane)
#pragma unroll
    for (int g = t0 / 8; g < (t0 + kSpan + 7) / 8; ++g) {
      if (8 * g < t0) continue;  // fixed before this span (scheme 3)
      const float m8 = quad_maxf(fmaxf(fabsf(v[2 * g]), fabsf(v[2 * g + 1])));
      e2g[g] = m8 > 3.5f * s;
      mw |= e2g[g] << (8 + g);
    }
    // level-3 exponents and element codes of the span's columns, E in place
#pragma unroll
    for (int m = t0 / 4; m < (t0 + kSpan) / 4; ++m) {
      const uint32_t e2 = e2g[m / 2];
      const float m4 = quad_maxf(fabsf(v[m]));
      const uint32_t e3 = m4 > (e2 ? 3.5f : 1.75f) * s;
      mw |= e3 << (16 + m);
      const float D = ldexpf(s, (int)(e2 + e3));
      const float ax = fabsf(v[m]);
      // k = midpoints (2t+1) D/8 below |x|; at a midpoint the even neighbour
      // wins (> for even t, >= for odd t); 7 beyond the last one
      uint32_t k = 0u;
#pragma unroll
      for (int t = 0; t < 7; ++t) {
        const float mid = D * (0.125f * (float)(2 * t + 1));
        k += (t & 1) ? (ax >= mid ? 1u : 0u) : (ax > mid ? 1u : 0u);
      }
      const uint32_t sgn = (v[m] < 0.0f && k != 0u) ? 8u : 0u;
      // element 4m + q: word m/2, byte q, high nibble for odd m
      cw[m / 2] |= (k | sgn) << (8 * q + 4 * (m & 1));
      const float mag = D * (0.25f * (float)k);
      v[m] = v[m] - (sgn ? -mag : mag);  // exact: within half a grid step
    }
    // F over the span, right-looking; the later columns updated as it goes
#pragma unroll
    for (int i = t0; i < t0 + kSpan; ++i) {
      const int mi = i >> 2, oi = i & 3;
      float vi;
      if (oi == 0) vi = quad_bcastf<0>(v[mi]);
      else if (oi == 1) vi = quad_bcastf<1>(v[mi]);
      else if (oi == 2) vi = quad_bcastf<2>(v[mi]);
      else vi = quad_bcastf<3>(v[mi]);
      const float fi = vi / us[64 * i + 16 * oi + mi];
      if (q == oi) v[mi] = fi;
      const float* ur = us + 64 * i + 16 * q;
      // column 4 mi + q is after i only on lanes q > oi
      if (q > oi) v[mi] = fmaf(-fi, ur[mi], v[mi]);
#pragma unroll
      for (int m = mi + 1; m < 16; ++m) v[m] = fmaf(-fi, ur[m], v[m]);
    }
  }
  // code words: OR of the four lanes' bytes; lane q stores words 2q, 2q + 1
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    cw[g] |= dpp<kDppQuadXor1>(cw[g]);
    cw[g] |= dpp<kDppQuadXor2>(cw[g]);
  }
  uint32_t w0 = cw[0], w1 = cw[1];
#pragma unroll
  for (int g = 1; g < 4; ++g)
    if (q == g) { w0 = cw[2 * g]; w1 = cw[2 * g + 1]; }
  *reinterpret_cast<uint2*>(codes32 + (r * units + unit) * 8 + 2 * q) = make_uint2(w0, w1);
  if (q == 0) meta[r * units + unit] = mw;
  float* fo = f + r * 64 + q;
#pragma unroll
  for (int m = 0; m < 16; ++m) fo[4 * m] = v[m];
}

// HiGPTQ group step, part 2: W[:, c0..k) -= F U[s0.., c0..k), a rank-64
// update on the fp32 matrix cores (v_mfma_f32_32x32x2_f32). Each element of
// W is read and written once and takes 128 flops, 16 per byte: the matrix
// cores would need more than HBM delivers, so the kernel is built to stream W
// and to keep enough of it in flight.
//
// The product is taken transposed, W^T -= U^T (-F)^T: in the instruction's
// output layout (lane l, register r: row 8(r/4) + 4(l/32) + r%4, column l%32)
// a lane then holds one row of W and, per register quad, four consecutive
// columns. The contraction index is split by lane half (step t: lanes 0-31
// contribute index t, lanes 32-63 index 32 + t), so a lane's -F operand is 32
// consecutive values of its F row and its U operand 32 rows of one column.
//
// Workgroup: 4 waves, each 64 rows x 64 columns (two 32-column blocks); the
// column range after a group is a multiple of 64, so every block is whole.
// W and the U block travel as 16-byte loads of whole 128-byte row pieces
// (instruction i: rows 8i + l/8, bytes 16 (l%8)) and are reordered through a
// wave-private LDS slice (no barrier): W rows padded to 36 floats; U rows 32..63
// shifted by 32 floats so that the two lane halves read different banks. The
// second block's loads are issued before the first block is computed, F's
// together with the first block's; the code is straight-line so that every
// wait counts exactly the loads it needs.
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4u_t __attribute__((ext_vector_type(4)));
constexpr int kRsrcWord3Upd = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kUpdWaveRows = 64, kUpdRows = 4 * kUpdWaveRows, kUpdCols = 64;
constexpr int kUpdWStride = 36;                        // floats per LDS row of the W block
constexpr int kUpdUFloats = 64 * 32 + 32;              // U block, rows 32..63 shifted by 32
constexpr int kUpdSlice = 64 * kUpdWStride + kUpdUFloats;  // floats per wave

template <bool kFull>
__device__ __forceinline__ void higptq_update_wave(float* __restrict__ w, int64_t ldw, int64_t n,
                                                   int64_t k, const float* __restrict__ u,
                                                   int64_t ldu, int64_t s0, int64_t cb0,
                                                   const float* __restrict__ f, int64_t r0,
                                                   float* __restrict__ sl) {
  const int lane = threadIdx.x & 63, li = lane & 31, h = lane >> 5;
  // F rows r0 + 32b + li, values 32h .. 32h + 31 (rows past n read as zero)
  float4 fr[2][8];
#pragma unroll
  for (int b = 0; b < 2; ++b) {
    const int64_t row = r0 + 32 * b + li;
    const float4* src = reinterpret_cast<const float4*>(f + row * 64 + 32 * h);
#pragma unroll
    for (int q = 0; q < 8; ++q)
      fr[b][q] = (kFull || row < n) ? src[q] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
  }
  // Buffer resources at the wave's corner of W and of the U panel; the lane
  // offsets are 32-bit (ldw, ldu < 2^22 keep every offset below 2^30).
  const int64_t wrows = n - r0 < kUpdWaveRows ? n - r0 : kUpdWaveRows;
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(w + r0 * ldw + cb0), (short)0, (int)(((wrows - 1) * ldw + (k - cb0)) * 4),
      kRsrcWord3Upd);
  const __amdgpu_buffer_rsrc_t ru = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(u + s0 * ldu + cb0), (short)0, (int)((63 * ldu + (k - cb0)) * 4), kRsrcWord3Upd);
  const int cr = lane >> 3, cc = 4 * (lane & 7);
  const int vw = (int)((cr * ldw + cc) * 4), sw8 = (int)(8 * ldw * 4);
  const int vu = (int)((cr * ldu + cc) * 4), su8 = (int)(8 * ldu * 4);
  const int64_t rem = n - r0 - cr;  // W row 8i + cr of the wave is live when 8i < rem
  float* const su = sl + 64 * kUpdWStride;
  struct Blk {
    f32x4u_t w[8], u[8];
  };
  auto load = [&](Blk& B, int j) {
#pragma unroll
    for (int i = 0; i < 8; ++i) B.u[i] = __builtin_amdgcn_raw_buffer_load_b128(ru, vu, i * su8 + 128 * j, 0);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      f32x4u_t x = {0.0f, 0.0f, 0.0f, 0.0f};
      if (kFull || 8 * i < rem) x = __builtin_amdgcn_raw_buffer_load_b128(rw, vw, i * sw8 + 128 * j, 0);
      B.w[i] = x;
    }
  };
  auto stage = [&](const Blk& B) {
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<f32x4u_t*>(sl + (8 * i + cr) * kUpdWStride + cc) = B.w[i];
#pragma unroll
    for (int i = 0; i < 8; ++i)
      *reinterpret_cast<f32x4u_t*>(su + (8 * i + cr) * 32 + cc + (i >= 4 ? 32 : 0)) = B.u[i];
  };
  float a[2][32];  // -F
  auto run = [&](int j) {
    // accumulators: register 4q + e of block b holds W[32b + li][8q + 4h + e]
    f32x16_t c[2];
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4u_t x =
            *reinterpret_cast<const f32x4u_t*>(sl + (32 * b + li) * kUpdWStride + 8 * q + 4 * h);
        c[b][4 * q] = x[0];
        c[b][4 * q + 1] = x[1];
        c[b][4 * q + 2] = x[2];
        c[b][4 * q + 3] = x[3];
      }
#pragma unroll
    for (int t = 0; t < 32; ++t) {
      const float uv = su[(32 * h + t) * 32 + li + 32 * h];
      c[0] = __builtin_amdgcn_mfma_f32_32x32x2f32(uv, a[0][t], c[0], 0, 0, 0);
      c[1] = __builtin_amdgcn_mfma_f32_32x32x2f32(uv, a[1][t], c[1], 0, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4u_t x = {c[b][4 * q], c[b][4 * q + 1], c[b][4 * q + 2], c[b][4 * q + 3]};
        *reinterpret_cast<f32x4u_t*>(sl + (32 * b + li) * kUpdWStride + 8 * q + 4 * h) = x;
      }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const f32x4u_t x = *reinterpret_cast<const f32x4u_t*>(sl + (8 * i + cr) * kUpdWStride + cc);
      if (kFull || 8 * i < rem) __builtin_amdgcn_raw_buffer_store_b128(x, rw, vw, i * sw8 + 128 * j, 0);
    }
  };
  // the scheduling barriers keep the loads ahead of the work they overlap
  Blk P, Q;
  load(P, 0);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      a[b][4 * q] = -fr[b][q].x;
      a[b][4 * q + 1] = -fr[b][q].y;
      a[b][4 * q + 2] = -fr[b][q].z;
      a[b][4 * q + 3] = -fr[b][q].w;
    }
  load(Q, 1);
  __builtin_amdgcn_sched_barrier(0);
  stage(P);
  __builtin_amdgcn_sched_barrier(0);
  run(0);
  __builtin_amdgcn_sched_barrier(0);
  stage(Q);
  __builtin_amdgcn_sched_barrier(0);
  run(1);
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void
higptq_update_kernel(float* __restrict__ w, int64_t ldw, int64_t n, int64_t k,
                     const float* __restrict__ u, int64_t ldu, int64_t s0, int64_t c0,
                     const float* __restrict__ f) {
  __shared__ __align__(16) float lds[4][kUpdSlice];
  // wave-uniform by construction; said so, the buffer resources stay scalar
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t r0 = (int64_t)blockIdx.y * kUpdRows + (int64_t)wave * kUpdWaveRows;
  if (r0 >= n) return;  // the whole wave lies below W
  const int64_t cb0 = c0 + (int64_t)blockIdx.x * kUpdCols;
  if (n - r0 >= kUpdWaveRows)
    higptq_update_wave<true>(w, ldw, n, k, u, ldu, s0, cb0, f, r0, lds[wave]);
  else
    higptq_update_wave<false>(w, ldw, n, k, u, ldu, s0, cb0, f, r0, lds[wave]);
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
  const dim3 gg((unsigned)((4 * n + 255) / 256)), gb(256);  // four lanes per row
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
