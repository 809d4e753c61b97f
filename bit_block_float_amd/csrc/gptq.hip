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

// HiGPTQ group step, part 1: one row of 16 lanes (a DPP row) per weight row,
// four weight rows per wave; lane p holds the group's columns p + 16 m in
// v[m] (m = 0..3). A level-3 group (4 consecutive columns) is then one
// register of a lane quad and a level-2 group one register of a half row, so
// the maxima are DPP reductions and a set of 4 or 8 columns is quantized by 4
// or 8 lanes at once. Writes unit `unit` of the row's codes and meta and the
// row's 64 values of F (at f + r ldf; the compensation of the columns after
// the group is F U_SR, part 2).
//   scheme 1: quantize the 64 values at once (all exponents from them), then
//             F = E U_SS^-1;
//   scheme 2: level-1 from the 64 values first; then per 8 columns: level-2
//             and level-3 from their current values, quantize, F over the 8,
//             and the group's later columns updated by F U before the next 8;
//   scheme 3: as scheme 2 per 4 columns, with each level-2 exponent fixed
//             from its 8 current values before its first 4 columns.
// F is formed right-looking, column i = 0, 1, ... in the order of the forward
// substitution: once column i holds its final value v_i, every later column
// takes v_j -= v_i (U_ij / U_ii), and f_i = v_i / U_ii. The workgroup stages
// -U_SS in LDS with each row scaled by its diagonal's reciprocal and zeros on
// and below the diagonal, so the step of column i is the same FMAs on every
// lane (v_i broadcast over the row from its owner lane, folded into the FMA):
// the columns up to i take v_i * 0 and keep their values, and F is v times
// the reciprocals once all steps are done. LDS holds row i of that matrix as lane p's four
// values (columns p + 16 m) side by side.
constexpr int kDppRowMirror = 0x140;  // row_mirror: lane i <-> 15-i in 16
__device__ __forceinline__ float quad_maxf(float x) {
  x = fmaxf(x, __uint_as_float(dpp<kDppQuadXor1>(__float_as_uint(x))));
  return fmaxf(x, __uint_as_float(dpp<kDppQuadXor2>(__float_as_uint(x))));
}
__device__ __forceinline__ float half_row_maxf(float quad_max) {  // over 8 lanes
  return fmaxf(quad_max, __uint_as_float(dpp<kDppHalfMirror>(__float_as_uint(quad_max))));
}
__device__ __forceinline__ float row_maxf(float x) {
  x = half_row_maxf(quad_maxf(x));
  return fmaxf(x, __uint_as_float(dpp<kDppRowMirror>(__float_as_uint(x))));
}
// lane `src` of each row of 16 broadcast over its row (row_newbcast); `src`
// is a constant once the caller's loop is unrolled, so the switch folds away
__device__ __forceinline__ float row_bcastf(float x, int src) {
  const uint32_t b = __float_as_uint(x);
  uint32_t y;
  switch (src) {
    case 0: y = dpp<0x150>(b); break;
    case 1: y = dpp<0x151>(b); break;
    case 2: y = dpp<0x152>(b); break;
    case 3: y = dpp<0x153>(b); break;
    case 4: y = dpp<0x154>(b); break;
    case 5: y = dpp<0x155>(b); break;
    case 6: y = dpp<0x156>(b); break;
    case 7: y = dpp<0x157>(b); break;
    case 8: y = dpp<0x158>(b); break;
    case 9: y = dpp<0x159>(b); break;
    case 10: y = dpp<0x15A>(b); break;
    case 11: y = dpp<0x15B>(b); break;
    case 12: y = dpp<0x15C>(b); break;
    case 13: y = dpp<0x15D>(b); break;
    case 14: y = dpp<0x15E>(b); break;
    default: y = dpp<0x15F>(b); break;
  }
  return __uint_as_float(y);
}
// the 16 bits of a wave-wide ballot that belong to this lane's row of 16
__device__ __forceinline__ uint32_t row_bits(uint64_t ballot) {
  return (uint32_t)(ballot >> (threadIdx.x & 48)) & 0xFFFFu;
}
// every fourth bit (0, 4, 8, 12) of x, packed into bits 0..3
__device__ __forceinline__ uint32_t every4th(uint32_t x) {
  x &= 0x1111u;
  x = (x | (x >> 3)) & 0x0303u;
  return (x | (x >> 6)) & 0x000Fu;
}

template <int kScheme>
__global__ __launch_bounds__(256) void higptq_group_kernel(
    const float* __restrict__ w, int64_t ldw, int64_t n, const float* __restrict__ u,
    int64_t ldu, int64_t s0, int64_t units, int64_t unit, uint32_t* __restrict__ codes32,
    uint32_t* __restrict__ meta, float* __restrict__ f, int64_t fsr, int64_t fsc) {
  __shared__ __align__(16) float us[64 * 64];  // row i: -U_ij / U_ii for j > i, else 0
  __shared__ __align__(16) float rinv[64];     // 1 / U_jj at 4 (j % 16) + j / 16
  const int p = threadIdx.x & 15;
  const int64_t r = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) >> 4;
  // the row's values first, so that their latency overlaps the staging
  float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (r < n) {
    const float* wr = w + r * ldw + s0 + p;
#pragma unroll
    for (int m = 0; m < 4; ++m) v[m] = wr[16 * m];
  }
  // U_SS: thread t stages rows i = t / 16 + 16 it (it = 0..3), columns
  // 4 (t % 16) .. + 3; all loads first, so that their latencies overlap
  float4 ux[4];
  float ud[4];
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int i = (threadIdx.x >> 4) + 16 * it, j = 4 * (threadIdx.x & 15);
    const float* ui = u + (s0 + i) * ldu + s0;
    ux[it] = *reinterpret_cast<const float4*>(ui + j);
    ud[it] = ui[i];
  }
#pragma unroll
  for (int it = 0; it < 4; ++it) {
    const int i = (threadIdx.x >> 4) + 16 * it, j = 4 * (threadIdx.x & 15);
    const float ri = 1.0f / ud[it];
    const float xs[4] = {ux[it].x, ux[it].y, ux[it].z, ux[it].w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int jj = j + e;  // lane jj % 16, register jj / 16
      us[64 * i + 4 * (jj & 15) + (jj >> 4)] = jj > i ? -(xs[e] * ri) : 0.0f;
    }
    if ((i >> 2) == (threadIdx.x & 15)) rinv[4 * (i & 15) + (i >> 4)] = ri;
  }
  __syncthreads();
  if (r >= n) return;  // the whole row of 16 lanes
  // level-1 from the 64 values as given (every scheme)
  const float a = row_maxf(fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3]))));
  const uint32_t c = level1_code(a);
  const float s = e6m2_f32(c);
  constexpr int kSpan = kScheme == 1 ? 64 : (kScheme == 2 ? 8 : 4);
  // per register: level-2 / level-3 bits of the lane's groups, element code
  uint32_t e2[4] = {0u, 0u, 0u, 0u}, e3[4] = {0u, 0u, 0u, 0u}, nib[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int sp = 0; sp < 64 / kSpan; ++sp) {
    // registers holding the set's columns sp kSpan .. + kSpan - 1
    constexpr int kRegs = kSpan == 64 ? 4 : 1;
#pragma unroll
    for (int mm = 0; mm < kRegs; ++mm) {
      const int m = kSpan == 64 ? mm : (sp * kSpan) / 16;
      const int col = p + 16 * m;
      const bool in = col / kSpan == sp;
      // the level-2 exponent of a half row is fixed at the first set that
      // reaches it (scheme 3: the first of its two sets of 4), from its 8
      // current values
      const float m4 = quad_maxf(fabsf(v[m]));
      if (kScheme != 3 || (sp & 1) == 0) {
        const bool fix2 = kScheme == 3 ? col / 8 == sp / 2 : in;
        const uint32_t t2 = half_row_maxf(m4) > 3.5f * s;
        if (fix2) e2[m] = t2;
      }
      // level-3 exponent and element code of the lane's column, E in place
      const uint32_t t3 = m4 > (e2[m] ? 3.5f : 1.75f) * s;
      const float D = ldexpf(s, (int)(e2[m] + t3));
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
      const float mag = D * (0.25f * (float)k);
      if (in) {
        e3[m] = t3;
        nib[m] = k | sgn;
        v[m] = v[m] - (sgn ? -mag : mag);  // exact: within half a grid step
      }
    }
    // the set's columns, right-looking: every later column updated (the
    // registers m < i / 16 hold only columns before i and keep their values)
#pragma unroll
    for (int i = sp * kSpan; i < sp * kSpan + kSpan; ++i) {
      const float vi = row_bcastf(v[i >> 4], i & 15);
      const float4 ur = *reinterpret_cast<const float4*>(us + 64 * i + 4 * p);
      if (i < 16) v[0] = fmaf(vi, ur.x, v[0]);
      if (i < 32) v[1] = fmaf(vi, ur.y, v[1]);
      if (i < 48) v[2] = fmaf(vi, ur.z, v[2]);
      v[3] = fmaf(vi, ur.w, v[3]);
    }
  }
  // code words: element j = p + 16 m sits in word j / 8 = 2 m + p / 8, byte
  // p % 4, high nibble for p % 8 >= 4; OR over the half row gives word
  // 2 m + p / 8 on all of its 8 lanes; lane 0 takes the odd words from lane 8
  const int sh = 8 * (p & 3) + 4 * ((p >> 2) & 1);
  uint32_t wd[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) wd[m] = or8_u32(nib[m] << sh);
  uint32_t wo[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) wo[m] = dpp<0x128>(wd[m]);  // row_ror:8: lane 0 <- lane 8
  if (p == 0) {
    uint4* dst = reinterpret_cast<uint4*>(codes32 + (r * units + unit) * 8);
    dst[0] = make_uint4(wd[0], wo[0], wd[1], wo[1]);
    dst[1] = make_uint4(wd[2], wo[2], wd[3], wo[3]);
  }
  // meta: level-3 group 4 m + p / 4 (one bit per quad), level-2 group
  // 2 m + p / 8 (one bit per half row)
  uint32_t b3 = 0u, b2 = 0u;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    b3 |= every4th(row_bits(__builtin_amdgcn_ballot_w64(e3[m] != 0u))) << (4 * m);
    const uint32_t h2 = row_bits(__builtin_amdgcn_ballot_w64(e2[m] != 0u));
    b2 |= ((h2 & 1u) | ((h2 >> 7) & 2u)) << (2 * m);
  }
  if (p == 0) meta[r * units + unit] = c | (b2 << 8) | (b3 << 16);
  const float4 ri = *reinterpret_cast<const float4*>(rinv + 4 * p);
  float* fr = f + r * fsr + p * fsc;
  fr[0] = v[0] * ri.x;
  fr[16 * fsc] = v[1] * ri.y;
  fr[32 * fsc] = v[2] * ri.z;
  fr[48 * fsc] = v[3] * ri.w;
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

// HiGPTQ block update: W[:, c0..c1) -= F[:, 0..R) U[sk..sk+R, c0..c1) with
// R = 64 units (the columns a block has quantized), F given transposed (F^T,
// row i at ft + i ldt), on the fp32 matrix cores (v_mfma_f32_32x32x2_f32). At
// R = 256 an element of W takes 512 flops per 8 bytes moved, so the matrix
// cores, not HBM, set the pace: the kernel keeps W in the accumulators and
// streams only the operands, from L2.
//
// Product taken transposed, W^T -= U^T F^T: in the output layout (lane l,
// register r: row 8(r/4) + 4(l/32) + r%4, column l%32) a lane holds one row of
// W and, per register quad, four consecutive columns, so the W tile moves as
// 16-byte loads and stores straight into and out of the accumulators. Step s
// contracts indices 2s (lanes 0-31) and 2s + 1 (lanes 32-63): a lane's U
// operand is U[sk + 2s + h][its column] and its -F operand F^T[2s + h][its
// row], so each operand load of a wave reads two rows of 32 consecutive
// floats (F transposed for this: row-major F would give a lane per row).
//
// Workgroup (x, y): 4 waves, wave v on rows 256 y + 64 v .. + 63, all on the
// columns c0 + 64 x .. + 63 (c1 - c0 is a multiple of 64). Each wave: four
// 32x32 accumulator tiles (2 row blocks x 2 column blocks). Rows of W past n
// load row n - 1 and are not stored; F^T's rows are padded to a multiple of
// 64, so its loads stay inside them. Operands go 16 contraction indices (8
// steps) at a time, two such chunks in flight; addresses are a wave-uniform
// base per chunk plus 32-bit lane offsets.
template <int kRB>
struct RankOps {
  float f[kRB][8];  // [row block][step]
  float u[2][8];    // [column block][step]
};

__device__ __forceinline__ float buf_ld(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}

template <int kRB>  // row blocks of 32 per wave
__global__ __launch_bounds__(256, 2) void higptq_rank_update_kernel(
    float* __restrict__ w, int64_t ldw, int64_t n, const float* __restrict__ u, int64_t ldu,
    int64_t sk, int64_t c0, const float* __restrict__ ft, int64_t ldt, int R) {
  constexpr int kRows = 32 * kRB;
  const int lane = threadIdx.x & 63, li = lane & 31, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
  const int64_t r0 = (int64_t)blockIdx.y * 4 * kRows + (int64_t)wave * kRows;
  if (r0 >= n) return;  // the whole wave lies below W
  const int64_t cb = c0 + (int64_t)blockIdx.x * 64;
  // the wave's W tile: rows r0 .. r0 + kRows - 1 (past n: row n - 1), columns cb ..
  const int last = n - r0 < kRows ? (int)(n - r0) - 1 : kRows - 1;
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(w + r0 * ldw + cb), (short)0, (int)((last * ldw + 64) * 4), kRsrcWord3Upd);
  int rl[kRB];
#pragma unroll
  for (int b = 0; b < kRB; ++b) rl[b] = 32 * b + li < last ? 32 * b + li : last;
  f32x16_t acc[kRB][2];  // [row block][column block]
#pragma unroll
  for (int b = 0; b < kRB; ++b)
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4u_t x = __builtin_amdgcn_raw_buffer_load_b128(
            rw, (int)((rl[b] * ldw + 4 * h) * 4), (32 * c + 8 * q) * 4, 0);
        acc[b][c][4 * q] = x[0];
        acc[b][c][4 * q + 1] = x[1];
        acc[b][c][4 * q + 2] = x[2];
        acc[b][c][4 * q + 3] = x[3];
      }
  // operand lane offsets (bytes): F^T[2s + h][r0 + 32b + li], U[sk + 2s + h][cb + 32c + li]
  const int fo = (int)((h * ldt + r0 + li) * 4), fs = (int)(2 * ldt * 4);
  const int uo = (int)((h * ldu + li) * 4), us2 = (int)(2 * ldu * 4);
  RankOps<kRB> A, B;
  // chunk T: steps 8T .. 8T + 7, contraction indices 16T .. 16T + 15
  auto load = [&](RankOps<kRB>& X, int T) {
    const __amdgpu_buffer_rsrc_t rf = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(ft + (int64_t)(16 * T) * ldt), (short)0, (int)(16 * ldt * 4), kRsrcWord3Upd);
    const __amdgpu_buffer_rsrc_t ru = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(u + (sk + 16 * T) * ldu + cb), (short)0, (int)(16 * ldu * 4), kRsrcWord3Upd);
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
      for (int b = 0; b < kRB; ++b) X.f[b][st] = buf_ld(rf, fo + 128 * b, st * fs);
#pragma unroll
    for (int st = 0; st < 8; ++st)
#pragma unroll
      for (int c = 0; c < 2; ++c) X.u[c][st] = buf_ld(ru, uo + 128 * c, st * us2);
  };
  auto run = [&](const RankOps<kRB>& X) {
#pragma unroll
    for (int st = 0; st < 8; ++st) {
      float nf[kRB];
#pragma unroll
      for (int b = 0; b < kRB; ++b) nf[b] = -X.f[b][st];
#pragma unroll
      for (int c = 0; c < 2; ++c)
#pragma unroll
        for (int b = 0; b < kRB; ++b)
          acc[b][c] = __builtin_amdgcn_mfma_f32_32x32x2f32(X.u[c][st], nf[b], acc[b][c], 0, 0, 0);
    }
  };
  // the loads are unconditional so that every wait counts exactly the loads
  // it needs across the loop (the last prefetch re-reads the last chunk); the
  // scheduling barriers keep each chunk's loads a whole chunk of work ahead
  const int chunks = R >> 4;  // even: R is a multiple of 64
  load(A, 0);
  for (int T = 0; T < chunks; T += 2) {
    load(B, T + 1);
    __builtin_amdgcn_sched_barrier(0);
    run(A);
    __builtin_amdgcn_sched_barrier(0);
    load(A, T + 2 < chunks ? T + 2 : chunks - 1);
    __builtin_amdgcn_sched_barrier(0);
    run(B);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int b = 0; b < kRB; ++b) {
    if (32 * b + li > last) continue;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const f32x4u_t x = {acc[b][c][4 * q], acc[b][c][4 * q + 1], acc[b][c][4 * q + 2],
                            acc[b][c][4 * q + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(x, rw, (int)(((32 * b + li) * ldw + 4 * h) * 4),
                                               (32 * c + 8 * q) * 4, 0);
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

namespace {
hipError_t launch_group(float* w, int64_t n, int64_t k, int64_t ldw, const float* u, int64_t ldu,
                        int64_t unit, int scheme, uint8_t* codes, uint32_t* meta, float* f,
                        int64_t fsr, int64_t fsc, hipStream_t stream) {
  const int64_t s0 = unit * 64, units = k / 64;
  const dim3 gg((unsigned)((16 * n + 255) / 256)), gb(256);  // 16 lanes per row
  uint32_t* c32 = reinterpret_cast<uint32_t*>(codes);
  if (scheme == 1)
    hipLaunchKernelGGL(higptq_group_kernel<1>, gg, gb, 0, stream, w, ldw, n, u, ldu, s0, units,
                       unit, c32, meta, f, fsr, fsc);
  else if (scheme == 2)
    hipLaunchKernelGGL(higptq_group_kernel<2>, gg, gb, 0, stream, w, ldw, n, u, ldu, s0, units,
                       unit, c32, meta, f, fsr, fsc);
  else
    hipLaunchKernelGGL(higptq_group_kernel<3>, gg, gb, 0, stream, w, ldw, n, u, ldu, s0, units,
                       unit, c32, meta, f, fsr, fsc);
  return hipGetLastError();
}

// W[:, c0..c1) -= F[:, 0..R) U[sk.., c0..c1), F given transposed (row stride ldt)
hipError_t launch_rank_update(float* w, int64_t n, int64_t ldw, const float* u, int64_t ldu,
                              int64_t sk, int64_t c0, int64_t c1, const float* ft, int64_t ldt,
                              int64_t R, hipStream_t stream) {
  if (c1 <= c0) return hipSuccess;
  const unsigned cols = (unsigned)((c1 - c0) / 64);
  if (c1 - c0 <= 512)  // narrow (in-block) updates: more and shorter waves
    hipLaunchKernelGGL(higptq_rank_update_kernel<1>, dim3(cols, (unsigned)((n + 127) / 128)),
                       dim3(256), 0, stream, w, ldw, n, u, ldu, sk, c0, ft, ldt, (int)R);
  else
    hipLaunchKernelGGL(higptq_rank_update_kernel<2>, dim3(cols, (unsigned)((n + 255) / 256)),
                       dim3(256), 0, stream, w, ldw, n, u, ldu, sk, c0, ft, ldt, (int)R);
  return hipGetLastError();
}
}  // namespace

hipError_t hif4_launch_higptq_unit(float* w, int64_t n, int64_t k, int64_t ldw, const float* u,
                                   int64_t ldu, int64_t unit, int scheme, uint8_t* codes,
                                   uint32_t* meta, float* f, hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t s0 = unit * 64;
  hipError_t e = launch_group(w, n, k, ldw, u, ldu, unit, scheme, codes, meta, f, 64, 1, stream);
  if (e != hipSuccess) return e;
  const int64_t c0 = s0 + 64;
  if (c0 >= k) return hipSuccess;
  const dim3 grid((unsigned)((k - c0 + kUpdCols - 1) / kUpdCols),
                  (unsigned)((n + kUpdRows - 1) / kUpdRows));
  hipLaunchKernelGGL(higptq_update_kernel, grid, dim3(256), 0, stream, w, ldw, n, k, u, ldu, s0,
                     c0, (const float*)f);
  return hipGetLastError();
}

// Groups lo .. hi - 1 of the block starting at unit0 (column s), in the
// nested order of blocked GPTQ: the first half of the range, then the second
// half's columns updated once with the first half's F (rank 64 (mid - lo)),
// then the second half. Every column of the block thus takes every earlier
// group's correction before its own group is quantized, with each in-block
// column read and written once per level instead of once per earlier group.
hipError_t block_range(float* w, int64_t n, int64_t k, int64_t ldw, const float* u, int64_t ldu,
                       int64_t unit0, int64_t lo, int64_t hi, int scheme, uint8_t* codes,
                       uint32_t* meta, float* ft, int64_t ldt, hipStream_t stream) {
  if (hi - lo == 1)
    return launch_group(w, n, k, ldw, u, ldu, unit0 + lo, scheme, codes, meta, ft + 64 * lo * ldt,
                        1, ldt, stream);
  const int64_t mid = lo + (hi - lo) / 2, s = unit0 * 64;
  hipError_t st = block_range(w, n, k, ldw, u, ldu, unit0, lo, mid, scheme, codes, meta, ft, ldt,
                              stream);
  if (st != hipSuccess) return st;
  st = launch_rank_update(w, n, ldw, u, ldu, s + 64 * lo, s + 64 * mid, s + 64 * hi,
                          ft + 64 * lo * ldt, ldt, 64 * (mid - lo), stream);
  if (st != hipSuccess) return st;
  return block_range(w, n, k, ldw, u, ldu, unit0, mid, hi, scheme, codes, meta, ft, ldt, stream);
}

// One block of `units` groups from unit0 (block_range for the groups), then
// the columns after the block take the whole block's F at once. F is kept
// transposed: F^T [64 units][ldt], ldt = n rounded up to a multiple of 64,
// group j's rows at 64 j.
hipError_t hif4_launch_higptq_block(float* w, int64_t n, int64_t k, int64_t ldw, const float* u,
                                    int64_t ldu, int64_t unit0, int64_t units, int scheme,
                                    uint8_t* codes, uint32_t* meta, float* ft,
                                    hipStream_t stream) {
  if (n == 0) return hipSuccess;
  const int64_t s = unit0 * 64, e = s + 64 * units, ldt = (n + 63) / 64 * 64;
  hipError_t st = block_range(w, n, k, ldw, u, ldu, unit0, 0, units, scheme, codes, meta, ft, ldt,
                              stream);
  if (st != hipSuccess) return st;
  return launch_rank_update(w, n, ldw, u, ldu, s, e, k, ft, ldt, 64 * units, stream);
}
