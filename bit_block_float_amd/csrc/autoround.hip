// autoround.hip -- HiF4 quantize with given HiAutoRound offsets.
//
// Method: HiFloat4 calibration article (hwcomputing.csdn.net), section 3.2
// "HiAutoRound": two sets of learnable offsets, K on the level-3 exponents
// (16 per unit, E' = E + RZ(K)) and M on the mantissas (shifted as
// M' = M >> RZ(K) before being added). Each iteration of its training loop
// quantizes the weight with the current offsets; this kernel is that step,
// with the offsets given (the loop that learns them is calibration-time
// training).
//
// Readings (the section gives the two formulas only; stated in hif4.h):
//   K [rows][k/4] (one per level-3 group) and M [rows][k] (one per element)
//   are fp32. The level-1 code and the level-2 bits come from the unit's
//   data as in hif4_quantize. Each level-3 bit e3 is computed as usual, then
//   e3' = clamp(e3 + trunc(K), 0, 1) (a 1-bit field). With d = e3' - e3,
//   M' = M 2^-d. An element's code is k = clamp(rint(fl(t + M')), 0, 7) with
//   t = fl(|x| / (D / 4)), D = v(c) 2^(e2 + e3'): every operation in IEEE
//   binary32, round to nearest even. The sign is kept; a zero code has none.
//
// Mapping: eight consecutive threads per unit, thread g of the unit owning
// level-2 group g (8 elements = one 16-byte load of x, two of M, one 8-byte
// load of K). The unit maximum and the meta word are combined across the
// eight lanes with xor shuffles. Every load and store is contiguous along the
// row across the lanes of a wave.
#include "hif4_dev.h"

namespace hif4 {

__device__ __forceinline__ uint32_t offset_e3(uint32_t e3, float kv) {
  const float t = (float)e3 + truncf(kv);
  return t >= 1.0f ? 1u : 0u;  // t is a whole number; NaN gives 0
}

__global__ __launch_bounds__(256) void quantize_offsets_kernel(
    const uint16_t* __restrict__ x, int64_t ld, int64_t rows, int64_t k,
    const float* __restrict__ koff, const float* __restrict__ moff,
    uint32_t* __restrict__ codes32, uint32_t* __restrict__ meta) {
  const int64_t groups = k / 8;     // level-2 groups per row (a multiple of 8)
  const int64_t total = rows * groups;  // a multiple of 8: units never split
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
       i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / groups, gi = i - row * groups;
    const uint32_t g = (uint32_t)(gi & 7);
    const uint4 xv = *reinterpret_cast<const uint4*>(x + row * ld + gi * 8);
    const uint32_t w[4] = {xv.x, xv.y, xv.z, xv.w};
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
    const float m4a = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    const float m4b = fmaxf(fmaxf(fabsf(v[4]), fabsf(v[5])), fmaxf(fabsf(v[6]), fabsf(v[7])));
    const float m8 = fmaxf(m4a, m4b);
    float a = m8;
    a = fmaxf(a, __shfl_xor(a, 1, 64));
    a = fmaxf(a, __shfl_xor(a, 2, 64));
    a = fmaxf(a, __shfl_xor(a, 4, 64));
    const uint32_t c = level1_code(a);
    const float s = e6m2_f32(c);
    // level-2 and level-3 bits from the data (exact compares), then K
    const uint32_t e2 = m8 > 3.5f * s;
    const float t3 = (e2 ? 3.5f : 1.75f) * s;
    const uint32_t e3a = m4a > t3, e3b = m4b > t3;
    const float2 kv = *reinterpret_cast<const float2*>(koff + row * (k / 4) + gi * 2);
    const uint32_t e3na = offset_e3(e3a, kv.x), e3nb = offset_e3(e3b, kv.y);
    const float4 ma = *reinterpret_cast<const float4*>(moff + row * k + gi * 8);
    const float4 mb = *reinterpret_cast<const float4*>(moff + row * k + gi * 8 + 4);
    const float mo[8] = {ma.x, ma.y, ma.z, ma.w, mb.x, mb.y, mb.z, mb.w};
    uint32_t word = 0u;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t e3 = e < 4 ? e3a : e3b, e3n = e < 4 ? e3na : e3nb;
      const float q = ldexpf(s, (int)(e2 + e3n)) * 0.25f;  // D / 4, exact
      const float mp = e3n > e3 ? mo[e] * 0.5f : (e3n < e3 ? mo[e] * 2.0f : mo[e]);
      const float t = __fdiv_rn(fabsf(v[e]), q);
      const float u = __fadd_rn(t, mp);
      uint32_t kq = 0u;
      if (u > 0.0f) {
        const float r = rintf(u);
        kq = r >= 7.0f ? 7u : (uint32_t)r;
      }
      const uint32_t sgn = (v[e] < 0.0f && kq != 0u) ? 8u : 0u;
      word |= (kq | sgn) << (e < 4 ? 8 * e : 8 * (e - 4) + 4);
    }
    codes32[row * groups + gi] = word;
    uint32_t mw = (e2 << (8 + g)) | (e3na << (16 + 2 * g)) | (e3nb << (17 + 2 * g));
    mw |= (uint32_t)__shfl_xor((int)mw, 1, 64);
    mw |= (uint32_t)__shfl_xor((int)mw, 2, 64);
    mw |= (uint32_t)__shfl_xor((int)mw, 4, 64);
    if (g == 0) meta[row * (k / 64) + gi / 8] = mw | c;
  }
}

}  // namespace hif4

using namespace hif4;

hipError_t hif4_launch_quantize_offsets(const uint16_t* x, int64_t rows, int64_t k, int64_t ld,
                                        const float* koff, const float* moff, uint8_t* codes,
                                        uint32_t* meta, hipStream_t stream) {
  const int64_t total = rows * (k / 8);
  if (total == 0) return hipSuccess;
  int64_t blocks = (total + 255) / 256;
  if (blocks > 256 * 64) blocks = 256 * 64;
  hipLaunchKernelGGL(quantize_offsets_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, x, ld,
                     rows, k, koff, moff, (uint32_t*)codes, meta);
  return hipGetLastError();
}
