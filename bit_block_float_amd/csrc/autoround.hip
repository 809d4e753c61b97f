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
// eight lanes with DPP moves. Every load and store is contiguous along the
// row across the lanes of a wave. Grid-stride over level-2 groups, the next
// group's loads issued before the current one is encoded (two register
// buffers; past the end the last group is read again, never encoded).
#include "hif4_dev.h"

namespace hif4 {

__device__ __forceinline__ uint32_t offset_e3(uint32_t e3, float kv) {
  const float t = (float)e3 + truncf(kv);
  return t >= 1.0f ? 1u : 0u;  // t is a whole number; NaN gives 0
}

struct OffsetsIn {
  uint4 x;
  float2 kv;
  float4 ma, mb;
};

// groups: level-2 groups per row (k / 8, a multiple of 8, so units never
// split); total = rows * groups < 2^31.
__global__ __launch_bounds__(256) void quantize_offsets_kernel(
    const uint16_t* __restrict__ x, int64_t ld, uint32_t groups, FastDiv gdiv, uint32_t total,
    const float* __restrict__ koff, const float* __restrict__ moff,
    uint32_t* __restrict__ codes32, uint32_t* __restrict__ meta) {
  const uint32_t stride = gridDim.x * blockDim.x;
  auto load = [&](OffsetsIn& in, uint32_t i) {
    i = min(i, total - 1u);
    const uint32_t row = fdiv(i, gdiv), gi = i - row * groups;
    in.x = *reinterpret_cast<const uint4*>(x + (int64_t)row * ld + gi * 8);
    // K [row][k/4] and M [row][k] are dense: group i's offsets sit at 2i and 8i
    in.kv = *reinterpret_cast<const float2*>(koff + (int64_t)i * 2);
    in.ma = *reinterpret_cast<const float4*>(moff + (int64_t)i * 8);
    in.mb = *reinterpret_cast<const float4*>(moff + (int64_t)i * 8 + 4);
  };
  auto encode = [&](const OffsetsIn& in, uint32_t i) {
    const uint32_t g = i & 7u;  // groups per row is a multiple of 8
    const uint32_t w[4] = {in.x.x, in.x.y, in.x.z, in.x.w};
    float v[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      v[2 * e] = __uint_as_float(w[e] << 16);
      v[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
    }
    const float m4a = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
    const float m4b = fmaxf(fmaxf(fabsf(v[4]), fabsf(v[5])), fmaxf(fabsf(v[6]), fabsf(v[7])));
    const float m8 = fmaxf(m4a, m4b);
    // unit maximum: |x| >= 0, so its bit pattern orders like its value
    const float a = __uint_as_float(max8_u32(__float_as_uint(m8)));
    const uint32_t c = level1_code(a);
    const float s = e6m2_f32(c);
    // level-2 and level-3 bits from the data (exact compares), then K
    const uint32_t e2 = m8 > 3.5f * s;
    const float t3 = (e2 ? 3.5f : 1.75f) * s;
    const uint32_t e3a = m4a > t3, e3b = m4b > t3;
    const uint32_t e3na = offset_e3(e3a, in.kv.x), e3nb = offset_e3(e3b, in.kv.y);
    const float mo[8] = {in.ma.x, in.ma.y, in.ma.z, in.ma.w, in.mb.x, in.mb.y, in.mb.z, in.mb.w};
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
    codes32[i] = word;
    const uint32_t mw = or8_u32((e2 << (8 + g)) | (e3na << (16 + 2 * g)) | (e3nb << (17 + 2 * g)));
    if (g == 0) meta[i >> 3] = mw | c;
  };
  uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  OffsetsIn a, b;
  load(a, i);
  while (i < total) {
    load(b, i + stride);
    encode(a, i);
    i += stride;
    if (i >= total) break;
    load(a, i + stride);
    encode(b, i);
    i += stride;
  }
}

}  // namespace hif4

using namespace hif4;

hipError_t hif4_launch_quantize_offsets(const uint16_t* x, int64_t rows, int64_t k, int64_t ld,
                                        const float* koff, const float* moff, uint8_t* codes,
                                        uint32_t* meta, hipStream_t stream) {
  if (rows == 0 || k == 0) return hipSuccess;
  const uint32_t groups = (uint32_t)(k / 8);
  const FastDiv fd = make_fastdiv(groups);
  // rows in chunks whose group indices stay below 2^31
  const int64_t max_rows = ((int64_t)1 << 30) / groups;
  for (int64_t r0 = 0; r0 < rows; r0 += max_rows) {
    const int64_t nr = rows - r0 < max_rows ? rows - r0 : max_rows;
    const uint32_t total = (uint32_t)(nr * groups);
    int64_t blocks = ((int64_t)total + 255) / 256;
    if (blocks > 256 * 64) blocks = 256 * 64;
    hipLaunchKernelGGL(quantize_offsets_kernel, dim3((unsigned)blocks), dim3(256), 0, stream,
                       x + r0 * ld, ld, groups, fd, total, koff + r0 * (k / 4), moff + r0 * k,
                       reinterpret_cast<uint32_t*>(codes + r0 * (k / 2)), meta + r0 * (k / 64));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
