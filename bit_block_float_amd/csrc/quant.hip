// quant.hip -- HiF4 quantize (bf16 -> codes + meta), its fake-quant variant
// (bf16 -> bf16 on the HiF4 grid), the protected-channel gather, and the
// dequantize kernel. All are HBM-streaming kernels for gfx950.
//
// Format: HiFloat4 calibration article (hwcomputing.csdn.net), section
// "一：HiFloat4 (HiF4) 格式". Exponent order and per-group statistics: same
// article, section 3.1 "HiGPTQ". No clipping: section 3.3 "HiFlatQuant".
// Protected channels: Tail-Aware HiFloat4 summary (agents-report.net),
// section "方法概述". The rule and layout readings are stated in hif4.h.
//
// Work mapping: one lane owns one level-2 group (8 consecutive elements along
// k, one 16-byte load); 8 aligned lanes own one unit; the unit maximum and the
// metadata word are formed with DPP moves inside the 8 lanes. Each lane emits
// one 32-bit code word (its two level-3 groups as low/high nibbles), so a
// wave writes 256 contiguous code bytes and 32 contiguous meta bytes.
#include "hif4_dev.h"

namespace hif4 {

// Fast unsigned division by a runtime-invariant divisor, valid for n < 2^31
// (Granlund & Montgomery, "Division by invariant integers using
// multiplication", 1994: q = (mulhi(n, m) + n) >> s).
struct FastDiv {
  uint32_t d, m, s;
};

static FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  const uint64_t m = ((1ull << 32) * ((1ull << s) - d)) / d + 1;
  return FastDiv{d, (uint32_t)m, s};
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  return (__umulhi(n, f.m) + n) >> f.s;
}

template <bool kMask, bool kCodes, bool kDeq>
__global__ __launch_bounds__(256) void quantize_kernel(
    const uint16_t* __restrict__ x, int64_t ld, uint32_t groups_per_row, FastDiv grp_div,
    uint32_t total_groups, const uint8_t* __restrict__ mask, uint32_t* __restrict__ codes32,
    uint32_t* __restrict__ meta, uint16_t* __restrict__ deq) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t grp = blockIdx.x * blockDim.x + threadIdx.x; grp < total_groups; grp += stride) {
    const uint32_t row = fdiv(grp, grp_div);
    const uint32_t gi = grp - row * groups_per_row;  // level-2 group index within the row
    const uint32_t g = gi & 7u;                     // level-2 group index within the unit

    const uint4 w = *reinterpret_cast<const uint4*>(x + (int64_t)row * ld + (int64_t)gi * 8);
    uint32_t bits[8] = {w.x << 16, w.x & 0xFFFF0000u, w.y << 16, w.y & 0xFFFF0000u,
                        w.z << 16, w.z & 0xFFFF0000u, w.w << 16, w.w & 0xFFFF0000u};
    if (kMask) {
      // Protected channels are quantized as +0 and do not enter the maxima.
      const uint2 mk = *reinterpret_cast<const uint2*>(mask + (size_t)gi * 8);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if ((mk.x >> (8 * i)) & 0xFFu) bits[i] = 0u;
        if ((mk.y >> (8 * i)) & 0xFFu) bits[4 + i] = 0u;
      }
    }

    // step 1: maxima of |x| (compared as bit patterns of non-negative floats)
    uint32_t m4a = 0u, m4b = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      m4a = max(m4a, bits[i] & 0x7FFFFFFFu);
      m4b = max(m4b, bits[4 + i] & 0x7FFFFFFFu);
    }
    const uint32_t m8 = max(m4a, m4b);
    const float amax = __uint_as_float(max8_u32(m8));

    // step 2: level-1 code; steps 3-4: level-2 / level-3 bits (exact compares)
    const uint32_t c = level1_code(amax);
    const float s = e6m2_f32(c);
    const uint32_t e2 = __uint_as_float(m8) > 3.5f * s;
    const float t3 = (e2 ? 3.5f : 1.75f) * s;
    const uint32_t e3a = __uint_as_float(m4a) > t3;
    const uint32_t e3b = __uint_as_float(m4b) > t3;

    // step 5: k = RNE(4|x| / D), D = s 2^E, computed as |x| * (4/D) in double
    const double rbase = inv_mant16(c & 3u);
    const int p = 31 - (int)(c >> 2);
    const double ra = ldexp(rbase, p - (int)(e2 + e3a));
    const double rb = ldexp(rbase, p - (int)(e2 + e3b));
    uint32_t k[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const double t = (double)__uint_as_float(bits[i] & 0x7FFFFFFFu) * (i < 4 ? ra : rb);
      k[i] = (uint32_t)fmin(rint(t), 7.0);
    }

    if (kCodes) {
      uint32_t word = 0u;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t sgn = (bits[i] >> 31) & (k[i] != 0u);
        const uint32_t nib = k[i] | (sgn << 3);
        word |= nib << (i < 4 ? 8 * i : 8 * (i - 4) + 4);
      }
      codes32[grp] = word;
      const uint32_t mb = (e2 << (8 + g)) | (e3a << (16 + 2 * g)) | (e3b << (17 + 2 * g));
      const uint32_t mw = or8_u32(mb) | c;
      if (g == 0u) meta[grp >> 3] = mw;
    }
    if (kDeq) {
      // Exact: k (3 bits) times D/4 (3 significant bits) fits bf16.
      const float da = ldexpf(s, (int)(e2 + e3a) - 2);
      const float db = ldexpf(s, (int)(e2 + e3b) - 2);
      uint32_t h[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float v = (float)k[i] * (i < 4 ? da : db);
        const uint32_t sgn = (bits[i] & 0x80000000u) & (k[i] != 0u ? 0xFFFFFFFFu : 0u);
        h[i] = (__float_as_uint(v) | sgn) >> 16;
      }
      uint4 o;
      o.x = h[0] | (h[1] << 16);
      o.y = h[2] | (h[3] << 16);
      o.z = h[4] | (h[5] << 16);
      o.w = h[6] | (h[7] << 16);
      *reinterpret_cast<uint4*>(deq + (int64_t)grp * 8) = o;
    }
  }
}

// Gather protected-channel entries into kept [rows][n_mask], ascending
// channel order. Each block first compacts the mask into a channel list in
// LDS (k <= 65536), then copies its rows.
__global__ __launch_bounds__(256) void gather_kept_kernel(const uint16_t* __restrict__ x,
                                                          int64_t rows, int k, int64_t ld,
                                                          const uint8_t* __restrict__ mask,
                                                          int n_mask, uint16_t* __restrict__ kept,
                                                          int rows_per_block) {
  extern __shared__ uint16_t chan[];  // n_mask entries
  __shared__ int counts[256];
  const int tid = threadIdx.x;
  const int chunk = (k + 255) / 256;
  const int c0 = min(k, tid * chunk), c1 = min(k, c0 + chunk);
  int cnt = 0;
  for (int ch = c0; ch < c1; ++ch) cnt += mask[ch] != 0;
  counts[tid] = cnt;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int i = 0; i < 256; ++i) {
      const int v = counts[i];
      counts[i] = run;
      run += v;
    }
  }
  __syncthreads();
  int pos = counts[tid];
  for (int ch = c0; ch < c1; ++ch) {
    if (mask[ch] != 0) {
      if (pos < n_mask) chan[pos] = (uint16_t)ch;
      ++pos;
    }
  }
  __shared__ int total;
  if (tid == 255) total = pos;  // exclusive prefix of the last thread + its own count
  __syncthreads();
  const int nf = min(total, n_mask);
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
  const int64_t r1 = min(rows, r0 + rows_per_block);
  for (int64_t r = r0; r < r1; ++r) {
    for (int i = tid; i < nf; i += 256) kept[r * n_mask + i] = x[r * ld + chan[i]];
  }
}

// Dequantize: one lane decodes one code word (8 elements of a level-2 group).
template <bool kBf16>
__global__ __launch_bounds__(256) void dequantize_kernel(const uint32_t* __restrict__ codes32,
                                                         const uint32_t* __restrict__ meta,
                                                         uint32_t total_groups,
                                                         void* __restrict__ out) {
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t grp = blockIdx.x * blockDim.x + threadIdx.x; grp < total_groups; grp += stride) {
    const uint32_t word = codes32[grp];
    const uint32_t mw = meta[grp >> 3];
    const uint32_t g = grp & 7u;
    const uint32_t c = mw & 255u;
    const float s = e6m2_f32(c);
    const uint32_t e2 = (mw >> (8 + g)) & 1u;
    const uint32_t e3a = (mw >> (16 + 2 * g)) & 1u;
    const uint32_t e3b = (mw >> (17 + 2 * g)) & 1u;
    const float da = ldexpf(s, (int)(e2 + e3a) - 2);
    const float db = ldexpf(s, (int)(e2 + e3b) - 2);
    uint32_t v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t nib = (word >> (i < 4 ? 8 * i : 8 * (i - 4) + 4)) & 15u;
      const float mag = (float)(nib & 7u) * (i < 4 ? da : db);
      v[i] = __float_as_uint(mag) | ((nib & 8u) << 28);
    }
    if (kBf16) {
      uint4 o;
      o.x = (v[0] >> 16) | (v[1] & 0xFFFF0000u);
      o.y = (v[2] >> 16) | (v[3] & 0xFFFF0000u);
      o.z = (v[4] >> 16) | (v[5] & 0xFFFF0000u);
      o.w = (v[6] >> 16) | (v[7] & 0xFFFF0000u);
      reinterpret_cast<uint4*>(out)[grp] = o;
    } else {
      uint4* o = reinterpret_cast<uint4*>(out) + 2 * (size_t)grp;
      o[0] = make_uint4(v[0], v[1], v[2], v[3]);
      o[1] = make_uint4(v[4], v[5], v[6], v[7]);
    }
  }
}

static unsigned grid_for(uint64_t threads) {
  const uint64_t blocks = (threads + 255) / 256;
  const uint64_t cap = 256ull * 64;  // enough blocks to fill 256 CUs many times over
  return (unsigned)(blocks < cap ? (blocks ? blocks : 1) : cap);
}

}  // namespace hif4

using namespace hif4;

// Rows are processed in chunks so that group indices stay below 2^31.
hipError_t hif4_launch_quantize(const uint16_t* x, int64_t rows, int64_t k, int64_t ld,
                                const uint8_t* mask, uint8_t* codes, uint32_t* meta,
                                uint16_t* deq_bf16, hipStream_t stream) {
  if (rows == 0 || k == 0) return hipSuccess;
  const uint32_t gpr = (uint32_t)(k / 8);
  const FastDiv fd = make_fastdiv(gpr);
  const int64_t max_rows = ((int64_t)1 << 30) / gpr;
  for (int64_t r0 = 0; r0 < rows; r0 += max_rows) {
    const int64_t nr = rows - r0 < max_rows ? rows - r0 : max_rows;
    const uint32_t total = (uint32_t)(nr * gpr);
    const uint16_t* xs = x + r0 * ld;
    uint32_t* cs = codes ? reinterpret_cast<uint32_t*>(codes + r0 * (k / 2)) : nullptr;
    uint32_t* ms = meta ? meta + r0 * (k / 64) : nullptr;
    uint16_t* ds = deq_bf16 ? deq_bf16 + r0 * k : nullptr;
    const dim3 grid(grid_for(total)), block(256);
    if (mask) {
      if (ds) return hipErrorInvalidValue;
      hipLaunchKernelGGL((quantize_kernel<true, true, false>), grid, block, 0, stream, xs, ld, gpr,
                         fd, total, mask, cs, ms, ds);
    } else if (ds && cs) {
      hipLaunchKernelGGL((quantize_kernel<false, true, true>), grid, block, 0, stream, xs, ld, gpr,
                         fd, total, mask, cs, ms, ds);
    } else if (ds) {
      hipLaunchKernelGGL((quantize_kernel<false, false, true>), grid, block, 0, stream, xs, ld,
                         gpr, fd, total, mask, cs, ms, ds);
    } else {
      hipLaunchKernelGGL((quantize_kernel<false, true, false>), grid, block, 0, stream, xs, ld,
                         gpr, fd, total, mask, cs, ms, ds);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t hif4_launch_gather_kept(const uint16_t* x, int64_t rows, int64_t k, int64_t ld,
                                   const uint8_t* mask, int64_t n_mask, uint16_t* kept,
                                   hipStream_t stream) {
  if (rows == 0 || n_mask == 0) return hipSuccess;
  const int rows_per_block = 16;
  const int64_t blocks = (rows + rows_per_block - 1) / rows_per_block;
  const size_t lds = (size_t)n_mask * sizeof(uint16_t);
  if (lds > 48 * 1024) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(gather_kept_kernel),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
  }
  for (int64_t b0 = 0; b0 < blocks; b0 += (1 << 30)) {
    const int64_t nb = blocks - b0 < (1 << 30) ? blocks - b0 : (1 << 30);
    const int64_t r0 = b0 * rows_per_block;
    hipLaunchKernelGGL(gather_kept_kernel, dim3((unsigned)nb), dim3(256),
                       (size_t)n_mask * sizeof(uint16_t), stream, x + r0 * ld, rows - r0, (int)k,
                       ld, mask, (int)n_mask, kept + r0 * n_mask, rows_per_block);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t hif4_launch_dequantize(const uint8_t* codes, const uint32_t* meta, int64_t rows,
                                  int64_t k, void* out, int out_bf16, hipStream_t stream) {
  if (rows == 0 || k == 0) return hipSuccess;
  const int64_t gpr = k / 8;
  const int64_t max_rows = ((int64_t)1 << 30) / gpr;
  for (int64_t r0 = 0; r0 < rows; r0 += max_rows) {
    const int64_t nr = rows - r0 < max_rows ? rows - r0 : max_rows;
    const uint32_t total = (uint32_t)(nr * gpr);
    const uint32_t* cs = reinterpret_cast<const uint32_t*>(codes + r0 * (k / 2));
    const uint32_t* ms = meta + r0 * (k / 64);
    const dim3 grid(grid_for(total)), block(256);
    if (out_bf16) {
      hipLaunchKernelGGL(dequantize_kernel<true>, grid, block, 0, stream, cs, ms, total,
                         (void*)((uint16_t*)out + r0 * k));
    } else {
      hipLaunchKernelGGL(dequantize_kernel<false>, grid, block, 0, stream, cs, ms, total,
                         (void*)((float*)out + r0 * k));
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}
