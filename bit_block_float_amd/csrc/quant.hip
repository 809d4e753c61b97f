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
// Work mapping (quantize): one lane owns 16 consecutive elements along k (two
// level-2 groups, two 16-byte loads); 4 aligned lanes own one unit; the unit
// maximum and the metadata word are formed with DPP moves inside the quad.
// Each lane emits two 32-bit code words (a level-2 group each, its two
// level-3 groups as low/high nibbles), so a wave writes 512 contiguous code
// bytes and 64 contiguous meta bytes. The element rounding runs in fp32 with
// a two-term reciprocal (inv_mant_hi/lo) that makes it exact.
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

// Max over the 4 lanes of an aligned quad (DPP quad_perm), and OR.
__device__ __forceinline__ uint32_t max4_u32(uint32_t v) {
  v = max(v, dpp<kDppQuadXor1>(v));
  v = max(v, dpp<kDppQuadXor2>(v));
  return v;
}
__device__ __forceinline__ uint32_t or4_u32(uint32_t v) {
  v |= dpp<kDppQuadXor1>(v);
  v |= dpp<kDppQuadXor2>(v);
  return v;
}

// One level-2 group (8 elements, one code word): steps 3-5 given the unit's
// level-1 scale. w: the group's 8 bf16 values (element 2i in the low half of
// word i). Returns the code word; e2 and e3 bits by reference.
__device__ __forceinline__ uint32_t encode_group(uint4 w, float s, int p, float rh, float rl,
                                                 uint32_t& e2, uint32_t& e3a, uint32_t& e3b) {
  const float v[8] = {bf16lo_to_f32(w.x), bf16hi_to_f32(w.x), bf16lo_to_f32(w.y),
                      bf16hi_to_f32(w.y), bf16lo_to_f32(w.z), bf16hi_to_f32(w.z),
                      bf16lo_to_f32(w.w), bf16hi_to_f32(w.w)};
  const float m4a = fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
  const float m4b = fmaxf(fmaxf(fabsf(v[4]), fabsf(v[5])), fmaxf(fabsf(v[6]), fabsf(v[7])));
  // steps 3-4: level-2 / level-3 bits (exact compares)
  e2 = fmaxf(m4a, m4b) > 3.5f * s;
  const float t3 = (e2 ? 3.5f : 1.75f) * s;
  e3a = m4a > t3;
  e3b = m4b > t3;
  // step 5: k = RNE(4|x| / D), D = s 2^E, 4/D = (16/(4+m)) 2^(31-e-E) (inv_mant_hi)
  const int pa = p - (int)(e2 + e3a), pb = p - (int)(e2 + e3b);
  const float rha = ldexpf(rh, pa), rla = ldexpf(rl, pa);
  const float rhb = ldexpf(rh, pb), rlb = ldexpf(rl, pb);
  float kf[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float ax = fabsf(v[i]);
    const float t = i < 4 ? fmaf(ax, rha, ax * rla) : fmaf(ax, rhb, ax * rlb);
    kf[i] = fminf(rintf(t), 7.0f);
  }
  // magnitudes: element b of the low level-3 group -> low nibble of byte b,
  // element 4+b -> high nibble of byte b
  uint32_t lo = 0u, hi = 0u;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    lo = __builtin_amdgcn_cvt_pk_u8_f32(kf[b], b, lo);
    hi = __builtin_amdgcn_cvt_pk_u8_f32(kf[4 + b], b, hi);
  }
  const uint32_t mag = lo | (hi << 4);
  // signs: the high byte of each bf16 carries its sign in bit 7
  const uint32_t sl = __builtin_amdgcn_perm(w.y, w.x, 0x07050301u);  // elements 0..3
  const uint32_t sh = __builtin_amdgcn_perm(w.w, w.z, 0x07050301u);  // elements 4..7
  const uint32_t sgn = ((sl >> 4) & 0x08080808u) | (sh & 0x80808080u);
  // a zero element keeps +0: sign only where the magnitude nibble is nonzero
  const uint32_t nz = (mag + 0x77777777u) & 0x88888888u;
  return mag | (sgn & nz);
}

// Nonzero bytes of a 32-bit word -> bits 0..3.
__device__ __forceinline__ uint32_t nonzero_bytes(uint32_t w) {
  const uint32_t hi = (((w & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) | w) & 0x80808080u;
  return ((hi >> 7) | (hi >> 14) | (hi >> 21) | (hi >> 28)) & 0xFu;
}

constexpr int kMaxMaskChunks = 65536 / 16;  // masked rows are at most 65536 wide

// Work mapping: one lane owns two level-2 groups (16 consecutive elements,
// two 16-byte loads), 4 aligned lanes own a unit; unit maximum and metadata
// word via DPP inside the quad. A wave covers 16 units.
//
// kMask: protected channels become +0 in the HiF4 stream and their bf16
// values go to kept[row][rank], rank = the channel's position among the
// masked channels. Each workgroup first builds the rank of every 16-channel
// chunk of the mask in LDS (a prefix count), so the lanes that meet masked
// channels store their values directly: no second pass over X.
template <bool kMask>
__global__ __launch_bounds__(256) void quantize_kernel(
    const uint16_t* __restrict__ x, int64_t ld, uint32_t items_per_row, FastDiv item_div,
    uint32_t total_items, const uint8_t* __restrict__ mask, uint32_t* __restrict__ codes32,
    uint32_t* __restrict__ meta, uint16_t* __restrict__ kept, int n_mask) {
  // per 16-channel chunk: rank of its first masked channel (low 16 bits) and
  // its 16 mask bits (high 16 bits)
  __shared__ uint32_t chunk_info[kMask ? kMaxMaskChunks : 1];
  __shared__ uint32_t part[kMask ? 256 : 1];
  if (kMask) {
    // chunks t*per .. t*per+per-1 belong to thread t
    const int chunks = (int)items_per_row, tid = threadIdx.x;
    const int per = (chunks + 255) / 256;
    const int c0 = min(chunks, tid * per), c1 = min(chunks, c0 + per);
    uint32_t run = 0;
    for (int c = c0; c < c1; ++c) {
      const uint4 mk = *reinterpret_cast<const uint4*>(mask + (size_t)c * 16);
      const uint32_t m16 = nonzero_bytes(mk.x) | (nonzero_bytes(mk.y) << 4) |
                           (nonzero_bytes(mk.z) << 8) | (nonzero_bytes(mk.w) << 12);
      chunk_info[c] = m16 << 16;
      run += __popc(m16);
    }
    part[tid] = run;
    __syncthreads();
    if (tid == 0) {  // exclusive prefix over the 256 thread totals
      uint32_t acc = 0;
      for (int i = 0; i < 256; ++i) {
        const uint32_t v = part[i];
        part[i] = acc;
        acc += v;
      }
    }
    __syncthreads();
    run = part[tid];
    for (int c = c0; c < c1; ++c) {
      const uint32_t m16 = chunk_info[c] >> 16;
      chunk_info[c] |= run & 0xFFFFu;
      run += __popc(m16);
    }
    __syncthreads();
  }
  const uint32_t stride = gridDim.x * blockDim.x;
  for (uint32_t it = blockIdx.x * blockDim.x + threadIdx.x; it < total_items; it += stride) {
    const uint32_t row = fdiv(it, item_div);
    const uint32_t j = it - row * items_per_row;  // 16-element item within the row
    const uint32_t q = j & 3u;                    // item within the unit (groups 2q, 2q+1)

    const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)row * ld + (int64_t)j * 16);
    uint4 w0 = src[0], w1 = src[1];
    if (kMask) {
      // Protected channels are quantized as +0 and do not enter the maxima;
      // their values go to kept (rare: only lanes whose chunk has any).
      const uint32_t info = chunk_info[j];
      const uint32_t m16 = info >> 16;
      if (m16) {
        uint32_t ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
        uint32_t mm = m16;
        while (mm) {
          const uint32_t e = __ffs(mm) - 1;
          const uint32_t rank = (info & 0xFFFFu) + __popc(m16 & ((1u << e) - 1u));
          if (rank < (uint32_t)n_mask)
            kept[(int64_t)row * n_mask + rank] = (uint16_t)(ww[e >> 1] >> (16 * (e & 1)));
          mm &= mm - 1;
        }
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const uint32_t lo = (m16 >> (2 * i)) & 1u, hi = (m16 >> (2 * i + 1)) & 1u;
          ww[i] &= ~((lo * 0x0000FFFFu) | (hi * 0xFFFF0000u));
        }
        w0 = make_uint4(ww[0], ww[1], ww[2], ww[3]);
        w1 = make_uint4(ww[4], ww[5], ww[6], ww[7]);
      }
    }

    // step 1: unit maximum of |x|, compared as bit patterns of non-negative
    // floats (sign bits dropped), over the lane's 16 values, then the quad
    uint32_t am = 0u;
    {
      const uint32_t ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        am = max(am, (ww[i] << 16) & 0x7FFFFFFFu);
        am = max(am, ww[i] & 0x7FFF0000u);
      }
    }
    const float amax = __uint_as_float(max4_u32(am));

    // step 2: level-1 code (shared by the quad)
    const uint32_t c = level1_code(amax);
    const float s = e6m2_f32(c);
    const int p = 31 - (int)(c >> 2);
    const float rh = inv_mant_hi(c & 3u), rl = inv_mant_lo(c & 3u);

    uint32_t e2a, e3a0, e3b0, e2b, e3a1, e3b1;
    const uint32_t cw0 = encode_group(w0, s, p, rh, rl, e2a, e3a0, e3b0);
    const uint32_t cw1 = encode_group(w1, s, p, rh, rl, e2b, e3a1, e3b1);

    reinterpret_cast<uint2*>(codes32)[it] = make_uint2(cw0, cw1);
    const uint32_t g0 = 2 * q, g1 = 2 * q + 1;
    const uint32_t mb = (e2a << (8 + g0)) | (e2b << (8 + g1)) | (e3a0 << (16 + 2 * g0)) |
                        (e3b0 << (17 + 2 * g0)) | (e3a1 << (16 + 2 * g1)) |
                        (e3b1 << (17 + 2 * g1));
    const uint32_t mw = or4_u32(mb) | c;
    if (q == 0u) meta[it >> 2] = mw;
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
                                const uint8_t* mask, int64_t n_mask, uint16_t* kept,
                                uint8_t* codes, uint32_t* meta, hipStream_t stream) {
  if (rows == 0 || k == 0) return hipSuccess;
  const uint32_t gpr = (uint32_t)(k / 16);  // 16-element items per row
  const FastDiv fd = make_fastdiv(gpr);
  const int64_t max_rows = ((int64_t)1 << 30) / gpr;
  for (int64_t r0 = 0; r0 < rows; r0 += max_rows) {
    const int64_t nr = rows - r0 < max_rows ? rows - r0 : max_rows;
    const uint32_t total = (uint32_t)(nr * gpr);
    const uint16_t* xs = x + r0 * ld;
    uint32_t* cs = reinterpret_cast<uint32_t*>(codes + r0 * (k / 2));
    uint32_t* ms = meta + r0 * (k / 64);
    const dim3 block(256);
    if (mask) {
      // fewer, longer-lived workgroups: each builds the mask's rank table once
      const unsigned g = grid_for(total);
      const dim3 grid(g < 256u * 8u ? g : 256u * 8u);
      hipLaunchKernelGGL(quantize_kernel<true>, grid, block, 0, stream, xs, ld, gpr, fd, total,
                         mask, cs, ms, kept ? kept + r0 * n_mask : nullptr, (int)n_mask);
    } else {
      hipLaunchKernelGGL(quantize_kernel<false>, dim3(grid_for(total)), block, 0, stream, xs, ld,
                         gpr, fd, total, mask, cs, ms, nullptr, 0);
    }
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
