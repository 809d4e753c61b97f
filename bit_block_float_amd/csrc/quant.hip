// quant.hip -- HiF4 quantize (bf16 -> codes + meta, optionally with
// protected channels), and the dequantize kernel. HBM-streaming kernels for
// gfx950.
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
// bytes and 64 contiguous meta bytes. Maxima, thresholds and the element
// rounding run on packed 16-bit pairs (bit-pattern maxima, an exact fp16
// quotient; see kpair): the kernel would otherwise be bound by its VALU work
// rather than by HBM.
#include <algorithm>

#include "hif4_dev.h"

namespace hif4 {

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

// ---- packed 16-bit element arithmetic
//
// The element step works on two bf16 values per 32-bit word with packed
// 16-bit instructions. For a level-3 quad with exponent sum E under a unit of
// code c (e = c >> 2, m = c & 3), the S1P2 magnitude is k = min(RNE(t), 7)
// with t = 4|x| / D = y * 4/(4+m), y = |x| 2^(33-e-E). Below range
// saturation every y lies under 7 * 1.75 (the level-3 rule bounds the quad
// maximum by 1.75 s 2^E), and any y of 16 or more gives k = 7, so y capped
// at 16 is an fp16 number: its bf16 bits become fp16 bits by one saturating
// subtract of ((e + E + 79) << 7) (exponent rebias and 2^(33-e-E) together;
// values too small for an fp16 normal saturate to 0 or land among the fp16
// subnormals, all of which round to k = 0) and a shift left by 3. Then
// t = fma(y, hi, y lo) in fp16, with hi = RN16(4/(4+m)) and
// lo = RN16(4/(4+m) - hi): within 2^-19 of the real quotient, while a
// non-tie quotient is at least 9 fp16 half-ulps from the nearest half-integer
// and a tie is an fp16 number, so t rounds on the same side as the real
// quotient and ties come out exact. Adding 1024 (fp16 spacing 1 there)
// rounds to nearest even; min(., 1031) saturates k at 7 and leaves k in the
// low byte of each half. (Checked on the CPU for every bf16 y below 14 and
// every m, and by the element-rounding parity tests.)
typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t kpair(uint32_t absw, uint32_t csub, uint32_t hi2,
                                          uint32_t lo2) {
  u16x2_t y = __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2_t, absw),
                                            __builtin_bit_cast(u16x2_t, csub));
  // range saturation (c = 255 below a unit maximum above 7 v(255)) lets y
  // exceed the fp16 range: cap it at 16 (pattern 0x0980 before the shift),
  // which still rounds to k = 7
  y = __builtin_elementwise_min(y, (u16x2_t)(0x0980));
  y = y << (u16x2_t)(3);
  const f16x2_t yf = __builtin_bit_cast(f16x2_t, y);
  const f16x2_t pl = yf * __builtin_bit_cast(f16x2_t, lo2);
  f16x2_t t = __builtin_elementwise_fma(yf, __builtin_bit_cast(f16x2_t, hi2), pl);
  t = t + (f16x2_t)((_Float16)1024.0f);
  t = __builtin_elementwise_min(t, (f16x2_t)((_Float16)1031.0f));
  return __builtin_bit_cast(uint32_t, t);  // k in bytes 0 and 2
}

// Larger of the two u16 halves.
__device__ __forceinline__ uint32_t hmax_u16(uint32_t v) { return max(v & 0xFFFFu, v >> 16); }
// Per-half maximum of two words of u16 halves.
__device__ __forceinline__ uint32_t pkmax_u16(uint32_t a, uint32_t b) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a),
                                                                __builtin_bit_cast(u16x2_t, b)));
}

// RN16(4/(4+m)) and the fp16 remainder, both halves.
__device__ __forceinline__ uint32_t kinv_hi2(uint32_t m) {
  return select4(m, 0x3C003C00u, 0x3A663A66u, 0x39553955u, 0x38923892u);
}
__device__ __forceinline__ uint32_t kinv_lo2(uint32_t m) {
  return select4(m, 0x00000000u, 0x0A660A66u, 0x09550955u, 0x08920892u);
}

// Level-3 quad maxima of a level-2 group, as |x| bf16 bits: `a` = the group's
// 4 words with the sign bits cleared.
struct QuadMax {
  uint32_t a, b;
};
__device__ __forceinline__ QuadMax quad_max(uint4 a) {
  return QuadMax{hmax_u16(pkmax_u16(a.x, a.y)), hmax_u16(pkmax_u16(a.z, a.w))};
}

// One level-2 group (8 elements, one code word): steps 3-5 given the unit's
// level-1 code. w: the group's 8 bf16 values (element 2i in the low half of
// word i), a: the same with the sign bits cleared, qm: its quad maxima;
// thr2 / thr175: bf16 bits of 3.5 s and 1.75 s (exact: s has at most three
// significant bits). Returns the code word; e2 and e3 bits by reference.
__device__ __forceinline__ uint32_t encode_group(uint4 w, uint4 a, QuadMax qm, uint32_t e,
                                                 uint32_t hi2, uint32_t lo2, uint32_t thr2,
                                                 uint32_t thr175, uint32_t& e2, uint32_t& e3a,
                                                 uint32_t& e3b) {
  // steps 3-4: level-2 / level-3 bits (exact compares of bf16 bit patterns)
  e2 = max(qm.a, qm.b) > thr2;
  const uint32_t t3 = e2 ? thr2 : thr175;
  e3a = qm.a > t3;
  e3b = qm.b > t3;
  // step 5: k = RNE(4|x| / D), two elements per packed operation
  const uint32_t ca = ((e + e2 + e3a + 79u) << 7) * 0x00010001u;
  const uint32_t cb = ((e + e2 + e3b + 79u) << 7) * 0x00010001u;
  const uint32_t k01 = kpair(a.x, ca, hi2, lo2), k23 = kpair(a.y, ca, hi2, lo2);
  const uint32_t k45 = kpair(a.z, cb, hi2, lo2), k67 = kpair(a.w, cb, hi2, lo2);
  // magnitudes: element b of the low level-3 group -> low nibble of byte b,
  // element 4+b -> high nibble of byte b
  const uint32_t lo = __builtin_amdgcn_perm(k23, k01, 0x06040200u);
  const uint32_t hi = __builtin_amdgcn_perm(k67, k45, 0x06040200u);
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

// One 16-element item (two level-2 groups, words v0 and v1, element 2i in
// the low half of word i; protected channels already cleared to +0, so they
// do not enter the maxima): item j of its row, it = its index over all rows
// (code words 2it, 2it+1; the unit's meta word it/4, written by the quad's
// first lane). Steps 1-5 of the rule.
__device__ __forceinline__ void quantize_item(uint4 v0, uint4 v1, uint32_t j, uint32_t it,
                                              uint32_t* __restrict__ codes32,
                                              uint32_t* __restrict__ meta) {
  const uint32_t q = j & 3u;  // item within the unit (groups 2q, 2q+1)

  // step 1: level-3 / level-2 maxima of |x| as bf16 bit patterns (sign bits
  // dropped; monotone in |x|), then the unit maximum over the quad of lanes
  const uint4 a0 = make_uint4(v0.x & 0x7FFF7FFFu, v0.y & 0x7FFF7FFFu, v0.z & 0x7FFF7FFFu,
                              v0.w & 0x7FFF7FFFu);
  const uint4 a1 = make_uint4(v1.x & 0x7FFF7FFFu, v1.y & 0x7FFF7FFFu, v1.z & 0x7FFF7FFFu,
                              v1.w & 0x7FFF7FFFu);
  const QuadMax q0 = quad_max(a0), q1 = quad_max(a1);
  const uint32_t am = max(max(q0.a, q0.b), max(q1.a, q1.b));
  const float amax = __uint_as_float(max4_u32(am) << 16);

  // step 2: level-1 code (shared by the quad)
  const uint32_t c = level1_code(amax);
  const float s = e6m2_f32(c);
  const uint32_t thr2 = __float_as_uint(3.5f * s) >> 16;
  const uint32_t thr175 = __float_as_uint(1.75f * s) >> 16;
  const uint32_t hi2 = kinv_hi2(c & 3u), lo2 = kinv_lo2(c & 3u);

  uint32_t e2a, e3a0, e3b0, e2b, e3a1, e3b1;
  const uint32_t cw0 = encode_group(v0, a0, q0, c >> 2, hi2, lo2, thr2, thr175, e2a, e3a0, e3b0);
  const uint32_t cw1 = encode_group(v1, a1, q1, c >> 2, hi2, lo2, thr2, thr175, e2b, e3a1, e3b1);

  reinterpret_cast<uint2*>(codes32)[it] = make_uint2(cw0, cw1);
  const uint32_t g0 = 2 * q, g1 = 2 * q + 1;
  const uint32_t mb = (e2a << (8 + g0)) | (e2b << (8 + g1)) | (e3a0 << (16 + 2 * g0)) |
                      (e3b0 << (17 + 2 * g0)) | (e3a1 << (16 + 2 * g1)) |
                      (e3b1 << (17 + 2 * g1));
  const uint32_t mw = or4_u32(mb) | c;
  if (q == 0u) meta[it >> 2] = mw;
}

// Kept values of one item of row `row`, one protected channel at a time:
// `info` = the item's 16 mask bits (high half) and the rank of its first
// masked channel among all masked channels (low half); the bf16 value of
// channel e goes to kept[row][rank of e].
__device__ __forceinline__ void keep_item_values(uint4 w0, uint4 w1, uint32_t info,
                                                 uint32_t row, uint16_t* __restrict__ kept,
                                                 int n_mask) {
  const uint32_t m16 = info >> 16;
  if (m16) {  // only lanes whose channels include masked ones
    const uint32_t ww[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
    uint32_t mm = m16;
    while (mm) {
      const uint32_t e = __ffs(mm) - 1;
      const uint32_t rank = (info & 0xFFFFu) + __popc(m16 & ((1u << e) - 1u));
      if (rank < (uint32_t)n_mask)
        kept[(int64_t)row * n_mask + rank] = (uint16_t)(ww[e >> 1] >> (16 * (e & 1)));
      mm &= mm - 1;
    }
  }
}

// Unmasked quantize. Work mapping: one lane owns one item (16 consecutive
// elements, two 16-byte loads), 4 aligned lanes own a unit; unit maximum and
// metadata word via DPP inside the quad. A wave covers 16 units.
__global__ __launch_bounds__(256) void quantize_kernel(
    const uint16_t* __restrict__ x, int64_t ld, uint32_t items_per_row, FastDiv item_div,
    uint32_t total_items, uint32_t* __restrict__ codes32, uint32_t* __restrict__ meta) {
  const uint32_t stride = gridDim.x * blockDim.x;
  // two register buffers: the loads of item it + stride go out before item
  // it is encoded, into the buffer that is not being read. Past the end the
  // last item is read again (never encoded): the loads are unconditional, so
  // the compiler can wait for one buffer while the other is in flight.
  auto load = [&](uint4& v0, uint4& v1, uint32_t it) {
    it = min(it, total_items - 1u);
    const uint32_t row = fdiv(it, item_div);
    const uint32_t j = it - row * items_per_row;
    const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)row * ld + (int64_t)j * 16);
    v0 = src[0];
    v1 = src[1];
  };
  auto encode = [&](uint4 v0, uint4 v1, uint32_t it) {
    const uint32_t row = fdiv(it, item_div);
    quantize_item(v0, v1, it - row * items_per_row, it, codes32, meta);
  };
  uint32_t it = blockIdx.x * blockDim.x + threadIdx.x;
  uint4 a0 = make_uint4(0, 0, 0, 0), a1 = a0, b0 = a0, b1 = a0;
  load(a0, a1, it);
  while (it < total_items) {
    load(b0, b1, it + stride);
    encode(a0, a1, it);
    it += stride;
    if (it >= total_items) break;
    load(a0, a1, it + stride);
    encode(b0, b1, it);
    it += stride;
  }
}

// Masked quantize, row-mapped. A workgroup of B threads (a multiple of 64)
// covers a row in kRounds rounds: thread t owns items t, t + B, ... of every
// row it visits, so the rank/mask word of its items is computed once, in
// registers, by a workgroup prefix count over the mask before the row loop:
// the loop itself has no table lookup. Workgroup g visits rows g, g + G, ...
//
// Kept values. The masked channels of a wave's items in one round hold the
// consecutive ranks [r0, r0 + cnt), the same in every row. When cnt <= 64
// the prologue assigns rank r0 + i to lane i and records where that value
// sits in the wave's LDS stage (source lane * 32 + element * 2); per row the
// lanes whose item holds masked channels write their 32 input bytes to the
// stage, every lane reads its slot back before the item is encoded, and
// lanes 0..cnt-1 store it after the encode, so the wave writes its kept run
// with one contiguous store and never waits for the LDS round trip. Waves
// with more masked channels keep the per-lane loop.
//
// Registers decide the occupancy of this HBM-streaming loop: with a single
// round the items' keep masks (32 bytes per thread) live in LDS and are read
// per item, which keeps the kernel at 8 waves per SIMD (measured on the
// FFN-up activation, 57600 x 5120 with 52 protected channels, at 4 rows per
// workgroup: 171 us with the per-lane loop and the masks in registers,
// 155-158 us this way).
template <int kRounds>
__global__ __launch_bounds__(1024) void quantize_masked_kernel(
    const uint16_t* __restrict__ x, int64_t ld, uint32_t rows, uint32_t items_per_row,
    const uint8_t* __restrict__ mask, uint32_t* __restrict__ codes32,
    uint32_t* __restrict__ meta, uint16_t* __restrict__ kept, int n_mask) {
  // dynamic LDS: per wave a stage of 64 lanes x the item's 2 words, then
  // (single round) the keep masks, 2 words per thread
  extern __shared__ uint4 stage[];
  constexpr bool kMasksInLds = kRounds == 1;
  uint4* const zs = stage + (blockDim.x >> 6) * 128;
  __shared__ uint32_t part[16];
  __shared__ uint16_t slot_src[kRounds][16][64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nwaves = blockDim.x >> 6;
  const uint32_t B = blockDim.x;
  // (loads past the last row or item read the last one again, unconditionally)
  auto load = [&](uint4& v0, uint4& v1, uint32_t row, int r) {
    const uint32_t j = min(tid + r * B, items_per_row - 1u);
    row = min(row, rows - 1u);
    const uint4* src = reinterpret_cast<const uint4*>(x + (int64_t)row * ld + (int64_t)j * 16);
    v0 = src[0];
    v1 = src[1];
  };
  // The mask words go out first, then the first item's loads, so that the
  // prologue below waits for the mask only while the item is in flight
  // (both loads unconditional: clamped indexes, out-of-range items masked
  // off afterwards).
  uint4 mk[kRounds];
#pragma unroll
  for (int r = 0; r < kRounds; ++r)
    mk[r] = *reinterpret_cast<const uint4*>(mask +
                                            (size_t)min(tid + r * B, items_per_row - 1u) * 16);
  uint4 a0 = make_uint4(0, 0, 0, 0), a1 = a0, b0 = a0, b1 = a0;
  load(a0, a1, blockIdx.x, 0);
  // info: the item's 16 mask bits (high half); low half: with the stage,
  // the stage byte offset of the lane's kept value (lanes < wcnt), else the
  // rank of the item's first masked channel
  uint32_t info[kRounds];
  uint4 zk0[kRounds], zk1[kRounds];  // keep masks of the item's words (several rounds)
  uint32_t wcnt[kRounds];            // masked channels of the wave's items (wave-uniform)
  uint32_t wrank[kRounds];           // rank of the first of them (wave-uniform)
  uint32_t run = 0;  // masked channels in the rounds before the current one
#pragma unroll
  for (int r = 0; r < kRounds; ++r) {
    const uint32_t j = tid + r * B;
    uint32_t m16 = nonzero_bytes(mk[r].x) | (nonzero_bytes(mk[r].y) << 4) |
                   (nonzero_bytes(mk[r].z) << 8) | (nonzero_bytes(mk[r].w) << 12);
    if (j >= items_per_row) m16 = 0;
    // exclusive prefix of the popcounts over the round's items (thread order)
    const uint32_t cnt = __popc(m16);
    uint32_t incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const uint32_t o = (uint32_t)__shfl_up((int)incl, d, 64);
      if (lane >= d) incl += o;
    }
    const uint32_t wc = (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
    wcnt[r] = wc;
    if (wc <= 64u) {
      // kept slot of each masked channel = its rank within the wave
      uint32_t mm = m16;
      while (mm) {
        const uint32_t e = __ffs(mm) - 1;
        slot_src[r][wave][incl - cnt + __popc(m16 & ((1u << e) - 1u))] =
            (uint16_t)(lane * 32 + e * 2);
        mm &= mm - 1;
      }
    }
    if (lane == 63) part[wave] = incl;
    __syncthreads();
    uint32_t base = run + incl - cnt, total = 0;
    for (int w = 0; w < nwaves; ++w) {
      const uint32_t pw = part[w];
      if (w < wave) base += pw;
      total += pw;
    }
    const uint32_t ksrc = (wc <= 64u && (uint32_t)lane < wc) ? slot_src[r][wave][lane] : 0u;
    wrank[r] = (uint32_t)__builtin_amdgcn_readfirstlane((int)(base - (incl - cnt)));
    __syncthreads();
    info[r] = (m16 << 16) | (wc <= 64u ? ksrc : (base & 0xFFFFu));
    run += total;
    uint32_t z[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint32_t lo = (m16 >> (2 * i)) & 1u, hi = (m16 >> (2 * i + 1)) & 1u;
      z[i] = ~((lo * 0x0000FFFFu) | (hi * 0xFFFF0000u));
    }
    if (kMasksInLds) {
      zs[2 * tid] = make_uint4(z[0], z[1], z[2], z[3]);
      zs[2 * tid + 1] = make_uint4(z[4], z[5], z[6], z[7]);
    } else {
      zk0[r] = make_uint4(z[0], z[1], z[2], z[3]);
      zk1[r] = make_uint4(z[4], z[5], z[6], z[7]);
    }
  }

  // items in the order (row, round); the next item's loads go out before the
  // current one is encoded, into the register buffer that is not being read
  uint4* const st = stage + wave * 128;
  auto encode = [&](uint4 w0, uint4 w1, uint32_t row, int r) {
    const uint32_t j = tid + r * B;
    uint16_t kv = 0;
    // kept values first: the raw words die at the masking below
    if (wcnt[r] > 64u) {
      keep_item_values(w0, w1, info[r], row, kept, n_mask);
    } else if (wcnt[r] != 0u) {
      if (info[r] >> 16) {
        st[2 * lane] = w0;
        st[2 * lane + 1] = w1;
      }
      // same-wave LDS accesses complete in order: the read sees the stage
      // writes above, and the next item's writes come after it
      __builtin_amdgcn_wave_barrier();
      kv = reinterpret_cast<const uint16_t*>(st)[(info[r] & 0xFFFFu) >> 1];
      __builtin_amdgcn_wave_barrier();
    }
    if (j < items_per_row) {
      uint4 z0, z1;
      if (kMasksInLds) {
        z0 = zs[2 * tid];
        z1 = zs[2 * tid + 1];
      } else {
        z0 = zk0[r];
        z1 = zk1[r];
      }
      quantize_item(make_uint4(w0.x & z0.x, w0.y & z0.y, w0.z & z0.z, w0.w & z0.w),
                    make_uint4(w1.x & z1.x, w1.y & z1.y, w1.z & z1.z, w1.w & z1.w), j,
                    row * items_per_row + j, codes32, meta);
    }
    const uint32_t rank = wrank[r] + lane;
    if (wcnt[r] <= 64u && (uint32_t)lane < wcnt[r] && rank < (uint32_t)n_mask)
      kept[(int64_t)row * n_mask + rank] = kv;
  };
  // (row, round) after (row, r)
  auto next = [&](uint32_t& row, int& r) {
    if (++r == kRounds) {
      r = 0;
      row += gridDim.x;
    }
  };
  uint32_t row = blockIdx.x;
  int r = 0;
  while (row < rows) {
    uint32_t row2 = row;
    int r2 = r;
    next(row2, r2);
    load(b0, b1, row2, r2);
    encode(a0, a1, row, r);
    row = row2;
    r = r2;
    if (row >= rows) break;
    next(row2, r2);
    load(a0, a1, row2, r2);
    encode(b0, b1, row, r);
    row = row2;
    r = r2;
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

// Blocks for a grid-stride launch over `threads` work items, at most `cap`.
// Far more blocks than fit at once (2048 of 256 threads on 256 CUs): as
// blocks retire, new ones land on whichever CUs are ahead, which balances
// CUs and XCDs that stream at different rates. Measured for the unmasked
// quantize (median of 20 calls, two runs on one box), FFN-up activation
// 57600 x 5120 / FFN-down activation 57600 x 13824: 8192 blocks 158 / 451 us,
// 32768 blocks 145 / 407 us, 131072 blocks 134-137 / 381-391 us, one item per
// thread (72000 / 194400 blocks) 135-136 / 377-388 us; the quantize takes a
// cap of 1024 blocks per CU, which leaves these shapes uncapped.
static unsigned grid_for(uint64_t threads, uint64_t cap = 256ull * 128) {
  const uint64_t blocks = (threads + 255) / 256;
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
    if (mask) {
      // one round per 1024 items of a row; B = the round's items rounded up to
      // a whole wave; enough workgroups to fill the chip several times
      const int rounds = (int)((gpr + 1023) / 1024);
      const uint32_t per = (gpr + rounds - 1) / rounds;
      const dim3 block((per + 63) / 64 * 64);
      // kept-value stage, and the keep masks with a single round
      const size_t lds = (size_t)block.x * 32 * (rounds == 1 ? 2 : 1);
      // at least ~6 rows per workgroup (the mask prologue is paid per
      // workgroup), at most 48 workgroups per CU. Measured on the FFN-up
      // activation (57600 x 5120, 52 protected channels; two runs on one
      // box): 1 row 235-242 us, 4 rows 157-162 us, 6 rows 153 us, 8 rows
      // 153-154 us, 12 rows 157-159 us, 24 rows 168 us
      const int64_t want = std::min<int64_t>(256 * 48, (nr + 5) / 6);
      const dim3 grid((unsigned)std::max<int64_t>(1, want));
      uint16_t* ks = kept ? kept + r0 * n_mask : nullptr;
      const uint32_t nrow = (uint32_t)nr;
      switch (rounds) {
        case 1:
          hipLaunchKernelGGL(quantize_masked_kernel<1>, grid, block, lds, stream, xs, ld, nrow,
                             gpr,
                             mask, cs, ms, ks, (int)n_mask);
          break;
        case 2:
          hipLaunchKernelGGL(quantize_masked_kernel<2>, grid, block, lds, stream, xs, ld, nrow,
                             gpr,
                             mask, cs, ms, ks, (int)n_mask);
          break;
        case 3:
          hipLaunchKernelGGL(quantize_masked_kernel<3>, grid, block, lds, stream, xs, ld, nrow,
                             gpr,
                             mask, cs, ms, ks, (int)n_mask);
          break;
        default:
          hipLaunchKernelGGL(quantize_masked_kernel<4>, grid, block, lds, stream, xs, ld, nrow,
                             gpr,
                             mask, cs, ms, ks, (int)n_mask);
          break;
      }
    } else {
      hipLaunchKernelGGL(quantize_kernel, dim3(grid_for(total, 256ull * 1024)), dim3(256), 0,
                         stream, xs, ld, gpr, fd, total, cs, ms);
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
