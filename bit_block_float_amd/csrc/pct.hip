// pct.hip -- tail-aware per-channel percentile and the channel-protection mask.
//
// Method: Tail-Aware HiFloat4 summary (agents-report.net), sections "方法概述"
// and "尾部百分位統計的動機": a per-channel percentile of the calibration
// activation magnitudes (instead of the maximum) builds a mask that protects
// the channels with the largest tail statistics. The percentile is read as
// the type-7 (linear) quantile; stated in hif4.h.
//
// Exact order statistics by radix select on the 15-bit magnitude key of a
// bf16 value (|x| bits, monotone in |x|):
//   pass 1  per-channel histogram of key >> 7 (256 coarse bins = the bf16
//           exponent field) -> the coarse bins holding ranks lo and hi;
//   pass 2  per-channel histogram of key & 127 inside the coarse bin of rank
//           lo, plus the smallest key of the coarse bin of rank hi when that
//           is a different bin -> the exact keys of ranks lo and hi;
//   final   type-7 interpolation in double, rounded once to fp32.
// Long columns first take a one-pass path (a window of keys placed by a
// sample of every S-th row; see the section further down) and compute only
// the channels the window missed exactly, from their own columns.
// Histograms are integers (LDS atomics per workgroup, then global atomics or
// per-segment partials): results do not depend on scheduling.
//
// Mapping: the work of a pass is the sequence of (channel block, row) pairs,
// a channel block being 128 channels. The grid is a whole number of waves of
// resident workgroups (one 16-wave workgroup per CU, the LDS bound of pass 1),
// and workgroup g takes the g-th equal contiguous slice of that sequence:
// every workgroup reads the same number of rows, so no partial last wave of
// workgroups idles the chip. A slice is one or a few segments (rows r0..r1 of
// one channel block); the LDS histogram is flushed to global memory at the end
// of each segment. In a segment each lane reads one 32-bit word (2 channels)
// per row, so every LDS atomic of an instruction targets a distinct channel.
// Channel p of the block is stored at LDS column (p & 1) * 64 + (p >> 1): the
// 64 lanes of a wave then hit 64 distinct columns, i.e. the 32 banks exactly
// twice. Lanes whose channels lie past the last channel read a valid word and
// count into their own columns, which are never flushed: the counting itself
// needs no per-lane validity test.
#include "hif4_dev.h"

namespace hif4 {

constexpr int kPctThreads = 1024;
constexpr int kPctWaves = kPctThreads / 64;
constexpr int kPctCh = 128;    // channels per workgroup
constexpr int kPctUnroll = 16; // rows per block of loads
constexpr int kRsrcWord3Pct = 0x00020000;  // raw buffer, 32-bit data format (gfx9)

struct PctSel {
  uint32_t b_lo, r_lo, b_hi, r_hi;
};

__device__ __forceinline__ int col_of(int p) { return (p & 1) * 64 + (p >> 1); }

// LDS column -> channel offset inside the block (inverse of col_of).
__device__ __forceinline__ int chan_of_col(int col) {
  return (col < 64) ? 2 * col : 2 * (col - 64) + 1;
}

// Element offset of the 32-bit word (channels ch, ch + 1) a lane reads in
// each row. Lanes past the last channel read channel 0 instead (a valid
// address); when c is odd the last lane's word also covers element c, which
// exists because ld >= c + 1 then (ld is a multiple of 8).
__device__ __forceinline__ uint32_t lane_offset(int ch, int c) {
  return ch < c ? (uint32_t)ch : 0u;
}

// Row streaming shared by the two passes (lane element offset loff inside a
// row): wave w of the workgroup reads rows
// r0 + w, r0 + w + 16, ... in blocks of kPctUnroll rows, the next block's
// loads issued before the current block is processed (two register buffers),
// so loads stay in flight while the histogram work runs. body(v, rb, tail)
// gets the block's words; the last partial block has its rows clamped to
// r1 - 1 and tail = true (the body must not count rows >= r1).
template <typename Body>
__device__ __forceinline__ void stream_rows(const uint16_t* x, uint32_t loff, int64_t ld,
                                            int64_t r0, int64_t r1, int wave, Body&& body) {
  constexpr int kWaves = kPctWaves;
  const int64_t step = (int64_t)kWaves * kPctUnroll;
  auto full = [&](int64_t rb) { return rb + (int64_t)(kPctUnroll - 1) * kWaves < r1; };
  // Buffer loads: the row base of a block is scalar, the lane offset and the
  // row step are 32-bit (ld <= 2^22 keeps every offset below 2^31).
  const uint32_t vbytes = loff * 2u;
  const int sstep = (int)(kWaves * ld * 2);
  auto word = [&](int64_t r) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(x + r * ld), (short)0, 0x7FFFFFFF, kRsrcWord3Pct);
    return (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, vbytes, 0, 0);
  };
  auto load = [&](uint32_t (&v)[kPctUnroll], int64_t rb) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(x + rb * ld), (short)0, 0x7FFFFFFF, kRsrcWord3Pct);
#pragma unroll
    for (int u = 0; u < kPctUnroll; ++u)
      v[u] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rs, vbytes, u * sstep, 0);
  };
  int64_t rb = r0 + wave;
  uint32_t va[kPctUnroll], vb[kPctUnroll];
  if (full(rb)) {
    load(va, rb);
    for (;;) {
      // the next block's loads are issued on every path (past the last full
      // block they repeat the current one, unused), so that the waits before
      // the current block count them exactly
      const bool nb = full(rb + step);
      load(vb, nb ? rb + step : rb);
      body(va, rb, false);
      rb += step;
      if (!nb) break;
      const bool na = full(rb + step);
      load(va, na ? rb + step : rb);
      body(vb, rb, false);
      rb += step;
      if (!na) break;
    }
  }
  if (rb < r1) {  // last partial block
#pragma unroll
    for (int u = 0; u < kPctUnroll; ++u) {
      const int64_t r = min(rb + (int64_t)u * kWaves, r1 - 1);
      va[u] = word(r);
    }
    body(va, rb, true);
  }
}

// Segments of workgroup g's slice [g * per_wg, (g + 1) * per_wg) of the
// (channel block, row) sequence; body(c0, r0, r1) runs once per segment, with
// values uniform over the workgroup. The sequence is ordered in slabs of
// per_wg rows (slab, then channel block, then row; the last slab may be
// shorter), so that workgroups g .. g + cblocks - 1 stream the same rows at
// the same time and the chip reads whole rows of X together.
template <typename Body>
__device__ __forceinline__ void for_segments(int64_t rows, int cblocks, int64_t per_wg,
                                             Body&& body) {
  const int64_t total = (int64_t)cblocks * rows;
  const int64_t slab_items = (int64_t)cblocks * per_wg;
  const int64_t full_slabs = rows / per_wg;
  int64_t pos = (int64_t)blockIdx.x * per_wg;
  const int64_t end = min(total, pos + per_wg);
  while (pos < end) {
    int64_t slab = pos / slab_items, rn = per_wg;
    if (slab >= full_slabs) {
      slab = full_slabs;
      rn = rows - full_slabs * per_wg;
    }
    const int64_t rs = slab * per_wg;
    const int64_t rem = pos - slab * slab_items;
    const int64_t cb = rem / rn;
    const int64_t off = rem - cb * rn;
    const int64_t r0 = rs + off;
    const int64_t r1 = rs + min(rn, off + (end - pos));
    body((int)cb * kPctCh, r0, r1);
    pos += r1 - r0;
  }
}

// Pass 1: coarse histograms, u32 counters, 256 bins x 128 channels = 128 KiB.
// The bin of the low channel of word v is bits 7..14, of the high channel
// bits 23..30: one bit-field extract and one shift-or per channel.
__global__ __launch_bounds__(kPctThreads) void pct_pass1_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int c, int64_t ld, int64_t per_wg,
    uint32_t* __restrict__ h1) {
  __shared__ uint32_t hist[256 * kPctCh];  // [bin][column]
  for (int i = threadIdx.x; i < 256 * kPctCh; i += kPctThreads) hist[i] = 0u;
  __syncthreads();

  // the wave index is uniform: row addresses then live in scalar registers
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int colA = col_of(2 * lane), colB = col_of(2 * lane + 1);
  const int cblocks = (c + kPctCh - 1) / kPctCh;

  for_segments(rows, cblocks, per_wg, [&](int c0, int64_t r0, int64_t r1) {
    auto count = [&](const uint32_t (&v)[kPctUnroll], int64_t rb, bool tail) {
#pragma unroll
      for (int u = 0; u < kPctUnroll; ++u) {
        if (tail && rb + (int64_t)u * kPctWaves >= r1) continue;  // clamped row
        atomicAdd(&hist[((v[u] >> 7) & 255u) * kPctCh + colA], 1u);
        atomicAdd(&hist[((v[u] >> 23) & 255u) * kPctCh + colB], 1u);
      }
    };
    stream_rows(x, lane_offset(c0 + 2 * lane, c), ld, r0, r1, wave, count);
    __syncthreads();
    // flush the segment's counts and clear the histogram for the next one
    for (int i = threadIdx.x; i < 256 * kPctCh; i += kPctThreads) {
      const uint32_t w = hist[i];
      if (!w) continue;
      hist[i] = 0u;
      const int chan = c0 + chan_of_col(i % kPctCh);
      if (chan < c) atomicAdd(&h1[(int64_t)chan * 256 + i / kPctCh], w);
    }
    __syncthreads();
  });
}

// Ranks lo and hi of the type-7 quantile: h = q (n-1), lo = floor(h).
__device__ __forceinline__ void type7_ranks(int64_t n, double q, int64_t* lo, int64_t* hi,
                                            double* f) {
  const double h = __dmul_rn(q, (double)(n - 1));
  const double fl = floor(h);
  *lo = (int64_t)fl;
  *hi = *lo + 1 < n ? *lo + 1 : n - 1;
  *f = __dsub_rn(h, fl);
}

// Inclusive prefix sum over the 64 lanes of a wave (Hillis-Steele with
// cross-lane reads; used only by the small per-channel kernels).
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint32_t o = __shfl_up(v, d, 64);
    if (lane >= d) v += o;
  }
  return v;
}

// First position (bin) whose running count exceeds `rank`, for counts laid
// out as `per` consecutive bins per lane; returns the bin and the count of
// all bins before it. Every lane gets the answer.
template <int kPer>
__device__ __forceinline__ void wave_find_rank(const uint32_t (&cnt)[kPer], int64_t rank,
                                               uint32_t* bin, int64_t* before) {
  const int lane = threadIdx.x & 63;
  uint32_t mine = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) mine += cnt[i];
  const uint32_t incl = wave_incl_scan(mine);
  const uint32_t excl = incl - mine;
  // the lane whose [excl, incl) range holds rank
  const bool here = (int64_t)excl <= rank && rank < (int64_t)incl;
  const uint64_t who = __ballot(here);
  const int src = who ? __ffsll((unsigned long long)who) - 1 : 63;
  uint32_t b = 0, run = excl;
  bool found = false;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if (!found && (int64_t)(run + cnt[i]) > rank) {
      b = (uint32_t)(lane * kPer + i);
      found = true;
    } else if (!found) {
      run += cnt[i];
    }
  }
  *bin = (uint32_t)__shfl((int)b, src, 64);
  *before = (int64_t)(uint32_t)__shfl((int)run, src, 64);
}

// Between passes: one wave per channel finds the coarse bins (and ranks
// inside them) of lo and hi; n_exact receives c (every channel's statistic
// comes from the two exact passes on this path).
__global__ __launch_bounds__(256) void pct_select_kernel(const uint32_t* __restrict__ h1,
                                                         int64_t rows, int c, double q,
                                                         PctSel* __restrict__ sel,
                                                         uint32_t* __restrict__ n_exact) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *n_exact = (uint32_t)c;
  const int ch = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (ch >= c) return;
  const int lane = threadIdx.x & 63;
  int64_t lo, hi;
  double f;
  type7_ranks(rows, q, &lo, &hi, &f);
  const uint4 w = reinterpret_cast<const uint4*>(h1 + (int64_t)ch * 256)[lane];
  const uint32_t cnt[4] = {w.x, w.y, w.z, w.w};
  uint32_t blo, bhi;
  int64_t before_lo, before_hi;
  wave_find_rank<4>(cnt, lo, &blo, &before_lo);
  wave_find_rank<4>(cnt, hi, &bhi, &before_hi);
  if (lane == 0) sel[ch] = PctSel{blo, (uint32_t)(lo - before_lo), bhi, (uint32_t)(hi - before_hi)};
}

// Pass 2: fine histograms inside bin b_lo and the minimum key of bin b_hi.
// With lo7 = b_lo << 7, a key k lies in bin b_lo exactly when t = k ^ lo7 is
// below 128, and t is then its fine index: min(t, 128) is the fine index, or
// the spare row 128 of the histogram (never flushed) for keys of other bins,
// so the count needs no branch. Likewise the smallest k ^ (b_hi << 7) below
// 128 gives the smallest key of bin b_hi; each lane keeps that minimum in a
// register (a lane owns its channels within its wave) and the workgroup
// merges it once per segment.
__global__ __launch_bounds__(kPctThreads) void pct_pass2_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int c, int64_t ld, int64_t per_wg,
    const PctSel* __restrict__ sel, uint32_t* __restrict__ h2, uint32_t* __restrict__ minkey) {
  __shared__ uint32_t hist[129 * kPctCh];  // [fine bin, spare][column]
  __shared__ uint32_t mins[kPctCh];
  for (int i = threadIdx.x; i < 129 * kPctCh; i += kPctThreads) hist[i] = 0u;
  for (int i = threadIdx.x; i < kPctCh; i += kPctThreads) mins[i] = 0xFFFFFFFFu;
  __syncthreads();

  // the wave index is uniform: row addresses then live in scalar registers
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int colA = col_of(2 * lane), colB = col_of(2 * lane + 1);
  const int cblocks = (c + kPctCh - 1) / kPctCh;

  for_segments(rows, cblocks, per_wg, [&](int c0, int64_t r0, int64_t r1) {
    const int ch = c0 + 2 * lane;
    // Bins to watch, shifted into key position; 0x1FF << 7 never matches a key
    // (keys are below 0x8000).
    uint32_t loA = 0x1FFu << 7, hiA = 0x1FFu << 7, loB = 0x1FFu << 7, hiB = 0x1FFu << 7;
    if (ch < c) {
      const PctSel s = sel[ch];
      loA = s.b_lo << 7;
      if (s.b_hi != s.b_lo) hiA = s.b_hi << 7;
    }
    if (ch + 1 < c) {
      const PctSel s = sel[ch + 1];
      loB = s.b_lo << 7;
      if (s.b_hi != s.b_lo) hiB = s.b_hi << 7;
    }
    uint32_t mnA = 0xFFFFFFFFu, mnB = 0xFFFFFFFFu;
    auto scan = [&](const uint32_t (&v)[kPctUnroll], int64_t rb, bool tail) {
#pragma unroll
      for (int u = 0; u < kPctUnroll; ++u) {
        // a clamped (repeated) row must not count: push it out of every bin
        const uint32_t kill = (!tail || rb + (int64_t)u * kPctWaves < r1) ? 0u : 0x1000000u;
        const uint32_t ka = (v[u] & 0x7FFFu) | kill, kb = ((v[u] >> 16) & 0x7FFFu) | kill;
        atomicAdd(&hist[min(ka ^ loA, 128u) * kPctCh + colA], 1u);
        atomicAdd(&hist[min(kb ^ loB, 128u) * kPctCh + colB], 1u);
        mnA = min(mnA, ka ^ hiA);
        mnB = min(mnB, kb ^ hiB);
      }
    };
    stream_rows(x, lane_offset(ch, c), ld, r0, r1, wave, scan);
    if (mnA < 128u) atomicMin(&mins[colA], mnA ^ hiA);
    if (mnB < 128u) atomicMin(&mins[colB], mnB ^ hiB);
    __syncthreads();
    // flush and clear for the next segment (the spare row is never read)
    for (int i = threadIdx.x; i < 128 * kPctCh; i += kPctThreads) {
      const uint32_t w = hist[i];
      if (!w) continue;
      hist[i] = 0u;
      const int chan = c0 + chan_of_col(i % kPctCh);
      if (chan < c) atomicAdd(&h2[(int64_t)chan * 128 + i / kPctCh], w);
    }
    for (int i = threadIdx.x; i < kPctCh; i += kPctThreads) {
      const uint32_t w = mins[i];
      if (w == 0xFFFFFFFFu) continue;
      mins[i] = 0xFFFFFFFFu;
      const int chan = c0 + chan_of_col(i);
      if (chan < c) atomicMin(&minkey[chan], w);
    }
    __syncthreads();
  });
}

// Exact keys of ranks lo / hi -> type-7 statistic, double then fp32 (RNE).
// One wave per channel.
__global__ __launch_bounds__(256) void pct_final_kernel(const uint32_t* __restrict__ h2,
                                                        const PctSel* __restrict__ sel,
                                                        const uint32_t* __restrict__ minkey,
                                                        int64_t rows, int c, double q,
                                                        float* __restrict__ stats) {
  const int ch = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (ch >= c) return;
  const int lane = threadIdx.x & 63;
  int64_t lo, hi;
  double f;
  type7_ranks(rows, q, &lo, &hi, &f);
  const PctSel s = sel[ch];
  const uint2 w = reinterpret_cast<const uint2*>(h2 + (int64_t)ch * 128)[lane];
  const uint32_t cnt[2] = {w.x, w.y};
  uint32_t flo, fhi;
  int64_t before;
  wave_find_rank<2>(cnt, (int64_t)s.r_lo, &flo, &before);
  const uint32_t klo = (s.b_lo << 7) | flo;
  uint32_t khi;
  if (s.b_hi == s.b_lo) {
    wave_find_rank<2>(cnt, (int64_t)s.r_hi, &fhi, &before);
    khi = (s.b_lo << 7) | fhi;
  } else {
    khi = minkey[ch];
  }
  if (lane == 0) {
    const double vlo = (double)__uint_as_float(klo << 16);
    const double vhi = (double)__uint_as_float(khi << 16);
    const double d = __dsub_rn(vhi, vlo);
    const double t = __dmul_rn(f, d);
    const double r = __dadd_rn(vlo, t);
    stats[ch] = __double2float_rn(r);
  }
}

// ---- one-pass path with a sampled window (large inputs)
//
// Pass 1 over every S-th row (S = max(8, ceil(rows / 8192)): at most ~8192
// sampled rows) gives each channel's coarse bin b_s of the quantile's rank
// in the sample; the window is the 512 consecutive keys of coarse bins
// b_s - 1 .. b_s + 2. One pass over all rows then counts, per channel, the
// keys below the window and a histogram of every key inside it. When ranks
// lo and hi of the full column both fall inside the window (their keys are
// then exact), the statistic is final; a channel whose ranks fall outside (a
// sample that misled) is computed exactly from its column in the same final
// kernel (pct_resolve_kernel), which also builds the mask.
constexpr int kWin = 512;          // keys in the window
// u32 per column of a partial: 256 packed words, below, pad to a whole number
// of 128-byte lines (so that the flush below writes whole lines)
constexpr int kPartStride = 288;
// LDS words per histogram row ([bin/2][column]): one pad word, so that the
// flush's lanes that read 8 consecutive quads of one column hit 8 banks
constexpr int kHistStride = kPctCh + 1;
constexpr int64_t kPartWords = (int64_t)kPctCh * kPartStride;  // one partial (a segment's counts)

// The window pass. A key below the window only adds to its lane's register
// count (most keys of a tail quantile do: as LDS atomics they would all hit
// one word per column, a chain of dependent read-modify-writes); a key inside
// adds to its bin, an LDS u16 pair counter (a segment never exceeds 65535
// rows) in 256 words per column; a key above is not counted. The atomic is
// issued under the lane mask of in-window keys. Lanes past the last channel
// see a window at 0xFFFF: every key is below, counted in registers whose
// partial is never read.
//
// Merging across workgroups without atomics: the (channel block, row) work
// sequence is cut into units, one per (slab, channel block) (see
// for_segments); a unit is at most per_wg rows long, so at most one slice
// boundary falls inside it and it is processed as one or two segments. Each
// segment stores its counts with plain 16-byte stores into its own partial:
// part[2 unit + 0] for the segment that starts the unit, part[2 unit + 1] for
// the other one. Partials are column-major ([column][word]): the final kernel
// reads a channel's 1 KiB of packed counts per partial contiguously.
// (Global atomics from the ~6 workgroups sharing a channel block, on lines
// that move between the chip's L2 caches, cost more than the streaming pass
// itself when every workgroup flushes at once.)
__global__ __launch_bounds__(kPctThreads) void pct_window_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int c, int64_t ld, int64_t per_wg,
    const uint32_t* __restrict__ wlo, uint32_t* __restrict__ part) {
  __shared__ uint32_t hist[(kWin / 2) * kHistStride];  // [bin/2][column]
  __shared__ uint32_t below[kPctCh];
  for (int i = threadIdx.x; i < (kWin / 2) * kHistStride; i += kPctThreads) hist[i] = 0u;
  for (int i = threadIdx.x; i < kPctCh; i += kPctThreads) below[i] = 0u;
  __syncthreads();

  // Lane layout: 16 lanes per row, each reading 16 bytes (channels 8p .. 8p + 7
  // of the block), so a wave's load covers 4 rows (row group g = lane / 16):
  // wave w reads rows rb + 4w + g + 64u of a block of kWinUnroll steps.
  constexpr int kWinUnroll = 4, kRowStep = 4 * kPctWaves;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4, p = lane & 15;
  const int rw = 4 * wave + g;  // row of the lane inside a step
  int col[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) col[e] = col_of(8 * p + e);
  const int cblocks = (c + kPctCh - 1) / kPctCh;

  for_segments(rows, cblocks, per_wg, [&](int c0, int64_t r0, int64_t r1) {
    const int ch = c0 + 8 * p;
    uint32_t wv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) wv[e] = ch + e < c ? wlo[ch + e] : 0xFFFFu;
    // lanes past the last channel read channel 0 of the row (a valid address;
    // their window start 0xFFFF keeps every key below it, and below counts of
    // channels >= c are never read)
    const uint32_t vb = (uint32_t)((rw * ld + (ch < c ? ch : 0)) * 2);
    const int sstep = (int)(kRowStep * ld * 2);
    uint32_t nb[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) nb[e] = 0u;
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    auto load = [&](u32x4_t (&v)[kWinUnroll], int64_t rb) {
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(x + rb * ld), (short)0, 0x7FFFFFFF, kRsrcWord3Pct);
#pragma unroll
      for (int u = 0; u < kWinUnroll; ++u) {
        const auto q = __builtin_amdgcn_raw_buffer_load_b128(rs, (int)vb, u * sstep, 2);
        v[u] = *reinterpret_cast<const u32x4_t*>(&q);
      }
    };
    auto count = [&](const u32x4_t (&v)[kWinUnroll], int64_t rb, bool tail) {
#pragma unroll
      for (int u = 0; u < kWinUnroll; ++u) {
        if (tail && rb + rw + (int64_t)u * kRowStep >= r1) continue;  // row past the segment
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t word = v[u][e >> 1];
          const uint32_t key = (e & 1) ? (word >> 16) & 0x7FFFu : word & 0x7FFFu;
          // keys and window starts are below 2^16: the difference wraps (top
          // bit set) exactly for keys below the window
          const uint32_t d = key - wv[e];
          nb[e] += d >> 31;
          if (d < (uint32_t)kWin)
            atomicAdd(&hist[(d >> 1) * kHistStride + col[e]], 1u << (16 * (d & 1u)));
        }
      }
    };
    // whole blocks of kWinUnroll steps (every lane's rows inside the segment),
    // the next block's loads issued on every path before the current block is
    // counted; then one partial block with rows past r1 clamped and skipped
    const int64_t blk = (int64_t)kWinUnroll * kRowStep;
    int64_t rb = r0;
    u32x4_t va[kWinUnroll], vc[kWinUnroll];
    if (rb + blk <= r1) {
      load(va, rb);
      for (;;) {
        const bool nxt = rb + 2 * blk <= r1;
        load(vc, nxt ? rb + blk : rb);
        count(va, rb, false);
        rb += blk;
        if (!nxt) break;
        const bool nxt2 = rb + 2 * blk <= r1;
        load(va, nxt2 ? rb + blk : rb);
        count(vc, rb, false);
        rb += blk;
        if (!nxt2) break;
      }
    }
    if (rb < r1) {
      // rows past r1 - 1 read row r1 - 1 again (skipped by count); offsets
      // from the block's row, below 256 rows
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(x + rb * ld), (short)0, 0x7FFFFFFF, kRsrcWord3Pct);
#pragma unroll
      for (int u = 0; u < kWinUnroll; ++u) {
        int64_t r = rb + rw + (int64_t)u * kRowStep;
        if (r > r1 - 1) r = r1 - 1;
        const auto q = __builtin_amdgcn_raw_buffer_load_b128(
            rs, (int)(((r - rb) * ld + (ch < c ? ch : 0)) * 2), 0, 2);
        va[u] = *reinterpret_cast<const u32x4_t*>(&q);
      }
      count(va, rb, true);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
      if (nb[e]) atomicAdd(&below[col[e]], nb[e]);
    __syncthreads();
    // this segment's partial: unit (slab, channel block), first or second part
    const int64_t slab = r0 / per_wg;
    const int64_t unit = slab * cblocks + c0 / kPctCh;
    uint32_t* dst = part + (2 * unit + (r0 == slab * per_wg ? 0 : 1)) * kPartWords;
    // Item i = (column, quad: words 4 quad .. 4 quad + 3). The 8 lanes of an
    // aligned group take 8 consecutive quads of one column, so each group
    // stores one whole 128-byte line of the partial (64 lanes: 8 columns).
    for (int i = threadIdx.x; i < (kWin / 8) * kPctCh; i += kPctThreads) {
      const int grp = i >> 6, l = i & 63;
      const int quad = (grp & 7) * 8 + (l & 7), col = (grp >> 3) * 8 + (l >> 3);
      uint4 w;
      w.x = hist[(4 * quad + 0) * kHistStride + col];
      w.y = hist[(4 * quad + 1) * kHistStride + col];
      w.z = hist[(4 * quad + 2) * kHistStride + col];
      w.w = hist[(4 * quad + 3) * kHistStride + col];
      hist[(4 * quad + 0) * kHistStride + col] = 0u;
      hist[(4 * quad + 1) * kHistStride + col] = 0u;
      hist[(4 * quad + 2) * kHistStride + col] = 0u;
      hist[(4 * quad + 3) * kHistStride + col] = 0u;
      *reinterpret_cast<uint4*>(dst + col * kPartStride + 4 * quad) = w;
    }
    for (int i = threadIdx.x; i < kPctCh; i += kPctThreads) {
      dst[i * kPartStride + kWin / 2] = below[i];
      below[i] = 0u;
    }
    __syncthreads();
  });
}

// Fill n words with a value (the buffers of the exact passes).
__global__ void pct_zero_kernel(uint32_t* __restrict__ p, int64_t n, uint32_t value) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = value;
}

// Top-n mask by radix select over the stats' bit patterns (stats are >= 0,
// so unsigned order = numeric order), run by one workgroup of kMaskThreads
// threads; thread t keeps the statistics of its contiguous chunk of channels
// [t * per, (t + 1) * per) (per <= kPer, c <= kMaskThreads * kPer) in
// registers. Four 8-bit digit passes (most significant first) find tau, the
// n-th largest value; channels above tau are protected, and of the channels
// equal to tau the lowest-indexed (n - count_above) are protected (ties go
// to the lower index).
constexpr int kMaskThreads = 1024;

struct TopnShared {
  uint32_t hist[256];
  uint32_t prefix, need;
  uint32_t part[kMaskThreads / 64], part_above[kMaskThreads / 64];
};

template <int kPer>
__device__ void topn_select(const float* __restrict__ stats, int c, int n_protect,
                            uint8_t* __restrict__ mask, TopnShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63;
  if (n_protect <= 0 || n_protect >= c) {
    const uint8_t v = n_protect <= 0 ? 0 : 1;
    for (int i = tid; i < c; i += kMaskThreads) mask[i] = v;
    return;
  }
  const int per = (c + kMaskThreads - 1) / kMaskThreads;  // uniform, <= kPer
  const int i0 = tid * per;
  uint32_t u[kPer];
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = i0 + j;
    u[j] = (j < per && i < c) ? __float_as_uint(stats[i]) : 0u;
  }
  // rank (0-based, descending) of the element we look for
  if (tid == 0) {
    sh.prefix = 0u;
    sh.need = (uint32_t)(n_protect - 1);
  }
  uint32_t prefix_mask = 0u;
#pragma unroll
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) sh.hist[tid] = 0u;
    __syncthreads();
    const uint32_t pre = sh.prefix;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      const int i = i0 + j;
      if (j < per && i < c && (u[j] & prefix_mask) == pre)
        atomicAdd(&sh.hist[(u[j] >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // the digit holding rank `need`, counting from the top digit down:
      // lane l holds digits 255 - 4l .. 252 - 4l
      const uint32_t need = sh.need;
      uint32_t cnt[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) cnt[i] = sh.hist[255 - (lane * 4 + i)];
      uint32_t pos;
      int64_t before;
      wave_find_rank<4>(cnt, (int64_t)need, &pos, &before);
      if (tid == 0) {
        sh.prefix = pre | ((255u - pos) << shift);
        sh.need = need - (uint32_t)before;
      }
    }
    prefix_mask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t tau = sh.prefix;
  // count_above, and the ties of each thread's chunk (thread order = channel
  // order, so an exclusive scan of the tie counts ranks the ties by index)
  uint32_t above = 0, ties = 0;
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const bool ok = j < per && i0 + j < c;
    above += (ok && u[j] > tau) ? 1u : 0u;
    ties += (ok && u[j] == tau) ? 1u : 0u;
  }
  const uint32_t incl = wave_incl_scan(ties);
  const uint32_t above_w = wave_incl_scan(above);  // lane 63: the wave's total
  if (lane == 63) {
    sh.part[tid >> 6] = incl;
    sh.part_above[tid >> 6] = above_w;
  }
  __syncthreads();
  uint32_t tie_rank = incl - ties, above_all = 0;
  for (int w = 0; w < kMaskThreads / 64; ++w) {
    if (w < (tid >> 6)) tie_rank += sh.part[w];
    above_all += sh.part_above[w];
  }
  const uint32_t take = (uint32_t)n_protect - above_all;  // ties to protect
#pragma unroll
  for (int j = 0; j < kPer; ++j) {
    const int i = i0 + j;
    if (j < per && i < c) {
      uint8_t m = 0;
      if (u[j] > tau) {
        m = 1;
      } else if (u[j] == tau) {
        m = tie_rank < take ? 1 : 0;
        ++tie_rank;
      }
      mask[i] = m;
    }
  }
}

template <int kPer>
__global__ __launch_bounds__(kMaskThreads) void topn_mask_kernel(const float* __restrict__ stats,
                                                                 int c, int n_protect,
                                                                 uint8_t* __restrict__ mask) {
  __shared__ TopnShared sh;
  topn_select<kPer>(stats, c, n_protect, mask, sh);
}

// Exact type-7 statistic of one channel by the whole workgroup: two passes over the channel's column, a 256-bin histogram of
// key >> 7, then a 128-bin histogram of key & 127 inside the coarse bin of
// rank lo with the smallest key of the coarse bin of rank hi when that
// differs; the interpolation as in pct_final_kernel. For the channels the
// sampled window missed: rare, and each is one column read twice.
struct ExactShared {
  uint32_t coarse[256];
  uint32_t fine[128];
  uint32_t minkey;
  PctSel sel;
};

__device__ void exact_channel(const uint16_t* __restrict__ x, int64_t ld, int64_t rows, int ch,
                              double q, float* __restrict__ stats, ExactShared& sh) {
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  constexpr int kU = 8;  // loads in flight per thread
  const int nthr = blockDim.x;
  for (int i = tid; i < 256; i += nthr) sh.coarse[i] = 0u;
  for (int i = tid; i < 128; i += nthr) sh.fine[i] = 0u;
  if (tid == 0) sh.minkey = 0xFFFFFFFFu;
  __syncthreads();
  const uint16_t* col = x + ch;
  const int64_t step = (int64_t)nthr * kU;
  for (int64_t r0 = tid; r0 < rows; r0 += step) {
    uint32_t v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t r = r0 + (int64_t)u * nthr;
      v[u] = r < rows ? (uint32_t)col[r * ld] : 0xFFFFFFFFu;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u)
      if (v[u] != 0xFFFFFFFFu) atomicAdd(&sh.coarse[(v[u] & 0x7FFFu) >> 7], 1u);
  }
  __syncthreads();
  int64_t lo, hi;
  double f;
  type7_ranks(rows, q, &lo, &hi, &f);
  if (wv == 0) {
    const uint32_t cnt[4] = {sh.coarse[4 * lane], sh.coarse[4 * lane + 1], sh.coarse[4 * lane + 2],
                             sh.coarse[4 * lane + 3]};
    uint32_t blo, bhi;
    int64_t before_lo, before_hi;
    wave_find_rank<4>(cnt, lo, &blo, &before_lo);
    wave_find_rank<4>(cnt, hi, &bhi, &before_hi);
    if (lane == 0) sh.sel = PctSel{blo, (uint32_t)(lo - before_lo), bhi, (uint32_t)(hi - before_hi)};
  }
  __syncthreads();
  const PctSel s = sh.sel;
  uint32_t mn = 0xFFFFFFFFu;
  for (int64_t r0 = tid; r0 < rows; r0 += step) {
    uint32_t v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int64_t r = r0 + (int64_t)u * nthr;
      v[u] = r < rows ? (uint32_t)col[r * ld] & 0x7FFFu : 0xFFFFFFFFu;
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (v[u] == 0xFFFFFFFFu) continue;
      if ((v[u] >> 7) == s.b_lo) atomicAdd(&sh.fine[v[u] & 127u], 1u);
      if ((v[u] >> 7) == s.b_hi) mn = min(mn, v[u]);
    }
  }
  if (s.b_hi != s.b_lo && mn != 0xFFFFFFFFu) atomicMin(&sh.minkey, mn);
  __syncthreads();
  if (wv == 0) {
    const uint32_t cnt[2] = {sh.fine[2 * lane], sh.fine[2 * lane + 1]};
    uint32_t flo, fhi;
    int64_t before;
    wave_find_rank<2>(cnt, (int64_t)s.r_lo, &flo, &before);
    const uint32_t klo = (s.b_lo << 7) | flo;
    uint32_t khi;
    if (s.b_hi == s.b_lo) {
      wave_find_rank<2>(cnt, (int64_t)s.r_hi, &fhi, &before);
      khi = (s.b_lo << 7) | fhi;
    } else {
      khi = sh.minkey;
    }
    if (lane == 0) {
      const double vlo = (double)__uint_as_float(klo << 16);
      const double vhi = (double)__uint_as_float(khi << 16);
      const double d = __dsub_rn(vhi, vlo);
      const double t = __dmul_rn(f, d);
      const double r = __dadd_rn(vlo, t);
      stats[ch] = __double2float_rn(r);
    }
  }
  __syncthreads();
}

// The window path's last kernel, one wave per channel (4 channels per
// workgroup of 256 threads):
//  1. each wave sums its channel's window counts over the partials of its
//     channel block; when ranks lo and hi both lie in the window their keys
//     are read off it and the statistic is final;
//  2. the channels whose ranks fell outside (a sample that misled) are then
//     computed exactly, one after another, by the whole workgroup
//     (exact_channel), and counted in n_failed.
constexpr int kResolveThreads = 256;

__global__ __launch_bounds__(kResolveThreads) void pct_resolve_kernel(
    const uint16_t* __restrict__ x, int64_t ld, const uint32_t* __restrict__ part,
    const uint32_t* __restrict__ wlo, int64_t rows, int c, int64_t per_wg, double q,
    float* __restrict__ stats, uint32_t* __restrict__ n_failed) {
  __shared__ ExactShared sh;
  __shared__ uint32_t s_fail;
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int ch = blockIdx.x * (kResolveThreads / 64) + wv;
  if (threadIdx.x == 0) s_fail = 0u;
  __syncthreads();
  if (ch < c) {
    const int cblocks = (c + kPctCh - 1) / kPctCh;
    const int cb = ch / kPctCh, col = col_of(ch % kPctCh);
    const int64_t full_slabs = rows / per_wg;
    const int64_t n_slabs = (rows + per_wg - 1) / per_wg;
    uint32_t cnt[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    int64_t nbelow = 0;
    // The channel's partials. A unit of a whole slab starts at a multiple of
    // per_wg and is per_wg rows long: it is one slice, one segment, and only
    // its first partial is written. Only the last slab's units (shorter than
    // per_wg) can straddle a slice boundary; then the unit's second partial
    // holds the rest. So the partials are p = 0 .. n_slabs - 1 (first
    // partial of slab p), plus, when the channel block's last unit straddles,
    // p = n_slabs (that unit's second partial): one wave-uniform test, no
    // division per partial.
    bool last_two = false;
    if (n_slabs > full_slabs) {
      const int64_t rn = rows - full_slabs * per_wg;
      const int64_t s0 = full_slabs * cblocks * per_wg + cb * rn;
      last_two = s0 / per_wg != (s0 + rn - 1) / per_wg;
    }
    const int64_t n_part = n_slabs + (last_two ? 1 : 0);
    // kBatch partials at a time, every load issued before any is summed;
    // indexes past the end read the last partial again, not summed. Batches
    // of 8 keep the kernel at 78 VGPRs (6 waves per SIMD: its one wave per
    // channel, 5 per SIMD at 5120 channels, fits the chip in one round).
    constexpr int kBatch = 8;
    for (int64_t pb = 0; pb < n_part; pb += kBatch) {
      uint4 w[kBatch];
      uint32_t bl[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        const int64_t p = min(pb + i, n_part - 1);
        const int64_t slab = p < n_slabs ? p : n_slabs - 1;
        const uint32_t* src = part + (2 * (slab * cblocks + cb) + (p < n_slabs ? 0 : 1)) * kPartWords +
                              (int64_t)col * kPartStride;
        w[i] = reinterpret_cast<const uint4*>(src)[lane];
        bl[i] = src[kWin / 2];
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (pb + i >= n_part) continue;
        cnt[0] += w[i].x & 0xFFFFu;
        cnt[1] += w[i].x >> 16;
        cnt[2] += w[i].y & 0xFFFFu;
        cnt[3] += w[i].y >> 16;
        cnt[4] += w[i].z & 0xFFFFu;
        cnt[5] += w[i].z >> 16;
        cnt[6] += w[i].w & 0xFFFFu;
        cnt[7] += w[i].w >> 16;
        nbelow += bl[i];
      }
    }
    int64_t lo, hi;
    double f;
    type7_ranks(rows, q, &lo, &hi, &f);
    uint32_t in_win = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) in_win += cnt[i];
    for (int d = 32; d >= 1; d >>= 1) in_win += (uint32_t)__shfl_xor((int)in_win, d, 64);
    if (!(lo >= nbelow && hi < nbelow + (int64_t)in_win)) {
      if (lane == 0) atomicOr(&s_fail, 1u << wv);
    } else {
      uint32_t blo, bhi;
      int64_t before;
      wave_find_rank<8>(cnt, lo - nbelow, &blo, &before);
      wave_find_rank<8>(cnt, hi - nbelow, &bhi, &before);
      if (lane == 0) {
        const uint32_t w0 = wlo[ch];
        const double vlo = (double)__uint_as_float((w0 + blo) << 16);
        const double vhi = (double)__uint_as_float((w0 + bhi) << 16);
        const double d = __dsub_rn(vhi, vlo);
        const double t = __dmul_rn(f, d);
        const double r = __dadd_rn(vlo, t);
        stats[ch] = __double2float_rn(r);
      }
    }
  }
  __syncthreads();
  const uint32_t fails = s_fail;
  for (uint32_t m = fails; m != 0u; m &= m - 1u)
    exact_channel(x, ld, rows, blockIdx.x * (kResolveThreads / 64) + __builtin_ctz(m), q, stats,
                  sh);
  if (threadIdx.x == 0 && fails) atomicAdd(n_failed, (uint32_t)__builtin_popcount(fails));
}

// The window path's first two kernels. pct_sample_kernel: workgroup (x, y)
// reads part y of the sampled rows (every S-th row; the parts are equal
// contiguous runs) for the block of 64 channels x, and stores its coarse
// histogram (key >> 7; u32 in LDS, u16 pairs in the partial) as sample
// partial (y, x), [channel][bin], with plain stores: no atomics across
// workgroups and nothing to clear beforehand.
// Lanes read 16 bytes (channels 8p .. 8p+7, p = lane & 7), 8 lanes per row, so
// a wave's load covers one 128-byte piece of each of 8 rows. In LDS the
// histogram is [bin][channel] with a row stride of 65 words, so the 8 rows of
// a wave's atomic land in distinct banks. Splitting the rows keeps every CU
// streaming (one workgroup per channel block alone ran 80 workgroups).
// pct_place_kernel: one wave per channel sums the channel's partials and finds
// the coarse bin b of rank floor(q (n_s - 1)) of the sample; the window starts
// one coarse bin below it. Its workgroup 0 also clears the flagged-channel
// count.
constexpr int kSampCh = 64;
constexpr int kSampStride = kSampCh + 1;
constexpr int kSampWords = kSampCh * 256;       // bins of one sample partial
constexpr int kSampPartWords = kSampWords / 2;  // its words (u16 counts)

__global__ __launch_bounds__(kPctThreads) void pct_sample_kernel(
    const uint16_t* __restrict__ x, int64_t rows_s, int c, int64_t ld, int parts,
    uint32_t* __restrict__ samp) {
  __shared__ uint32_t hist[256 * kSampStride];
  for (int i = threadIdx.x; i < 256 * kSampStride; i += kPctThreads) hist[i] = 0u;
  __syncthreads();
  // Single-buffered blocks of kUnroll steps (8 rows per wave per step,
  // 128 rows per step): all of a block's loads go out at once and are counted
  // as they arrive. 11 steps (1408 rows) cover a part at 5120 channels (1200
  // rows at FFN-up, at most 1366) in one block, and the kernel stays within
  // 64 VGPRs, so two workgroups share a CU and its grid (480 workgroups at
  // 5120 channels) runs in one round. Double-buffered blocks of 8 needed 80
  // VGPRs: one workgroup per CU, about two rounds.
  constexpr int kUnroll = 11, kHalf = 6, kRowStep = 8 * kPctWaves;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 3, p = lane & 7;
  const int rw = 8 * wave + g;  // row of the lane inside a step
  const int c0 = blockIdx.x * kSampCh;
  const int ch = c0 + 8 * p;
  // this part's sampled rows [rbeg, rend)
  const int64_t rbeg = rows_s * blockIdx.y / parts, rend = rows_s * (blockIdx.y + 1) / parts;
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  // Lanes past the last channel read channel 0 (a valid address); their
  // columns are never read back. Offsets are 32-bit from a wave-uniform row
  // base: steps 0..kHalf-1 of a block from its first row, the others from
  // row kHalf * kRowStep, so that an offset spans at most kHalf * 128 rows of
  // ld <= 2^20 elements (below 2^31 bytes). Each base's buffer range ends
  // with the part's last row: loads of rows past it return zeros (and are
  // not counted); a base at or past the end gets an empty range.
  const uint32_t vb = (uint32_t)((rw * ld + (ch < c ? ch : 0)) * 2);
  const uint32_t sstep = (uint32_t)(kRowStep * ld * 2);
  const int64_t blk = (int64_t)kUnroll * kRowStep;
  for (int64_t rb = rbeg; rb < rend; rb += blk) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int64_t hb = rb + (int64_t)h * kHalf * kRowStep;
      const int64_t nrec = hb < rend ? min((rend - hb) * ld * 2, (int64_t)0x7FFFFFFF) : 0;
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(x + min(hb, rend - 1) * ld), (short)0, (int)nrec, kRsrcWord3Pct);
#pragma unroll
      for (int u = h * kHalf; u < (h == 0 ? kHalf : kUnroll); ++u) {
        const auto qq =
            __builtin_amdgcn_raw_buffer_load_b128(rs, (int)vb, (int)((u - h * kHalf) * sstep), 2);
        v[u] = *reinterpret_cast<const u32x4_t*>(&qq);
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      if (rb + rw + (int64_t)u * kRowStep >= rend) continue;  // row past the part
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t word = v[u][e >> 1];
        const uint32_t bin = (e & 1) ? (word >> 23) & 255u : (word >> 7) & 255u;
        atomicAdd(&hist[bin * kSampStride + 8 * p + e], 1u);
      }
    }
  }
  __syncthreads();
  // [channel][bin]: consecutive threads store consecutive bins of a channel
  // as u16 pairs (a part holds at most ~8192 sampled rows, so no count
  // reaches 2^16): word w of a channel holds bins 2w (low) and 2w + 1 (high)
  uint32_t* dst = samp + ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * kSampPartWords;
  for (int i = threadIdx.x; i < kSampPartWords; i += kPctThreads) {
    const int ch = i >> 7, w = i & 127;
    dst[i] = hist[(2 * w) * kSampStride + ch] | (hist[(2 * w + 1) * kSampStride + ch] << 16);
  }
}

constexpr int kPlaceThreads = 256;

__global__ __launch_bounds__(kPlaceThreads) void pct_place_kernel(
    const uint32_t* __restrict__ samp, int parts, int c, int64_t rows_s, double q,
    uint32_t* __restrict__ wlo, uint32_t* __restrict__ n_failed) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *n_failed = 0u;
  const int lane = threadIdx.x & 63;
  const int ch = blockIdx.x * (kPlaceThreads / 64) + (threadIdx.x >> 6);
  if (ch >= c) return;  // the whole wave
  const int cblocks = (c + kSampCh - 1) / kSampCh;
  const uint32_t* src =
      samp + (int64_t)(ch / kSampCh) * kSampPartWords + (ch % kSampCh) * 128 + 2 * lane;
  uint32_t cnt[4] = {0u, 0u, 0u, 0u};
  for (int y = 0; y < parts; ++y) {
    const uint2 v = *reinterpret_cast<const uint2*>(src + (int64_t)y * cblocks * kSampPartWords);
    cnt[0] += v.x & 0xFFFFu;
    cnt[1] += v.x >> 16;
    cnt[2] += v.y & 0xFFFFu;
    cnt[3] += v.y >> 16;
  }
  int64_t lo, hi;
  double f;
  type7_ranks(rows_s, q, &lo, &hi, &f);
  uint32_t b;
  int64_t before;
  wave_find_rank<4>(cnt, lo, &b, &before);
  if (lane == 0) wlo[ch] = (b > 0 ? b - 1 : 0u) << 7;
}

}  // namespace hif4

using namespace hif4;

namespace {
// Compute units of the current device (cached per device; 256 on MI355X).
int g_cus[64];
int cu_count() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 256;
  if (dev < 64 && g_cus[dev] > 0) return g_cus[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    n = 256;
  if (dev < 64) g_cus[dev] = n;
  return n;
}
}  // namespace

namespace {
// Grid of a streaming pass over `rows` rows: a whole number of waves of
// `resident` workgroups (one per CU), each taking an equal slice of the
// (channel block, row) sequence of at most 65535 rows.
bool pass_grid(int64_t rows, int ci, int64_t resident, int64_t* per_wg, int64_t* grid) {
  const int cblocks = (ci + kPctCh - 1) / kPctCh;
  const int64_t total = (int64_t)cblocks * rows;
  const int64_t waves = (total + resident * 65535 - 1) / (resident * 65535);
  *per_wg = (total + resident * waves - 1) / (resident * waves);
  *grid = (total + *per_wg - 1) / *per_wg;
  return *grid <= 0x7FFFFFFF;
}

// The window pass runs on a grid for 256 resident workgroups (MI355X's CU
// count) whatever the device reports, so that its partials -- two per unit,
// one unit per (slab of per_wg rows, channel block) -- depend only on rows
// and c and the workspace size can be stated without a device.
constexpr int64_t kWindowResident = 256;
constexpr int64_t kWindowMinRows = 8192;

// Row stride of the window path's sample: every 8th row, and at most ~8192
// sampled rows for very long columns.
int64_t sample_stride(int64_t rows) {
  const int64_t s = (rows + 8191) / 8192;
  return s > 8 ? s : 8;
}

int64_t window_partials(int64_t rows, int64_t c) {
  if (rows < kWindowMinRows) return 0;
  int64_t per_wg, grid;
  pass_grid(rows, (int)c, kWindowResident, &per_wg, &grid);
  const int64_t cblocks = (c + kPctCh - 1) / kPctCh;
  return 2 * ((rows + per_wg - 1) / per_wg) * cblocks;
}

// Parts of the window path's sample: about two workgroups per CU of a
// 256-CU device over all channel blocks, at least 256 sampled rows each, at
// most 16 (a function of rows and c only, so the workspace is too).
int sample_parts(int64_t rows_s, int64_t c) {
  const int64_t cblocks = (c + kSampCh - 1) / kSampCh;
  int64_t parts = 512 / cblocks;
  if (parts > rows_s / 256) parts = rows_s / 256;
  if (parts > 16) parts = 16;
  return parts < 1 ? 1 : (int)parts;
}

// Bytes of the region that holds the window pass's partials and, before that
// pass, the sample partials.
size_t window_region_bytes(int64_t rows, int64_t c) {
  if (rows < kWindowMinRows) return 0;
  const int64_t rows_s = (rows + sample_stride(rows) - 1) / sample_stride(rows);
  const size_t win = (size_t)window_partials(rows, c) * kPartWords * 4;
  const size_t smp = (size_t)sample_parts(rows_s, c) * ((c + kSampCh - 1) / kSampCh) * kSampWords * 4;
  return win > smp ? win : smp;
}
}  // namespace

size_t hif4_percentile_ws_bytes(int64_t rows, int64_t c) {
  // h1 [c][256] + h2 [c][128] + minkey [c] + sel [c] (16 B) + window start [c]
  // + window partials + the exact-channel count (last part), 256-B aligned
  // parts
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  return al((size_t)c * 256 * 4) + al((size_t)c * 128 * 4) + al((size_t)c * 4) +
         al((size_t)c * sizeof(PctSel)) + al((size_t)c * 4) +
         al(window_region_bytes(rows, c)) + al(4);
}

hipError_t hif4_launch_percentile(const uint16_t* x, int64_t rows, int64_t c, int64_t ld,
                                  double q, int64_t n_protect, float* stats, uint8_t* mask,
                                  void* workspace, hipStream_t stream) {
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  char* ws = (char*)workspace;
  uint32_t* h1 = (uint32_t*)ws;
  ws += al((size_t)c * 256 * 4);
  uint32_t* h2 = (uint32_t*)ws;
  ws += al((size_t)c * 128 * 4);
  uint32_t* minkey = (uint32_t*)ws;
  ws += al((size_t)c * 4);
  PctSel* sel = (PctSel*)ws;
  ws += al((size_t)c * sizeof(PctSel));
  uint32_t* wlo = (uint32_t*)ws;
  ws += al((size_t)c * 4);
  uint32_t* part = (uint32_t*)ws;
  ws += al(window_region_bytes(rows, c));
  uint32_t* n_exact = (uint32_t*)ws;  // channels resolved by exact passes

  const int ci = (int)c;
  hipError_t e;
  const int64_t stride_s = sample_stride(rows);
  // The sampled window pays off on long columns; the sample is read with an
  // S-fold row stride, and the sample kernel's 32-bit buffer offsets span
  // 512 sampled rows: ld * S <= 2^20 keeps them below 2^31.
  const bool window = rows >= kWindowMinRows && ld * stride_s <= ((int64_t)1 << 20);
  if (window) {
    const int64_t rows_s = (rows + stride_s - 1) / stride_s;
    int64_t per_w, grid_w;
    if (!pass_grid(rows, ci, kWindowResident, &per_w, &grid_w)) return hipErrorInvalidValue;
    const int parts = sample_parts(rows_s, c);
    hipLaunchKernelGGL(pct_sample_kernel, dim3((unsigned)((ci + kSampCh - 1) / kSampCh), parts),
                       dim3(kPctThreads), 0, stream, x, rows_s, ci, ld * stride_s, parts, part);
    hipLaunchKernelGGL(pct_place_kernel,
                       dim3((unsigned)((ci + kPlaceThreads / 64 - 1) / (kPlaceThreads / 64))),
                       dim3(kPlaceThreads), 0, stream, (const uint32_t*)part, parts, ci, rows_s, q,
                       wlo, n_exact);
    hipLaunchKernelGGL(pct_window_kernel, dim3((unsigned)grid_w), dim3(kPctThreads), 0, stream, x,
                       rows, ci, ld, per_w, (const uint32_t*)wlo, part);
    hipLaunchKernelGGL(pct_resolve_kernel,
                       dim3((unsigned)((ci + kResolveThreads / 64 - 1) / (kResolveThreads / 64))),
                       dim3(kResolveThreads), 0, stream, x, ld, (const uint32_t*)part,
                       (const uint32_t*)wlo, rows, ci, per_w, q, stats, n_exact);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  } else {
    // Short columns: the two exact passes for every channel.
    int64_t per_wg, grid;
    if (!pass_grid(rows, ci, cu_count(), &per_wg, &grid)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(pct_zero_kernel, dim3(256), dim3(256), 0, stream, h1, (int64_t)c * 256, 0u);
    hipLaunchKernelGGL(pct_zero_kernel, dim3(256), dim3(256), 0, stream, h2, (int64_t)c * 128, 0u);
    hipLaunchKernelGGL(pct_zero_kernel, dim3(64), dim3(256), 0, stream, minkey, (int64_t)c,
                       0xFFFFFFFFu);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(pct_pass1_kernel, dim3((unsigned)grid), dim3(kPctThreads), 0, stream, x,
                       rows, ci, ld, per_wg, h1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(pct_select_kernel, dim3((ci + 3) / 4), dim3(256), 0, stream, h1, rows, ci,
                       q, sel, n_exact);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(pct_pass2_kernel, dim3((unsigned)grid), dim3(kPctThreads), 0, stream, x,
                       rows, ci, ld, per_wg, sel, h2, minkey);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(pct_final_kernel, dim3((ci + 3) / 4), dim3(256), 0, stream, h2, sel,
                       minkey, rows, ci, q, stats);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (ci <= 8 * kMaskThreads)
    hipLaunchKernelGGL(topn_mask_kernel<8>, dim3(1), dim3(kMaskThreads), 0, stream, stats, ci,
                       (int)n_protect, mask);
  else
    hipLaunchKernelGGL(topn_mask_kernel<64>, dim3(1), dim3(kMaskThreads), 0, stream, stats, ci,
                       (int)n_protect, mask);
  return hipGetLastError();
}
