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
// Histograms are integers (LDS atomics per workgroup, then global atomics):
// results do not depend on scheduling.
//
// Mapping: a workgroup of 8 waves owns 128 channels and a slice of rows; each
// lane reads one 32-bit word (2 channels) per row, so every LDS atomic of an
// instruction targets a distinct channel. Channel p of the block is stored at
// LDS column (p & 1) * 64 + (p >> 1): the 64 lanes of a wave then hit 64
// distinct columns, i.e. the 32 banks exactly twice.
#include "hif4_dev.h"

namespace hif4 {

constexpr int kPctThreads = 512;
constexpr int kPctCh = 128;    // channels per workgroup
constexpr int kPctUnroll = 16; // rows in flight per lane

struct PctSel {
  uint32_t b_lo, r_lo, b_hi, r_hi;
};

__device__ __forceinline__ int col_of(int p) { return (p & 1) * 64 + (p >> 1); }

// Zero the histograms, reset the per-channel minimum keys.
__global__ void pct_init_kernel(uint32_t* __restrict__ h1, uint32_t* __restrict__ h2,
                                uint32_t* __restrict__ minkey, int c) {
  const int64_t n1 = (int64_t)c * 256, n2 = (int64_t)c * 128;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n1; i += stride) {
    h1[i] = 0u;
    if (i < n2) h2[i] = 0u;
    if (i < c) minkey[i] = 0xFFFFFFFFu;
  }
}

// Per-lane channel setup: the lane reads the 32-bit word of channels ch and
// ch+1 of every row. Lanes past the last channel read channel 0 instead (a
// valid address) and mark both halves invalid; when c is odd the last lane's
// word also covers element c, which exists because ld >= c + 1 then (ld is a
// multiple of 8), and its high half is marked invalid. Loads stay branch-free.
struct LaneCh {
  uint32_t off;     // element offset of the word inside a row
  uint32_t valid;   // bit 0: low half (ch) valid, bit 1: high half (ch+1) valid
};
__device__ __forceinline__ LaneCh lane_channels(int ch, int c) {
  LaneCh l;
  l.off = ch < c ? (uint32_t)ch : 0u;
  l.valid = (ch < c ? 1u : 0u) | (ch + 1 < c ? 2u : 0u);
  return l;
}

// Row streaming shared by the two passes: wave w of the workgroup reads rows
// r0 + w, r0 + w + 8, ... in blocks of kPctUnroll rows, the next block's
// loads issued before the current block is processed (two register buffers),
// so loads stay in flight while the histogram work runs. body(v, rb, tail)
// gets the block's words; the last partial block has its rows clamped to
// r1 - 1 and tail = true (the body must not count rows >= r1).
template <typename Body>
__device__ __forceinline__ void stream_rows(const uint16_t* xl, int64_t ld, int64_t r0,
                                            int64_t r1, int wave, Body&& body) {
  constexpr int kWaves = kPctThreads / 64;
  const int64_t step = (int64_t)kWaves * kPctUnroll, rstride = (int64_t)kWaves * ld;
  auto full = [&](int64_t rb) { return rb + (int64_t)(kPctUnroll - 1) * kWaves < r1; };
  auto load = [&](uint32_t (&v)[kPctUnroll], int64_t rb) {
    const uint16_t* p = xl + rb * ld;
#pragma unroll
    for (int u = 0; u < kPctUnroll; ++u) v[u] = *reinterpret_cast<const uint32_t*>(p + u * rstride);
  };
  int64_t rb = r0 + wave;
  uint32_t va[kPctUnroll], vb[kPctUnroll];
  if (full(rb)) {
    load(va, rb);
    for (;;) {
      const bool nb = full(rb + step);
      if (nb) load(vb, rb + step);
      body(va, rb, false);
      rb += step;
      if (!nb) break;
      const bool na = full(rb + step);
      if (na) load(va, rb + step);
      body(vb, rb, false);
      rb += step;
      if (!na) break;
    }
  }
  if (rb < r1) {  // last partial block
#pragma unroll
    for (int u = 0; u < kPctUnroll; ++u) {
      const int64_t r = min(rb + (int64_t)u * kWaves, r1 - 1);
      va[u] = *reinterpret_cast<const uint32_t*>(xl + r * ld);
    }
    body(va, rb, true);
  }
}

// Pass 1: coarse histograms. LDS counters are u16 pairs (rows per workgroup
// never exceed 65535), 256 bins x 128 channels = 64 KiB.
__global__ __launch_bounds__(kPctThreads) void pct_pass1_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int c, int64_t ld, int rows_per_block,
    uint32_t* __restrict__ h1) {
  __shared__ uint32_t hist[128 * kPctCh];  // [bin/2][column]
  for (int i = threadIdx.x; i < 128 * kPctCh; i += kPctThreads) hist[i] = 0u;
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = blockIdx.x * kPctCh;
  const LaneCh lc = lane_channels(c0 + 2 * lane, c);
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r1 = min(rows, r0 + rows_per_block);
  const int colA = col_of(2 * lane), colB = col_of(2 * lane + 1);
  constexpr int kWaves = kPctThreads / 64;
  const uint16_t* xl = x + lc.off;

  auto count = [&](const uint32_t (&v)[kPctUnroll], int64_t rb, bool tail) {
#pragma unroll
    for (int u = 0; u < kPctUnroll; ++u) {
      const bool row_ok = !tail || rb + (int64_t)u * kWaves < r1;
      const uint32_t ka = v[u] & 0x7FFFu, kb = (v[u] >> 16) & 0x7FFFu;
      const uint32_t ba = ka >> 7, bb = kb >> 7;
      const uint32_t ia = (row_ok && (lc.valid & 1u)) ? 1u << (16 * (ba & 1u)) : 0u;
      const uint32_t ib = (row_ok && (lc.valid & 2u)) ? 1u << (16 * (bb & 1u)) : 0u;
      atomicAdd(&hist[(ba >> 1) * kPctCh + colA], ia);
      atomicAdd(&hist[(bb >> 1) * kPctCh + colB], ib);
    }
  };
  stream_rows(xl, ld, r0, r1, wave, count);
  __syncthreads();
  for (int i = threadIdx.x; i < 128 * kPctCh; i += kPctThreads) {
    const uint32_t w = hist[i];
    if (!w) continue;
    const int col = i % kPctCh, bin2 = i / kPctCh;
    const int p = (col < 64) ? 2 * col : 2 * (col - 64) + 1;
    const int chan = c0 + p;
    if (chan >= c) continue;
    if (w & 0xFFFFu) atomicAdd(&h1[(int64_t)chan * 256 + 2 * bin2], w & 0xFFFFu);
    if (w >> 16) atomicAdd(&h1[(int64_t)chan * 256 + 2 * bin2 + 1], w >> 16);
  }
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
// inside them) of lo and hi.
__global__ __launch_bounds__(256) void pct_select_kernel(const uint32_t* __restrict__ h1,
                                                         int64_t rows, int c, double q,
                                                         PctSel* __restrict__ sel) {
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
__global__ __launch_bounds__(kPctThreads) void pct_pass2_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int c, int64_t ld, int rows_per_block,
    const PctSel* __restrict__ sel, uint32_t* __restrict__ h2, uint32_t* __restrict__ minkey) {
  __shared__ uint32_t hist[128 * kPctCh];  // [fine bin][column]
  __shared__ uint32_t mins[kPctCh];
  for (int i = threadIdx.x; i < 128 * kPctCh; i += kPctThreads) hist[i] = 0u;
  for (int i = threadIdx.x; i < kPctCh; i += kPctThreads) mins[i] = 0xFFFFFFFFu;
  __syncthreads();

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c0 = blockIdx.x * kPctCh;
  const int ch = c0 + 2 * lane;
  const LaneCh lc = lane_channels(ch, c);
  const int colA = col_of(2 * lane), colB = col_of(2 * lane + 1);
  // Bins to watch; 0x1FF never matches a bin (at most 255).
  uint32_t loA = 0x1FFu, hiA = 0x1FFu, loB = 0x1FFu, hiB = 0x1FFu;
  if (lc.valid & 1u) {
    loA = sel[ch].b_lo;
    hiA = sel[ch].b_hi != sel[ch].b_lo ? sel[ch].b_hi : 0x1FFu;
  }
  if (lc.valid & 2u) {
    loB = sel[ch + 1].b_lo;
    hiB = sel[ch + 1].b_hi != sel[ch + 1].b_lo ? sel[ch + 1].b_hi : 0x1FFu;
  }
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r1 = min(rows, r0 + rows_per_block);
  constexpr int kWaves = kPctThreads / 64;
  const uint16_t* xl = x + lc.off;

  auto scan = [&](const uint32_t (&v)[kPctUnroll], int64_t rb, bool tail) {
#pragma unroll
    for (int u = 0; u < kPctUnroll; ++u) {
      // a clamped (repeated) row must not count: push its bins out of range
      const uint32_t kill = (!tail || rb + (int64_t)u * kWaves < r1) ? 0u : 0x1000000u;
      const uint32_t ka = (v[u] & 0x7FFFu) | kill, kb = ((v[u] >> 16) & 0x7FFFu) | kill;
      if ((ka >> 7) == loA) atomicAdd(&hist[(ka & 127u) * kPctCh + colA], 1u);
      if ((ka >> 7) == hiA) atomicMin(&mins[colA], ka);
      if ((kb >> 7) == loB) atomicAdd(&hist[(kb & 127u) * kPctCh + colB], 1u);
      if ((kb >> 7) == hiB) atomicMin(&mins[colB], kb);
    }
  };
  stream_rows(xl, ld, r0, r1, wave, scan);
  __syncthreads();
  for (int i = threadIdx.x; i < 128 * kPctCh; i += kPctThreads) {
    const uint32_t w = hist[i];
    if (!w) continue;
    const int col = i % kPctCh, fb = i / kPctCh;
    const int p = (col < 64) ? 2 * col : 2 * (col - 64) + 1;
    const int chan = c0 + p;
    if (chan < c) atomicAdd(&h2[(int64_t)chan * 128 + fb], w);
  }
  for (int i = threadIdx.x; i < kPctCh; i += kPctThreads) {
    const int p = (i < 64) ? 2 * i : 2 * (i - 64) + 1;
    const int chan = c0 + p;
    if (chan < c && mins[i] != 0xFFFFFFFFu) atomicMin(&minkey[chan], mins[i]);
  }
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

// Top-n mask by radix select over the stats' bit patterns (stats are >= 0,
// so unsigned order = numeric order). One workgroup: four 8-bit digit passes
// (most significant first) find tau, the n-th largest value; channels above
// tau are protected, and of the channels equal to tau the lowest-indexed
// (n - count_above) are protected (ties go to the lower index).
constexpr int kMaskThreads = 1024;
__global__ __launch_bounds__(kMaskThreads) void topn_mask_kernel(const float* __restrict__ stats,
                                                                 int c, int n_protect,
                                                                 uint8_t* __restrict__ mask) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t s_prefix, s_need, s_above;
  __shared__ uint32_t part[kMaskThreads];
  const int tid = threadIdx.x;
  if (n_protect <= 0 || n_protect >= c) {
    const uint8_t v = n_protect <= 0 ? 0 : 1;
    for (int i = tid; i < c; i += kMaskThreads) mask[i] = v;
    return;
  }
  // rank (0-based, descending) of the element we look for
  if (tid == 0) {
    s_prefix = 0u;
    s_need = (uint32_t)(n_protect - 1);
  }
  uint32_t prefix_mask = 0u;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0u;
    __syncthreads();
    const uint32_t pre = s_prefix;
    for (int i = tid; i < c; i += kMaskThreads) {
      const uint32_t u = __float_as_uint(stats[i]);
      if ((u & prefix_mask) == pre) atomicAdd(&hist[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (tid == 0) {
      // walk digits from the top: find the digit holding rank s_need (descending)
      uint32_t need = s_need, d = 255;
      for (int dd = 255; dd >= 0; --dd) {
        if (need < hist[dd]) {
          d = (uint32_t)dd;
          break;
        }
        need -= hist[dd];
      }
      s_prefix = pre | (d << shift);
      s_need = need;
    }
    prefix_mask |= 255u << shift;
    __syncthreads();
  }
  const uint32_t tau = s_prefix;
  // count_above and, per thread chunk, the number of ties (for the index-ordered tie rank)
  const int chunk = (c + kMaskThreads - 1) / kMaskThreads;
  const int b0 = min(c, tid * chunk), b1 = min(c, b0 + chunk);
  uint32_t above = 0, ties = 0;
  for (int i = b0; i < b1; ++i) {
    const uint32_t u = __float_as_uint(stats[i]);
    above += u > tau;
    ties += u == tau;
  }
  part[tid] = ties;
  if (tid == 0) s_above = 0u;
  __syncthreads();
  atomicAdd(&s_above, above);
  // exclusive scan of the tie counts (thread order = channel order)
  if (tid == 0) {
    uint32_t run = 0;
    for (int i = 0; i < kMaskThreads; ++i) {
      const uint32_t v = part[i];
      part[i] = run;
      run += v;
    }
  }
  __syncthreads();
  const uint32_t take = (uint32_t)n_protect - s_above;  // ties to protect
  uint32_t tie_rank = part[tid];
  for (int i = b0; i < b1; ++i) {
    const uint32_t u = __float_as_uint(stats[i]);
    uint8_t m = 0;
    if (u > tau) {
      m = 1;
    } else if (u == tau) {
      m = tie_rank < take ? 1 : 0;
      ++tie_rank;
    }
    mask[i] = m;
  }
}

}  // namespace hif4

using namespace hif4;

size_t hif4_percentile_ws_bytes(int64_t c) {
  // h1 [c][256] + h2 [c][128] + minkey [c] (u32) + sel [c] (16 B), 256-B aligned parts
  auto al = [](size_t b) { return (b + 255) & ~(size_t)255; };
  return al((size_t)c * 256 * 4) + al((size_t)c * 128 * 4) + al((size_t)c * 4) +
         al((size_t)c * sizeof(PctSel));
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

  const int ci = (int)c;
  hipLaunchKernelGGL(pct_init_kernel, dim3(256), dim3(256), 0, stream, h1, h2, minkey, ci);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;

  // Rows per workgroup: enough workgroups to fill the chip (>= ~1024), at
  // most 65535 rows each (u16 LDS counters in pass 1).
  const int cblocks = (ci + kPctCh - 1) / kPctCh;
  int64_t splits = (1024 + cblocks - 1) / cblocks;
  if (splits > rows) splits = rows;
  int64_t rpb = (rows + splits - 1) / splits;
  if (rpb > 65535) rpb = 65535;
  if (rpb < 1) rpb = 1;
  const int64_t nsplit = (rows + rpb - 1) / rpb;
  for (int64_t s0 = 0; s0 < nsplit; s0 += 65535) {
    const int64_t ns = nsplit - s0 < 65535 ? nsplit - s0 : 65535;
    const int64_t rbase = s0 * rpb;
    hipLaunchKernelGGL(pct_pass1_kernel, dim3(cblocks, (unsigned)ns), dim3(kPctThreads), 0, stream,
                       x + rbase * ld, rows - rbase, ci, ld, (int)rpb, h1);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(pct_select_kernel, dim3((ci + 3) / 4), dim3(256), 0, stream, h1, rows, ci, q,
                     sel);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  for (int64_t s0 = 0; s0 < nsplit; s0 += 65535) {
    const int64_t ns = nsplit - s0 < 65535 ? nsplit - s0 : 65535;
    const int64_t rbase = s0 * rpb;
    hipLaunchKernelGGL(pct_pass2_kernel, dim3(cblocks, (unsigned)ns), dim3(kPctThreads), 0, stream,
                       x + rbase * ld, rows - rbase, ci, ld, (int)rpb, sel, h2, minkey);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(pct_final_kernel, dim3((ci + 3) / 4), dim3(256), 0, stream, h2, sel, minkey,
                     rows, ci, q, stats);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(topn_mask_kernel, dim3(1), dim3(kMaskThreads), 0, stream, stats, ci,
                     (int)n_protect, mask);
  return hipGetLastError();
}
