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

// Load the magnitude keys of this lane's (up to) two channels for one row.
__device__ __forceinline__ uint32_t load_pair(const uint16_t* __restrict__ xr, int ch, int c) {
  if (ch + 1 < c) return *reinterpret_cast<const uint32_t*>(xr + ch) & 0x7FFF7FFFu;
  if (ch < c) return (uint32_t)(xr[ch] & 0x7FFFu) | 0xFFFF0000u;  // high half: no channel
  return 0xFFFFFFFFu;
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
  const int ch = c0 + 2 * lane;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r1 = min(rows, r0 + rows_per_block);
  const int colA = col_of(2 * lane), colB = col_of(2 * lane + 1);
  constexpr int kWaves = kPctThreads / 64;

  for (int64_t rb = r0 + wave; rb < r1; rb += (int64_t)kWaves * kPctUnroll) {
    uint32_t v[kPctUnroll];
#pragma unroll
    for (int u = 0; u < kPctUnroll; ++u) {
      const int64_t r = rb + (int64_t)u * kWaves;
      v[u] = r < r1 ? load_pair(x + r * ld, ch, c) : 0xFFFFFFFFu;
    }
#pragma unroll
    for (int u = 0; u < kPctUnroll; ++u) {
      const uint32_t ka = v[u] & 0xFFFFu, kb = v[u] >> 16;
      if (ka != 0xFFFFu) {
        const uint32_t bin = ka >> 7;
        atomicAdd(&hist[(bin >> 1) * kPctCh + colA], 1u << (16 * (bin & 1)));
      }
      if (kb != 0xFFFFu) {
        const uint32_t bin = kb >> 7;
        atomicAdd(&hist[(bin >> 1) * kPctCh + colB], 1u << (16 * (bin & 1)));
      }
    }
  }
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

// Between passes: find the coarse bins (and ranks inside them) of lo and hi.
__global__ void pct_select_kernel(const uint32_t* __restrict__ h1, int64_t rows, int c, double q,
                                  PctSel* __restrict__ sel) {
  const int ch = blockIdx.x * blockDim.x + threadIdx.x;
  if (ch >= c) return;
  int64_t lo, hi;
  double f;
  type7_ranks(rows, q, &lo, &hi, &f);
  const uint32_t* h = h1 + (int64_t)ch * 256;
  int64_t cum = 0;
  uint32_t blo = 255, bhi = 255, rlo = 0, rhi = 0;
  bool got_lo = false, got_hi = false;
  for (int b = 0; b < 256; ++b) {
    const int64_t nxt = cum + h[b];
    if (!got_lo && nxt > lo) {
      blo = b;
      rlo = (uint32_t)(lo - cum);
      got_lo = true;
    }
    if (!got_hi && nxt > hi) {
      bhi = b;
      rhi = (uint32_t)(hi - cum);
      got_hi = true;
    }
    cum = nxt;
  }
  sel[ch] = PctSel{blo, rlo, bhi, rhi};
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
  const int colA = col_of(2 * lane), colB = col_of(2 * lane + 1);
  // Bins to watch; 0xFFFF never matches a key >> 7 (at most 255).
  uint32_t loA = 0xFFFFu, hiA = 0xFFFFu, loB = 0xFFFFu, hiB = 0xFFFFu;
  if (ch < c) {
    loA = sel[ch].b_lo;
    hiA = sel[ch].b_hi != sel[ch].b_lo ? sel[ch].b_hi : 0xFFFFu;
  }
  if (ch + 1 < c) {
    loB = sel[ch + 1].b_lo;
    hiB = sel[ch + 1].b_hi != sel[ch + 1].b_lo ? sel[ch + 1].b_hi : 0xFFFFu;
  }
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r1 = min(rows, r0 + rows_per_block);
  constexpr int kWaves = kPctThreads / 64;

  for (int64_t rb = r0 + wave; rb < r1; rb += (int64_t)kWaves * kPctUnroll) {
    uint32_t v[kPctUnroll];
#pragma unroll
    for (int u = 0; u < kPctUnroll; ++u) {
      const int64_t r = rb + (int64_t)u * kWaves;
      v[u] = r < r1 ? load_pair(x + r * ld, ch, c) : 0xFFFFFFFFu;
    }
#pragma unroll
    for (int u = 0; u < kPctUnroll; ++u) {
      const uint32_t ka = v[u] & 0xFFFFu, kb = v[u] >> 16;
      if ((ka >> 7) == loA) atomicAdd(&hist[(ka & 127u) * kPctCh + colA], 1u);
      if ((ka >> 7) == hiA) atomicMin(&mins[colA], ka);
      if ((kb >> 7) == loB) atomicAdd(&hist[(kb & 127u) * kPctCh + colB], 1u);
      if ((kb >> 7) == hiB) atomicMin(&mins[colB], kb);
    }
  }
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
__global__ void pct_final_kernel(const uint32_t* __restrict__ h2, const PctSel* __restrict__ sel,
                                 const uint32_t* __restrict__ minkey, int64_t rows, int c,
                                 double q, float* __restrict__ stats) {
  const int ch = blockIdx.x * blockDim.x + threadIdx.x;
  if (ch >= c) return;
  int64_t lo, hi;
  double f;
  type7_ranks(rows, q, &lo, &hi, &f);
  const PctSel s = sel[ch];
  const uint32_t* h = h2 + (int64_t)ch * 128;
  uint32_t klo = 0, khi = 0;
  bool got_lo = false, got_hi = false;
  int64_t cum = 0;
  for (int b = 0; b < 128; ++b) {
    const int64_t nxt = cum + h[b];
    if (!got_lo && nxt > (int64_t)s.r_lo) {
      klo = (s.b_lo << 7) | (uint32_t)b;
      got_lo = true;
    }
    if (!got_hi && s.b_hi == s.b_lo && nxt > (int64_t)s.r_hi) {
      khi = (s.b_lo << 7) | (uint32_t)b;
      got_hi = true;
    }
    cum = nxt;
  }
  if (s.b_hi != s.b_lo) khi = minkey[ch];
  const double vlo = (double)__uint_as_float(klo << 16);
  const double vhi = (double)__uint_as_float(khi << 16);
  const double d = __dsub_rn(vhi, vlo);
  const double t = __dmul_rn(f, d);
  const double r = __dadd_rn(vlo, t);
  stats[ch] = __double2float_rn(r);
}

// Top-n mask: rank of ch = #{j : s[j] > s[ch] or (s[j] == s[ch] and j < ch)};
// protected iff rank < n_protect. Stats are staged through LDS in tiles.
__global__ __launch_bounds__(256) void topn_mask_kernel(const float* __restrict__ stats, int c,
                                                        int n_protect, uint8_t* __restrict__ mask) {
  __shared__ float tile[1024];
  const int ch = blockIdx.x * blockDim.x + threadIdx.x;
  const float mine = ch < c ? stats[ch] : 0.0f;
  int rank = 0;
  for (int t0 = 0; t0 < c; t0 += 1024) {
    const int n = min(1024, c - t0);
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += blockDim.x) tile[i] = stats[t0 + i];
    __syncthreads();
    for (int i = 0; i < n; ++i) {
      const float o = tile[i];
      const int j = t0 + i;
      rank += (o > mine) || (o == mine && j < ch);
    }
  }
  if (ch < c) mask[ch] = rank < n_protect ? 1 : 0;
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
  hipLaunchKernelGGL(pct_select_kernel, dim3((ci + 255) / 256), dim3(256), 0, stream, h1, rows,
                     ci, q, sel);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  for (int64_t s0 = 0; s0 < nsplit; s0 += 65535) {
    const int64_t ns = nsplit - s0 < 65535 ? nsplit - s0 : 65535;
    const int64_t rbase = s0 * rpb;
    hipLaunchKernelGGL(pct_pass2_kernel, dim3(cblocks, (unsigned)ns), dim3(kPctThreads), 0, stream,
                       x + rbase * ld, rows - rbase, ci, ld, (int)rpb, sel, h2, minkey);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  hipLaunchKernelGGL(pct_final_kernel, dim3((ci + 255) / 256), dim3(256), 0, stream, h2, sel,
                     minkey, rows, ci, q, stats);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(topn_mask_kernel, dim3((ci + 255) / 256), dim3(256), 0, stream, stats, ci,
                     (int)n_protect, mask);
  return hipGetLastError();
}
