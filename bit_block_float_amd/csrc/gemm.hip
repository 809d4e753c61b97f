// gemm.hip -- the W4A4 contraction Y = A B^T on gfx950 matrix cores.
//
// Layer form Y = X W^T: HiFloat4 calibration article (hwcomputing.csdn.net),
// section 2.3 "FlatQuant"; W4A4 fake quantization of the main linear layers:
// Tail-Aware HiFloat4 (arXiv 2605.26628 record, abstract).
//
// Operands are the HiF4-decoded values of X and W in bf16. Every decoded HiF4
// value k/4 * 2^(e2+e3) * v(c) has at most 6 significant bits (3 from k, 3 from
// the E6M2 mantissa) and an exponent in [-33, 35], so it is EXACT in bf16, every
// product is exact in fp32, and the only rounding is the fp32 accumulation
// inside the MFMA. The per-unit level-1 scales are therefore already inside
// the operands: no per-unit rescale is needed in the K loop.
//
// Tiling: 256x256 output tile per workgroup (4 waves, 2x2, each 128x128 =
// 4x4 blocks of v_mfma_f32_32x32x16_bf16, 256 fp32 accumulators per lane in
// AGPRs). K advances 32 per stage through a 4-stage LDS ring (4 x (A + B) x
// 256 rows x 64 B = 128 KiB of the 160 KiB), filled by direct-to-LDS buffer
// DMA (buffer_load_dwordx4 ... lds): no VGPR staging, the K offset rides in
// an SGPR, rows past M / N read as zero through the buffer range check.
// Stages are issued three ahead of the one being consumed; one barrier per
// stage.
//
// LDS layout: a row is 4 chunks of 16 B (8 bf16 of K). Chunk c of row r is
// stored in slot c ^ ((r >> 2) & 3). gfx950's LDS serves a 16-byte read for
// 16 lanes per cycle across 64 banks; the fragment reads of 16 consecutive
// rows then land in 16 distinct bank groups (rows r, r+4, r+8, r+12 share a
// bank base, and the XOR separates them). The DMA writes a wave's 64 lanes to
// 1 KiB of consecutive LDS, so the swizzle is applied on the global side: the
// lane that lands in slot j of row r fetches chunk j ^ ((r >> 2) & 3).
#include "hif4_dev.h"

namespace hif4 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kBM = 256, kBN = 256;
constexpr int kBK = 32;                          // K per stage
constexpr int kStages = 4;
constexpr int kRowBytes = kBK * 2;               // 64 B per LDS row
constexpr int kTileBytes = kBM * kRowBytes;      // one operand, one stage: 16 KiB
constexpr int kStageBytes = 2 * kTileBytes;      // A + B
constexpr int kLdsBytes = kStages * kStageBytes; // 128 KiB
constexpr int kRsrcWord3 = 0x00020000;           // raw buffer, 32-bit data format (gfx9)

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  if constexpr (N == 16) asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
  else if constexpr (N == 8) asm volatile("s_waitcnt vmcnt(8)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every DMA stage in flight, i.e. vmcnt(0)). Each wave first waits
// for its own DMA of the stage it is about to read (wait_vmcnt); after the
// barrier every wave's part of that stage is in LDS. The asm statements keep
// the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_bf16_nt_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B, int M,
                         int N, int K, void* __restrict__ Y, int64_t ldy, int y_bf16, int tiles_m,
                         int tiles_n) {
  __shared__ __attribute__((aligned(1024))) char lds[kLdsBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // XCD-aware tile order: consecutive workgroup ids land on different XCDs
  // (round-robin over 8), so give each XCD a contiguous run of tiles, and
  // walk that run column-major in groups of 8 tile-rows so that tiles in
  // flight on one XCD share A and B panels in its L2.
  const int ntiles = tiles_m * tiles_n;
  int t = blockIdx.x;
  {
    const int per_xcd = ntiles / 8;
    if (t < per_xcd * 8) t = (t & 7) * per_xcd + (t >> 3);
    const int group = 8;
    const int tiles_per_group = group * tiles_n;
    const int gidx = t / tiles_per_group;
    const int first_m = gidx * group;
    const int gsize = min(tiles_m - first_m, group);
    const int in = t - gidx * tiles_per_group;
    t = (first_m + in % gsize) * tiles_n + in / gsize;
  }
  const int tm = t / tiles_n, tn = t - (t / tiles_n) * tiles_n;
  const int m0 = tm * kBM, n0 = tn * kBN;

  // DMA mapping: per stage and operand, wave w fills rows 64w .. 64w+63 with
  // 4 instructions of 1 KiB (16 rows x 64 B). Lane l lands in row 16i + l/4,
  // slot l%4, and fetches chunk (l%4) ^ ((row >> 2) & 3) = (l%4) ^ ((l>>4)&3).
  const __amdgpu_buffer_rsrc_t rsA =
      __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, M * K * 2, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rsB =
      __builtin_amdgcn_make_buffer_rsrc((void*)B, (short)0, N * K * 2, kRsrcWord3);
  const int dchunk = (lane & 3) ^ ((lane >> 4) & 3);
  uint32_t voffA[4], voffB[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t r = (uint32_t)(wave * 64 + 16 * i + (lane >> 2));
    voffA[i] = ((uint32_t)(m0 + r) * (uint32_t)K + dchunk * 8) * 2;
    voffB[i] = ((uint32_t)(n0 + r) * (uint32_t)K + dchunk * 8) * 2;
  }
  // DMA of quarter i of a stage (one A and one B instruction).
  auto dma_i = [&](int stage, int kt, int i) {
    char* As = lds + stage * kStageBytes + wave * 64 * kRowBytes;
    char* Bs = As + kTileBytes;
    const int soff = kt * kRowBytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsA, (lds_void_t*)(As + i * 1024), 16, voffA[i], soff,
                                             0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, (lds_void_t*)(Bs + i * 1024), 16, voffB[i], soff,
                                             0, 0);
  };
  auto dma = [&](int stage, int kt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) dma_i(stage, kt, i);
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  // Fragment addressing: lane l supplies row (l % 32) and K values
  // 8*(l/32) .. +7 of each 16-wide K step s, i.e. chunk 2s + l/32 (same
  // mapping for A and B, so the contraction pairs matching K indices
  // whatever the hardware's K order inside an instruction).
  const int frow = lane & 31;
  const int fsw = (frow >> 2) & 3;
  const int fhalf = lane >> 5;
  const int slot0 = ((0 + fhalf) ^ fsw) * 16;
  const int slot1 = ((2 + fhalf) ^ fsw) * 16;

  const int KT = K / kBK;
  dma(0, 0);
  if (KT > 1) dma(1, 1);
  if (KT > 2) dma(2, 2);
  for (int kt = 0; kt < KT; ++kt) {
    const int rem = KT - 1 - kt;  // stages issued after this one (at most 2)
    if (rem >= 2) wait_vmcnt<16>();
    else if (rem == 1) wait_vmcnt<8>();
    else wait_vmcnt<0>();
    stage_barrier();
    // The DMA of stage kt+3 is spread over this stage's MFMAs (a burst of
    // eight DMA instructions ahead of them stalls the wave's issue).
    const bool prefetch = kt + 3 < KT;
    const char* st = lds + (kt & 3) * kStageBytes;
    const char* As = st + (wm * 128 + frow) * kRowBytes;
    const char* Bs = st + kTileBytes + (wn * 128 + frow) * kRowBytes;
    // All 16 fragments of the stage go into distinct registers first, so the
    // LDS latency is exposed once per stage, not once per 4 MFMAs.
    bf16x8_t af[2][4], bfr[2][4];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int slot = s ? slot1 : slot0;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[s][i] = *reinterpret_cast<const bf16x8_t*>(As + i * 32 * kRowBytes + slot);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[s][j] = *reinterpret_cast<const bf16x8_t*>(Bs + j * 32 * kRowBytes + slot);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (s == 0 && prefetch) dma_i((kt + 3) & 3, kt + 3, i);
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[s][i], bfr[s][j], acc[i][j], 0, 0, 0);
      }
    __builtin_amdgcn_sched_barrier(0);
  }

  // Epilogue. 32x32 block output layout: lane l holds column l % 32 and,
  // in register r, row 8*(r/4) + 4*(l/32) + r%4.
  const int col_in = lane & 31, row_in = (lane >> 5) * 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int col = n0 + wn * 128 + j * 32 + col_in;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + row_in + (r & 3);
        if (row < M) {
          if (y_bf16)
            reinterpret_cast<uint16_t*>(Y)[(size_t)row * ldy + col] =
                (uint16_t)f32_to_bf16_rne(acc[i][j][r]);
          else
            reinterpret_cast<float*>(Y)[(size_t)row * ldy + col] = acc[i][j][r];
        }
      }
    }
  }
}

// Y = 0 for an empty contraction (k == 0). A kernel rather than a memset so
// the call stays capturable in a graph. Works in 16-bit words (bf16 or half
// an fp32).
__global__ void zero_fill_kernel(uint16_t* __restrict__ p, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

}  // namespace hif4

using namespace hif4;

hipError_t hif4_launch_zero(void* p, size_t bytes, hipStream_t stream) {
  const size_t n = bytes / 2;
  if (n == 0) return hipSuccess;
  const size_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(zero_fill_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256),
                     0, stream, (uint16_t*)p, n);
  return hipGetLastError();
}

// The DMA addresses are 32-bit byte offsets inside a buffer resource, so each
// launch covers at most 2^31 bytes of A rows and of B rows; larger problems
// are split into row blocks of A and of B (Y sub-blocks with stride n).
hipError_t hif4_launch_gemm_bf16_nt(const uint16_t* a, const uint16_t* b, int64_t m, int64_t n,
                                    int64_t k, void* y, int y_bf16, hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  if (k == 0) return hipErrorInvalidValue;  // handled by the caller (zero fill)
  const int64_t max_rows = (((int64_t)1 << 31) / (2 * k)) / kBM * kBM;
  if (max_rows < kBM) return hipErrorInvalidValue;
  const size_t ysz = y_bf16 ? 2 : 4;
  for (int64_t m0 = 0; m0 < m; m0 += max_rows) {
    const int64_t mc = m - m0 < max_rows ? m - m0 : max_rows;
    for (int64_t n0 = 0; n0 < n; n0 += max_rows) {
      const int64_t nc = n - n0 < max_rows ? n - n0 : max_rows;
      const int tiles_m = (int)((mc + kBM - 1) / kBM), tiles_n = (int)((nc + kBN - 1) / kBN);
      void* ys = (char*)y + ((size_t)m0 * n + n0) * ysz;
      hipLaunchKernelGGL(gemm_bf16_nt_kernel, dim3((unsigned)(tiles_m * tiles_n)), dim3(256), 0,
                         stream, a + m0 * k, b + n0 * k, (int)mc, (int)nc, (int)k, ys, n, y_bf16,
                         tiles_m, tiles_n);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}
