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
// 4x4 blocks of v_mfma_f32_32x32x16_bf16), K step 64 (one HiF4 unit). Tiles
// go global -> LDS by direct-to-LDS DMA (global_load_lds_dwordx4, no VGPR
// staging), double-buffered: 2 stages x (A + B) x 256 rows x 128 B = 128 KiB.
// Each LDS row holds 8 16-byte chunks of K; chunk c of row r is stored in
// slot c ^ (r & 7), so the 16-byte fragment reads of 8 consecutive rows hit
// 8 different slots (all 32 banks once). The DMA writes a wave's 64 lanes to
// 1 KiB of consecutive LDS, so the swizzle is applied on the global side:
// the lane that lands in slot j of row r fetches chunk j ^ (r & 7).
#include "hif4_dev.h"

namespace hif4 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;

constexpr int kBM = 256, kBN = 256, kBK = 64;
constexpr int kRowBytes = kBK * 2;               // 128 B per LDS row
constexpr int kTileBytes = kBM * kRowBytes;      // one operand, one stage: 32 KiB
constexpr int kLdsBytes = 2 * 2 * kTileBytes;    // 2 stages x (A, B)

typedef __attribute__((address_space(3))) void lds_void_t;

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

  // Global load mapping: 8 lanes cover one 128-byte row chunk (64 bf16),
  // 32 rows per pass, 8 passes per operand.
  // DMA mapping: wave w fills rows 64w .. 64w+63 of each operand tile, 8 rows
  // (1 KiB) per instruction. Lane l lands in row 8i + l/8, slot l%8, and
  // fetches K chunk (l%8) ^ (l/8) of that row. Rows past M (N) are clamped to
  // the last valid row: they only feed outputs that are never stored.
  const int drow = wave * 64 + (lane >> 3);
  const int dchunk = (lane & 7) ^ (lane >> 3);
  uint32_t offA[8], offB[8];  // byte offsets of this lane's chunk at kt = 0
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    offA[i] = (uint32_t)(((size_t)min(m0 + drow + 8 * i, M - 1) * K + dchunk * 8) * 2);
    offB[i] = (uint32_t)(((size_t)min(n0 + drow + 8 * i, N - 1) * K + dchunk * 8) * 2);
  }
  const char* Ab = reinterpret_cast<const char*>(A);
  const char* Bb = reinterpret_cast<const char*>(B);
  auto dma = [&](int kt, int stage) {
    char* As = lds + stage * 2 * kTileBytes + wave * 64 * kRowBytes;
    char* Bs = As + kTileBytes;
    const size_t kofs = (size_t)kt * kRowBytes;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      __builtin_amdgcn_global_load_lds(Ab + kofs + offA[i], (lds_void_t*)(As + i * 1024), 16, 0, 0);
      __builtin_amdgcn_global_load_lds(Bb + kofs + offB[i], (lds_void_t*)(Bs + i * 1024), 16, 0, 0);
    }
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int KT = K / kBK;
  dma(0, 0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();

  // Fragment addressing: lane l supplies row (l % 32) and K values
  // 8*(l/32) .. +7 of each 16-wide K step, i.e. chunk 2s + l/32 (same
  // mapping for A and B, so the contraction pairs matching K indices
  // whatever the hardware's K order inside an instruction).
  const int frow = lane & 31;
  const int fsw = lane & 7;  // (row & 7) of every row this lane reads
  const int fhalf = lane >> 5;
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) dma(kt + 1, cur ^ 1);
    const char* As = lds + cur * 2 * kTileBytes + (wm * 128 + frow) * kRowBytes;
    const char* Bs = lds + cur * 2 * kTileBytes + kTileBytes + (wn * 128 + frow) * kRowBytes;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int slot = ((2 * s + fhalf) ^ fsw) * 16;
      bf16x8_t af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = *reinterpret_cast<const bf16x8_t*>(As + i * 32 * kRowBytes + slot);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bfr[j] = *reinterpret_cast<const bf16x8_t*>(Bs + j * 32 * kRowBytes + slot);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
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

// The DMA addresses are 32-bit byte offsets from the operand base, so each
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
