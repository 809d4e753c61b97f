// gemm.hip -- the W4A4 contraction Y = deq(Q(X)) deq(Q(W))^T on gfx950
// matrix cores.
//
// Layer form Y = X W^T: HiFloat4 calibration article (hwcomputing.csdn.net),
// section 2.3 "FlatQuant"; W4A4 fake quantization of the main linear layers:
// Tail-Aware HiFloat4 (arXiv 2605.26628 record, abstract).
//
// Operands are HiF4-decoded values in bf16. Every decoded HiF4 value
// k/4 * 2^(e2+e3) * v(c) has at most 6 significant bits (3 from k, 3 from the
// E6M2 mantissa) and an exponent in [-33, 35], so it is EXACT in bf16, every
// product is exact in fp32, and the only rounding is the fp32 accumulation
// inside the MFMA. The per-unit level-1 scales are therefore already inside
// the operands: no per-unit rescale is needed in the K loop.
//
// Tiling: 256x256 output tile per workgroup, 4 waves, v_mfma_f32_32x32x16_bf16,
// 256 fp32 accumulators per lane in AGPRs, one workgroup per CU. Two kernels:
// gemm_w4a4_rd_kernel (K a multiple of 256, 16-byte meta rows: every
// workload here) steps one HiF4 unit (64 K values) per barrier, with the
// waves splitting the tile by rows and each lane decoding its A fragments
// straight into registers; gemm_w4a4_kernel (any other K) steps half a unit
// with a 2x2 wave split and the activation decoded once into an LDS tile.
// Operands reach LDS by direct-to-LDS buffer DMA (buffer_load ... lds): no
// VGPR staging, rows past M / N read as zero through the buffer range check.
//
// LDS rows of bf16 operands are 64 B (32 K values) = 4 chunks of 16 B; chunk
// c of row r sits in slot c ^ ((r >> 2) & 3). gfx950's LDS serves a 16-byte
// read for 16 lanes per cycle across 64 banks; the fragment reads of 16
// consecutive rows then land in 16 distinct bank groups (rows r, r+4, r+8,
// r+12 share a bank base, and the XOR separates them). The DMA writes a
// wave's 64 lanes to 1 KiB of consecutive LDS, so the swizzle is applied on
// the global side: the lane that lands in slot j of row r fetches chunk
// j ^ ((r >> 2) & 3).
#include <type_traits>

#include "hif4_dev.h"

namespace hif4 {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2_t;
typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kBM = 256, kBN = 256;
constexpr int kBK = 32;                          // K per stage
constexpr int kRowBytes = kBK * 2;               // 64 B per LDS row
constexpr int kTileBytes = kBM * kRowBytes;      // one operand, one stage: 16 KiB
constexpr int kRsrcWord3 = 0x00020000;           // raw buffer, 32-bit data format (gfx9)

__device__ __forceinline__ void wait_vmcnt0() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier without the memory fence of __syncthreads (which would
// wait for every DMA stage in flight, i.e. vmcnt(0)). Each wave first waits
// for its own DMA of the stage it is about to read (s_waitcnt vmcnt); after
// the barrier every wave's part of that stage is in LDS. The asm statements
// keep the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// ---------------------------------------------------------------------------
// W4A4 GEMM with the activation operand in HiF4: Y = deq(A_codes) B^T.
//
// A arrives as HiF4 codes + meta (0.5625 B per element) through the DMA ring
// and is decoded ONCE per workgroup into a bf16 LDS tile; B (the weight,
// decoded to bf16 once per call) arrives as bf16. Fetching 4.5 KiB of A
// codes instead of 16 KiB of bf16 per 32-wide K step cuts the global->LDS
// traffic, which bounds a kernel fed with bf16 on both sides.
//
// Decode (HiF4 element = S1P2 nibble k/4 x 2^E x v(c), E = e2 + e3 in
// {0, 1, 2}, v(c) = 2^(e-31) (1 + m/4) with e = c >> 2, m = c & 3): write
// e = 2a + p. Then |x| = [k (1 + m/4) 2^(E + p - 33)] 2^(2a), and the bracket
// depends on m and s = E + p only (s in 0..3) and takes one of 16 x 8
// values, all exact in bf16 (k (4 + m) <= 49). A 16-entry LDS table holds,
// per (m, s), the low and high bytes of the bracket's bf16 for k = 0..7 as
// two byte planes. Multiplying by 2^(2a) adds a to the
// high byte of every non-zero value (the exponent's low bit stays put), so a
// level-3 quad decodes as: add a to the high plane (sparing k = 0), two
// v_perm_b32 plane lookups by the 4 magnitudes, OR the 4 signs into the high
// bytes, two v_perm_b32 to interleave into 4 bf16. The table is 256 B, one
// entry per 16-byte bank group: the 16 lanes served together either share an
// entry (broadcast) or hit distinct bank groups.
//
// Thread t decodes row t of the tile, whose codes its own wave fetched.
// LDS map (bytes):
//   [0, 64K)          B ring: 4 stages x 256 rows x 64 B (16-row swizzle)
//   [64K, 96K)        decoded A: 2 buffers x 256 rows x 64 B (same swizzle)
//   [96K, 144K)       A code ring: 3 slots x 2 units x 256 rows x 32 B
//   [144K, 152K)      A meta ring: 2 slots x 4 units x 256 rows x 4 B
//   [152K, +256)      decode table
// Code bytes are fetched two units (64 B) per row and meta four units (16 B)
// per row, so that one DMA instruction touches 16 (codes) or 64 (meta) rows
// instead of 32-64 rows for 32 or 4 bytes each: the vector L1 looks up far
// fewer lines per instruction.
//
// Step h covers K = 32h .. 32h+31 (half h&1 of unit h>>1) as two 16-wide
// MFMA K-chunks with one barrier between them, so that the fragments of the
// next chunk always load under the MFMAs of the current one (one wave per
// SIMD: nothing else would hide the LDS latency). The loop runs a multiple
// of 8 steps; halves past the end of K decode as zeros, and loads past the
// end read clamped or range-checked (zero) data into ring slots no one reads
// again, which keeps the loop free of branches; the vmcnt accounting is
// spelled out at the loop.
constexpr int kLdsB = 0;
constexpr int kLdsADec = 4 * kTileBytes;                     // 65536
constexpr int kLdsACodes = kLdsADec + 2 * kTileBytes;        // 98304
constexpr int kCodeSlotBytes = 256 * 64;                     // 16384: 2 units
constexpr int kLdsAMeta = kLdsACodes + 3 * kCodeSlotBytes;   // 147456
constexpr int kMetaSlotBytes = 256 * 16;                     // 4096: 4 units
constexpr int kLdsTable = kLdsAMeta + 2 * kMetaSlotBytes;    // 155648
constexpr int kLdsW4A4Bytes = kLdsTable + 16 * 16;           // 155904

// 16-byte LDS access through a native vector type. (Through the uint4
// struct it is split into four i32 accesses and re-merged, and the compiler
// then makes it wait for every LDS-DMA in flight, draining the ring.)
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 lds_u32x4(const char* p) {
  const u32x4_t q = *reinterpret_cast<const u32x4_t*>(p);
  return make_uint4(q.x, q.y, q.z, q.w);
}

// One level-3 quad: `nib` holds 4 nibbles in its bytes' low halves
// (magnitude bits 0-2, sign bit 3); t = table entry (lo plane k0-3, k4-7,
// hi plane k0-3, k4-7) with the exponent offset already in the hi plane.
__device__ __forceinline__ uint2 decode_quad(uint32_t nib, uint4 t) {
  const uint32_t sel = nib & 0x07070707u;
  const uint32_t lob = __builtin_amdgcn_perm(t.y, t.x, sel);  // low bytes of the 4 bf16
  uint32_t hib = __builtin_amdgcn_perm(t.w, t.z, sel);        // high bytes
  hib |= (nib << 4) & 0x80808080u;                             // signs
  return make_uint2(__builtin_amdgcn_perm(hib, lob, 0x05010400u),
                    __builtin_amdgcn_perm(hib, lob, 0x07030602u));
}

// This 32-wide schedule serves the shapes the register-decoded kernel below
// does not take (K not a multiple of 256, or meta rows not 16-byte aligned):
// a unit quad of meta is four 4-byte loads per row, one per unit.
//
// kResid: protected channels ([TA-method]: kept in high precision). Xr [M][KR]
// and Wr [N][KR] hold their bf16 values, zero-padded to KR (a multiple of
// 64); Y += Xr Wr^T is computed after the main loop, 64 columns at a time,
// in the B ring: the first 64 columns are fetched by the last four steps of
// the loop (whose B stages would lie past K), the rest after it.
template <bool kResid>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_w4a4_kernel(const uint16_t* __restrict__ Xr, const uint16_t* __restrict__ Wr, int KR,
                      const uint8_t* __restrict__ Ac, const uint32_t* __restrict__ Am,
                      const uint16_t* __restrict__ B, int M, int N, int K, void* __restrict__ Y,
                      int64_t ldy, int y_bf16, int tiles_m, int tiles_n) {
  __shared__ __attribute__((aligned(1024))) char lds[kLdsW4A4Bytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  // wave-uniform: the DMA destinations (M0) then come from scalar arithmetic
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // Tile order: consecutive workgroup ids go to different XCDs (round
  // robin), so give each XCD a contiguous run of tiles; within the order,
  // groups of 8 tile-rows are walked column by column so that the B tiles
  // in flight are shared by 8 neighbouring workgroups through L2.
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

  // ---- decode table: entry (m, s = E + p) at 16 (4m + s), built by threads 0..15
  if (tid < 16) {
    const int m = tid >> 2, sx = tid & 3;
    const float d = ldexpf(1.0f + 0.25f * (float)m, sx - 33);  // value of k = 1
    uint32_t lo0 = 0, lo1 = 0, hi0 = 0, hi1 = 0;
#pragma unroll
    for (int k = 1; k < 8; ++k) {
      const uint32_t bits = __float_as_uint((float)k * d) >> 16;  // exact bf16
      const uint32_t lb = bits & 0xFFu, hb = bits >> 8;
      if (k < 4) {
        lo0 |= lb << (8 * k);
        hi0 |= hb << (8 * k);
      } else {
        lo1 |= lb << (8 * (k - 4));
        hi1 |= hb << (8 * (k - 4));
      }
    }
    const u32x4_t v = {lo0, lo1, hi0, hi1};
    *reinterpret_cast<u32x4_t*>(lds + kLdsTable + 16 * tid) = v;
  }

  // ---- DMA setup
  const __amdgpu_buffer_rsrc_t rsAc =
      __builtin_amdgcn_make_buffer_rsrc((void*)Ac, (short)0, M * (K / 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rsAm =
      __builtin_amdgcn_make_buffer_rsrc((void*)Am, (short)0, M * (K / 64) * 4, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rsB =
      __builtin_amdgcn_make_buffer_rsrc((void*)B, (short)0, N * K * 2, kRsrcWord3);
  // B: wave w rows 64w.., 4 x 1 KiB per stage, chunk swizzle on the global side
  const int dchunk = (lane & 3) ^ ((lane >> 4) & 3);
  uint32_t voffB[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t r = (uint32_t)(wave * 64 + 16 * i + (lane >> 2));
    voffB[i] = ((uint32_t)(n0 + r) * (uint32_t)K + dchunk * 8) * 2;
  }
  // A: wave w fetches (and later decodes) rows 64w..64w+63, so its code
  // reads need no barrier, only its own vmcnt. Codes, unit pair P (64 B per
  // row), block i = rows 64w+16i..+15 (1 KiB): lane l -> row 64w+16i+(l>>2),
  // LDS chunk l&3 holding global chunk (l&3) ^ ((row>>2)&3), so that the
  // decode reads of 16 consecutive rows hit 16 distinct bank groups. Meta,
  // unit quad Q: four 4-byte loads per row, lane l -> row 64w+l. The K offsets ride in
  // the range-checked vector offset: past the end of a row they read the
  // next row (never decoded), past the end of the matrix they read zeros.
  const uint32_t KU = (uint32_t)(K / 64);  // units per row
  uint32_t voffAc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t r = (uint32_t)(wave * 64 + 16 * i + (lane >> 2));
    voffAc[i] = (uint32_t)(m0 + r) * (uint32_t)(K / 2) + (((lane & 3) ^ ((lane >> 4) & 3)) * 16);
  }
  const uint32_t voffAm = (uint32_t)(m0 + wave * 64 + lane) * KU * 4;

  const int KH = K / kBK;  // half-unit steps (even)
  auto dma_b_part = [&](int h, int i) {  // rows 16i.. of stage min(h, KH-1) into slot h & 3
    char* Bs = lds + kLdsB + (h & 3) * kTileBytes + wave * 64 * kRowBytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, (lds_void_t*)(Bs + i * 1024), 16, voffB[i],
                                             min(h, KH - 1) * kRowBytes, 0, 0);
  };
  auto dma_b = [&](int h) {
#pragma unroll
    for (int i = 0; i < 4; ++i) dma_b_part(h, i);
  };
  auto dma_codes = [&](int P, int i) {  // block i of unit pair P into slot P % 3
    char* slot = lds + kLdsACodes + (P % 3) * kCodeSlotBytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsAc, (lds_void_t*)(slot + wave * 4096 + i * 1024),
                                             16, voffAc[i] + (uint32_t)P * 64u, 0, 0, 0);
  };
  // meta slot layout: [wave][unit][64 rows]
  auto dma_meta = [&](int Q) {  // unit quad Q into slot Q % 2
    char* slot = lds + kLdsAMeta + (Q & 1) * kMetaSlotBytes + wave * 1024;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rsAm, (lds_void_t*)(slot + j * 256), 4,
                                               voffAm + (uint32_t)(4 * Q + j) * 4u, 0, 0, 0);
  };
  constexpr int kMetaLoads = 4;

  // Residual tiles, laid out like B stages (16-row swizzle) in B-ring slot
  // `slot`: part = 0/1 -> Wr columns 64c + 32part.., 2/3 -> Xr columns
  // 64c + 32(part-2).. . Rows past M / N read zeros (range check).
  auto dma_resid = [&](int c, int part, int i) {
    const bool is_x = part >= 2;
    const uint32_t row = (uint32_t)((is_x ? m0 : n0) + wave * 64 + 16 * i + (lane >> 2));
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(is_x ? (const void*)Xr : (const void*)Wr), (short)0, (is_x ? M : N) * KR * 2,
        kRsrcWord3);
    char* dst = lds + kLdsB + (part & 3) * kTileBytes + wave * 64 * kRowBytes + i * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (lds_void_t*)dst, 16, row * (uint32_t)(KR * 2) + (uint32_t)(dchunk * 16),
        (64 * c + 32 * (part & 1)) * 2, 0, 0);
  };

  // ---- decode state: thread tid decodes row tid of a half hn
  const int dsw = (tid >> 2) & 3;
  uint32_t dmw = 0;              // meta word of the row's unit
  uint4 dcw = make_uint4(0, 0, 0, 0);  // the row's 16 code bytes of half hn
  uint4 t8[8];                   // table entries of the 8 quads
  const char* dbase = lds;       // table entry (m, 0, p) of the unit
  uint32_t dd = 0, dd0 = 0;      // a in every byte; the same but not for k = 0
  uint2 dq0 = make_uint2(0, 0);  // decoded low quad of the current group
  auto dec_in = [&](int hn) {    // meta + codes of half hn (all zero past the end of K)
    const char* ms = lds + kLdsAMeta + ((hn >> 3) & 1) * kMetaSlotBytes;
    const char* cs = lds + kLdsACodes + ((hn >> 2) % 3) * kCodeSlotBytes;
    dmw = *reinterpret_cast<const uint32_t*>(ms + (tid >> 6) * 1024 + ((hn >> 1) & 3) * 256 +
                                             (tid & 63) * 4);
    const uint4 w = lds_u32x4(cs + tid * 64 + (((hn & 3) ^ dsw) * 16));
    const bool live = hn < KH;
    dcw = make_uint4(live ? w.x : 0u, live ? w.y : 0u, live ? w.z : 0u, live ? w.w : 0u);
  };
  auto dec_unit = [&]() {
    const uint32_t c = dmw & 255u;
    const uint32_t a = c >> 3, p = (c >> 2) & 1u, m = c & 3u;
    dbase = lds + kLdsTable + (m * 4u + p) * 16u;  // entry (m, p); + E selects s = E + p
    dd = __builtin_amdgcn_perm(a, a, 0u);
    dd0 = dd & 0xFFFFFF00u;
  };
  // table read of quad q (group g = 4 (hn & 1) + q / 2, half q & 1)
  auto dec_tab = [&](int hn_odd, int q) {
    const int g = hn_odd * 4 + (q >> 1);
    const uint32_t E = ((dmw >> (8 + g)) & 1u) + ((dmw >> (16 + 2 * g + (q & 1))) & 1u);
    t8[q] = lds_u32x4(dbase + 16 * E);
  };
  // decode quad q of half hn; the second quad of a group writes the group
  auto dec_quad = [&](int hn, int q) {
    const uint32_t words[4] = {dcw.x, dcw.y, dcw.z, dcw.w};
    uint4 tq = t8[q];
    tq.z += dd0;
    tq.w += dd;
    const uint2 v = decode_quad(words[q >> 1] >> (4 * (q & 1)), tq);
    if ((q & 1) == 0) {
      dq0 = v;
    } else {
      char* dst = lds + kLdsADec + (hn & 1) * kTileBytes + tid * kRowBytes;
      const u32x4_t w = {dq0.x, dq0.y, v.x, v.y};
      *reinterpret_cast<u32x4_t*>(dst + (((q >> 1) ^ dsw) * 16)) = w;
    }
  };

  // the same in two halves, to spread a quad over two MFMAs: (a) plane
  // lookups, (b) signs, interleave, write
  uint32_t qlo = 0, qhi = 0, qnib = 0;
  auto dec_quad_a = [&](int q) {
    const uint32_t words[4] = {dcw.x, dcw.y, dcw.z, dcw.w};
    qnib = words[q >> 1] >> (4 * (q & 1));
    uint4 tq = t8[q];
    tq.z += dd0;
    tq.w += dd;
    const uint32_t sel = qnib & 0x07070707u;
    qlo = __builtin_amdgcn_perm(tq.y, tq.x, sel);
    qhi = __builtin_amdgcn_perm(tq.w, tq.z, sel);
  };
  auto dec_quad_b = [&](int hn, int q) {
    const uint32_t hib = qhi | ((qnib << 4) & 0x80808080u);
    const uint2 v = make_uint2(__builtin_amdgcn_perm(hib, qlo, 0x05010400u),
                               __builtin_amdgcn_perm(hib, qlo, 0x07030602u));
    if ((q & 1) == 0) {
      dq0 = v;
    } else {
      char* dst = lds + kLdsADec + (hn & 1) * kTileBytes + tid * kRowBytes;
      const u32x4_t w = {dq0.x, dq0.y, v.x, v.y};
      *reinterpret_cast<u32x4_t*>(dst + (((q >> 1) ^ dsw) * 16)) = w;
    }
  };

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int frow = lane & 31;
  const int fsw = (frow >> 2) & 3;
  const int fhalf = lane >> 5;
  const int fslot[2] = {((0 + fhalf) ^ fsw) * 16, ((2 + fhalf) ^ fsw) * 16};
  // fragment f of K-chunk s of step h: f < 4 -> A rows wm*128 + 32f, else B rows wn*128 + 32(f-4)
  // (h only enters through h & 3: callers pass the step's phase, a constant)
  auto frag = [&](int h, int s, int f) {
    const char* p = f < 4
        ? lds + kLdsADec + (h & 1) * kTileBytes + (wm * 128 + f * 32 + frow) * kRowBytes
        : lds + kLdsB + (h & 3) * kTileBytes + (wn * 128 + (f - 4) * 32 + frow) * kRowBytes;
    return *reinterpret_cast<const bf16x8_t*>(p + fslot[s]);
  };
  bf16x8_t f0[8], f1[8];  // fragments of K-chunks 0 and 1 of the current step

  // ---- prologue: unit pairs 0..2, unit quads 0..1, B stages 0..3, all
  // landed; half 0 decoded, half 1 read and its first group decoded; chunk-0
  // fragments of step 0.
#pragma unroll
  for (int P = 0; P < 3; ++P)
#pragma unroll
    for (int i = 0; i < 4; ++i) dma_codes(P, i);
  dma_meta(0);
  dma_meta(1);
#pragma unroll
  for (int st = 0; st < 4; ++st) dma_b(st);
  wait_vmcnt0();
  __syncthreads();  // table + every wave's stage loads visible
  dec_in(0);
  dec_unit();
#pragma unroll
  for (int q = 0; q < 8; ++q) dec_tab(0, q);
#pragma unroll
  for (int q = 0; q < 8; ++q) dec_quad(0, q);
  dec_in(1);
  dec_unit();
#pragma unroll
  for (int q = 0; q < 8; ++q) dec_tab(1, q);
  dec_quad(1, 0);
  dec_quad(1, 1);
  __syncthreads();  // half 0 decoded by every wave
#pragma unroll
  for (int f = 0; f < 8; ++f) f0[f] = frag(0, 0, f);

  // ---- main loop. Step h: phase 1 = 16 MFMAs on K-chunk 0 (f0) while the
  // chunk-1 fragments load and quads 2..7 of half h+1 are decoded; then
  // vmcnt wait, lgkmcnt(0), barrier; phase 2 = 16 MFMAs on K-chunk 1 (f1)
  // while the chunk-0 fragments of step h+1 load, half h+2 is read and its
  // first group decoded, and the step's loads go out one per MFMA pair:
  // B stage h+4 (4 loads), block (h+2)&3 of unit pair (h+10)/4 (1 load) and,
  // when h = 6 mod 8, unit quad (h+10)/8 (1 load). Every load is needed at
  // least 3 barriers later (B stage h+1 at B_h; the pair holding half h+2 was
  // issued by step h-5, its quad by step h-8), so "vmcnt <= loads of steps
  // h-1 and h-2" at B_h is enough; that count depends on h mod 8 only.
  // Ring reuse: B stage h+4 overwrites stage h (last read before B_h); pair
  // P+3 overwrites pair P (last read at step 4P+1, first overwritten at step
  // 4P+2); quad Q+2 overwrites quad Q (last read at step 8Q+5, overwritten
  // at step 8Q+6).
  auto step = [&](int h, auto phase, auto last) {
    constexpr int kPh = decltype(phase)::value;  // h mod 8
    constexpr bool kPrefetchResid = kResid && decltype(last)::value && kPh >= 4;
    constexpr int kOdd = kPh & 1;
    constexpr int kLoads1 = 5 + (((kPh + 7) & 7) == 6 ? kMetaLoads : 0);  // loads of step h-1
    constexpr int kLoads2 = 5 + (((kPh + 6) & 7) == 6 ? kMetaLoads : 0);  // ... of step h-2
    // phase 1: one MFMA per slot, at most a few VALU ops between two MFMAs
    // (a longer run would leave the matrix pipe idle)
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      if (c < 8) f1[c] = frag(kPh, 1, c);
      if (c >= 2 && c < 14) {
        if (((c - 2) & 1) == 0) dec_quad_a(2 + ((c - 2) >> 1));
        else dec_quad_b(h + 1, 2 + ((c - 2) >> 1));
      }
      const int i = c >> 2, j = c & 3;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f0[i], f0[4 + j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    static_assert(kLoads1 + kLoads2 == 10 || kLoads1 + kLoads2 == 14, "vmcnt");
    if constexpr (kLoads1 + kLoads2 == 10) asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(14)" ::: "memory");
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    stage_barrier();
    dec_in(h + 2);
    __builtin_amdgcn_sched_barrier(0);
    // phase 2
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      if (c < 8 && (c & 1) == 0) {
        // past the loop's end: the first residual chunk instead of stage h + 4
        if constexpr (kPrefetchResid) dma_resid(0, kPh - 4, c >> 1);
        else dma_b_part(h + 4, c >> 1);
      }
      if (c == 8) dma_codes((h + 10) >> 2, (kPh + 2) & 3);
      if constexpr (kPh == 6) {
        if (c == 10) dma_meta((h + 10) >> 3);
      }
      if (c < 8) f0[c] = frag(kPh + 1, 0, c);
      if (c == 4) dec_unit();
      if (c >= 5 && c < 13) dec_tab(kOdd, c - 5);
      if (c >= 12) {
        if ((c & 1) == 0) dec_quad_a((c - 12) >> 1);
        else dec_quad_b(h + 2, (c - 12) >> 1);
      }
      const int i = c >> 2, j = c & 3;
      acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f1[i], f1[4 + j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  };
  const int KHp = (KH + 7) & ~7;
  using F = std::false_type;
  using T = std::true_type;
  auto eight = [&](int h, auto last) {
    step(h + 0, std::integral_constant<int, 0>{}, last);
    step(h + 1, std::integral_constant<int, 1>{}, last);
    step(h + 2, std::integral_constant<int, 2>{}, last);
    step(h + 3, std::integral_constant<int, 3>{}, last);
    step(h + 4, std::integral_constant<int, 4>{}, last);
    step(h + 5, std::integral_constant<int, 5>{}, last);
    step(h + 6, std::integral_constant<int, 6>{}, last);
    step(h + 7, std::integral_constant<int, 7>{}, last);
  };
  if constexpr (kResid) {
    for (int h = 0; h < KHp - 8; h += 8) eight(h, F{});
    eight(KHp - 8, T{});
  } else {
    for (int h = 0; h < KHp; h += 8) eight(h, F{});
  }
  wait_vmcnt0();  // no LDS-DMA may outlive the workgroup

  if constexpr (kResid) {
    // Y += Xr Wr^T, 64 columns per chunk: B-ring slots 0/1 = Wr halves,
    // 2/3 = Xr halves (chunk 0 already fetched by the last loop steps).
    const int chunks = KR / 64;
    for (int c = 0; c < chunks; ++c) {
      if (c > 0) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        stage_barrier();  // every wave is done with chunk c-1
#pragma unroll
        for (int part = 0; part < 4; ++part)
#pragma unroll
          for (int i = 0; i < 4; ++i) dma_resid(c, part, i);
        wait_vmcnt0();
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      stage_barrier();
#pragma unroll
      for (int r = 0; r < 2; ++r) {
#pragma unroll
        for (int sk = 0; sk < 2; ++sk) {
          bf16x8_t fa[4], fb[4];
#pragma unroll
          for (int f = 0; f < 4; ++f) {
            fa[f] = *reinterpret_cast<const bf16x8_t*>(
                lds + kLdsB + (2 + r) * kTileBytes + (wm * 128 + f * 32 + frow) * kRowBytes + fslot[sk]);
            fb[f] = *reinterpret_cast<const bf16x8_t*>(
                lds + kLdsB + r * kTileBytes + (wn * 128 + f * 32 + frow) * kRowBytes + fslot[sk]);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
              acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
      }
    }
  }

  // Epilogue. In the 32x32 MFMA output a lane holds one column and, per
  // group g of 4 accumulator registers, 4 consecutive rows. A 4x4 transpose
  // across each aligned quad of lanes (two DPP exchange steps) gives every
  // lane 4 consecutive columns of one row instead, stored as one 16-byte
  // (fp32) or 8-byte (bf16) write: a quarter of the store instructions of
  // element-wise stores, each row segment written whole. Rows are
  // 16-byte aligned when ldy % 4 == 0 (and Y is); otherwise, and for a
  // column group that crosses N, the values go out one by one.
  const int col_in = lane & 31, row_in = (lane >> 5) * 4, qt = lane & 3;
  const bool q_odd = (qt & 1) != 0, q_hi = (qt & 2) != 0;
  const bool vec_ok = (ldy & 3) == 0 && ((uintptr_t)Y & 15) == 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int colq = n0 + wn * 128 + j * 32 + (col_in & ~3);  // the quad's first column
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float v0 = acc[i][j][4 * g], v1 = acc[i][j][4 * g + 1];
        const float v2 = acc[i][j][4 * g + 2], v3 = acc[i][j][4 * g + 3];
        // step 1 (lanes t, t^1): c[t][k] = a[t^1][k^1] where bit 0 of k and t differ
        const float x0 = __uint_as_float(dpp<kDppQuadXor1>(__float_as_uint(v1)));
        const float x1 = __uint_as_float(dpp<kDppQuadXor1>(__float_as_uint(v0)));
        const float x2 = __uint_as_float(dpp<kDppQuadXor1>(__float_as_uint(v3)));
        const float x3 = __uint_as_float(dpp<kDppQuadXor1>(__float_as_uint(v2)));
        const float c0 = q_odd ? x0 : v0, c1 = q_odd ? v1 : x1;
        const float c2 = q_odd ? x2 : v2, c3 = q_odd ? v3 : x3;
        // step 2 (lanes t, t^2): d[t][k] = c[t^2][k^2] where bit 1 of k and t differ
        const float y0 = __uint_as_float(dpp<kDppQuadXor2>(__float_as_uint(c2)));
        const float y1 = __uint_as_float(dpp<kDppQuadXor2>(__float_as_uint(c3)));
        const float y2 = __uint_as_float(dpp<kDppQuadXor2>(__float_as_uint(c0)));
        const float y3 = __uint_as_float(dpp<kDppQuadXor2>(__float_as_uint(c1)));
        const float d0 = q_hi ? y0 : c0, d1 = q_hi ? y1 : c1;
        const float d2 = q_hi ? c2 : y2, d3 = q_hi ? c3 : y3;
        // lane t of the quad: row (group row + t), columns colq .. colq + 3
        const int row = m0 + wm * 128 + i * 32 + 8 * g + row_in + qt;
        if (row >= M || colq >= N) continue;
        const size_t off = (size_t)row * ldy + colq;
        if (vec_ok && colq + 4 <= N) {
          // non-temporal: Y is written once and read by no one in this
          // kernel, so it should not push the operand tiles out of L2/MALL
          if (y_bf16) {
            const uint32_t lo = f32_to_bf16_rne(d0) | (f32_to_bf16_rne(d1) << 16);
            const uint32_t hi = f32_to_bf16_rne(d2) | (f32_to_bf16_rne(d3) << 16);
            __builtin_nontemporal_store(
                u32x2_t{lo, hi}, reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(Y) + off));
          } else {
            __builtin_nontemporal_store(
                f32x4_t{d0, d1, d2, d3}, reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(Y) + off));
          }
        } else {
          const float d[4] = {d0, d1, d2, d3};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (colq + e >= N) break;
            if (y_bf16)
              reinterpret_cast<uint16_t*>(Y)[off + e] = (uint16_t)f32_to_bf16_rne(d[e]);
            else
              reinterpret_cast<float*>(Y)[off + e] = d[e];
          }
        }
      }
    }
  }
}

// bf16 operand rows of one HiF4 unit (64 K values) in LDS
constexpr int kRowBytes2 = 128;
constexpr int kTileBytes2 = 256 * kRowBytes2;              // 32 KiB

// ---------------------------------------------------------------------------
// The unit-step contraction with the activation decoded straight into the
// MFMA's operand registers (K % 256 == 0, 16-byte meta rows).
//
// The four waves split the 256x256 tile by rows: wave w owns rows
// 64w..64w+63 and all 256 columns (2 x 8 blocks of 32x32, the same 256 fp32
// accumulators per lane). No wave then needs another wave's A rows, so each
// lane decodes its own A fragments from HiF4 into the registers the MFMA
// reads: the decoded tile is neither written to nor read back from LDS, and
// the decode is not tied to the step barrier. B fragments are read from LDS
// as before (8 per K-chunk per wave instead of 4 A + 4 B).
//
// K order: in unit u, lane half h (lanes 32h..32h+31) supplies K values
// 64u + 32h + 8s .. +7 of MFMA K-chunk s, for both operands. Every
// assignment of K values to chunks gives the same sum up to the order of the
// fp32 roundings; this one makes a lane's codes for the four chunks of a
// unit one 16-byte run of its row (code word 4h + s = level-2 group 4h + s).
//
// Decode table: 512 entries, one per (a, m, s = p + E), the high plane
// already multiplied by 2^(2a), so a quad decodes without the two adds of
// the exponent (a = e >> 1, e = 2a + p the level-1 exponent). Entry
// (a, m, s) sits at 256a + 16((4m + s + a) & 15): rotating each a-block by a
// spreads the entries 16 rows of different a read together over bank
// groups. For a row and unit the lane precomputes, per quad it decodes, the
// byte 16((4m + p + E + a) & 15) (E = e2 + e3 of the quad); these 8 bytes sit
// in two words, and a quad's entry address is one v_perm of a byte of them
// and a. The table lives at LDS address 0 for that reason.
//
// LDS map (bytes):
//   [0, 8K)           decode table, entry (a, m, s) at 256a + 16((4m + s + a) & 15)
//   [8192, +64K)      B ring: 2 stages x 256 rows x 128 B, chunk c of row r in
//                     slot c ^ ((r >> 1) & 7)
//   [73728, +64K)     code ring: 2 groups of 4 units x 256 rows x 128 B, chunk
//                     c (= 2 x unit-in-group + half) of row r in slot
//                     c ^ ((r >> 1) & 7)
//   [139264, +16K)    meta ring: 2 groups of 8 units x 256 rows x 32 B, half c
//                     (units 4c..4c+3) of row r in slot c ^ ((r >> 3) & 1)
// Codes, meta and the table entries a lane reads are its own wave's rows,
// fetched by its own wave: those reads need the wave's own vmcnt only.
// Codes are fetched four units (one 128-byte line) per row, 8 rows per DMA
// instruction: the cost of a DMA instruction grows with the cache lines it
// touches, and one unit per row (32 rows of 32 B per instruction) made the
// code fetch cost as much as the eight times larger B fetch. Meta words
// likewise come 8 units (32 B) per row, 32 rows per instruction.
//
// Step u (one unit, 64 MFMAs per wave, one barrier):
//   L0  chunk 0 of unit u; B chunk-1 fragments; decode A(u) chunk 3;
//       table entries for A(u+1) chunk 0 (decode halves in the even MFMA
//       slots, table reads and the per-unit preparation pieces in the odd
//       ones, so that at most ~6 VALU ops sit between two MFMAs: more than
//       that leaves the matrix core idle)
//   L1  chunk 1; B chunk 2; decode A(u+1) chunk 0; entries for chunk 1
//   L2  chunk 2; B chunk 3; decode A(u+1) chunk 1; entries for chunk 2
//   s_waitcnt vmcnt(0 or 1) + lgkmcnt(0) + barrier
//   L3  chunk 3; B chunk-0 fragments of stage u+1; decode A(u+1) chunk 2;
//       entries for chunk 3; codes + meta of unit u+2 read and prepared;
//       DMA: B stage u+2, a quarter of code group (u+6)/4 (parts
//       2((u+2)%4), +1 of 8), (u % 4 == 2) half ((u+10)/4 % 2) of meta
//       group (u+10)/8
// A chunk s of unit u+1 overwrites chunk s of unit u once the MFMAs that
// read it have issued, so one set of A registers serves (32 VGPRs).
// Ring reuse: B slot u&1 held stage u (last read in L2 of step u, before the
// barrier); code group g = (u+6)/4 goes to slot g&1, which held group g-2,
// whose last unit 4g-5 was read in step 4g-7 (the group's parts go out in
// steps 4g-6 .. 4g-3, and unit 4g is first read in step 4g-2); meta group
// G goes out in steps 8G-10 and 8G-6 to slot G&1, which held group G-2,
// whose last unit 8G-9 was read in step 8G-11 (unit 8G is read in 8G-2).
// vmcnt: at the barrier of step u, B stage u+1 and the codes of unit u+2
// (all issued by step u-1) must be in; only a meta part issued in step u-1
// (u % 4 == 3, issued last) may still be in flight: vmcnt(1), else vmcnt(0).
// In the last steps the B DMA of stages past K reads clamped data into slots
// no one reads; with protected channels the two such DMAs of the last two
// steps fetch the first 64 residual columns of Wr and Xr into slots 0 and 1.
constexpr int kRdT = 0;
constexpr int kRdB = 8192;
constexpr int kRdC = kRdB + 2 * kTileBytes2;       // 73728
constexpr int kRdCodeGroup = 256 * 128;            // 4 units x 256 rows
constexpr int kRdM = kRdC + 2 * kRdCodeGroup;      // 139264
constexpr int kRdMetaGroup = 256 * 32;             // 8 units x 256 rows
constexpr int kRdBytes = kRdM + 2 * kRdMetaGroup;  // 155648

// bits 0..3 of x -> the low bit of bytes 0..3 (the partial products of the
// multiply land on disjoint bits, so nothing carries)
__device__ __forceinline__ uint32_t spread4(uint32_t x) {
  return ((x & 15u) * 0x204081u) & 0x01010101u;
}
// bit 0 of x -> bytes 0 and 1, bit 1 -> bytes 2 and 3
__device__ __forceinline__ uint32_t spread2x2(uint32_t x) {
  return ((x & 3u) * 0x808101u) & 0x01010101u;
}

__device__ __forceinline__ u32x4_t lds_v4(const char* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

// kNB: 32-column blocks per wave. 8 is the 256x256 tile; 4 is a 256x128 half
// tile, launched (two per tile) only for the tiles of a last partial round of
// workgroups, tile_base being the first of them in the tile order below: a
// half tile decodes as much as a whole one but does half the MFMAs, DMA and
// fragment reads, so the last round ends sooner than with whole tiles.
template <bool kResid, int kNB>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1)))
void gemm_w4a4_rd_kernel(const uint16_t* __restrict__ Xr, const uint16_t* __restrict__ Wr, int KR,
                         const uint8_t* __restrict__ Ac, const uint32_t* __restrict__ Am,
                         const uint16_t* __restrict__ B, int M, int N, int K,
                         void* __restrict__ Y, int64_t ldy, int y_bf16, int tiles_m, int tiles_n,
                         int tile_base) {
  static_assert(kNB == 8 || kNB == 4, "whole or half tiles");
  __shared__ __attribute__((aligned(1024))) char lds[kRdBytes];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int ntiles = tiles_m * tiles_n;
  int t = kNB == 8 ? (int)blockIdx.x : tile_base + (int)(blockIdx.x >> 1);
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
  const int m0 = tm * kBM, n0 = tn * kBN + (kNB == 8 ? 0 : (int)(blockIdx.x & 1) * 128);

  // decode table: entry (a, m, s = E + p) at 256a + 16((4m + s + a) & 15), its high
  // plane already multiplied by 2^(2a) (a added to every non-zero high byte);
  // rotating each a-block by a spreads rows of different a over bank groups
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int e = 2 * tid + h;  // a = e >> 4, 4m + s = e & 15
    const int a = e >> 4, m = (e >> 2) & 3, sx = e & 3;
    const float d = ldexpf(1.0f + 0.25f * (float)m, sx - 33);
    uint32_t lo0 = 0, lo1 = 0, hi0 = 0, hi1 = 0;
#pragma unroll
    for (int k = 1; k < 8; ++k) {
      const uint32_t bits = __float_as_uint((float)k * d) >> 16;
      const uint32_t lb = bits & 0xFFu, hb = (bits >> 8) + (uint32_t)a;
      if (k < 4) {
        lo0 |= lb << (8 * k);
        hi0 |= hb << (8 * k);
      } else {
        lo1 |= lb << (8 * (k - 4));
        hi1 |= hb << (8 * (k - 4));
      }
    }
    const u32x4_t v = {lo0, lo1, hi0, hi1};
    *reinterpret_cast<u32x4_t*>(lds + kRdT + 256 * a + 16 * (((e & 15) + a) & 15)) = v;
  }

  const __amdgpu_buffer_rsrc_t rsAc =
      __builtin_amdgcn_make_buffer_rsrc((void*)Ac, (short)0, M * (K / 2), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rsAm =
      __builtin_amdgcn_make_buffer_rsrc((void*)Am, (short)0, M * (K / 64) * 4, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rsB =
      __builtin_amdgcn_make_buffer_rsrc((void*)B, (short)0, N * K * 2, kRsrcWord3);
  // B: wave w rows 8 kNB w.. of the stage, kNB x 1 KiB (8 rows each); lane l ->
  // row 8i + (l >> 3), LDS slot l & 7 holding global chunk (l & 7) ^ ((row >> 1) & 7)
  uint32_t voffB[8];  // (arrays sized by kNB break the host-side instantiation)
#pragma unroll
  for (int i = 0; i < kNB; ++i) {
    const uint32_t r = (uint32_t)(wave * 8 * kNB + 8 * i + (lane >> 3));
    voffB[i] = ((uint32_t)(n0 + r) * (uint32_t)K + (((uint32_t)(lane & 7) ^ ((r >> 1) & 7u)) * 8u)) * 2u;
  }
  // codes: a group of 4 units of wave w's rows 64w.. is 8 x 1 KiB (8 rows of
  // 128 B each); part p: lane l -> row 8p + (l >> 3), slot l & 7 holding chunk
  // (l & 7) ^ ((row >> 1) & 7). The swizzle depends on p only through p & 1.
  uint32_t voffC[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const uint32_t r = (uint32_t)(wave * 64 + 8 * e + (lane >> 3));
    voffC[e] = (uint32_t)(m0 + r) * (uint32_t)(K / 2) + (((uint32_t)(lane & 7) ^ ((r >> 1) & 7u)) * 16u);
  }
  const uint32_t KU = (uint32_t)(K / 64);
  // meta: half p of a group of 8 units: lane l -> row 32p + (l >> 1) of
  // wave w's rows, slot l & 1 holding half (l & 1) ^ ((row >> 3) & 1)
  const uint32_t voffM = (uint32_t)(m0 + wave * 64 + (lane >> 1)) * KU * 4u +
                         (((uint32_t)(lane & 1) ^ ((uint32_t)(lane >> 4) & 1u)) * 16u);
  const int KUi = K / 64;

  auto dma_b = [&](int st, int i) {  // part i of B stage min(st, KU-1) into slot st & 1
    char* dst = lds + kRdB + (st & 1) * kTileBytes2 + wave * 8 * kNB * kRowBytes2 + i * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsB, (lds_void_t*)dst, 16, voffB[i],
                                             min(st, KUi - 1) * kRowBytes2, 0, 0);
  };
  // part p of code group g (units 4g..4g+3) into slot g & 1; the whole offset
  // rides in the range-checked vector offset (rows past M and bytes past the
  // end read zeros)
  auto dma_codes = [&](int g, int p) {
    char* dst = lds + kRdC + (g & 1) * kRdCodeGroup + wave * 8192 + p * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsAc, (lds_void_t*)dst, 16,
        voffC[p & 1] + (uint32_t)(p & ~1) * 8u * (uint32_t)(K / 2) + (uint32_t)g * 128u, 0, 0, 0);
  };
  // part p (rows 32p..) of meta group G (units 8G..8G+7) into slot G & 1
  auto dma_meta = [&](int G, int p) {
    char* dst = lds + kRdM + (G & 1) * kRdMetaGroup + wave * 2048 + p * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rsAm, (lds_void_t*)dst, 16, voffM + (uint32_t)p * 32u * KU * 4u + (uint32_t)G * 32u, 0, 0, 0);
  };
  // residual chunk c: Wr (is_x false) or Xr columns 64c.. into B slot `slot`,
  // with the stage swizzle; rows past M / N read zeros
  auto dma_resid = [&](int c, bool is_x, int i, int slot) {
    const uint32_t r = (uint32_t)(wave * 64 + 8 * i + (lane >> 3));
    const uint32_t row = (uint32_t)((is_x ? m0 : n0)) + r;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(is_x ? (const void*)Xr : (const void*)Wr), (short)0, (is_x ? M : N) * KR * 2,
        kRsrcWord3);
    char* dst = lds + kRdB + slot * kTileBytes2 + wave * 64 * kRowBytes2 + i * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        rs, (lds_void_t*)dst, 16,
        row * (uint32_t)(KR * 2) + (((uint32_t)(lane & 7) ^ ((r >> 1) & 7u)) * 16u),
        c * 128, 0, 0);
  };

  // ---- per-lane constants: row 64*wave + 32*rb + r32 of the tile, K half hh
  const uint32_t r32 = (uint32_t)(lane & 31), hh = (uint32_t)(lane >> 5);
  const uint32_t fsw = (r32 >> 1) & 7u;
  // fragment address of K-chunk s for lane row r32 (slot and column block
  // in the DS offset field)
  uint32_t fbo[4];
#pragma unroll
  for (int s = 0; s < 4; ++s)
    fbo[s] = (uint32_t)kRdB + r32 * kRowBytes2 + (((4u * hh + (uint32_t)s) ^ fsw) << 4);
  // code run of unit j (0..3) of a group for lane row r32, half hh
  uint32_t cb4[4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
    cb4[j] = (uint32_t)kRdC + ((uint32_t)wave * 64u + r32) * 128u +
             (((2u * (uint32_t)j + hh) ^ fsw) << 4);
  // meta word of lane row r32: half c of the row's group at slot c ^ msw
  const uint32_t msw = (r32 >> 3) & 1u;
  const uint32_t mb0 = (uint32_t)kRdM + ((uint32_t)wave * 64u + r32) * 32u + (msw << 4);
  const uint32_t mb1 = (uint32_t)kRdM + ((uint32_t)wave * 64u + r32) * 32u + ((msw ^ 1u) << 4);
  const uint32_t sh2 = 8u + 4u * hh, sh3 = 16u + 8u * hh;

  auto fragB = [&](int slot, int s, int cb) -> bf16x8_t {
    const uint32_t a = fbo[s] + (uint32_t)((slot & 1) * kTileBytes2 + cb * 32 * kRowBytes2);
    return *reinterpret_cast<const bf16x8_t*>(lds + a);
  };

  // ---- decode state, two sets (unit parity): meta word, code run, per-quad
  // table offsets, exponent add for the high plane
  uint32_t mw[2][2];
  u32x4_t cw[2][2];
  uint32_t ew[2][2][2], dd[2][2];  // per set and row: entry offsets of the 8 quads, a
  u32x4_t tq[8];
  u32x4_t fa[2][4];
  uint32_t qlo = 0, qhi = 0;

  // unit un's meta and codes into set S; j = un & 3 (a compile-time constant)
  auto dec_in = [&](int un, int S, int j) {
    const uint32_t msl = (((un >> 2) & 1) ? mb1 : mb0) + (uint32_t)((un >> 3) & 1) * (uint32_t)kRdMetaGroup;
    const uint32_t csl = cb4[j] + (uint32_t)((un >> 2) & 1) * (uint32_t)kRdCodeGroup;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      mw[S][rb] = *reinterpret_cast<const uint32_t*>(lds + msl + j * 4 + rb * 1024);
      cw[S][rb] = lds_v4(lds + csl + rb * 4096);
    }
  };
  // Per row and unit, in five pieces of 3..6 VALU ops (each has an MFMA slot
  // of its own): piece 0 puts 4m + p + a in every byte of both offset words
  // and keeps a (dd); pieces 1..4 add e2 and e3 of quads 0..3 and 4..7, and
  // pieces 2 and 4 turn each byte into 16 ((4m + p + E + a) & 15).
  auto prep = [&](int S, int rb, int piece) {
    const uint32_t w = mw[S][rb];
    if (piece == 0) {  // 4m + p + a in every byte of both offset words, a apart
      const uint32_t c = w & 255u;
      const uint32_t base = ((c & 3u) << 2) + ((c >> 2) & 1u) + (c >> 3);
      ew[S][rb][0] = ew[S][rb][1] = __builtin_amdgcn_perm(base, base, 0u);
      dd[S][rb] = c >> 3;
    } else if (piece == 1) {
      ew[S][rb][0] += spread2x2(w >> sh2);
    } else if (piece == 2) {
      ew[S][rb][0] = ((ew[S][rb][0] + spread4(w >> sh3)) & 0x0F0F0F0Fu) << 4;
    } else if (piece == 3) {
      ew[S][rb][1] += spread2x2(w >> (sh2 + 2u));
    } else if (piece == 4) {
      ew[S][rb][1] = ((ew[S][rb][1] + spread4(w >> (sh3 + 4u))) & 0x0F0F0F0Fu) << 4;
    }
  };
  // table entry of quad j (0..7) of row block rb, set S, into tq[slot]
  // entry address 256a + (byte j&3 of the offset word): one v_perm
  auto tab = [&](int S, int rb, int j, int slot) {
    const uint32_t off = __builtin_amdgcn_perm(dd[S][rb], ew[S][rb][j >> 2], 0x0C0C0400u | (uint32_t)(j & 3));
    tq[slot] = lds_v4(lds + kRdT + off);
  };
  // quad j (even: low nibbles of code word j/2, odd: high nibbles), two halves
  auto dq_a = [&](int S, int rb, int j, int slot) {
    const uint32_t word = cw[S][rb][j >> 1];
    const uint32_t sel = ((j & 1) ? (word >> 4) : word) & 0x07070707u;
    const u32x4_t tv = tq[slot];
    qlo = __builtin_amdgcn_perm(tv.y, tv.x, sel);
    qhi = __builtin_amdgcn_perm(tv.w, tv.z, sel);
  };
  auto dq_b = [&](int S, int rb, int j) {
    const uint32_t word = cw[S][rb][j >> 1];
    const uint32_t hib = qhi | (((j & 1) ? word : (word << 4)) & 0x80808080u);
    const uint32_t v0 = __builtin_amdgcn_perm(hib, qlo, 0x05010400u);
    const uint32_t v1 = __builtin_amdgcn_perm(hib, qlo, 0x07030602u);
    const int s = j >> 1;
    if (j & 1) {
      fa[rb][s].z = v0;
      fa[rb][s].w = v1;
    } else {
      fa[rb][s].x = v0;
      fa[rb][s].y = v1;
    }
  };
  // half i (0..7) of the decode of chunk s of set S: quad (rb, j) =
  // (i >> 2, 2s + ((i >> 1) & 1)), first or second half; entries in tq[tb..tb+3]
  auto dec_half = [&](int S, int s, int tb, int i) {
    const int rb = i >> 2, jj = (i >> 1) & 1;
    if ((i & 1) == 0) dq_a(S, rb, 2 * s + jj, tb + rb * 2 + jj);
    else dq_b(S, rb, 2 * s + jj);
  };
  // table entry i (0..3) for chunk s of set S into tq[tb + i]
  auto tab_chunk = [&](int S, int s, int tb, int i) {
    const int rb = i >> 1, jj = i & 1;
    tab(S, rb, 2 * s + jj, tb + i);
  };

  f32x16_t acc[2][8];  // the first kNB blocks used
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < kNB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int s = 0; s < 4; ++s) fa[rb][s] = u32x4_t{0u, 0u, 0u, 0u};

  bf16x8_t fb0[8], fb1[8];
  auto mfma = [&](int c, int s, const bf16x8_t* fb) {
    const int rb = c / kNB, cb = c % kNB;
    acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
        __builtin_bit_cast(bf16x8_t, fa[rb][s]), fb[cb], acc[rb][cb], 0, 0, 0);
  };

  // ---- prologue: meta group 0, code group 0, B stages 0 and 1, the first
  // half of meta group 1 (step -2's) and the parts 0..3 of code group 1 that
  // steps -2 and -1 would have issued (parts 4..7 follow in steps 0 and 1)
  dma_meta(0, 0);
  dma_meta(0, 1);
#pragma unroll
  for (int p = 0; p < 8; ++p) dma_codes(0, p);
#pragma unroll
  for (int i = 0; i < kNB; ++i) dma_b(0, i);
  dma_meta(1, 0);
#pragma unroll
  for (int i = 0; i < kNB; ++i) dma_b(1, i);
#pragma unroll
  for (int p = 0; p < 4; ++p) dma_codes(1, p);
  // meta group 0, code group 0 and B 0 in (5 + kNB loads issued after them)
  if constexpr (kNB == 8) asm volatile("s_waitcnt vmcnt(13)" ::: "memory");
  else asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  stage_barrier();  // table and every wave's B stage 0 visible
  dec_in(0, 0, 0);
  dec_in(1, 1, 1);
#pragma unroll
  for (int S = 0; S < 2; ++S)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      if (S == 0) {
#pragma unroll
        for (int piece = 0; piece < 5; ++piece) prep(S, rb, piece);
      } else {  // set 1 gets the pieces step -1 would have made (0, 1)
        prep(S, rb, 0);
        prep(S, rb, 1);
      }
    }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) tab_chunk(0, s, (s & 1) * 4, i);
    if (s < 3) {
#pragma unroll
      for (int i = 0; i < 8; ++i) dec_half(0, s, (s & 1) * 4, i);
    }
  }
#pragma unroll
  for (int c = 0; c < kNB; ++c) fb0[c] = fragB(0, 0, c);

  auto step = [&](int u, auto phase, auto tail) {
    constexpr int kPh = decltype(phase)::value;  // u mod 4
    constexpr bool kTail = decltype(tail)::value;  // the last four steps, residual ahead
    constexpr int Sc = kPh & 1, Sn = Sc ^ 1;     // sets of units u (and u+2), u+1
    if constexpr (kNB == 8) {
    // L0: chunk 0; B chunk 1 -> fb1; decode A(u) chunk 3 (tq 4..7); entries
    // of A(u+1) chunk 0 -> tq 0..3
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      if (c < 8) fb1[c] = fragB(kPh, 1, c);
      if ((c & 1) == 0) dec_half(Sc, 3, 4, c >> 1);
      if (c == 1 || c == 3) prep(Sn, c >> 1, 2);
      if (c >= 5 && c <= 11 && (c & 1)) tab_chunk(Sn, 0, 0, (c - 5) >> 1);
      mfma(c, 0, fb0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // L1: chunk 1; B chunk 2 -> fb0; decode A(u+1) chunk 0; entries of chunk 1
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      if (c < 8) fb0[c] = fragB(kPh, 2, c);
      if ((c & 1) == 0) dec_half(Sn, 0, 0, c >> 1);
      if ((c & 1) && c < 8) tab_chunk(Sn, 1, 4, c >> 1);
      if (c == 9 || c == 11) prep(Sn, (c - 9) >> 1, 3);
      if (c == 13 || c == 15) prep(Sn, (c - 13) >> 1, 4);
      mfma(c, 1, fb1);
      __builtin_amdgcn_sched_barrier(0);
    }
    // L2: chunk 2; B chunk 3 -> fb1; decode A(u+1) chunk 1; entries of chunk 2
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      if (c < 8) fb1[c] = fragB(kPh, 3, c);
      if ((c & 1) == 0) dec_half(Sn, 1, 4, c >> 1);
      if ((c & 1) && c < 8) tab_chunk(Sn, 2, 0, c >> 1);
      mfma(c, 2, fb0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kPh == 3) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    stage_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // L3: chunk 3; B chunk 0 of stage u+1 -> fb0; decode A(u+1) chunk 2;
    // entries of chunk 3; unit u+2 read and prepared; DMA codes u+3, meta,
    // B stage u+4 (or the first residual columns)
#pragma unroll
    for (int c = 0; c < 16; ++c) {
      if (c == 0) dec_in(u + 2, Sc, (kPh + 2) & 3);
      if (c < 8) fb0[c] = fragB((kPh + 1) & 3, 0, c);
      if ((c & 1) == 0) dec_half(Sn, 2, 0, c >> 1);
      if ((c & 1) && c < 8) tab_chunk(Sn, 3, 4, c >> 1);
      if (c == 9 || c == 11) prep(Sc, (c - 9) >> 1, 0);
      if (c == 13 || c == 15) prep(Sc, (c - 13) >> 1, 1);
      if (c >= 2 && c < 10) {
        if constexpr (kResid && kTail && kPh == 2) dma_resid(0, false, c - 2, 0);
        else if constexpr (kResid && kTail && kPh == 3) dma_resid(0, true, c - 2, 1);
        else dma_b(u + 2, c - 2);
      }
      if (c == 10) dma_codes((u + 6) >> 2, 2 * ((kPh + 2) & 3));
      if (c == 11) dma_codes((u + 6) >> 2, 2 * ((kPh + 2) & 3) + 1);
      if constexpr (kPh == 2) {
        if (c == 12) dma_meta((u + 10) >> 3, ((u + 10) >> 2) & 1);
      }
      mfma(c, 3, fb1);
      __builtin_amdgcn_sched_barrier(0);
    }
    } else {
    // Half tile: 8 MFMAs per K-chunk, one slot each, the same work per step
    // otherwise (the decode of 8 halves per chunk fills every slot).
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if (c < 4) fb1[c] = fragB(kPh, 1, c);
      dec_half(Sc, 3, 4, c);
      if (c < 2) prep(Sn, c, 2);
      if (c >= 4) tab_chunk(Sn, 0, 0, c - 4);
      mfma(c, 0, fb0);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if (c < 4) fb0[c] = fragB(kPh, 2, c);
      dec_half(Sn, 0, 0, c);
      if (c < 2) prep(Sn, c, 3);
      else if (c < 4) prep(Sn, c - 2, 4);
      if (c >= 4) tab_chunk(Sn, 1, 4, c - 4);
      mfma(c, 1, fb1);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if (c < 4) fb1[c] = fragB(kPh, 3, c);
      dec_half(Sn, 1, 4, c);
      if (c >= 4) tab_chunk(Sn, 2, 0, c - 4);
      mfma(c, 2, fb0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if constexpr (kPh == 3) asm volatile("s_waitcnt vmcnt(1)" ::: "memory");
    else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    stage_barrier();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      if (c == 0) dec_in(u + 2, Sc, (kPh + 2) & 3);
      if (c < 4) fb0[c] = fragB((kPh + 1) & 3, 0, c);
      dec_half(Sn, 2, 0, c);
      if (c >= 4) tab_chunk(Sn, 3, 4, c - 4);
      if (c == 4 || c == 5) prep(Sc, c - 4, 0);
      if (c == 6 || c == 7) prep(Sc, c - 6, 1);
      if constexpr (kResid && kTail && (kPh == 2 || kPh == 3)) dma_resid(0, kPh == 3, c, kPh - 2);
      else if (c < 4) dma_b(u + 2, c);
      if (c == 4) dma_codes((u + 6) >> 2, 2 * ((kPh + 2) & 3));
      if (c == 5) dma_codes((u + 6) >> 2, 2 * ((kPh + 2) & 3) + 1);
      if constexpr (kPh == 2) {
        if (c == 7) dma_meta((u + 10) >> 3, ((u + 10) >> 2) & 1);
      }
      mfma(c, 3, fb1);
      __builtin_amdgcn_sched_barrier(0);
    }
    }
  };
  // with protected channels the last four steps are a copy whose last two
  // B DMAs (stages past K) fetch residual chunk 0 instead
  const int KUmain = kResid ? KUi - 4 : KUi;
  for (int u = 0; u < KUmain; u += 4) {
    step(u + 0, std::integral_constant<int, 0>{}, std::false_type{});
    step(u + 1, std::integral_constant<int, 1>{}, std::false_type{});
    step(u + 2, std::integral_constant<int, 2>{}, std::false_type{});
    step(u + 3, std::integral_constant<int, 3>{}, std::false_type{});
  }
  if constexpr (kResid) {
    const int u = KUi - 4;
    step(u + 0, std::integral_constant<int, 0>{}, std::true_type{});
    step(u + 1, std::integral_constant<int, 1>{}, std::true_type{});
    step(u + 2, std::integral_constant<int, 2>{}, std::true_type{});
    step(u + 3, std::integral_constant<int, 3>{}, std::true_type{});
  }
  wait_vmcnt0();  // no LDS-DMA may outlive the workgroup (or overlap the residual's)

  if constexpr (kResid) {
    // Y += Xr Wr^T, 64 columns per chunk: Wr in B slot 0, Xr in B slot 1
    // (chunk 0 was fetched by the last steps of the loop)
    const int chunks = KR / 64;
    for (int c = 0; c < chunks; ++c) {
      if (c > 0) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        stage_barrier();  // every wave is done with the previous contents
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          dma_resid(c, false, i, 0);
          dma_resid(c, true, i, 1);
        }
        wait_vmcnt0();
      }
      stage_barrier();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8_t fr[8], xa[2];
#pragma unroll
        for (int cb = 0; cb < kNB; ++cb) fr[cb] = fragB(0, s, cb);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          xa[rb] = *reinterpret_cast<const bf16x8_t*>(
              lds + fbo[s] + kTileBytes2 + (wave * 64 + rb * 32) * kRowBytes2);
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int cb = 0; cb < kNB; ++cb)
            acc[rb][cb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xa[rb], fr[cb], acc[rb][cb], 0, 0, 0);
      }
    }
  }

  // Epilogue: as in the kernels above (4x4 lane-quad transpose, one 16- or
  // 8-byte store per lane and group), for the row blocks rb of this wave and
  // its kNB column blocks.
  const int col_in = lane & 31, row_in = (lane >> 5) * 4, qt = lane & 3;
  const bool q_odd = (qt & 1) != 0, q_hi = (qt & 2) != 0;
  const bool vec_ok = (ldy & 3) == 0 && ((uintptr_t)Y & 15) == 0;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
#pragma unroll
    for (int cb = 0; cb < kNB; ++cb) {
      const int colq = n0 + cb * 32 + (col_in & ~3);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const float v0 = acc[rb][cb][4 * g], v1 = acc[rb][cb][4 * g + 1];
        const float v2 = acc[rb][cb][4 * g + 2], v3 = acc[rb][cb][4 * g + 3];
        const float x0 = __uint_as_float(dpp<kDppQuadXor1>(__float_as_uint(v1)));
        const float x1 = __uint_as_float(dpp<kDppQuadXor1>(__float_as_uint(v0)));
        const float x2 = __uint_as_float(dpp<kDppQuadXor1>(__float_as_uint(v3)));
        const float x3 = __uint_as_float(dpp<kDppQuadXor1>(__float_as_uint(v2)));
        const float c0 = q_odd ? x0 : v0, c1 = q_odd ? v1 : x1;
        const float c2 = q_odd ? x2 : v2, c3 = q_odd ? v3 : x3;
        const float y0 = __uint_as_float(dpp<kDppQuadXor2>(__float_as_uint(c2)));
        const float y1 = __uint_as_float(dpp<kDppQuadXor2>(__float_as_uint(c3)));
        const float y2 = __uint_as_float(dpp<kDppQuadXor2>(__float_as_uint(c0)));
        const float y3 = __uint_as_float(dpp<kDppQuadXor2>(__float_as_uint(c1)));
        const float d0 = q_hi ? y0 : c0, d1 = q_hi ? y1 : c1;
        const float d2 = q_hi ? c2 : y2, d3 = q_hi ? c3 : y3;
        const int row = m0 + wave * 64 + rb * 32 + 8 * g + row_in + qt;
        if (row >= M || colq >= N) continue;
        const size_t off = (size_t)row * ldy + colq;
        if (vec_ok && colq + 4 <= N) {
          if (y_bf16) {
            const uint32_t lo = f32_to_bf16_rne(d0) | (f32_to_bf16_rne(d1) << 16);
            const uint32_t hi = f32_to_bf16_rne(d2) | (f32_to_bf16_rne(d3) << 16);
            __builtin_nontemporal_store(
                u32x2_t{lo, hi}, reinterpret_cast<u32x2_t*>(reinterpret_cast<uint16_t*>(Y) + off));
          } else {
            __builtin_nontemporal_store(
                f32x4_t{d0, d1, d2, d3}, reinterpret_cast<f32x4_t*>(reinterpret_cast<float*>(Y) + off));
          }
        } else {
          const float d[4] = {d0, d1, d2, d3};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (colq + e >= N) break;
            if (y_bf16)
              reinterpret_cast<uint16_t*>(Y)[off + e] = (uint16_t)f32_to_bf16_rne(d[e]);
            else
              reinterpret_cast<float*>(Y)[off + e] = d[e];
          }
        }
      }
    }
  }
}

// Protected-channel values for the residual: kept [rows][nk] (dense, any
// nk) -> out [rows][kr] zero-padded, kr a multiple of 64, so that the
// residual tiles load like B stages (16-byte rows chunks, 16-byte aligned).
__global__ __launch_bounds__(256) void pack_kept_kernel(const uint16_t* __restrict__ kept,
                                                        int64_t rows, int nk, int kr,
                                                        uint16_t* __restrict__ out) {
  const int64_t groups = rows * (kr / 8);  // 8 outputs (16 bytes) per item
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < groups; g += stride) {
    const int64_t r = g / (kr / 8);
    const int c0 = (int)(g - r * (kr / 8)) * 8;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int ca = c0 + 2 * e, cb = ca + 1;
      const uint32_t lo = ca < nk ? kept[r * nk + ca] : 0u;
      const uint32_t hi = cb < nk ? kept[r * nk + cb] : 0u;
      w[e] = lo | (hi << 16);
    }
    *reinterpret_cast<uint4*>(out + r * kr + c0) = make_uint4(w[0], w[1], w[2], w[3]);
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
// A in HiF4 codes (+ meta), B bf16. Same row-block split as the bf16 kernel;
// the code/meta offsets stay far inside 32 bits whenever the bf16 B offsets do.
hipError_t hif4_launch_pack_kept(const uint16_t* kept, int64_t rows, int64_t nk, int64_t kr,
                                 uint16_t* out, hipStream_t stream) {
  if (rows == 0 || kr == 0) return hipSuccess;
  const int64_t items = rows * (kr / 8);
  const int64_t blocks = (items + 255) / 256;
  hipLaunchKernelGGL(pack_kept_kernel, dim3((unsigned)(blocks < 65536 ? blocks : 65536)), dim3(256),
                     0, stream, kept, rows, (int)nk, (int)kr, out);
  return hipGetLastError();
}

// A in HiF4 codes (+ meta), B bf16, optional residual xr/wr [.][kr] (kr = 0:
// none). Same row-block split as before: all 32-bit offsets stay in range.
template <bool kResid>
static void launch_w4a4(dim3 grid, hipStream_t stream, const uint16_t* xr, const uint16_t* wr,
                        int kr, const uint8_t* ac, const uint32_t* am, const uint16_t* b, int mc,
                        int nc, int k, void* ys, int64_t ldy, int y_bf16, int tiles_m,
                        int tiles_n) {
  hipLaunchKernelGGL((gemm_w4a4_kernel<kResid>), grid, dim3(256), 0, stream, xr, wr, kr,
                     ac, am, b, mc, nc, k, ys, ldy, y_bf16, tiles_m, tiles_n);
}

// The register-decoded kernel over tiles_m x tiles_n tiles. When at most two
// whole rounds of tiles (one workgroup per CU) leave a last partial round of
// at most half the CUs, those tiles go to a second launch as half tiles, two
// workgroups each, which end that round sooner; the split follows the
// kernel's own tile order, so the two launches cover every tile exactly once.
// After more rounds the CUs finish at times spread widely enough that the
// leftover tiles of a single launch, started by the first CUs to free up,
// end sooner than a second launch could start (measured: 8192 x 5120 x 5120,
// 640 tiles, 0.377 -> 0.359 ms split; FFN-up, 12,150 tiles, 6.10 -> 6.17 ms).
template <bool kResid>
static void launch_rd(int tiles_m, int tiles_n, hipStream_t stream, const uint16_t* xr,
                      const uint16_t* wr, int kr, const uint8_t* ac, const uint32_t* am,
                      const uint16_t* b, int mc, int nc, int k, void* ys, int64_t ldy, int y_bf16) {
  static int cu_count[64];  // per device, queried once (0: not yet, or unknown)
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
    cus = cu_count[dev];
    if (cus == 0 &&
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess)
      cu_count[dev] = cus;
  }
  if (cus < 0) cus = 0;
  const int ntiles = tiles_m * tiles_n;
  const int tail = cus > 0 ? ntiles % cus : 0;
  const bool split = tail != 0 && 2 * tail <= cus && ntiles - tail <= 2 * cus;
  const int whole = split ? ntiles - tail : ntiles;
  if (whole > 0)
    hipLaunchKernelGGL((gemm_w4a4_rd_kernel<kResid, 8>), dim3((unsigned)whole), dim3(256), 0,
                       stream, xr, wr, kr, ac, am, b, mc, nc, k, ys, ldy, y_bf16, tiles_m, tiles_n,
                       0);
  if (split)
    hipLaunchKernelGGL((gemm_w4a4_rd_kernel<kResid, 4>), dim3((unsigned)(2 * tail)), dim3(256), 0,
                       stream, xr, wr, kr, ac, am, b, mc, nc, k, ys, ldy, y_bf16, tiles_m, tiles_n,
                       whole);
}

hipError_t hif4_launch_gemm_w4a4(const uint8_t* a_codes, const uint32_t* a_meta,
                                 const uint16_t* b, int64_t m, int64_t n, int64_t k, void* y,
                                 int y_bf16, const uint16_t* xr, const uint16_t* wr, int64_t kr,
                                 hipStream_t stream) {
  if (m == 0 || n == 0) return hipSuccess;
  if (k == 0) return hipErrorInvalidValue;
  const int64_t max_rows = (((int64_t)1 << 31) / (2 * (k + kr))) / kBM * kBM;
  if (max_rows < kBM) return hipErrorInvalidValue;
  const size_t ysz = y_bf16 ? 2 : 4;
  for (int64_t m0 = 0; m0 < m; m0 += max_rows) {
    const int64_t mc = m - m0 < max_rows ? m - m0 : max_rows;
    for (int64_t n0 = 0; n0 < n; n0 += max_rows) {
      const int64_t nc = n - n0 < max_rows ? n - n0 : max_rows;
      const int tiles_m = (int)((mc + kBM - 1) / kBM), tiles_n = (int)((nc + kBN - 1) / kBN);
      const dim3 grid((unsigned)(tiles_m * tiles_n));
      void* ys = (char*)y + ((size_t)m0 * n + n0) * ysz;
      const uint32_t* am = a_meta + m0 * (k / 64);
      const uint8_t* ac = a_codes + m0 * (k / 2);
      const uint16_t* bs = b + n0 * k;
      const uint16_t* xs = kr ? xr + m0 * kr : nullptr;
      const uint16_t* ws = kr ? wr + n0 * kr : nullptr;
      const bool meta16 = (k / 64) % 4 == 0 && ((uintptr_t)am & 15) == 0;
      // K % 256 == 0 with 16-byte meta rows: the register-decoded unit-step kernel; other
      // shapes take the 32-wide schedule
      if (meta16 && kr)
        launch_rd<true>(tiles_m, tiles_n, stream, xs, ws, (int)kr, ac, am, bs, (int)mc, (int)nc,
                        (int)k, ys, (int64_t)n, y_bf16);
      else if (meta16)
        launch_rd<false>(tiles_m, tiles_n, stream, xs, ws, 0, ac, am, bs, (int)mc, (int)nc, (int)k,
                         ys, (int64_t)n, y_bf16);
      else if (kr)
        launch_w4a4<true>(grid, stream, xs, ws, (int)kr, ac, am, bs, (int)mc, (int)nc,
                                 (int)k, ys, n, y_bf16, tiles_m, tiles_n);
      else
        launch_w4a4<false>(grid, stream, xs, ws, 0, ac, am, bs, (int)mc, (int)nc, (int)k,
                                  ys, n, y_bf16, tiles_m, tiles_n);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return hipSuccess;
}
