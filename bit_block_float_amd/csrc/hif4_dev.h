// hif4_dev.h -- device helpers and internal launcher declarations of libhif4.
// gfx950 (CDNA4) only: 64-lane wavefronts, DPP cross-lane moves.
//
// Format: HiFloat4 calibration article (hwcomputing.csdn.net), section
// "一：HiFloat4 (HiF4) 格式" -- 64-element units, one E6M2 level-1 scale, E1
// level-2 (per 8) and level-3 (per 4) exponents, S1P2 elements. The readings
// of what the article leaves open (E6M2 bias, E1 direction, nibble layout,
// scale rule, rounding) are stated in include/hif4.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hif4 {

constexpr int kUnit = 64;  // elements per HiF4 unit

// E6M2 level-1 value v(c) = 2^((c>>2) - 31) * (1 + (c&3)/4), built as fp32
// bits: biased exponent (c>>2) - 31 + 127, two mantissa bits on top.
__device__ __forceinline__ float e6m2_f32(uint32_t c) {
  return __uint_as_float((((c >> 2) + 96u) << 23) | ((c & 3u) << 21));
}

// Smallest level-1 code c with 7 v(c) >= a (a >= 0, exact bf16 value), 255 if
// none. An estimate from a/7 is off by at most one code; two exact
// comparisons settle it (7 v(c) has at most 6 significant bits: exact in
// fp32). Branch-free.
__device__ __forceinline__ uint32_t level1_code(float a) {
  const float r = a * (1.0f / 7.0f);
  const uint32_t b = __float_as_uint(r);
  const int e = (int)(b >> 23) - 96;
  const uint32_t m = b & 0x7FFFFFu;
  int c = 4 * e + (int)(m >> 21) + ((m & 0x1FFFFFu) != 0u);
  c = c < 0 ? 0 : (c > 255 ? 255 : c);
  // bitwise & (not &&): no short-circuit, no branch; e6m2_f32 of an
  // out-of-range code is a harmless finite float that the mask discards
  const uint32_t down = (uint32_t)(c > 0) & (uint32_t)(7.0f * e6m2_f32((uint32_t)(c - 1)) >= a);
  const uint32_t up = (uint32_t)(c < 255) & (uint32_t)(7.0f * e6m2_f32((uint32_t)c) < a);
  return (uint32_t)c - down + up;
}

// 16 / (4 + m) as an unevaluated fp32 sum hi + lo (hi = RN(16/(4+m)),
// lo = RN(16/(4+m) - hi)): the HiF4 element quotient 4|x| / D is
// t = fma(|x|, hi 2^p, |x| lo 2^p) with D's power of two folded into p. For
// every bf16 |x| this t is within half an fp32 ulp of the real quotient, so
// exact half-integers (the ties) come out exact and rintf() rounds to nearest
// even exactly as on the reals (checked exhaustively for all four mantissas).
// 4-way select by bit masks (v_bfi_b32), no branches.
__device__ __forceinline__ uint32_t select4(uint32_t m, uint32_t t0, uint32_t t1, uint32_t t2,
                                            uint32_t t3) {
  const uint32_t b0 = 0u - (m & 1u), b1 = 0u - ((m >> 1) & 1u);
  const uint32_t t01 = (t1 & b0) | (t0 & ~b0);
  const uint32_t t23 = (t3 & b0) | (t2 & ~b0);
  return (t23 & b1) | (t01 & ~b1);
}
__device__ __forceinline__ float inv_mant_hi(uint32_t m) {
  return __uint_as_float(select4(m, 0x40800000u, 0x404CCCCDu, 0x402AAAABu, 0x40124925u));
}
__device__ __forceinline__ float inv_mant_lo(uint32_t m) {
  return __uint_as_float(select4(m, 0x00000000u, 0xB34CCCCDu, 0xB3AAAAABu, 0xB3DB6DB7u));
}

// Fast unsigned division by a runtime-invariant divisor, valid for n < 2^31
// (Granlund & Montgomery, "Division by invariant integers using
// multiplication", 1994: q = (mulhi(n, m) + n) >> s).
struct FastDiv {
  uint32_t d, m, s;
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t s = 0;
  while ((1ull << s) < d) ++s;
  const uint64_t m = ((1ull << 32) * ((1ull << s) - d)) / d + 1;
  return FastDiv{d, (uint32_t)m, s};
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
  return (__umulhi(n, f.m) + n) >> f.s;
}

// DPP lane moves within a row of 16 lanes (gfx9 encodings).
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // row_half_mirror: lane i <-> 7-i in 8

template <int Ctrl>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, Ctrl, 0xF, 0xF, false);
}

// Max / OR over the 8 lanes of an aligned group of 8.
__device__ __forceinline__ uint32_t max8_u32(uint32_t v) {
  v = max(v, dpp<kDppQuadXor1>(v));
  v = max(v, dpp<kDppQuadXor2>(v));
  v = max(v, dpp<kDppHalfMirror>(v));
  return v;
}
__device__ __forceinline__ uint32_t or8_u32(uint32_t v) {
  v |= dpp<kDppQuadXor1>(v);
  v |= dpp<kDppQuadXor2>(v);
  v |= dpp<kDppHalfMirror>(v);
  return v;
}

__device__ __forceinline__ float bf16lo_to_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi_to_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

}  // namespace hif4

// ---------------------------------------------------------------- launchers
// Internal (hidden) host launchers; argument checks happen in api.hip.
hipError_t hif4_launch_quantize(const uint16_t* x, int64_t rows, int64_t k, int64_t ld,
                                const uint8_t* mask, int64_t n_mask, uint16_t* kept,
                                uint8_t* codes, uint32_t* meta, hipStream_t stream);
hipError_t hif4_launch_dequantize(const uint8_t* codes, const uint32_t* meta, int64_t rows,
                                  int64_t k, void* out, int out_bf16, hipStream_t stream);
hipError_t hif4_launch_gemm_w4a4(const uint8_t* a_codes, const uint32_t* a_meta,
                                 const uint16_t* b, int64_t m, int64_t n, int64_t k, void* y,
                                 int y_bf16, const uint16_t* xr, const uint16_t* wr, int64_t kr,
                                 hipStream_t stream);
hipError_t hif4_launch_pack_kept(const uint16_t* kept, int64_t rows, int64_t nk, int64_t kr,
                                 uint16_t* out, hipStream_t stream);
hipError_t hif4_launch_percentile(const uint16_t* x, int64_t rows, int64_t c, int64_t ld,
                                  double q, int64_t n_protect, float* stats, uint8_t* mask,
                                  void* workspace, hipStream_t stream);
size_t hif4_percentile_ws_bytes(int64_t rows, int64_t c);
hipError_t hif4_launch_zero(void* p, size_t bytes, hipStream_t stream);
hipError_t hif4_launch_quantize_offsets(const uint16_t* x, int64_t rows, int64_t k, int64_t ld,
                                        const float* koff, const float* moff, uint8_t* codes,
                                        uint32_t* meta, hipStream_t stream);
hipError_t hif4_launch_quantize_f32(const float* x, int64_t rows, int64_t k, int64_t ld,
                                    uint8_t* codes, uint32_t* meta, hipStream_t stream);
hipError_t hif4_launch_higptq_unit(float* w, int64_t n, int64_t k, int64_t ldw, const float* u,
                                   int64_t ldu, int64_t unit, int scheme, uint8_t* codes,
                                   uint32_t* meta, float* f, hipStream_t stream);
hipError_t hif4_launch_higptq_block(float* w, int64_t n, int64_t k, int64_t ldw, const float* u,
                                    int64_t ldu, int64_t unit0, int64_t units, int scheme,
                                    uint8_t* codes, uint32_t* meta, float* f,
                                    hipStream_t stream);
