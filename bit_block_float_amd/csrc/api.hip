// api.hip -- the C ABI of libhif4.so (declared and documented in
// include/hif4.h). Every argument check runs before any HIP call, so invalid
// calls return a status without touching the device or the outputs.
#include <hip/hip_runtime.h>
#include <string.h>

#include <atomic>

#include "../../include/hif4.h"
#include "hif4_dev.h"

namespace {

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// 0 = unknown, 1 = gfx950, 2 = other. Benign race: every writer stores the
// same value for a device.
int g_dev_kind[64];

hif4_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return HIF4_ERR_DEVICE;
  if (dev < 64 && g_dev_kind[dev] != 0) return g_dev_kind[dev] == 1 ? HIF4_OK : HIF4_ERR_DEVICE;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return HIF4_ERR_DEVICE;
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_dev_kind[dev] = ok ? 1 : 2;
  return ok ? HIF4_OK : HIF4_ERR_DEVICE;
}

hif4_status launched(hipError_t e) { return e == hipSuccess ? HIF4_OK : HIF4_ERR_LAUNCH; }

size_t align256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

const char* hif4_status_string(int status) {
  switch (status) {
    case HIF4_OK: return "ok";
    case HIF4_ERR_NULL: return "a required pointer is NULL";
    case HIF4_ERR_SHAPE: return "invalid shape (negative size, k % 64 != 0, ld < k, ...)";
    case HIF4_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case HIF4_ERR_WORKSPACE: return "workspace missing or too small";
    case HIF4_ERR_DTYPE: return "unknown dtype";
    case HIF4_ERR_DEVICE: return "current device is not gfx950 (MI355X)";
    case HIF4_ERR_LAUNCH: return "kernel launch failed";
    case HIF4_ERR_ARG: return "argument out of range";
    case HIF4_ERR_SCRATCH:
      return "problem needs more than the allocation-free entry point's static scratch";
    default: return "unknown status";
  }
}

int hif4_version(void) { return HIF4_API_VERSION; }

hif4_status hif4_quantize(const void* x, int64_t rows, int64_t k, int64_t ld, const uint8_t* mask,
                          int64_t n_mask, void* kept, uint8_t* codes, uint32_t* meta,
                          hipStream_t stream) {
  if (rows < 0 || k < 0 || k % 64 != 0 || ld < k || n_mask < 0) return HIF4_ERR_SHAPE;
  if (mask && (k > 65536 || n_mask > k)) return HIF4_ERR_SHAPE;
  if (rows == 0 || k == 0) return HIF4_OK;
  if (!x || !codes || !meta) return HIF4_ERR_NULL;
  if (mask && n_mask > 0 && !kept) return HIF4_ERR_NULL;
  if (!aligned(x, 16) || ld % 8 != 0 || !aligned(codes, 16) || !aligned(meta, 4))
    return HIF4_ERR_ALIGN;
  if (mask && !aligned(mask, 16)) return HIF4_ERR_ALIGN;
  if (mask && n_mask > 0 && !aligned(kept, 2)) return HIF4_ERR_ALIGN;
  hif4_status st = check_device();
  if (st != HIF4_OK) return st;
  const uint16_t* xb = (const uint16_t*)x;
  return launched(hif4_launch_quantize(xb, rows, k, ld, mask, mask ? n_mask : 0,
                                       (uint16_t*)kept, codes, meta, stream));
}

hif4_status hif4_dequantize(const uint8_t* codes, const uint32_t* meta, int64_t rows, int64_t k,
                            void* out, int out_dtype, hipStream_t stream) {
  if (rows < 0 || k < 0 || k % 64 != 0) return HIF4_ERR_SHAPE;
  if (out_dtype != HIF4_F32 && out_dtype != HIF4_BF16) return HIF4_ERR_DTYPE;
  if (rows == 0 || k == 0) return HIF4_OK;
  if (!codes || !meta || !out) return HIF4_ERR_NULL;
  if (!aligned(codes, 16) || !aligned(meta, 4) || !aligned(out, 16)) return HIF4_ERR_ALIGN;
  hif4_status st = check_device();
  if (st != HIF4_OK) return st;
  return launched(hif4_launch_dequantize(codes, meta, rows, k, out, out_dtype == HIF4_BF16, stream));
}

// Workspace of the linear entry points, in order (each part 256-byte aligned):
//   X codes [m][k/2], X meta [m][k/64]   (X given in bf16)
//   W~ bf16 [n][k]                        (hif4_linear_w4a4: W decoded once)
//   X kept bf16 [m][n_kept]               (X given in bf16 with a mask)
//   Xr bf16 [m][kr], Wr bf16 [n][kr]      (protected channels zero-padded to
//                                          kr = n_kept rounded up to 64)
// With k = 0 the same formula gives what hif4_linear_xcodes_wbf16 needs.
static int64_t resid_cols(int64_t n_kept) { return (n_kept + 63) / 64 * 64; }
static size_t ws_x_codes(int64_t m, int64_t k) { return align256((size_t)m * (size_t)(k / 2)); }
static size_t ws_x_meta(int64_t m, int64_t k) { return align256((size_t)m * (size_t)(k / 64) * 4); }
static size_t ws_w_deq(int64_t n, int64_t k) { return align256((size_t)n * (size_t)k * 2); }
static size_t ws_x_kept(int64_t m, int64_t nk) { return align256((size_t)m * (size_t)nk * 2); }
static size_t ws_resid(int64_t rows, int64_t nk) {
  return align256((size_t)rows * (size_t)resid_cols(nk) * 2);
}
size_t hif4_linear_workspace_bytes(int64_t m, int64_t n, int64_t k, int64_t n_kept) {
  // 0 for sizes no linear entry point accepts (so the sums below never wrap)
  if (m < 0 || n < 0 || k < 0 || n_kept < 0) return 0;
  if (m >= (1ll << 31) || n >= (1ll << 31) || k >= (1ll << 31) || n_kept > 65536) return 0;
  return ws_x_codes(m, k) + ws_x_meta(m, k) + ws_w_deq(n, k) + ws_x_kept(m, n_kept) +
         ws_resid(m, n_kept) + ws_resid(n, n_kept);
}

// Shared tail of both linear entry points: pack the protected channels (if
// any) into the zero-padded residual operands, then the W4A4 kernel.
static hif4_status linear_tail(const uint8_t* x_codes, const uint32_t* x_meta, const uint16_t* w,
                               const uint16_t* x_kept, const uint16_t* w_kept, int64_t n_kept,
                               int64_t m, int64_t n, int64_t k, void* y, int y_dtype,
                               char* resid_ws, hipStream_t stream) {
  uint16_t* xr = nullptr;
  uint16_t* wr = nullptr;
  const int64_t kr = n_kept ? resid_cols(n_kept) : 0;
  if (n_kept) {
    xr = (uint16_t*)resid_ws;
    wr = (uint16_t*)(resid_ws + ws_resid(m, n_kept));
    hif4_status st = launched(hif4_launch_pack_kept(x_kept, m, n_kept, kr, xr, stream));
    if (st != HIF4_OK) return st;
    st = launched(hif4_launch_pack_kept(w_kept, n, n_kept, kr, wr, stream));
    if (st != HIF4_OK) return st;
  }
  return launched(hif4_launch_gemm_w4a4(x_codes, x_meta, w, m, n, k, y, y_dtype == HIF4_BF16, xr,
                                        wr, kr, stream));
}

static hif4_status check_linear_common(int64_t m, int64_t n, int64_t k, int64_t n_kept,
                                       int y_dtype) {
  if (m < 0 || n < 0 || k < 0 || k % 64 != 0) return HIF4_ERR_SHAPE;
  if (m >= (1ll << 31) || n >= (1ll << 31) || k >= (1ll << 31)) return HIF4_ERR_SHAPE;
  if (n_kept < 0 || n_kept > k || n_kept > 65536) return HIF4_ERR_SHAPE;
  if (y_dtype != HIF4_F32 && y_dtype != HIF4_BF16) return HIF4_ERR_DTYPE;
  return HIF4_OK;
}

hif4_status hif4_linear_w4a4(const void* x, const uint8_t* x_codes, const uint32_t* x_meta,
                             const uint8_t* w_codes, const uint32_t* w_meta, const uint8_t* mask,
                             const void* x_kept, const void* w_kept, int64_t n_kept, int64_t m,
                             int64_t n, int64_t k, void* y, int y_dtype, void* workspace,
                             size_t workspace_bytes, hipStream_t stream) {
  hif4_status st = check_linear_common(m, n, k, n_kept, y_dtype);
  if (st != HIF4_OK) return st;
  if (m == 0 || n == 0) return HIF4_OK;
  if (!y) return HIF4_ERR_NULL;
  if (k > 0) {
    if (!w_codes || !w_meta) return HIF4_ERR_NULL;
    if (!x && (!x_codes || !x_meta)) return HIF4_ERR_NULL;
    if (n_kept > 0 && (!w_kept || (x ? !mask : !x_kept))) return HIF4_ERR_NULL;
    if (x && n_kept > 0 && k > 65536) return HIF4_ERR_SHAPE;  // channel list of the gather
  }
  if (!aligned(y, 16)) return HIF4_ERR_ALIGN;
  if (k > 0) {
    if (x && !aligned(x, 16)) return HIF4_ERR_ALIGN;
    if (!x && (!aligned(x_codes, 16) || !aligned(x_meta, 4))) return HIF4_ERR_ALIGN;
    if (!aligned(w_codes, 16) || !aligned(w_meta, 4)) return HIF4_ERR_ALIGN;
    if (n_kept > 0) {
      if (!aligned(w_kept, 2) || (!x && !aligned(x_kept, 2))) return HIF4_ERR_ALIGN;
      if (x && !aligned(mask, 16)) return HIF4_ERR_ALIGN;
    }
    if (!workspace || workspace_bytes < hif4_linear_workspace_bytes(m, n, k, n_kept))
      return HIF4_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return HIF4_ERR_ALIGN;
  }
  st = check_device();
  if (st != HIF4_OK) return st;
  if (k == 0) {
    // Empty contraction: Y = 0.
    const size_t bytes = (size_t)m * (size_t)n * (y_dtype == HIF4_BF16 ? 2 : 4);
    return launched(hif4_launch_zero(y, bytes, stream));
  }
  char* ws = (char*)workspace;
  uint8_t* xc = (uint8_t*)ws;
  uint32_t* xm = (uint32_t*)(ws + ws_x_codes(m, k));
  uint16_t* wb = (uint16_t*)(ws + ws_x_codes(m, k) + ws_x_meta(m, k));
  uint16_t* xk = (uint16_t*)(ws + ws_x_codes(m, k) + ws_x_meta(m, k) + ws_w_deq(n, k));
  char* rws = ws + ws_x_codes(m, k) + ws_x_meta(m, k) + ws_w_deq(n, k) + ws_x_kept(m, n_kept);
  if (x) {
    // X in bf16: quantize it to HiF4 first (the same codes hif4_quantize
    // gives), with the protected channels masked out and gathered.
    const uint8_t* xmask = n_kept ? mask : nullptr;
    st = launched(hif4_launch_quantize((const uint16_t*)x, m, k, k, xmask, n_kept, xk, xc, xm,
                                       stream));
    if (st != HIF4_OK) return st;
    if (n_kept) x_kept = xk;
    x_codes = xc;
    x_meta = xm;
  }
  // W decoded to bf16 once; X codes are decoded tile by tile inside the GEMM.
  st = launched(hif4_launch_dequantize(w_codes, w_meta, n, k, wb, 1, stream));
  if (st != HIF4_OK) return st;
  return linear_tail(x_codes, x_meta, wb, (const uint16_t*)x_kept, (const uint16_t*)w_kept, n_kept,
                     m, n, k, y, y_dtype, rws, stream);
}

hif4_status hif4_linear_xcodes_wbf16(const uint8_t* x_codes, const uint32_t* x_meta,
                                     const void* w, const void* x_kept, const void* w_kept,
                                     int64_t n_kept, int64_t m, int64_t n, int64_t k, void* y,
                                     int y_dtype, void* workspace, size_t workspace_bytes,
                                     hipStream_t stream) {
  hif4_status st = check_linear_common(m, n, k, n_kept, y_dtype);
  if (st != HIF4_OK) return st;
  if (m == 0 || n == 0) return HIF4_OK;
  if (!y) return HIF4_ERR_NULL;
  if (k > 0 && (!x_codes || !x_meta || !w)) return HIF4_ERR_NULL;
  if (n_kept > 0 && (!x_kept || !w_kept)) return HIF4_ERR_NULL;
  if (!aligned(y, 16)) return HIF4_ERR_ALIGN;
  if (k > 0 && (!aligned(x_codes, 16) || !aligned(x_meta, 4) || !aligned(w, 16)))
    return HIF4_ERR_ALIGN;
  if (n_kept > 0) {
    if (!aligned(x_kept, 2) || !aligned(w_kept, 2)) return HIF4_ERR_ALIGN;
    if (!workspace || workspace_bytes < hif4_linear_workspace_bytes(m, n, 0, n_kept))
      return HIF4_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return HIF4_ERR_ALIGN;
  }
  st = check_device();
  if (st != HIF4_OK) return st;
  if (k == 0) {
    const size_t bytes = (size_t)m * (size_t)n * (y_dtype == HIF4_BF16 ? 2 : 4);
    return launched(hif4_launch_zero(y, bytes, stream));
  }
  return linear_tail(x_codes, x_meta, (const uint16_t*)w, (const uint16_t*)x_kept,
                     (const uint16_t*)w_kept, n_kept, m, n, k, y, y_dtype,
                     (char*)workspace + ws_x_kept(m, 0), stream);
}

}  // extern "C"

// Static scratch of the allocation-free entry point: the zero-padded
// protected-channel operands Xr [m][kr] and Wr [n][kr] of one call. Host code
// never passes `scratch` itself to a kernel (in host code that name is a
// host-side stand-in, not the device address): each device's copy is looked
// up once with hipGetSymbolAddress, with that device current, and the cached
// address is what the kernels receive.
static __device__ __attribute__((aligned(256))) char scratch[HIF4_NOALLOC_SCRATCH_BYTES];

namespace {
std::atomic<void*> g_scratch_ptr[64];

// The current device's copy of `scratch` (looked up on first use). Two
// threads racing on the first lookup both store the same address.
hif4_status scratch_of_current_device(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return HIF4_ERR_DEVICE;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return HIF4_ERR_LAUNCH;
    g_scratch_ptr[dev].store(p, std::memory_order_release);
  }
  *out = (char*)p;
  return HIF4_OK;
}
}  // namespace

extern "C" {

hif4_status hif4_linear_xcodes_wbf16_noalloc(const uint8_t* x_codes, const uint32_t* x_meta,
                                             const void* w, const void* x_kept,
                                             const void* w_kept, int64_t n_kept, int64_t m,
                                             int64_t n, int64_t k, void* y, int y_dtype,
                                             hipStream_t stream) {
  hif4_status st = check_linear_common(m, n, k, n_kept, y_dtype);
  if (st != HIF4_OK) return st;
  if (m == 0 || n == 0) return HIF4_OK;
  if (!y) return HIF4_ERR_NULL;
  if (k > 0 && (!x_codes || !x_meta || !w)) return HIF4_ERR_NULL;
  if (n_kept > 0 && (!x_kept || !w_kept)) return HIF4_ERR_NULL;
  if (!aligned(y, 16)) return HIF4_ERR_ALIGN;
  if (k > 0 && (!aligned(x_codes, 16) || !aligned(x_meta, 4) || !aligned(w, 16)))
    return HIF4_ERR_ALIGN;
  if (n_kept > 0 && (!aligned(x_kept, 2) || !aligned(w_kept, 2))) return HIF4_ERR_ALIGN;
  if (ws_resid(m, n_kept) + ws_resid(n, n_kept) > HIF4_NOALLOC_SCRATCH_BYTES)
    return HIF4_ERR_SCRATCH;
  st = check_device();
  if (st != HIF4_OK) return st;
  if (k == 0) {
    const size_t bytes = (size_t)m * (size_t)n * (y_dtype == HIF4_BF16 ? 2 : 4);
    return launched(hif4_launch_zero(y, bytes, stream));
  }
  char* ws = nullptr;
  if (n_kept > 0) {
    st = scratch_of_current_device(&ws);
    if (st != HIF4_OK) return st;
  }
  return linear_tail(x_codes, x_meta, (const uint16_t*)w, (const uint16_t*)x_kept,
                     (const uint16_t*)w_kept, n_kept, m, n, k, y, y_dtype, ws, stream);
}

size_t hif4_percentile_workspace_bytes(int64_t rows, int64_t c) {
  // 0 beyond the entry point's limits (rows below 2^32, at most 65536 channels)
  if (c < 0 || rows < 0 || rows > 0xFFFFFFFFll || c > 65536) return 0;
  return hif4_percentile_ws_bytes(rows, c);
}

hif4_status hif4_percentile_mask(const void* x, int64_t rows, int64_t c, int64_t ld, double q,
                                 int64_t n_protect, float* stats, uint8_t* mask, void* workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  if (rows < 1 || rows > 0xFFFFFFFFll || c < 1 || c > 65536 || ld < c || ld > (1 << 22))
    return HIF4_ERR_SHAPE;
  if (n_protect < 0 || n_protect > c) return HIF4_ERR_SHAPE;
  if (!(q >= 0.0 && q <= 1.0)) return HIF4_ERR_ARG;
  if (!x || !stats || !mask) return HIF4_ERR_NULL;
  if (!aligned(x, 16) || ld % 8 != 0 || !aligned(stats, 4)) return HIF4_ERR_ALIGN;
  if (!workspace || workspace_bytes < hif4_percentile_workspace_bytes(rows, c))
    return HIF4_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return HIF4_ERR_ALIGN;
  hif4_status st = check_device();
  if (st != HIF4_OK) return st;
  return launched(hif4_launch_percentile((const uint16_t*)x, rows, c, ld, q, n_protect, stats, mask,
                                         workspace, stream));
}

hif4_status hif4_quantize_f32(const float* x, int64_t rows, int64_t k, int64_t ld,
                              uint8_t* codes, uint32_t* meta, hipStream_t stream) {
  if (rows < 0 || k < 0 || k % 64 != 0 || ld < k) return HIF4_ERR_SHAPE;
  if (rows == 0 || k == 0) return HIF4_OK;
  if (!x || !codes || !meta) return HIF4_ERR_NULL;
  if (!aligned(x, 16) || ld % 4 != 0 || !aligned(codes, 16) || !aligned(meta, 4))
    return HIF4_ERR_ALIGN;
  hif4_status st = check_device();
  if (st != HIF4_OK) return st;
  return launched(hif4_launch_quantize_f32(x, rows, k, ld, codes, meta, stream));
}

hif4_status hif4_quantize_offsets(const void* x, int64_t rows, int64_t k, int64_t ld,
                                  const float* koff, const float* moff, uint8_t* codes,
                                  uint32_t* meta, hipStream_t stream) {
  if (rows < 0 || k < 0 || k % 64 != 0 || ld < k) return HIF4_ERR_SHAPE;
  if (rows == 0 || k == 0) return HIF4_OK;
  if (!x || !koff || !moff || !codes || !meta) return HIF4_ERR_NULL;
  if (!aligned(x, 16) || ld % 8 != 0 || !aligned(koff, 16) || !aligned(moff, 16) ||
      !aligned(codes, 16) || !aligned(meta, 4))
    return HIF4_ERR_ALIGN;
  hif4_status st = check_device();
  if (st != HIF4_OK) return st;
  return launched(hif4_launch_quantize_offsets((const uint16_t*)x, rows, k, ld, koff, moff, codes,
                                               meta, stream));
}

size_t hif4_higptq_workspace_bytes(int64_t n) {
  if (n < 0 || n >= (int64_t(1) << 24)) return 0;  // the entry point's row limit
  return align256((size_t)n * 64 * sizeof(float));
}

hif4_status hif4_higptq_unit(float* w, int64_t n, int64_t k, int64_t ldw, const float* u,
                             int64_t ldu, int64_t unit, int scheme, uint8_t* codes,
                             uint32_t* meta, void* workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  if (n < 0 || n >= (int64_t(1) << 24) || k <= 0 || k % 64 != 0 || ldw < k || ldu < k ||
      ldw >= (int64_t(1) << 22) || ldu >= (int64_t(1) << 22))
    return HIF4_ERR_SHAPE;
  if (unit < 0 || unit >= k / 64 || scheme < 1 || scheme > 3) return HIF4_ERR_ARG;
  if (n == 0) return HIF4_OK;
  if (!w || !u || !codes || !meta) return HIF4_ERR_NULL;
  if (!aligned(w, 16) || ldw % 4 != 0 || !aligned(u, 16) || ldu % 4 != 0 || !aligned(codes, 16) ||
      !aligned(meta, 4))
    return HIF4_ERR_ALIGN;
  if (!workspace || workspace_bytes < hif4_higptq_workspace_bytes(n)) return HIF4_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return HIF4_ERR_ALIGN;
  hif4_status st = check_device();
  if (st != HIF4_OK) return st;
  return launched(hif4_launch_higptq_unit(w, n, k, ldw, u, ldu, unit, scheme, codes, meta,
                                          (float*)workspace, stream));
}

size_t hif4_higptq_block_workspace_bytes(int64_t n, int64_t units) {
  if (n < 0 || n >= (int64_t(1) << 24) || units < 1 || units > HIF4_HIGPTQ_MAX_BLOCK_UNITS)
    return 0;
  return align256((size_t)((n + 63) / 64 * 64) * 64 * (size_t)units * sizeof(float));
}

hif4_status hif4_higptq_block(float* w, int64_t n, int64_t k, int64_t ldw, const float* u,
                              int64_t ldu, int64_t unit0, int64_t units, int scheme,
                              uint8_t* codes, uint32_t* meta, void* workspace,
                              size_t workspace_bytes, hipStream_t stream) {
  if (n < 0 || n >= (int64_t(1) << 24) || k <= 0 || k % 64 != 0 || ldw < k || ldu < k ||
      ldw >= (int64_t(1) << 22) || ldu >= (int64_t(1) << 22))
    return HIF4_ERR_SHAPE;
  if (units < 1 || units > HIF4_HIGPTQ_MAX_BLOCK_UNITS || unit0 < 0 || unit0 > k / 64 - units ||
      scheme < 1 || scheme > 3)
    return HIF4_ERR_ARG;
  if (n == 0) return HIF4_OK;
  if (!w || !u || !codes || !meta) return HIF4_ERR_NULL;
  if (!aligned(w, 16) || ldw % 4 != 0 || !aligned(u, 16) || ldu % 4 != 0 || !aligned(codes, 16) ||
      !aligned(meta, 4))
    return HIF4_ERR_ALIGN;
  if (!workspace || workspace_bytes < hif4_higptq_block_workspace_bytes(n, units))
    return HIF4_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return HIF4_ERR_ALIGN;
  hif4_status st = check_device();
  if (st != HIF4_OK) return st;
  return launched(hif4_launch_higptq_block(w, n, k, ldw, u, ldu, unit0, units, scheme, codes,
                                           meta, (float*)workspace, stream));
}

}  // extern "C"
