"""Python binding of libhif4.so (the C ABI in include/hif4.h).

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch provides device memory and the current HIP stream. There is no CPU
fallback: if the library or a gfx950 device is missing, calls raise.

Tensors: bf16 inputs are torch.bfloat16 on the GPU; codes are uint8
[rows][k/2]; meta is int32 [rows][k/64] holding the u32 metadata words bit
for bit; masks are uint8.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libhif4.so")

HIF4_F32, HIF4_BF16 = 0, 1
_lib = None


class Hif4Error(RuntimeError):
    def __init__(self, status, what):
        super().__init__(f"{what}: {lib().hif4_status_string(status).decode()} (status {status})")
        self.status = status


def lib():
    """The loaded library (ctypes). Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m bit_block_float_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        p, i64, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        L.hif4_status_string.argtypes = [ctypes.c_int]
        L.hif4_status_string.restype = ctypes.c_char_p
        L.hif4_version.argtypes = []
        L.hif4_version.restype = ctypes.c_int
        L.hif4_quantize.argtypes = [p, i64, i64, i64, p, i64, p, p, p, p]
        L.hif4_quantize.restype = ctypes.c_int
        L.hif4_dequantize.argtypes = [p, p, i64, i64, p, ctypes.c_int, p]
        L.hif4_dequantize.restype = ctypes.c_int
        L.hif4_linear_workspace_bytes.argtypes = [i64, i64, i64, i64]
        L.hif4_linear_workspace_bytes.restype = sz
        L.hif4_linear_w4a4.argtypes = [p, p, p, p, p, p, p, p, i64, i64, i64, i64, p, ctypes.c_int,
                                       p, sz, p]
        L.hif4_linear_w4a4.restype = ctypes.c_int
        L.hif4_linear_xcodes_wbf16.argtypes = [p, p, p, p, p, i64, i64, i64, i64, p, ctypes.c_int, p,
                                               sz, p]
        L.hif4_linear_xcodes_wbf16.restype = ctypes.c_int
        L.hif4_linear_xcodes_wbf16_noalloc.argtypes = [p, p, p, p, p, i64, i64, i64, i64, p,
                                                       ctypes.c_int, p]
        L.hif4_linear_xcodes_wbf16_noalloc.restype = ctypes.c_int
        L.hif4_percentile_workspace_bytes.argtypes = [i64, i64]
        L.hif4_percentile_workspace_bytes.restype = sz
        L.hif4_percentile_mask.argtypes = [p, i64, i64, i64, ctypes.c_double, i64, p, p, p, sz, p]
        L.hif4_percentile_mask.restype = ctypes.c_int
        L.hif4_quantize_f32.argtypes = [p, i64, i64, i64, p, p, p]
        L.hif4_quantize_offsets.argtypes = [p, i64, i64, i64, p, p, p, p, p]
        L.hif4_quantize_offsets.restype = ctypes.c_int
        L.hif4_quantize_f32.restype = ctypes.c_int
        L.hif4_higptq_workspace_bytes.argtypes = [i64]
        L.hif4_higptq_workspace_bytes.restype = sz
        L.hif4_higptq_unit.argtypes = [p, i64, i64, i64, p, i64, i64, ctypes.c_int, p, p, p, sz, p]
        L.hif4_higptq_unit.restype = ctypes.c_int
        L.hif4_higptq_block_workspace_bytes.argtypes = [i64, i64]
        L.hif4_higptq_block_workspace_bytes.restype = sz
        L.hif4_higptq_block.argtypes = [p, i64, i64, i64, p, i64, i64, i64, ctypes.c_int, p, p, p,
                                        sz, p]
        L.hif4_higptq_block.restype = ctypes.c_int
        _lib = L
    return _lib


def require_gpu():
    """Raise unless a gfx950 GPU is visible and the library loads."""
    lib()
    if not torch.cuda.is_available():
        raise RuntimeError("no GPU visible: libhif4 runs only on gfx950 (MI355X)")
    arch = torch.cuda.get_device_properties(torch.cuda.current_device()).gcnArchName
    if not arch.startswith("gfx950"):
        raise RuntimeError(f"libhif4 needs gfx950, found {arch}")


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else None


def _stream(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _ok(status, what):
    if status != 0:
        raise Hif4Error(status, what)


def _check_bf16_rows(x, name):
    if x.dtype != torch.bfloat16 or not x.is_cuda or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D bf16 CUDA tensor with unit column stride")


def quantize(x, mask=None, codes=None, meta=None, kept=None, stream=None):
    """HiF4-quantize bf16 x [rows][k] along k -> (codes u8, meta int32, kept bf16)."""
    _check_bf16_rows(x, "x")
    rows, k = x.shape
    dev = x.device
    codes = codes if codes is not None else torch.empty((rows, k // 2), dtype=torch.uint8, device=dev)
    meta = meta if meta is not None else torch.empty((rows, k // 64), dtype=torch.int32, device=dev)
    n_mask = 0
    if mask is not None:
        n_mask = int(torch.count_nonzero(mask).item())
        if kept is None:
            kept = torch.empty((rows, n_mask), dtype=torch.bfloat16, device=dev)
    st = lib().hif4_quantize(_ptr(x), rows, k, x.stride(0), _ptr(mask), n_mask,
                             _ptr(kept) if n_mask else None, _ptr(codes), _ptr(meta), _stream(stream))
    _ok(st, "hif4_quantize")
    return codes, meta, kept


def dequantize(codes, meta, out_dtype=torch.float32, out=None, stream=None):
    """Decode codes [rows][k/2] + meta [rows][k/64] -> [rows][k] fp32 or bf16."""
    rows, k = codes.shape[0], codes.shape[1] * 2
    dt = HIF4_F32 if out_dtype == torch.float32 else HIF4_BF16
    out = out if out is not None else torch.empty((rows, k), dtype=out_dtype, device=codes.device)
    st = lib().hif4_dequantize(_ptr(codes), _ptr(meta), rows, k, _ptr(out), dt, _stream(stream))
    _ok(st, "hif4_dequantize")
    return out


def linear_workspace_bytes(m, n, k, n_kept=0):
    return int(lib().hif4_linear_workspace_bytes(m, n, k, n_kept))


def _kept_count(x_kept, w_kept, m, n):
    """n_kept from the kept-value tensors, after checking their shapes: a
    short tensor would be read past its end by the library."""
    if w_kept is None:
        if x_kept is not None:
            raise ValueError("x_kept given without w_kept")
        return 0
    if (w_kept.dtype != torch.bfloat16 or not w_kept.is_contiguous() or w_kept.dim() != 2
            or w_kept.shape[0] != n or not w_kept.is_cuda):
        raise ValueError(f"w_kept must be a contiguous bf16 CUDA tensor [n={n}][n_kept]")
    if x_kept is not None and (x_kept.dtype != torch.bfloat16 or not x_kept.is_contiguous()
                               or x_kept.dim() != 2 or x_kept.shape[0] != m
                               or x_kept.shape[1] != w_kept.shape[1] or not x_kept.is_cuda):
        raise ValueError(f"x_kept must be a contiguous bf16 CUDA tensor [m={m}][n_kept]")
    return w_kept.shape[1]


def _check_mask(mask, k, n_kept):
    """The protection mask: uint8 [k] on the GPU with exactly n_kept nonzeros
    (the count the kept values were gathered for)."""
    if mask is None:
        if n_kept:
            raise ValueError("n_kept > 0 with a bf16 x needs the mask that selects the channels")
        return
    if mask.dtype != torch.uint8 or mask.shape != (k,) or not mask.is_contiguous() or not mask.is_cuda:
        raise ValueError(f"mask must be a contiguous uint8 CUDA tensor [k={k}]")
    nz = int(torch.count_nonzero(mask).item())
    if nz != n_kept:
        raise ValueError(f"mask has {nz} protected channels but the kept values have {n_kept}")


def linear_w4a4(w_codes, w_meta, x=None, x_codes=None, x_meta=None, mask=None, x_kept=None,
                w_kept=None, y_dtype=torch.float32, y=None, workspace=None, stream=None):
    """Y = deq(Q(X)) deq(Q(W))^T (+ x_kept w_kept^T over protected channels).
    X as bf16 x [m][k] (with `mask` when there are protected channels) or as
    (x_codes, x_meta[, x_kept])."""
    n, k = w_codes.shape[0], w_codes.shape[1] * 2
    if x is not None:
        _check_bf16_rows(x, "x")
        if not x.is_contiguous():
            raise ValueError("x must be contiguous (row stride k)")
        m = x.shape[0]
    else:
        m = x_codes.shape[0]
    n_kept = _kept_count(x_kept, w_kept, m, n)
    if x is not None:
        _check_mask(mask, k, n_kept)
    elif n_kept and x_kept is None:
        raise ValueError("X given as codes with protected channels needs x_kept")
    dev = w_codes.device
    dt = HIF4_F32 if y_dtype == torch.float32 else HIF4_BF16
    y = y if y is not None else torch.empty((m, n), dtype=y_dtype, device=dev)
    need = linear_workspace_bytes(m, n, k, n_kept)
    if workspace is None:
        workspace = torch.empty((max(need, 1),), dtype=torch.uint8, device=dev)
    st = lib().hif4_linear_w4a4(_ptr(x), _ptr(x_codes), _ptr(x_meta), _ptr(w_codes), _ptr(w_meta),
                                _ptr(mask), _ptr(x_kept), _ptr(w_kept), n_kept, m, n, k, _ptr(y),
                                dt, _ptr(workspace), workspace.numel(), _stream(stream))
    _ok(st, "hif4_linear_w4a4")
    return y


def linear_xcodes_wbf16(x_codes, x_meta, w, x_kept=None, w_kept=None, y_dtype=torch.float32,
                        y=None, workspace=None, stream=None):
    """Y = deq(X codes) w^T (+ x_kept w_kept^T) with w bf16 [n][k] (e.g. a
    weight decoded once)."""
    _check_bf16_rows(w, "w")
    if not w.is_contiguous():
        raise ValueError("w must be contiguous (row stride k)")
    m, n, k = x_codes.shape[0], w.shape[0], w.shape[1]
    n_kept = _kept_count(x_kept, w_kept, m, n)
    if n_kept and x_kept is None:
        raise ValueError("protected channels need x_kept")
    dt = HIF4_F32 if y_dtype == torch.float32 else HIF4_BF16
    y = y if y is not None else torch.empty((m, n), dtype=y_dtype, device=w.device)
    if workspace is None and n_kept:
        workspace = torch.empty((linear_workspace_bytes(m, n, 0, n_kept),), dtype=torch.uint8,
                                device=w.device)
    ws_bytes = workspace.numel() if workspace is not None else 0
    st = lib().hif4_linear_xcodes_wbf16(_ptr(x_codes), _ptr(x_meta), _ptr(w), _ptr(x_kept),
                                        _ptr(w_kept), n_kept, m, n, k, _ptr(y), dt,
                                        _ptr(workspace), ws_bytes, _stream(stream))
    _ok(st, "hif4_linear_xcodes_wbf16")
    return y


NOALLOC_SCRATCH_BYTES = 32 << 20  # HIF4_NOALLOC_SCRATCH_BYTES


def linear_xcodes_wbf16_noalloc(x_codes, x_meta, w, y, x_kept=None, w_kept=None, stream=None):
    """hif4_linear_xcodes_wbf16 without a workspace (the library's static
    scratch holds the protected-channel operands): Y into the caller's `y`
    ([m][n], fp32 or bf16). Allocates no device memory."""
    _check_bf16_rows(w, "w")
    if not w.is_contiguous():
        raise ValueError("w must be contiguous (row stride k)")
    m, n, k = x_codes.shape[0], w.shape[0], w.shape[1]
    if y.shape != (m, n) or not y.is_contiguous() or y.dtype not in (torch.float32, torch.bfloat16):
        raise ValueError("y must be a contiguous fp32 or bf16 tensor [m][n]")
    n_kept = _kept_count(x_kept, w_kept, m, n)
    if n_kept and x_kept is None:
        raise ValueError("protected channels need x_kept")
    dt = HIF4_F32 if y.dtype == torch.float32 else HIF4_BF16
    st = lib().hif4_linear_xcodes_wbf16_noalloc(_ptr(x_codes), _ptr(x_meta), _ptr(w),
                                                _ptr(x_kept), _ptr(w_kept), n_kept, m, n, k,
                                                _ptr(y), dt, _stream(stream))
    _ok(st, "hif4_linear_xcodes_wbf16_noalloc")
    return y


def percentile_workspace_bytes(rows, c):
    return int(lib().hif4_percentile_workspace_bytes(rows, c))


def percentile_exact_channels(workspace, rows, c):
    """Channels of the last hif4_percentile_mask call on `workspace` whose
    statistic came from the two exact passes (c unless the one-pass window
    path ran; then the channels it missed). Reads the count from the device."""
    off = percentile_workspace_bytes(rows, c) - 256
    return int(workspace[off:off + 4].view(torch.int32).item())


def percentile_mask(x, q, n_protect, stats=None, mask=None, workspace=None, stream=None):
    """Per-channel type-7 quantile of |x| over rows -> (stats fp32 [c], mask u8 [c])."""
    _check_bf16_rows(x, "x")
    rows, c = x.shape
    dev = x.device
    stats = stats if stats is not None else torch.empty((c,), dtype=torch.float32, device=dev)
    mask = mask if mask is not None else torch.empty((c,), dtype=torch.uint8, device=dev)
    if workspace is None:
        workspace = torch.empty((percentile_workspace_bytes(rows, c),), dtype=torch.uint8, device=dev)
    st = lib().hif4_percentile_mask(_ptr(x), rows, c, x.stride(0), float(q), int(n_protect),
                                    _ptr(stats), _ptr(mask), _ptr(workspace), workspace.numel(),
                                    _stream(stream))
    _ok(st, "hif4_percentile_mask")
    return stats, mask


def _check_f32_rows(x, name):
    if x.dtype != torch.float32 or not x.is_cuda or x.dim() != 2 or x.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D fp32 CUDA tensor with unit column stride")


def quantize_offsets(x, koff, moff, codes=None, meta=None, stream=None):
    """HiF4-quantize bf16 x [rows][k] with given HiAutoRound offsets: koff fp32
    [rows][k/4] (level-3 exponents), moff fp32 [rows][k] (mantissas).
    Returns (codes u8, meta int32)."""
    _check_bf16_rows(x, "x")
    rows, k = x.shape
    for t, name, shape in ((koff, "koff", (rows, k // 4)), (moff, "moff", (rows, k))):
        if (t.dtype != torch.float32 or not t.is_cuda or tuple(t.shape) != shape
                or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous fp32 CUDA tensor of shape {shape}")
    dev = x.device
    codes = codes if codes is not None else torch.empty((rows, k // 2), dtype=torch.uint8, device=dev)
    meta = meta if meta is not None else torch.empty((rows, k // 64), dtype=torch.int32, device=dev)
    st = lib().hif4_quantize_offsets(_ptr(x), rows, k, x.stride(0), _ptr(koff), _ptr(moff),
                                     _ptr(codes), _ptr(meta), _stream(stream))
    _ok(st, "hif4_quantize_offsets")
    return codes, meta


def quantize_f32(x, codes=None, meta=None, stream=None):
    """HiF4-quantize fp32 x [rows][k] along k -> (codes u8, meta int32)."""
    _check_f32_rows(x, "x")
    rows, k = x.shape
    dev = x.device
    codes = codes if codes is not None else torch.empty((rows, k // 2), dtype=torch.uint8, device=dev)
    meta = meta if meta is not None else torch.empty((rows, k // 64), dtype=torch.int32, device=dev)
    st = lib().hif4_quantize_f32(_ptr(x), rows, k, x.stride(0), _ptr(codes), _ptr(meta),
                                 _stream(stream))
    _ok(st, "hif4_quantize_f32")
    return codes, meta


def higptq_workspace_bytes(n):
    return int(lib().hif4_higptq_workspace_bytes(n))


def higptq_unit(w, u, unit, codes, meta, workspace=None, stream=None, scheme=1):
    """One HiGPTQ group step (scheme 1, 2 or 3) in place on the fp32 working
    weights w [n][k] with the upper factor u [k][k] (H^-1 = u^T u): writes
    unit ``unit`` of codes/meta and updates the later columns of w."""
    _check_f32_rows(w, "w")
    _check_f32_rows(u, "u")
    n, k = w.shape
    if workspace is None:
        workspace = torch.empty((higptq_workspace_bytes(n),), dtype=torch.uint8, device=w.device)
    st = lib().hif4_higptq_unit(_ptr(w), n, k, w.stride(0), _ptr(u), u.stride(0), int(unit),
                                int(scheme), _ptr(codes), _ptr(meta), _ptr(workspace),
                                workspace.numel(), _stream(stream))
    _ok(st, "hif4_higptq_unit")


HIGPTQ_MAX_BLOCK_UNITS = 16


def higptq_block_workspace_bytes(n, units):
    return int(lib().hif4_higptq_block_workspace_bytes(n, units))


def higptq_block(w, u, unit0, units, codes, meta, workspace=None, stream=None, scheme=1):
    """One HiGPTQ block step (blocksize 64 * units columns, groups unit0 ..
    unit0 + units - 1, scheme 1, 2 or 3) in place on the fp32 working weights
    w [n][k]: writes those units of codes/meta and updates the later columns
    of w, the block's own later columns after each group and the columns after
    the block once."""
    _check_f32_rows(w, "w")
    _check_f32_rows(u, "u")
    n, k = w.shape
    if workspace is None:
        nbytes = max(higptq_block_workspace_bytes(n, units), 1)
        workspace = torch.empty((nbytes,), dtype=torch.uint8, device=w.device)
    st = lib().hif4_higptq_block(_ptr(w), n, k, w.stride(0), _ptr(u), u.stride(0), int(unit0),
                                 int(units), int(scheme), _ptr(codes), _ptr(meta),
                                 _ptr(workspace), workspace.numel(), _stream(stream))
    _ok(st, "hif4_higptq_block")


def higptq(w, u, stream=None, scheme=1, block_units=8):
    """HiGPTQ over all groups in blocks of ``block_units`` groups (1 = one
    group at a time through hif4_higptq_unit): returns (codes, meta); w is
    updated in place (its final contents are the compensated working
    weights)."""
    n, k = w.shape
    units = k // 64
    codes = torch.empty((n, k // 2), dtype=torch.uint8, device=w.device)
    meta = torch.empty((n, units), dtype=torch.int32, device=w.device)
    if block_units == 1:
        ws = torch.empty((higptq_workspace_bytes(n),), dtype=torch.uint8, device=w.device)
        for unit in range(units):
            higptq_unit(w, u, unit, codes, meta, workspace=ws, stream=stream, scheme=scheme)
        return codes, meta
    ws = torch.empty((max(higptq_block_workspace_bytes(n, block_units), 1),), dtype=torch.uint8,
                     device=w.device)
    for unit0 in range(0, units, block_units):
        higptq_block(w, u, unit0, min(block_units, units - unit0), codes, meta, workspace=ws,
                     stream=stream, scheme=scheme)
    return codes, meta
