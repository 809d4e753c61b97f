"""The HiF4 oracle: a plain, slow, obviously correct CPU reference.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. The HIP library
never calls it; the two share no code.

The arithmetic lives in ``hif4_oracle.c`` (plain C, IEEE double); this module
only marshals numpy arrays through ctypes. bf16 tensors are passed as their
uint16 bit patterns. Every function cites the page passage it follows in the
C source.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_LIB = None


def _lib():
    global _LIB
    if _LIB is None:
        if not os.path.exists(_build.LIB):
            _build.build()
        lib = ctypes.CDLL(_build.LIB)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        lib.hif4o_e6m2_value.argtypes = [ctypes.c_int]
        lib.hif4o_e6m2_value.restype = ctypes.c_double
        lib.hif4o_quantize.argtypes = [p, i64, i64, i64, p, i64, p, p, p]
        lib.hif4o_quantize.restype = ctypes.c_int
        lib.hif4o_dequantize.argtypes = [p, p, i64, i64, p]
        lib.hif4o_dequantize.restype = ctypes.c_int
        lib.hif4o_linear.argtypes = [p, p, p, p, i64, i64, i64, p, p]
        lib.hif4o_linear_protected.argtypes = [p, p, p, p, p, p, i64, i64, i64, i64, p, p]
        lib.hif4o_linear.restype = ctypes.c_int
        lib.hif4o_percentile.argtypes = [p, i64, i64, i64, ctypes.c_double, p]
        lib.hif4o_percentile.restype = ctypes.c_int
        lib.hif4o_topn_mask.argtypes = [p, i64, i64, p]
        lib.hif4o_topn_mask.restype = ctypes.c_int
        lib.hif4o_quantize_f32.argtypes = [p, i64, i64, i64, p, p]
        lib.hif4o_quantize_offsets.argtypes = [p, i64, i64, i64, p, p, p, p]
        lib.hif4o_quantize_f32.restype = ctypes.c_int
        lib.hif4o_higptq_unit.argtypes = [p, i64, i64, p, i64, p, p]
        lib.hif4o_higptq_unit.restype = ctypes.c_int
        lib.hif4o_higptq_unit_scheme.argtypes = [p, i64, i64, p, i64, ctypes.c_int, p, p]
        lib.hif4o_higptq_unit_scheme.restype = ctypes.c_int
        lib.hif4o_higptq_unit_scheme_margin.argtypes = [p, i64, i64, p, i64, ctypes.c_int, p, p, p]
        lib.hif4o_higptq_unit_scheme_margin.restype = ctypes.c_int
        lib.hif4o_higptq_run_margin.argtypes = [p, i64, i64, p, i64, i64, ctypes.c_int, p, p, p, p]
        lib.hif4o_higptq_run_margin.restype = ctypes.c_int
        _LIB = lib
    return _LIB


class OracleError(RuntimeError):
    pass


def _check(rc, what):
    if rc == 1:
        raise OracleError(f"{what}: invalid argument")
    if rc == 2:
        raise OracleError(f"{what}: non-finite input (out of contract)")
    if rc != 0:
        raise OracleError(f"{what}: status {rc}")


def _shape(a, shape, what):
    if tuple(a.shape) != tuple(shape):
        raise OracleError(f"{what}: shape {tuple(a.shape)}, expected {tuple(shape)}")


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def e6m2_value(c: int) -> float:
    """Value of the level-1 E6M2 code c (0..255)."""
    return _lib().hif4o_e6m2_value(int(c))


def quantize(x_bits: np.ndarray, mask: np.ndarray = None):
    """HiF4-quantize rows of bf16 bits [rows][k] along k.

    Returns (codes u8 [rows][k/2], meta u32 [rows][k/64], kept u16 [rows][n_mask]).
    ``mask`` (u8 [k], nonzero = protected) zeroes those channels in the HiF4
    stream and copies their bf16 bits into ``kept`` in ascending channel order.
    """
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, k = x.shape
    if mask is not None:
        _shape(np.asarray(mask), (k,), "mask")
    codes = np.zeros((rows, k // 2), dtype=np.uint8)
    meta = np.zeros((rows, k // 64), dtype=np.uint32)
    n_mask = 0
    m = None
    kept = np.zeros((rows, 0), dtype=np.uint16)
    if mask is not None:
        m = np.ascontiguousarray(mask, dtype=np.uint8)
        n_mask = int(np.count_nonzero(m))
        kept = np.zeros((rows, n_mask), dtype=np.uint16)
    rc = _lib().hif4o_quantize(_ptr(x), rows, k, k, _ptr(m), n_mask,
                               _ptr(kept) if n_mask else None, _ptr(codes), _ptr(meta))
    _check(rc, "quantize")
    return codes, meta, kept


def dequantize(codes: np.ndarray, meta: np.ndarray) -> np.ndarray:
    """Decode HiF4 codes [rows][k/2] + meta [rows][k/64] into float64 [rows][k]."""
    c = np.ascontiguousarray(codes, dtype=np.uint8)
    m = np.ascontiguousarray(meta, dtype=np.uint32)
    rows, k = c.shape[0], c.shape[1] * 2
    _shape(m, (rows, k // 64), "meta")
    out = np.zeros((rows, k), dtype=np.float64)
    _check(_lib().hif4o_dequantize(_ptr(c), _ptr(m), rows, k, _ptr(out)), "dequantize")
    return out


def linear(xc, xm, wc, wm, with_mag: bool = True):
    """Y = deq(Q(X)) deq(Q(W))^T in float64 from codes, plus S = sum |a||b|."""
    xc = np.ascontiguousarray(xc, dtype=np.uint8)
    xm = np.ascontiguousarray(xm, dtype=np.uint32)
    wc = np.ascontiguousarray(wc, dtype=np.uint8)
    wm = np.ascontiguousarray(wm, dtype=np.uint32)
    m, n, k = xc.shape[0], wc.shape[0], xc.shape[1] * 2
    if wc.shape[1] * 2 != k:
        raise OracleError("linear: K mismatch")
    _shape(xm, (m, k // 64), "x meta")
    _shape(wm, (n, k // 64), "w meta")
    y = np.zeros((m, n), dtype=np.float64)
    s = np.zeros((m, n), dtype=np.float64) if with_mag else None
    _check(_lib().hif4o_linear(_ptr(xc), _ptr(xm), _ptr(wc), _ptr(wm), m, n, k, _ptr(y), _ptr(s)),
           "linear")
    return (y, s) if with_mag else y


def linear_protected(xc, xm, xk, wc, wm, wk, with_mag: bool = True):
    """Y = deq(Q(X)) deq(Q(W))^T + xk wk^T in float64 (protected channels kept
    in bf16: xk [m][nk], wk [n][nk] as uint16 bit patterns), plus S."""
    xc = np.ascontiguousarray(xc, dtype=np.uint8)
    xm = np.ascontiguousarray(xm, dtype=np.uint32)
    wc = np.ascontiguousarray(wc, dtype=np.uint8)
    wm = np.ascontiguousarray(wm, dtype=np.uint32)
    m, n, k = xc.shape[0], wc.shape[0], xc.shape[1] * 2
    if wc.shape[1] * 2 != k:
        raise OracleError("linear_protected: K mismatch")
    _shape(xm, (m, k // 64), "x meta")
    _shape(wm, (n, k // 64), "w meta")
    nk = 0 if xk is None else xk.shape[1]
    xk = np.ascontiguousarray(xk if xk is not None else np.zeros((m, 0)), dtype=np.uint16)
    wk = np.ascontiguousarray(wk if wk is not None else np.zeros((n, 0)), dtype=np.uint16)
    _shape(xk, (m, nk), "x kept")
    _shape(wk, (n, nk), "w kept")
    y = np.zeros((m, n), dtype=np.float64)
    s = np.zeros((m, n), dtype=np.float64) if with_mag else None
    _check(_lib().hif4o_linear_protected(_ptr(xc), _ptr(xm), _ptr(xk), _ptr(wc), _ptr(wm), _ptr(wk),
                                         m, n, k, nk, _ptr(y), _ptr(s)), "linear_protected")
    return (y, s) if with_mag else y


def percentile(x_bits: np.ndarray, q: float) -> np.ndarray:
    """Per-channel type-7 quantile at level q of |x| over the rows -> float32 [c]."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, c = x.shape
    stats = np.zeros((c,), dtype=np.float32)
    _check(_lib().hif4o_percentile(_ptr(x), rows, c, c, float(q), _ptr(stats)), "percentile")
    return stats


def topn_mask(stats: np.ndarray, n_protect: int) -> np.ndarray:
    """u8 mask [c]: 1 for the n_protect largest stats, ties to the lower index."""
    s = np.ascontiguousarray(stats, dtype=np.float32)
    mask = np.zeros((s.shape[0],), dtype=np.uint8)
    _check(_lib().hif4o_topn_mask(_ptr(s), s.shape[0], int(n_protect), _ptr(mask)), "topn_mask")
    return mask


def bf16_bits_to_float(bits: np.ndarray) -> np.ndarray:
    """Exact float32 values of bf16 bit patterns (a plain bit move)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def quantize_f32(x: np.ndarray):
    """HiF4-quantize rows of float32 values [rows][k] along k (same rule as
    ``quantize``, on the exact values of the floats). Returns (codes, meta)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    rows, k = x.shape
    codes = np.zeros((rows, k // 2), np.uint8)
    meta = np.zeros((rows, k // 64), np.uint32)
    _check(_lib().hif4o_quantize_f32(_ptr(x), rows, k, k, _ptr(codes), _ptr(meta)),
           "quantize_f32")
    return codes, meta


def quantize_offsets(x_bits: np.ndarray, koff: np.ndarray, moff: np.ndarray):
    """HiF4-quantize bf16 rows [rows][k] with given HiAutoRound offsets
    (HiFloat4 calibration article, section 3.2): koff float32 [rows][k/4], one
    per level-3 group, shifts the level-3 exponent by RZ(K); moff float32
    [rows][k] is added to each element's scaled magnitude before rounding.
    Returns (codes, meta)."""
    x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
    rows, k = x_bits.shape
    koff = np.ascontiguousarray(koff, dtype=np.float32)
    moff = np.ascontiguousarray(moff, dtype=np.float32)
    if koff.shape != (rows, k // 4) or moff.shape != (rows, k):
        raise ValueError("koff must be [rows][k/4] and moff [rows][k]")
    codes = np.zeros((rows, k // 2), np.uint8)
    meta = np.zeros((rows, k // 64), np.uint32)
    _check(_lib().hif4o_quantize_offsets(_ptr(x_bits), rows, k, k, _ptr(koff), _ptr(moff),
                                         _ptr(codes), _ptr(meta)), "quantize_offsets")
    return codes, meta


def higptq_unit(w: np.ndarray, u: np.ndarray, unit: int, codes: np.ndarray, meta: np.ndarray,
                scheme: int = 1, margin: np.ndarray = None):
    """One HiGPTQ step (scheme 1, 2 or 3) in place (see hif4_oracle.c):
    quantize group ``unit`` of the working weights ``w`` (float64 [n][k],
    C-contiguous) and compensate the later columns with the upper factor
    ``u`` (H^-1 = u^T u). ``margin`` (float64 [n], optional) receives each
    row's smallest relative distance of a decision on updated values to its
    boundary (+inf when no decision reads updated values)."""
    n, k = w.shape
    if w.dtype != np.float64 or not w.flags.c_contiguous:
        raise OracleError("higptq_unit: w must be C-contiguous float64")
    uu = np.ascontiguousarray(u, dtype=np.float64)
    _shape(uu, (k, k), "higptq_unit u")
    _shape(codes, (n, k // 2), "higptq_unit codes")
    _shape(meta, (n, k // 64), "higptq_unit meta")
    if margin is not None:
        if margin.dtype != np.float64 or margin.shape != (n,) or not margin.flags.c_contiguous:
            raise OracleError("higptq_unit: margin must be a contiguous float64 array [n]")
    _check(_lib().hif4o_higptq_unit_scheme_margin(_ptr(w), n, k, _ptr(uu), int(unit), int(scheme),
                                                  _ptr(codes), _ptr(meta),
                                                  _ptr(margin) if margin is not None else None),
           "higptq_unit")


def higptq_run(w: np.ndarray, u: np.ndarray, unit0: int, units: int, codes: np.ndarray,
               meta: np.ndarray, scheme: int, margin: np.ndarray, accmag: np.ndarray):
    """Groups ``unit0 .. unit0 + units - 1`` in order, each exactly the step of
    ``higptq_unit``, in place on ``w`` (float64 [n][k]); ``margin`` (float64
    [n], start it at +inf) receives each row's smallest relative distance of a
    decision on a moved value to its boundary over the whole run, and
    ``accmag`` (float64 [n][k], start it at 0) the accumulated update sizes
    sum |f||U| per entry (see hif4_oracle.c)."""
    n, k = w.shape
    if w.dtype != np.float64 or not w.flags.c_contiguous:
        raise OracleError("higptq_run: w must be C-contiguous float64")
    uu = np.ascontiguousarray(u, dtype=np.float64)
    _shape(uu, (k, k), "higptq_run u")
    _shape(codes, (n, k // 2), "higptq_run codes")
    _shape(meta, (n, k // 64), "higptq_run meta")
    for a, shp, name in ((margin, (n,), "margin"), (accmag, (n, k), "accmag")):
        if a.dtype != np.float64 or a.shape != shp or not a.flags.c_contiguous:
            raise OracleError(f"higptq_run: {name} must be a contiguous float64 array {shp}")
    _check(_lib().hif4o_higptq_run_margin(_ptr(w), n, k, _ptr(uu), int(unit0), int(units),
                                          int(scheme), _ptr(codes), _ptr(meta), _ptr(margin),
                                          _ptr(accmag)),
           "higptq_run")


def higptq(w: np.ndarray, u: np.ndarray, scheme: int = 1):
    """HiGPTQ over every group of ``w`` [n][k] (any float dtype): returns
    (codes, meta, final working weights as float64)."""
    ww = np.array(w, dtype=np.float64, order="C")
    n, k = ww.shape
    codes = np.zeros((n, k // 2), np.uint8)
    meta = np.zeros((n, k // 64), np.uint32)
    for unit in range(k // 64):
        higptq_unit(ww, u, unit, codes, meta, scheme)
    return codes, meta, ww
