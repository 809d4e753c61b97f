"""C-ABI contract of libhif4.so, checked without a GPU.

Loads the built library, checks that it exports exactly the entry points
declared in include/hif4.h, and that invalid arguments return the documented
status codes before any device work (no compute call reaches a kernel here).
"""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "hif4.h")
LIB = os.path.join(ROOT, "bit_block_float_amd", "libhif4.so")

OK, NULL, SHAPE, ALIGN, WORKSPACE, DTYPE, DEVICE, LAUNCH, ARG, SCRATCH = range(10)
A = 0x100000  # a 256-byte-aligned stand-in address; never dereferenced here


def declared():
    text = open(HEADER, encoding="utf-8").read()
    return set(re.findall(r"HIF4_EXPORT\s+[\w\s\*]+?\b(hif4_\w+)\s*\(", text))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(LIB):
        from bit_block_float_amd import build
        build.build()
    from bit_block_float_amd import hif4
    return hif4.lib()


def test_header_declares_the_four_entry_points():
    names = declared()
    for fn in ("hif4_quantize", "hif4_dequantize", "hif4_linear_w4a4", "hif4_percentile_mask",
               "hif4_linear_xcodes_wbf16", "hif4_linear_xcodes_wbf16_noalloc",
               "hif4_quantize_f32", "hif4_higptq_unit", "hif4_higptq_block",
               "hif4_quantize_offsets",
               "hif4_higptq_workspace_bytes", "hif4_higptq_block_workspace_bytes",
               "hif4_linear_workspace_bytes", "hif4_percentile_workspace_bytes",
               "hif4_status_string", "hif4_version"):
        assert fn in names


def test_library_exports_exactly_the_declared_symbols(L):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    hif4_syms = {s for s in exported if s.startswith("hif4_")}
    assert hif4_syms == declared()
    for s in declared():
        assert hasattr(L, s)


def test_probe_library_exports_exactly_its_header():
    """libhif4_probe.so (the measurement probes bench.py --ceilings runs)
    exports exactly the functions include/hif4_probe.h declares."""
    probe = os.path.join(ROOT, "bit_block_float_amd", "libhif4_probe.so")
    if not os.path.exists(probe):
        from bit_block_float_amd import build
        build.build_probe()
    text = open(os.path.join(ROOT, "include", "hif4_probe.h"), encoding="utf-8").read()
    want = set(re.findall(r'visibility\("default"\)\)\)\s+int\s+(hif4_probe_\w+)\s*\(', text))
    assert want >= {"hif4_probe_mfma_bf16", "hif4_probe_copy", "hif4_probe_read",
                    "hif4_probe_read4_write1"}
    out = subprocess.run(["nm", "-D", "--defined-only", probe], capture_output=True, text=True,
                         check=True).stdout
    got = {line.split()[-1] for line in out.splitlines()
           if " T " in line and line.split()[-1].startswith("hif4_")}
    assert got == want


def test_version_and_status_strings(L):
    assert L.hif4_version() == 1
    for s in range(10):
        assert L.hif4_status_string(s) and L.hif4_status_string(s) != b"unknown status"
    assert L.hif4_status_string(12345) == b"unknown status"


def test_quantize_argument_checks(L):
    q = L.hif4_quantize
    assert q(A, -1, 64, 64, None, 0, None, A, A, None) == SHAPE
    assert q(A, 4, 65, 72, None, 0, None, A, A, None) == SHAPE
    assert q(A, 4, 128, 64, None, 0, None, A, A, None) == SHAPE   # ld < k
    assert q(A, 0, 64, 64, None, 0, None, None, None, None) == OK  # empty: no work
    assert q(A, 4, 0, 0, None, 0, None, None, None, None) == OK
    assert q(None, 4, 64, 64, None, 0, None, A, A, None) == NULL
    assert q(A, 4, 64, 64, None, 0, None, None, A, None) == NULL
    assert q(A, 4, 64, 64, A, 3, None, A, A, None) == NULL         # kept missing
    assert q(A + 2, 4, 64, 64, None, 0, None, A, A, None) == ALIGN
    assert q(A, 4, 64, 68, None, 0, None, A, A, None) == ALIGN     # ld % 8
    assert q(A, 4, 64, 64, None, 0, None, A + 4, A, None) == ALIGN
    assert q(A, 4, 64, 64, None, 0, None, A, A + 2, None) == ALIGN
    assert q(A, 4, 64, 64, A + 8, 1, A, A, A, None) == ALIGN
    assert q(A, 4, 65536 + 64, 65536 + 64, A, 1, A, A, A, None) == SHAPE  # masked k limit
    assert q(A, 4, 64, 64, A, 65, A, A, A, None) == SHAPE          # n_mask > k


def test_dequantize_argument_checks(L):
    d = L.hif4_dequantize
    assert d(A, A, 4, 100, A, 0, None) == SHAPE
    assert d(A, A, 4, 64, A, 7, None) == DTYPE
    assert d(None, A, 4, 64, A, 0, None) == NULL
    assert d(A, A, 4, 64, A + 8, 0, None) == ALIGN
    assert d(A, A, 0, 64, None, 1, None) == OK


def test_linear_argument_checks(L):
    f = L.hif4_linear_w4a4
    ws = L.hif4_linear_workspace_bytes(8, 8, 64, 0)
    assert ws == 256 + 256 + 1024  # X codes, X meta, W bf16 (each 256-B aligned)
    assert L.hif4_linear_workspace_bytes(-1, 8, 64, 0) == 0
    assert L.hif4_linear_workspace_bytes(8, 8, 64, -1) == 0
    # protected channels add X kept, and Xr / Wr padded to 64 columns
    assert L.hif4_linear_workspace_bytes(8, 8, 64, 3) == ws + 256 + 1024 + 1024
    assert L.hif4_linear_workspace_bytes(8, 8, 0, 3) == 256 + 1024 + 1024

    def call(x=A, xc=None, xm=None, wc=A, wm=A, mask=None, xk=None, wk=None, nk=0, m=8, n=8, k=64,
             y=A, dt=0, w=A, wb=None):
        return f(x, xc, xm, wc, wm, mask, xk, wk, nk, m, n, k, y, dt, w,
                 ws if wb is None else wb, None)

    assert call(k=60) == SHAPE
    assert call(dt=3) == DTYPE
    assert call(x=None) == NULL
    assert call(wc=None) == NULL
    assert call(y=None) == NULL
    assert call(wb=ws - 1) == WORKSPACE
    assert call(w=None) == WORKSPACE
    assert call(w=A + 16) == ALIGN
    assert call(x=A + 2) == ALIGN
    assert call(m=0, w=None, wb=0) == OK
    # protected channels
    assert call(nk=65) == SHAPE                          # n_kept > k
    assert call(nk=-1) == SHAPE
    wsk = L.hif4_linear_workspace_bytes(8, 8, 64, 3)
    assert call(nk=3, mask=A, wk=None, wb=wsk) == NULL   # w_kept missing
    assert call(nk=3, mask=None, wk=A, wb=wsk) == NULL   # bf16 X needs the mask
    assert call(x=None, xc=A, xm=A, nk=3, wk=A, wb=wsk) == NULL  # codes X needs x_kept
    assert call(nk=3, mask=A + 8, wk=A, wb=wsk) == ALIGN
    assert call(nk=3, mask=A, wk=A + 1, wb=wsk) == ALIGN
    assert call(nk=3, mask=A, wk=A, wb=wsk - 1) == WORKSPACE
    assert call(nk=3, mask=A, wk=A, k=65536 + 64, wb=1 << 40) == SHAPE  # gather limit


def test_linear_xcodes_wbf16_argument_checks(L):
    f = L.hif4_linear_xcodes_wbf16

    def call(xc=A, xm=A, w=A, xk=None, wk=None, nk=0, m=8, n=8, k=64, y=A, dt=0, ws=None, wb=0):
        return f(xc, xm, w, xk, wk, nk, m, n, k, y, dt, ws, wb, None)

    assert call(k=60) == SHAPE
    assert call(m=-1) == SHAPE
    assert call(dt=2) == DTYPE
    assert call(xc=None) == NULL
    assert call(xm=None) == NULL
    assert call(w=None) == NULL
    assert call(y=None) == NULL
    assert call(w=A + 8) == ALIGN
    assert call(xc=A + 8) == ALIGN
    assert call(xm=A + 2) == ALIGN
    assert call(m=0, y=None) == OK
    wsk = L.hif4_linear_workspace_bytes(8, 8, 0, 5)
    assert call(nk=5, xk=A) == NULL                      # w_kept missing
    assert call(nk=5, xk=A, wk=A) == WORKSPACE           # workspace missing
    assert call(nk=5, xk=A, wk=A, ws=A, wb=wsk - 1) == WORKSPACE
    assert call(nk=5, xk=A, wk=A, ws=A + 16, wb=wsk) == ALIGN
    assert call(nk=65, xk=A, wk=A, ws=A, wb=wsk) == SHAPE


def test_linear_xcodes_wbf16_noalloc_argument_checks(L):
    """The allocation-free variant: the same checks minus the workspace, and
    problems whose protected-channel operands exceed the static scratch
    (32 MiB) are refused before any device work."""
    f = L.hif4_linear_xcodes_wbf16_noalloc
    limit = 32 << 20

    def call(xc=A, xm=A, w=A, xk=None, wk=None, nk=0, m=8, n=8, k=64, y=A, dt=0):
        return f(xc, xm, w, xk, wk, nk, m, n, k, y, dt, None)

    assert call(k=60) == SHAPE
    assert call(dt=2) == DTYPE
    assert call(xc=None) == NULL
    assert call(y=None) == NULL
    assert call(w=A + 8) == ALIGN
    assert call(m=0, y=None) == OK
    assert call(nk=5, xk=A) == NULL                      # w_kept missing
    assert call(nk=5, xk=A, wk=A + 1) == ALIGN
    assert call(nk=65, xk=A, wk=A) == SHAPE
    # (m + n) * 2 * kr bytes (256-byte aligned parts) against the limit
    rows = limit // (2 * 64)  # kr = 64: exactly the limit for m + n = rows
    assert call(nk=64, xk=A, wk=A, m=rows - 256 + 1, n=256, k=64) == SCRATCH
    assert call(nk=128, xk=A, wk=A, m=rows // 2, n=8, k=128) == SCRATCH
    assert call(nk=65, xk=A, wk=A, m=rows // 2, n=8, k=128) == SCRATCH  # kr = 128


def test_percentile_argument_checks(L):
    f = L.hif4_percentile_mask
    ws = L.hif4_percentile_workspace_bytes(100, 256)
    assert ws >= 256 * (256 + 128 + 1) * 4
    assert f(A, 0, 256, 256, 0.5, 1, A, A, A, ws, None) == SHAPE
    assert f(A, 100, 256, 256, 0.5, 257, A, A, A, ws, None) == SHAPE
    assert f(A, 100, 256, 200, 0.5, 1, A, A, A, ws, None) == SHAPE
    assert f(A, 100, 256, (1 << 22) + 8, 0.5, 1, A, A, A, ws, None) == SHAPE  # ld limit
    assert f(A, 100, 256, 256, 1.5, 1, A, A, A, ws, None) == ARG
    assert f(A, 100, 256, 256, float("nan"), 1, A, A, A, ws, None) == ARG
    assert f(A, 100, 256, 256, 0.5, 1, None, A, A, ws, None) == NULL
    assert f(A, 100, 256, 260, 0.5, 1, A, A, A, ws, None) == ALIGN
    assert f(A, 100, 256, 256, 0.5, 1, A, A, A, ws - 1, None) == WORKSPACE
    assert f(A, 1 << 32, 256, 256, 0.5, 1, A, A, A, ws, None) == SHAPE  # u32 counters


def test_percentile_workspace_grows_with_rows(L):
    """Long columns (>= 8192 rows) add the one-pass path's per-segment
    partials: 2 per (slab, 128-channel block), 128 x 288 u32 each (per
    channel 256 packed bin words, the below count and padding to whole
    128-byte lines). For
    57,600 x 5120 the slabs are 9000 rows (57,600 x 40 blocks over 256
    workgroups): 7 slabs x 40 blocks x 2 = 560 partials."""
    w = L.hif4_percentile_workspace_bytes
    assert w(8191, 5120) == w(100, 5120)
    assert w(57600, 5120) - w(100, 5120) == 560 * 128 * 288 * 4


def test_quantize_f32_argument_checks(L):
    q = L.hif4_quantize_f32
    assert q(A, 4, 65, 72, A, A, None) == SHAPE
    assert q(A, 4, 128, 64, A, A, None) == SHAPE            # ld < k
    assert q(A, 0, 64, 64, None, None, None) == OK         # empty: no work
    assert q(None, 4, 64, 64, A, A, None) == NULL
    assert q(A, 4, 64, 64, None, A, None) == NULL
    assert q(A + 4, 4, 64, 64, A, A, None) == ALIGN
    assert q(A, 4, 64, 66, A, A, None) == ALIGN             # ld % 4
    assert q(A, 4, 64, 64, A + 8, A, None) == ALIGN


def test_quantize_offsets_argument_checks(L):
    q = L.hif4_quantize_offsets

    def call(x=A, rows=4, k=64, ld=64, ko=A, mo=A, c=A, m=A):
        return q(x, rows, k, ld, ko, mo, c, m, None)
    assert call(k=65, ld=72) == SHAPE
    assert call(k=128, ld=64) == SHAPE                      # ld < k
    assert call(rows=-1) == SHAPE
    assert call(rows=0, x=None, ko=None, mo=None, c=None, m=None) == OK  # empty
    assert call(x=None) == NULL
    assert call(ko=None) == NULL
    assert call(mo=None) == NULL
    assert call(c=None) == NULL
    assert call(x=A + 8) == ALIGN
    assert call(ld=68) == ALIGN                             # ld % 8
    assert call(ko=A + 8) == ALIGN
    assert call(mo=A + 4) == ALIGN
    assert call(m=A + 2) == ALIGN


def test_higptq_argument_checks(L):
    f = L.hif4_higptq_unit
    ws = L.hif4_higptq_workspace_bytes(10)
    assert ws == 2560  # 10 rows x 64 fp32 (a multiple of 256 bytes)
    assert L.hif4_higptq_workspace_bytes(-1) == 0

    def call(w=A, n=10, k=128, ldw=128, u=A, ldu=128, unit=0, scheme=1, c=A, m=A, wsp=A, wb=None):
        return f(w, n, k, ldw, u, ldu, unit, scheme, c, m, wsp, ws if wb is None else wb, None)

    assert call(k=96) == SHAPE
    assert call(k=0) == SHAPE
    assert call(ldw=64) == SHAPE
    assert call(ldu=64) == SHAPE
    assert call(ldw=1 << 22) == SHAPE  # strides below 2^22 (32-bit buffer offsets)
    assert call(ldu=1 << 22) == SHAPE
    assert call(ldw=(1 << 22) - 4) != SHAPE
    assert call(n=1 << 24) == SHAPE  # the compensation's grid holds 2^16 tiles of 256 rows
    assert call(unit=2) == ARG
    assert call(unit=-1) == ARG
    assert call(scheme=0) == ARG
    assert call(scheme=4) == ARG
    assert call(n=0, w=None) == OK
    assert call(w=None) == NULL
    assert call(u=None) == NULL
    assert call(w=A + 4) == ALIGN
    assert call(ldw=130) == ALIGN
    assert call(wsp=None) == WORKSPACE
    assert call(wb=ws - 1) == WORKSPACE
    assert call(wsp=A + 16) == ALIGN


def test_higptq_block_argument_checks(L):
    f = L.hif4_higptq_block
    ws = L.hif4_higptq_block_workspace_bytes(10, 3)
    assert ws == 3 * 64 * 64 * 4  # F^T: 3 groups x 64 rows of 64 (10 rows padded to 64) fp32
    assert L.hif4_higptq_block_workspace_bytes(65, 1) == 64 * 128 * 4
    assert L.hif4_higptq_block_workspace_bytes(10, 0) == 0
    assert L.hif4_higptq_block_workspace_bytes(10, 17) == 0
    assert L.hif4_higptq_block_workspace_bytes(-1, 2) == 0

    def call(w=A, n=10, k=256, ldw=256, u=A, ldu=256, unit0=1, units=3, scheme=1, c=A, m=A,
             wsp=A, wb=None):
        return f(w, n, k, ldw, u, ldu, unit0, units, scheme, c, m, wsp, ws if wb is None else wb,
                 None)

    assert call(k=96) == SHAPE
    assert call(ldw=128) == SHAPE
    assert call(ldu=1 << 22) == SHAPE
    assert call(n=1 << 24) == SHAPE
    assert call(units=0) == ARG
    assert call(units=17) == ARG
    assert call(unit0=2) == ARG  # 2 + 3 > 256 / 64
    assert call(unit0=-1) == ARG
    assert call(scheme=4) == ARG
    assert call(n=0, w=None) == OK
    assert call(u=None) == NULL
    assert call(w=A + 4) == ALIGN
    assert call(wsp=None) == WORKSPACE
    assert call(wb=ws - 1) == WORKSPACE
    assert call(units=2, wb=ws) != WORKSPACE  # a smaller block needs less
    assert call(wsp=A + 16) == ALIGN


def test_valid_call_without_gfx950_reports_device_error():
    """With no GPU visible a well-formed call must stop at the device check."""
    code = (
        "import ctypes, sys; sys.path.insert(0, %r)\n"
        "from bit_block_float_amd import hif4\n"
        "L = hif4.lib(); A = 0x100000\n"
        "print(L.hif4_dequantize(A, A, 4, 64, A, 0, None))\n" % ROOT)
    env = dict(os.environ, HIP_VISIBLE_DEVICES="-1", ROCR_VISIBLE_DEVICES="-1")
    try:
        import torch
        if torch.cuda.is_available():
            pytest.skip("a GPU is visible in this process environment")
    except ImportError:
        pass
    out = subprocess.run(["python", "-c", code], capture_output=True, text=True, env=env, timeout=120)
    assert out.returncode == 0, out.stderr
    assert int(out.stdout.strip().splitlines()[-1]) == DEVICE
