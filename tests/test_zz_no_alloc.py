"""The allocation-free linear entry point against the one with a workspace.

hif4_linear_xcodes_wbf16_noalloc stages the protected-channel operands in
the library's static device scratch instead of a caller workspace; it runs
the same kernels, so its Y must equal hif4_linear_xcodes_wbf16's bit for bit.
Two calls in a row share the scratch: the second (smaller) must not see the
first's contents. A call without protected channels needs no scratch.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from bit_block_float_amd import hif4 as H

pytestmark = pytest.mark.gpu


def _problem(m, n, k, n_kept, seed):
    x = workloads.heavy_tailed_x(m, k, device="cuda", seed=seed)
    wt = workloads.normal_bf16(n, k, 0.02, device="cuda", seed=seed + 1000)
    mask = torch.zeros(k, dtype=torch.uint8, device="cuda")
    if n_kept:
        g = torch.Generator(device="cpu")
        g.manual_seed(seed)
        mask[torch.randperm(k, generator=g)[:n_kept].cuda()] = 1
        xc, xm, xk = H.quantize(x, mask)
        wc, wm, wk = H.quantize(wt, mask)
    else:
        (xc, xm, _), (wc, wm, _) = H.quantize(x), H.quantize(wt)
        xk = wk = None
    wdeq = H.dequantize(wc, wm, out_dtype=torch.bfloat16)
    return dict(x=x, wt=wt, mask=mask, xc=xc, xm=xm, xk=xk, wc=wc, wm=wm, wk=wk, wdeq=wdeq)


def _with_workspace(p, y_dtype):
    return H.linear_xcodes_wbf16(p["xc"], p["xm"], p["wdeq"], x_kept=p["xk"], w_kept=p["wk"],
                                 y_dtype=y_dtype)


@pytest.mark.parametrize("y_dtype", [torch.float32, torch.bfloat16])
def test_noalloc_matches_workspace_entry_twice_in_a_row(hip, y_dtype):
    big = _problem(1000, 700, 512, 70, 31)     # 128 residual columns
    small = _problem(300, 260, 256, 13, 32)    # 64 residual columns, fewer rows
    y_big = torch.full((1000, 700), float("nan"), dtype=y_dtype, device="cuda")
    y_small = torch.full((300, 260), float("nan"), dtype=y_dtype, device="cuda")
    H.linear_xcodes_wbf16_noalloc(big["xc"], big["xm"], big["wdeq"], y_big,
                                  x_kept=big["xk"], w_kept=big["wk"])
    H.linear_xcodes_wbf16_noalloc(small["xc"], small["xm"], small["wdeq"], y_small,
                                  x_kept=small["xk"], w_kept=small["wk"])
    ref_big = _with_workspace(big, y_dtype)
    ref_small = _with_workspace(small, y_dtype)
    torch.cuda.synchronize()
    assert torch.equal(y_big, ref_big)
    assert torch.equal(y_small, ref_small)
    if y_dtype == torch.float32:
        # the small call against the oracle as well (protected channels in bf16)
        mk = small["mask"].cpu().numpy()
        xc, xm, xk = oracle.quantize(workloads.bits(small["x"]), mk)
        wc, wm, wk = oracle.quantize(workloads.bits(small["wt"]), mk)
        y_ref, s_ref = oracle.linear_protected(xc, xm, xk, wc, wm, wk)
        err = np.abs(y_small.cpu().numpy().astype(np.float64) - y_ref)
        assert np.all(err <= 1e-5 * s_ref)


def test_noalloc_without_protected_channels_and_limit(hip):
    p = _problem(257, 129, 320, 0, 33)
    y = torch.empty((257, 129), dtype=torch.float32, device="cuda")
    H.linear_xcodes_wbf16_noalloc(p["xc"], p["xm"], p["wdeq"], y)
    ref = _with_workspace(p, torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y, ref)
    # a problem whose residual operands exceed the static scratch is refused
    # before any work: (m + n) * 2 * 128 > 32 MiB
    m_big = (H.NOALLOC_SCRATCH_BYTES // 256) + 1
    st = H.lib().hif4_linear_xcodes_wbf16_noalloc(1 << 20, 1 << 20, 1 << 20, 1 << 20, 1 << 20,
                                                  100, m_big, 64, 256, 1 << 20, 0, None)
    assert st == 9
