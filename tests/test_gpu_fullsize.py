"""GPU parity at the full workload sizes (the shapes bench.py runs).

Quantize outputs and masks are compared in full, bit for bit. The linear
layer is compared on sampled rows (64 evenly spaced rows plus the rows that
hold the largest |x| of the outlier channels) over all N columns, since the
fp64 oracle cannot afford all M rows. The calibration percentile is compared
on sampled channels (all protected ones plus a spread of others) and checked
at every channel through properties that hold at any size.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu


def host_u32(t):
    return t.cpu().numpy().view(np.uint32)


def sample_rows(x, n=64):
    m = x.shape[0]
    rows = set(np.linspace(0, m - 1, n).astype(np.int64).tolist())
    amax = x.float().abs().amax(dim=1)
    rows.update(torch.topk(amax, 8).indices.cpu().tolist())  # outlier rows
    return np.array(sorted(rows), dtype=np.int64)


@pytest.mark.parametrize("name", ["attn", "ffn_up", "ffn_down"])
def test_quantize_full_activation(hip, name):
    w = workloads.WORKLOADS[name]
    print(f"[case] quantize X {name} {w['M']}x{w['K']}", flush=True)
    x = (workloads.heavy_tailed_x(w["M"], w["K"], device="cuda", seed=w["index"])
         if name != "ffn_down" else workloads.gelu_x(w["M"], w["K"], device="cuda", seed=w["index"]))
    codes, meta, _ = hip.quantize(x)
    xb = workloads.bits(x)
    del x
    c_o, m_o, _ = oracle.quantize(xb)
    assert np.array_equal(host_u32(meta), m_o)
    assert np.array_equal(codes.cpu().numpy(), c_o)


@pytest.mark.parametrize("name,y_dtype,via_codes", [("attn", torch.float32, False),
                                                    ("attn", torch.bfloat16, False),
                                                    ("ffn_up", torch.float32, True),
                                                    ("ffn_down", torch.float32, False)])
def test_linear_full_shape_sampled_rows(hip, name, y_dtype, via_codes):
    w = workloads.WORKLOADS[name]
    M, N, K = w["M"], w["N"], w["K"]
    print(f"[case] linear {name} {M}x{N}x{K} {y_dtype} codes={via_codes}", flush=True)
    x = (workloads.heavy_tailed_x(M, K, device="cuda", seed=w["index"])
         if name != "ffn_down" else workloads.gelu_x(M, K, device="cuda", seed=w["index"]))
    wt = workloads.normal_bf16(N, K, 0.015 if name == "ffn_down" else 0.02, device="cuda",
                               seed=w["index"] + 1000)
    wcodes, wmeta, _ = hip.quantize(wt)
    if via_codes:
        xcodes, xmeta, _ = hip.quantize(x)
        y = hip.linear_w4a4(wcodes, wmeta, x_codes=xcodes, x_meta=xmeta, y_dtype=y_dtype)
    else:
        y = hip.linear_w4a4(wcodes, wmeta, x=x, y_dtype=y_dtype)
    rows = sample_rows(x)
    xs = workloads.bits(x[torch.from_numpy(rows).cuda()])
    wb = workloads.bits(wt)
    y_rows = y[torch.from_numpy(rows).cuda()].float().cpu().numpy().astype(np.float64)
    del x, y
    xc, xm, _ = oracle.quantize(xs)
    wc, wm, _ = oracle.quantize(wb)
    assert np.array_equal(wcodes.cpu().numpy(), wc)
    y_ref, s_ref = oracle.linear(xc, xm, wc, wm)
    tol = 1e-5 * s_ref + (2.0 ** -8 * np.abs(y_ref) if y_dtype == torch.bfloat16 else 0.0)
    err = np.abs(y_rows - y_ref)
    assert np.all(err <= tol), f"max excess {np.max(err - tol)}"


def test_linear_ffn_down_same_sign_full_k(hip, capsys):
    """Same-sign contraction at the full FFN-down depth (K = 13,824: 864
    sequential fp32 MFMA accumulations per output, whose worst-case bound
    ~864 * 2^-24 = 5.1e-5 of sum |a||b| exceeds the tolerance): GELU
    activations against |W|, so partial sums grow monotonically and rounding
    errors cannot cancel by sign; eight rows are near-constant (every entry
    within a few bf16 steps of 1). Sampled rows against the oracle within
    1e-5 * sum |a||b|; the measured ratio is printed."""
    w = workloads.WORKLOADS["ffn_down"]
    M, N, K = w["M"], w["N"], w["K"]
    print(f"[case] same-sign linear {M}x{N}x{K}", flush=True)
    x = workloads.gelu_x(M, K, device="cuda", seed=w["index"])
    # near-constant rows: every entry within a few bf16 steps of 1.0
    g = torch.Generator(device="cuda")
    g.manual_seed(7)
    x[:8] = (1.0 + torch.randint(0, 4, (8, K), generator=g, device="cuda") * 2.0 ** -7).to(torch.bfloat16)
    wt = workloads.normal_bf16(N, K, 0.015, device="cuda", seed=w["index"] + 1000).abs()
    wcodes, wmeta, _ = hip.quantize(wt)
    y = hip.linear_w4a4(wcodes, wmeta, x=x)
    rows = np.unique(np.concatenate([np.arange(8), sample_rows(x)]))
    xs = workloads.bits(x[torch.from_numpy(rows).cuda()])
    y_rows = y[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    wb = workloads.bits(wt)
    del x, y
    xc, xm, _ = oracle.quantize(xs)
    wc, wm, _ = oracle.quantize(wb)
    y_ref, s_ref = oracle.linear(xc, xm, wc, wm)
    ratio = np.abs(y_rows - y_ref) / s_ref
    with capsys.disabled():
        print(f"\n[same-sign K=13824] max |dY|/S = {ratio.max():.3e}, mean {ratio.mean():.3e}, "
              f"near-constant rows max {ratio[:8].max():.3e}, "
              f"|Y|/S min {np.min(np.abs(y_ref) / s_ref):.3f}", flush=True)
    assert np.all(ratio <= 1e-5), f"max |dY|/S {ratio.max():.3e}"


def test_linear_ffn_up_protected_channels(hip):
    """The whole method at the FFN-up shape: the percentile mask of X (52
    channels), W and X quantized with it, the linear with the bf16 residual;
    sampled rows against the oracle."""
    w = workloads.WORKLOADS["ffn_up"]
    M, N, K = w["M"], w["N"], w["K"]
    x = workloads.heavy_tailed_x(M, K, device="cuda", seed=w["index"])
    wt = workloads.normal_bf16(N, K, 0.02, device="cuda", seed=w["index"] + 1000)
    _, mask = hip.percentile_mask(x, w["q"], w["n_protect"])
    wcodes, wmeta, wkept = hip.quantize(wt, mask)
    xcodes, xmeta, xkept = hip.quantize(x, mask)
    w_deq = hip.dequantize(wcodes, wmeta, out_dtype=torch.bfloat16)
    y = hip.linear_xcodes_wbf16(xcodes, xmeta, w_deq, x_kept=xkept, w_kept=wkept)
    rows = sample_rows(x)
    mk = mask.cpu().numpy()
    xs = workloads.bits(x[torch.from_numpy(rows).cuda()])
    y_rows = y[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    wb = workloads.bits(wt)
    del x, y
    xc, xm, xk = oracle.quantize(xs, mk)
    wc, wm, wk = oracle.quantize(wb, mk)
    assert np.array_equal(wkept.cpu().view(torch.int16).numpy().view(np.uint16), wk)
    y_ref, s_ref = oracle.linear_protected(xc, xm, xk, wc, wm, wk)
    err = np.abs(y_rows - y_ref)
    assert np.all(err <= 1e-5 * s_ref), f"max excess {np.max(err - 1e-5 * s_ref)}"


def _check_mask_properties(stats, mask, n_protect):
    assert int(mask.sum()) == n_protect
    on, off = stats[mask == 1], stats[mask == 0]
    if on.size and off.size:
        lo_on = on.min()
        assert lo_on >= off.max()
        # ties at the boundary go to the lower channel index
        tied_off = np.nonzero((mask == 0) & (stats == lo_on))[0]
        tied_on = np.nonzero((mask == 1) & (stats == lo_on))[0]
        if tied_off.size:
            assert tied_on.max() < tied_off.min()


def test_percentile_bench_batch(hip):
    """The bench's percentile call: one FFN-up batch (57600 x 5120), q=0.999."""
    w = workloads.WORKLOADS["ffn_up"]
    x = workloads.heavy_tailed_x(w["M"], w["K"], device="cuda", seed=w["index"])
    stats, mask = hip.percentile_mask(x, w["q"], w["n_protect"])
    s, mk = stats.cpu().numpy(), mask.cpu().numpy()
    _check_mask_properties(s, mk, w["n_protect"])
    chans = np.unique(np.concatenate([np.nonzero(mk)[0], np.linspace(0, w["K"] - 1, 200).astype(int)]))
    cols = workloads.bits(x[:, torch.from_numpy(chans).cuda()])
    ref = oracle.percentile(cols, w["q"])
    assert np.array_equal(s[chans].view(np.uint32), ref.view(np.uint32))


def test_percentile_calibration_pass_and_masked_weight(hip):
    """Calibration at full size: 16 x 57600 tokens x 5120 channels (9.4 GB),
    q = 0.999, top-1% mask; then the FFN-up weight quantized with that mask."""
    w = workloads.WORKLOADS["calib"]
    rows = w["batches"] * w["rows_per_batch"]
    print(f"[case] calibration {rows}x{w['C']}", flush=True)
    x = workloads.calib_x(w["batches"], w["rows_per_batch"], w["C"], device="cuda", seed=w["index"])
    stats, mask = hip.percentile_mask(x, w["q"], w["n_protect"])
    s, mk = stats.cpu().numpy(), mask.cpu().numpy()
    _check_mask_properties(s, mk, w["n_protect"])
    r = np.random.default_rng(0)
    chans = np.unique(np.concatenate([np.nonzero(mk)[0][:12], r.choice(w["C"], 12, replace=False)]))
    cols = workloads.bits(x[:, torch.from_numpy(chans).cuda()])
    del x
    ref = oracle.percentile(cols, w["q"])
    assert np.array_equal(s[chans].view(np.uint32), ref.view(np.uint32))

    wt = workloads.normal_bf16(w["N"], w["C"], 0.02, device="cuda", seed=w["index"] + 1000)
    codes, meta, kept = hip.quantize(wt, mask)
    c_o, m_o, k_o = oracle.quantize(workloads.bits(wt), mk)
    assert np.array_equal(host_u32(meta), m_o)
    assert np.array_equal(codes.cpu().numpy(), c_o)
    assert np.array_equal(kept.cpu().view(torch.int16).numpy().view(np.uint16), k_o)


def test_higptq_full_weight_sampled_rows(hip):
    """HiGPTQ scheme 1 over the full 13,824 x 5120 weight (80 groups) with a
    random inverse-Hessian factor: every step checked on 96 sampled rows
    against the oracle started from the GPU's own weights (the rows of the
    method are independent of each other)."""
    from test_gpu_higptq import _check_steps

    spec = workloads.WORKLOADS["higptq"]
    n, k = spec["N"], spec["K"]
    w = workloads.normal_bf16(n, k, 0.02, device="cpu", seed=spec["index"]).float().numpy()
    u = workloads.higptq_factor(k, device="cpu", seed=spec["index"]).numpy()
    rows = np.linspace(0, n - 1, 96).astype(np.int64)
    _check_steps(hip, w, u, rows=rows)


def test_higptq_scheme3_full_weight_sampled_rows(hip, capsys):
    """Scheme 3 (4 columns at a time) over the full weight: every step checked
    on 64 sampled rows against the oracle's step from the same rows (the
    trajectory check for rows within rounding of a decision; see
    test_gpu_higptq)."""
    from test_gpu_higptq import _check_scheme_step_oracle

    spec = workloads.WORKLOADS["higptq"]
    n, k = spec["N"], spec["K"]
    w = workloads.normal_bf16(n, k, 0.02, device="cuda", seed=spec["index"]).float().contiguous()
    u = workloads.higptq_factor(k, device="cuda", seed=spec["index"])
    U64 = u.cpu().numpy().astype(np.float64)
    codes = torch.zeros((n, k // 2), dtype=torch.uint8, device="cuda")
    meta = torch.zeros((n, k // 64), dtype=torch.int32, device="cuda")
    ws = torch.empty((hip.higptq_workspace_bytes(n),), dtype=torch.uint8, device="cuda")
    rows = torch.from_numpy(np.linspace(0, n - 1, 64).astype(np.int64)).cuda()
    fallback = 0
    for unit in range(k // 64):
        before = w[rows].cpu().numpy()
        hip.higptq_unit(w, u, unit, codes, meta, workspace=ws, scheme=3)
        torch.cuda.synchronize()
        F = ws[:n * 64 * 4].view(torch.float32).view(n, 64)[rows].cpu().numpy().astype(np.float64)
        fallback += _check_scheme_step_oracle(before, w[rows].cpu().numpy(),
                                              codes[rows, 32 * unit:32 * unit + 32].cpu().numpy(),
                                              host_u32(meta[rows])[:, unit], F, U64, unit, 3)
    with capsys.disabled():
        print(f"\n[higptq scheme 3, full weight] row-steps checked on the trajectory instead of "
              f"exactly against the oracle: {fallback} of {64 * (k // 64)}", flush=True)
    assert fallback < 64 * (k // 64) // 20
