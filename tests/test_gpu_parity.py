"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Sizes here are small enough for the oracle to finish in seconds while still
spanning several tiles and ragged tails. Codes, meta, masks and percentile
statistics must be bit-exact; the linear layer must satisfy
|Y - Y_ref| <= 1e-5 * sum_t |a||b| per output (fp32 output), plus 2^-8 |Y_ref|
for bf16 output (its own rounding).
"""
import numpy as np
import pytest
import torch

import oracle
import unit_cases as uc
import workloads

pytestmark = pytest.mark.gpu


def dev_bf16(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16).cuda()


def host_u32(t):
    return t.cpu().numpy().view(np.uint32)


def host_bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def gpu_quantize(hip, bits, mask=None):
    x = dev_bf16(bits)
    m = torch.from_numpy(mask).cuda() if mask is not None else None
    codes, meta, kept = hip.quantize(x, m)
    torch.cuda.synchronize()
    return codes.cpu().numpy(), host_u32(meta), (host_bits(kept) if kept is not None else None)


def assert_same_quant(hip, bits, mask=None):
    c_g, m_g, k_g = gpu_quantize(hip, bits, mask)
    c_o, m_o, k_o = oracle.quantize(bits, mask)
    bad = np.nonzero(m_g != m_o)
    assert np.array_equal(m_g, m_o), f"meta differs at {bad[0][:5]}, {bad[1][:5]}"
    assert np.array_equal(c_g, c_o), f"codes differ at {np.nonzero(c_g != c_o)[0][:5]}"
    if mask is not None and k_o.shape[1]:
        assert np.array_equal(k_g, k_o)


# ---------------------------------------------------------------- quantize

def test_quantize_tiny_workload(hip):
    t = workloads.workload("tiny")
    assert_same_quant(hip, workloads.bits(t["x"]))
    assert_same_quant(hip, workloads.bits(t["w"]))


def test_quantize_every_bf16_magnitude_as_unit_max(hip):
    assert_same_quant(hip, uc.all_magnitudes_as_unit_max())
    assert_same_quant(hip, uc.all_magnitudes_as_unit_max(position=63, negative=True))


@pytest.mark.parametrize("c", [0, 1, 2, 3, 60, 101, 102, 103, 124, 126, 127, 200, 251, 254, 255])
def test_quantize_every_bf16_rounded_under_each_mantissa(hip, c):
    assert_same_quant(hip, uc.all_magnitudes_under_code(c, oracle.e6m2_value))


def test_quantize_random_and_tie_units(hip):
    assert_same_quant(hip, uc.random_bits(4096, seed=1))
    assert_same_quant(hip, uc.random_bits(4096, seed=2, spread=12.0))
    assert_same_quant(hip, uc.midpoint_bits(512, seed=3, e6m2_value=oracle.e6m2_value))
    assert_same_quant(hip, uc.special_values_bits())


@pytest.mark.parametrize("rows,k", [(1, 64), (3, 320), (257, 192), (1000, 5120), (7, 13824)])
def test_quantize_ragged_shapes(hip, rows, k):
    bits = uc.random_bits(rows * k // 64, seed=rows + k).reshape(rows, k)
    assert_same_quant(hip, bits)


def test_quantize_strided_rows(hip):
    bits = uc.random_bits(50 * 12, seed=9).reshape(50, 768)
    x = dev_bf16(bits)[:, :512]  # row stride 768, k = 512
    codes, meta, _ = hip.quantize(x)
    c_o, m_o, _ = oracle.quantize(np.ascontiguousarray(bits[:, :512]))
    assert np.array_equal(host_u32(meta), m_o)
    assert np.array_equal(codes.cpu().numpy(), c_o)


def test_quantize_empty_is_a_no_op(hip):
    x = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    codes, meta, _ = hip.quantize(x)
    assert codes.shape == (0, 64) and meta.shape == (0, 2)


def test_quantize_with_mask_and_kept(hip):
    bits = uc.random_bits(64 * 8, seed=11).reshape(64, 512)
    r = np.random.default_rng(12)
    for n in (0, 1, 7, 26):
        mask = np.zeros(512, np.uint8)
        mask[r.choice(512, size=n, replace=False)] = 1 + r.integers(0, 200, size=n)
        assert_same_quant(hip, bits, mask)


@pytest.mark.parametrize("rows,k,n", [(3, 13824, 52), (2, 16384, 100), (5, 16448, 300),
                                      (2, 40960, 9), (2, 65536, 655), (4, 1024, 1024)])
def test_quantize_with_mask_wide_rows(hip, rows, k, n):
    """Masked rows of 1 to 4 rounds of the row-mapped masked kernel, with idle
    lanes in the last wave (k / 16 not a multiple of 64), the widest
    single-round row (1024 items: the largest LDS stage), and a fully masked
    row."""
    bits = uc.random_bits(rows * k // 64, seed=k + n).reshape(rows, k)
    r = np.random.default_rng(k)
    mask = np.zeros(k, np.uint8)
    mask[r.choice(k, size=n, replace=False)] = 1
    assert_same_quant(hip, bits, mask)


@pytest.mark.parametrize("dense", [63, 64, 65, 200])
def test_quantize_with_mask_dense_and_sparse_waves(hip, dense):
    """A wave whose items hold `dense` masked channels (the first 1024
    channels: one wave's items) beside waves with a few: the kept values of
    waves with at most 64 go through the wave's LDS stage, the others one
    lane at a time, and the ranks run on across both."""
    k = 5120
    bits = uc.random_bits(9 * k // 64, seed=dense).reshape(9, k)
    r = np.random.default_rng(dense)
    mask = np.zeros(k, np.uint8)
    mask[r.choice(1024, size=dense, replace=False)] = 1
    mask[1024 + r.choice(k - 1024, size=40, replace=False)] = 1
    assert_same_quant(hip, bits, mask)


def test_quantize_deterministic(hip):
    bits = uc.random_bits(2048, seed=13).reshape(256, 512)
    a = gpu_quantize(hip, bits)
    b = gpu_quantize(hip, bits)
    assert all(np.array_equal(u, v) for u, v in zip(a[:2], b[:2]))


# -------------------------------------------------------------- dequantize

@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_dequantize_matches_oracle_exactly(hip, dtype):
    bits = uc.random_bits(1024, seed=21, spread=8.0).reshape(128, 512)
    c_o, m_o, _ = oracle.quantize(bits)
    # plus arbitrary (non-canonical) codes: every nibble, every meta word
    r = np.random.default_rng(22)
    c_r = r.integers(0, 256, size=(64, 256), dtype=np.uint8)
    m_r = r.integers(0, 2**32, size=(64, 8), dtype=np.uint64).astype(np.uint32)
    for codes, meta in ((c_o, m_o), (c_r, m_r)):
        ref = oracle.dequantize(codes, meta)
        out = hip.dequantize(torch.from_numpy(codes).cuda(),
                             torch.from_numpy(meta.view(np.int32)).cuda(), out_dtype=dtype)
        got = out.float().cpu().numpy().astype(np.float64)
        assert np.array_equal(got, ref)
        assert np.array_equal(np.signbit(got), np.signbit(ref))


# ------------------------------------------------------------------ linear

def check_linear(y_gpu, y_ref, s_ref, bf16_out=False):
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    tol = 1e-5 * s_ref + (2.0 ** -8 * np.abs(y_ref) if bf16_out else 0.0)
    worst = np.max(err - tol)
    assert np.all(err <= tol), f"max excess {worst}"


def run_linear_case(hip, xb, wb, y_dtype=torch.float32, via_codes=False):
    xc, xm, _ = oracle.quantize(xb)
    wc, wm, _ = oracle.quantize(wb)
    y_ref, s_ref = oracle.linear(xc, xm, wc, wm)
    w_codes = torch.from_numpy(wc).cuda()
    w_meta = torch.from_numpy(wm.view(np.int32)).cuda()
    if via_codes:
        y = hip.linear_w4a4(w_codes, w_meta, x_codes=torch.from_numpy(xc).cuda(),
                            x_meta=torch.from_numpy(xm.view(np.int32)).cuda(), y_dtype=y_dtype)
    else:
        y = hip.linear_w4a4(w_codes, w_meta, x=dev_bf16(xb), y_dtype=y_dtype)
    check_linear(y.float().cpu().numpy(), y_ref, s_ref, bf16_out=(y_dtype == torch.bfloat16))


def test_linear_tiny_workload(hip):
    t = workloads.workload("tiny")
    xb, wb = workloads.bits(t["x"]), workloads.bits(t["w"])
    run_linear_case(hip, xb, wb)
    run_linear_case(hip, xb, wb, via_codes=True)
    run_linear_case(hip, xb, wb, y_dtype=torch.bfloat16)


@pytest.mark.parametrize("m,n,k", [(300, 200, 320), (1, 1, 64), (257, 513, 128), (512, 256, 1024),
                                   (33, 700, 192)])
@pytest.mark.parametrize("via_codes", [False, True])
def test_linear_ragged_shapes(hip, m, n, k, via_codes):
    xb = workloads.bits(workloads.heavy_tailed_x(m, k, seed=m + n, outlier_channels=1))
    wb = workloads.bits(workloads.normal_bf16(n, k, 0.02, seed=k))
    run_linear_case(hip, xb, wb, via_codes=via_codes)


@pytest.mark.parametrize("m,n,k,n_kept", [(1, 1, 256, 0), (300, 260, 256, 0), (300, 260, 256, 5),
                                          (257, 130, 512, 0), (257, 130, 512, 70),
                                          (520, 300, 1280, 0), (64, 520, 2304, 129)])
def test_linear_unit_step_kernel_edges(hip, m, n, k, n_kept):
    """The unit-step contraction (K % 256 == 0) at its loop-structure edges:
    K = 256 (one block of four unit steps; with protected channels only the
    copy of the last four steps that fetches the residual), K = 512 (the first
    full 8-unit meta group), K = 1280 and 2304 (20 and 36 units: code groups
    and meta groups that end mid-group), one-output and ragged tiles, and 1 to
    3 residual chunks. Against the oracle, through the decoded-weight entry
    point (the bench's) and the codes entry point."""
    print(f"[case] unit-step {m}x{n}x{k} n_kept={n_kept}", flush=True)
    r = np.random.default_rng(m * 7 + n + k + n_kept)
    xb = workloads.bits(workloads.heavy_tailed_x(m, k, seed=m + k, outlier_channels=2))
    wb = workloads.bits(workloads.normal_bf16(n, k, 0.02, seed=n + k))
    if n_kept:
        mask = np.zeros(k, np.uint8)
        mask[r.choice(k, n_kept, replace=False)] = 1
        xc, xm, xk = oracle.quantize(xb, mask)
        wc, wm, wk = oracle.quantize(wb, mask)
        y_ref, s_ref = oracle.linear_protected(xc, xm, xk, wc, wm, wk)
        xkd, wkd = _bf16_dev(xk), _bf16_dev(wk)
    else:
        xc, xm, _ = oracle.quantize(xb)
        wc, wm, _ = oracle.quantize(wb)
        y_ref, s_ref = oracle.linear(xc, xm, wc, wm)
        xkd = wkd = None
    xcd, xmd = torch.from_numpy(xc).cuda(), torch.from_numpy(xm.view(np.int32)).cuda()
    wcd, wmd = torch.from_numpy(wc).cuda(), torch.from_numpy(wm.view(np.int32)).cuda()
    w_deq = hip.dequantize(wcd, wmd, out_dtype=torch.bfloat16)
    y1 = hip.linear_xcodes_wbf16(xcd, xmd, w_deq, x_kept=xkd, w_kept=wkd)
    check_linear(y1.cpu().numpy(), y_ref, s_ref)
    y2 = hip.linear_w4a4(wcd, wmd, x_codes=xcd, x_meta=xmd, x_kept=xkd, w_kept=wkd)
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


@pytest.mark.parametrize("m,n,k,n_kept", [(2304, 4096, 512, 0), (2304, 4096, 512, 70),
                                          (2304, 4093, 256, 3),   # odd N: element-wise stores
                                          (4608, 4096, 256, 0), (4608, 4096, 256, 5)])
def test_linear_whole_and_half_tiles(hip, m, n, k, n_kept):
    """Enough 256x256 tiles for the whole-tile kernel: 144 tiles (more than half
    of the MI355X's 256 CUs: whole tiles only) and 288 (one round of whole tiles,
    then the last 32 as 64 half tiles). Two rows of every tile row are checked
    against the oracle over all columns, so every tile and half tile is."""
    print(f"[case] tiles {m}x{n}x{k} n_kept={n_kept}", flush=True)
    r = np.random.default_rng(m + n + k + n_kept)
    xb = workloads.bits(workloads.heavy_tailed_x(m, k, seed=m + k + 1, outlier_channels=2))
    wb = workloads.bits(workloads.normal_bf16(n, k, 0.02, seed=n + k + 1))
    rows = np.sort(np.concatenate([np.arange(0, m, 256) + 17, np.arange(0, m, 256) + 230]))
    rows = rows[rows < m]
    if n_kept:
        mask = np.zeros(k, np.uint8)
        mask[r.choice(k, n_kept, replace=False)] = 1
        xc, xm, xk = oracle.quantize(xb, mask)
        wc, wm, wk = oracle.quantize(wb, mask)
        y_ref, s_ref = oracle.linear_protected(xc[rows], xm[rows], xk[rows], wc, wm, wk)
        xkd, wkd = _bf16_dev(xk), _bf16_dev(wk)
    else:
        xc, xm, _ = oracle.quantize(xb)
        wc, wm, _ = oracle.quantize(wb)
        y_ref, s_ref = oracle.linear(xc[rows], xm[rows], wc, wm)
        xkd = wkd = None
    xcd, xmd = torch.from_numpy(xc).cuda(), torch.from_numpy(xm.view(np.int32)).cuda()
    wcd, wmd = torch.from_numpy(wc).cuda(), torch.from_numpy(wm.view(np.int32)).cuda()
    w_deq = hip.dequantize(wcd, wmd, out_dtype=torch.bfloat16)
    y = hip.linear_xcodes_wbf16(xcd, xmd, w_deq, x_kept=xkd, w_kept=wkd)
    check_linear(y[torch.from_numpy(rows).cuda()].cpu().numpy(), y_ref, s_ref)


def random_units(rows, k, seed):
    """Arbitrary well-formed HiF4 units: every level-1 code, every micro-exponent
    pattern, every nibble (both signs, both zeros)."""
    r = np.random.default_rng(seed)
    codes = r.integers(0, 256, size=(rows, k // 2), dtype=np.uint8)
    c = r.integers(0, 256, size=(rows, k // 64), dtype=np.uint32)
    c.flat[:256] = np.arange(min(256, c.size), dtype=np.uint32)[: c.size]
    e2 = r.integers(0, 256, size=c.shape, dtype=np.uint32)
    e3 = r.integers(0, 1 << 16, size=c.shape, dtype=np.uint32)
    return codes, c | (e2 << 8) | (e3 << 16)


@pytest.mark.parametrize("m,n,k,y_dtype", [(300, 200, 320, torch.float32), (513, 257, 640, torch.float32),
                                           (260, 300, 128, torch.bfloat16),
                                           (300, 200, 512, torch.float32),   # K % 256 == 0: the
                                           (129, 257, 768, torch.bfloat16)])  # unit-step kernel
def test_linear_random_codes(hip, m, n, k, y_dtype):
    """Decode inside the GEMM over every level-1 code and exponent pattern."""
    xc, xm = random_units(m, k, 5)
    wc, wm = random_units(n, k, 6)
    y_ref, s_ref = oracle.linear(xc, xm, wc, wm)
    y = hip.linear_w4a4(torch.from_numpy(wc).cuda(), torch.from_numpy(wm.view(np.int32)).cuda(),
                        x_codes=torch.from_numpy(xc).cuda(),
                        x_meta=torch.from_numpy(xm.view(np.int32)).cuda(), y_dtype=y_dtype)
    check_linear(y.float().cpu().numpy(), y_ref, s_ref, bf16_out=(y_dtype == torch.bfloat16))


@pytest.mark.parametrize("m,n,k,y_dtype", [(300, 200, 320, torch.float32), (257, 513, 1024, torch.float32),
                                           (64, 96, 192, torch.bfloat16)])
def test_linear_with_decoded_weight_matches(hip, m, n, k, y_dtype):
    """hif4_linear_xcodes_wbf16 on W decoded by hif4_dequantize: the same
    bits as hif4_linear_w4a4, and the oracle's values."""
    xb = workloads.bits(workloads.heavy_tailed_x(m, k, seed=m + 7, outlier_channels=1))
    wb = workloads.bits(workloads.normal_bf16(n, k, 0.02, seed=n + 7))
    xc, xm, _ = oracle.quantize(xb)
    wc, wm, _ = oracle.quantize(wb)
    y_ref, s_ref = oracle.linear(xc, xm, wc, wm)
    xcd, xmd = torch.from_numpy(xc).cuda(), torch.from_numpy(xm.view(np.int32)).cuda()
    wcd, wmd = torch.from_numpy(wc).cuda(), torch.from_numpy(wm.view(np.int32)).cuda()
    w_deq = hip.dequantize(wcd, wmd, out_dtype=torch.bfloat16)
    y1 = hip.linear_xcodes_wbf16(xcd, xmd, w_deq, y_dtype=y_dtype)
    y2 = hip.linear_w4a4(wcd, wmd, x_codes=xcd, x_meta=xmd, y_dtype=y_dtype)
    assert torch.equal(y1.view(torch.int16 if y_dtype == torch.bfloat16 else torch.int32),
                       y2.view(torch.int16 if y_dtype == torch.bfloat16 else torch.int32))
    check_linear(y1.float().cpu().numpy(), y_ref, s_ref, bf16_out=(y_dtype == torch.bfloat16))


def _bf16_dev(bits_2d):
    return torch.from_numpy(np.ascontiguousarray(bits_2d).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("m,n,k,n_kept", [(300, 200, 320, 1), (257, 513, 640, 13), (64, 96, 256, 64),
                                          (33, 700, 192, 65), (260, 300, 1024, 139), (1, 1, 64, 64)])
@pytest.mark.parametrize("path", ["bf16_x", "codes", "decoded_w"])
def test_linear_protected_channels(hip, m, n, k, n_kept, path):
    """[TA-method]: protected channels stay in high precision. The HiF4
    product plus the bf16 residual over the masked channels, against the
    oracle, through each entry point (1 to 3 residual chunks of 64)."""
    print(f"[case] protected {path} {m}x{n}x{k} n_kept={n_kept}", flush=True)
    r = np.random.default_rng(m + n + k + n_kept)
    mask = np.zeros(k, np.uint8)
    mask[r.choice(k, n_kept, replace=False)] = 1
    xb = workloads.bits(workloads.heavy_tailed_x(m, k, seed=m + 3, outlier_channels=2))
    wb = workloads.bits(workloads.normal_bf16(n, k, 0.02, seed=n + 5))
    xc, xm, xk = oracle.quantize(xb, mask)
    wc, wm, wk = oracle.quantize(wb, mask)
    y_ref, s_ref = oracle.linear_protected(xc, xm, xk, wc, wm, wk)
    wcd, wmd = torch.from_numpy(wc).cuda(), torch.from_numpy(wm.view(np.int32)).cuda()
    xcd, xmd = torch.from_numpy(xc).cuda(), torch.from_numpy(xm.view(np.int32)).cuda()
    xkd, wkd = _bf16_dev(xk), _bf16_dev(wk)
    if path == "bf16_x":
        y = hip.linear_w4a4(wcd, wmd, x=dev_bf16(xb), mask=torch.from_numpy(mask).cuda(), w_kept=wkd)
    elif path == "codes":
        y = hip.linear_w4a4(wcd, wmd, x_codes=xcd, x_meta=xmd, x_kept=xkd, w_kept=wkd)
    else:
        w_deq = hip.dequantize(wcd, wmd, out_dtype=torch.bfloat16)
        y = hip.linear_xcodes_wbf16(xcd, xmd, w_deq, x_kept=xkd, w_kept=wkd)
    check_linear(y.cpu().numpy(), y_ref, s_ref)


def test_linear_binding_rejects_inconsistent_protection(hip):
    """The binding checks that the mask and the kept values agree before the
    library reads them (a short mask or kept tensor would be read past its
    end, and a mask with fewer channels than n_kept would feed uninitialized
    workspace into the residual)."""
    m, n, k, n_kept = 40, 24, 128, 3
    r = np.random.default_rng(5)
    mask = np.zeros(k, np.uint8)
    mask[r.choice(k, n_kept, replace=False)] = 1
    xb = workloads.bits(workloads.heavy_tailed_x(m, k, seed=9))
    wb = workloads.bits(workloads.normal_bf16(n, k, 0.02, seed=10))
    xc, xm, xk = oracle.quantize(xb, mask)
    wc, wm, wk = oracle.quantize(wb, mask)
    wcd, wmd = torch.from_numpy(wc).cuda(), torch.from_numpy(wm.view(np.int32)).cuda()
    xcd, xmd = torch.from_numpy(xc).cuda(), torch.from_numpy(xm.view(np.int32)).cuda()
    xkd, wkd = _bf16_dev(xk), _bf16_dev(wk)
    x, md = dev_bf16(xb), torch.from_numpy(mask).cuda()
    hip.linear_w4a4(wcd, wmd, x=x, mask=md, w_kept=wkd)  # consistent: accepted
    bad_calls = [
        lambda: hip.linear_w4a4(wcd, wmd, x=x, mask=md, w_kept=wkd[:, :2].contiguous()),
        lambda: hip.linear_w4a4(wcd, wmd, x=x, mask=md[:k - 1].contiguous(), w_kept=wkd),
        lambda: hip.linear_w4a4(wcd, wmd, x=x, mask=md.to(torch.int32), w_kept=wkd),
        lambda: hip.linear_w4a4(wcd, wmd, x=x, w_kept=wkd),
        lambda: hip.linear_w4a4(wcd, wmd, x=x, mask=md, w_kept=wkd[:n - 1].contiguous()),
        lambda: hip.linear_w4a4(wcd, wmd, x_codes=xcd, x_meta=xmd, w_kept=wkd),
        lambda: hip.linear_w4a4(wcd, wmd, x_codes=xcd, x_meta=xmd, x_kept=xkd[:m - 1].contiguous(),
                                w_kept=wkd),
        lambda: hip.linear_xcodes_wbf16(xcd, xmd, hip.dequantize(wcd, wmd, out_dtype=torch.bfloat16),
                                        w_kept=wkd),
    ]
    for i, call in enumerate(bad_calls):
        with pytest.raises(ValueError):
            call()
        print(f"[case] inconsistent protection {i} rejected", flush=True)


def test_linear_one_hot_weight_is_exact(hip):
    """W row j = a single 7 at column t: Y[:, j] = 7 * deq(Q(X))[:, t] exactly
    (one exact product per output, no rounding)."""
    xb = workloads.bits(workloads.heavy_tailed_x(300, 256, seed=3))
    xc, xm, _ = oracle.quantize(xb)
    a = oracle.dequantize(xc, xm)
    cols = [0, 5, 77, 128, 255, 31]
    w = np.zeros((len(cols), 256), np.uint16)
    for j, t in enumerate(cols):
        w[j, t] = uc.to_bits([7.0])[0]
    wc, wm, _ = oracle.quantize(w)
    y = hip.linear_w4a4(torch.from_numpy(wc).cuda(), torch.from_numpy(wm.view(np.int32)).cuda(),
                        x=dev_bf16(xb)).cpu().numpy()
    for j, t in enumerate(cols):
        assert np.array_equal(y[:, j].astype(np.float64), 7.0 * a[:, t])


def test_linear_empty_k_gives_zero(hip):
    w_codes = torch.zeros((5, 0), dtype=torch.uint8, device="cuda")
    w_meta = torch.zeros((5, 0), dtype=torch.int32, device="cuda")
    x = torch.zeros((3, 0), dtype=torch.bfloat16, device="cuda")
    y = torch.full((3, 5), 7.0, device="cuda")
    hip.linear_w4a4(w_codes, w_meta, x=x, y=y)
    assert torch.count_nonzero(y).item() == 0


# -------------------------------------------------------------- percentile

def window_misses(bits, q):
    """Channels the one-pass window path leaves to the exact passes, by the
    rule the header states: the window is the 512 keys starting one coarse bin
    (128 keys) below the coarse bin of rank floor(q (n_s - 1)) among every
    S-th row, S = max(8, ceil(rows / 8192)); a channel misses when its ranks
    lo or hi fall outside the window."""
    rows, c = bits.shape
    if rows < 8192:
        return c
    stride = max(8, -(-rows // 8192))
    k = (bits & 0x7FFF).astype(np.int64)
    s = np.sort(k[::stride], axis=0)
    b = s[int(np.floor(q * (s.shape[0] - 1)))] >> 7
    w = np.maximum(b - 1, 0) << 7
    lo = int(np.floor(q * (rows - 1)))
    hi = min(lo + 1, rows - 1)
    below = (k < w).sum(axis=0)
    inside = ((k >= w) & (k < w + 512)).sum(axis=0)
    return int((~((lo >= below) & (hi < below + inside))).sum())


def run_pct_case(hip, bits, q, n_protect, ld=None):
    x = dev_bf16(bits)
    if ld is not None:
        full = torch.zeros((bits.shape[0], ld), dtype=torch.bfloat16, device="cuda")
        full[:, :bits.shape[1]] = x
        x = full[:, :bits.shape[1]]
    rows, c = bits.shape
    ws = torch.empty((hip.percentile_workspace_bytes(rows, c),), dtype=torch.uint8, device="cuda")
    stats, mask = hip.percentile_mask(x, q, n_protect, workspace=ws)
    s_ref = oracle.percentile(bits, q)
    m_ref = oracle.topn_mask(s_ref, n_protect)
    s_gpu = stats.cpu().numpy()
    assert np.array_equal(s_gpu.view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(mask.cpu().numpy(), m_ref)
    # which path produced each statistic: the count is exact integer work too
    exact = hip.percentile_exact_channels(ws, rows, c)
    assert exact == window_misses(bits, q), (exact, window_misses(bits, q))
    return exact


def test_percentile_tiny_workload(hip):
    t = workloads.workload("tiny")
    run_pct_case(hip, workloads.bits(t["x"]), t["q"], t["n_protect"])


@pytest.mark.parametrize("rows,c,q,n", [(1, 64, 0.99, 3), (2, 128, 0.5, 0), (1000, 200, 0.999, 2),
                                        (777, 77, 0.0, 77), (4096, 384, 1.0, 10),
                                        (5000, 256, 0.75, 13), (50, 9000, 0.9, 90),
                                        (3, 65536, 0.5, 655)])
def test_percentile_ragged(hip, rows, c, q, n):
    bits = workloads.bits(workloads.heavy_tailed_x(rows, c, seed=rows + c, outlier_channels=2))
    ld = ((c + 7) // 8) * 8 if c % 8 else None
    run_pct_case(hip, bits, q, n, ld=ld)


def test_percentile_constant_and_tied_channels(hip):
    r = np.random.default_rng(31)
    x = uc.truncate_to_bits(r.standard_t(3, size=(3000, 256)))
    x[:, 10] = uc.to_bits([2.5])[0]          # constant channel
    x[:, 20] = x[:, 30]                       # duplicated channels -> tied stats
    x[:, 40] = x[:, 30] ^ np.uint16(0x8000)   # sign-flipped duplicate: same |x|
    run_pct_case(hip, x, 0.99, 40)
    run_pct_case(hip, x, 0.5, 128)


@pytest.mark.parametrize("rows,c,q,n", [(8192, 64, 0.999, 3), (10000, 300, 0.999, 3),
                                        (20000, 130, 0.5, 13), (9000, 64, 1.0, 5),
                                        (9001, 200, 0.0, 7), (12345, 77, 0.9, 1),
                                        (70001, 64, 0.999, 3), (200000, 24, 0.99, 2)])
def test_percentile_sampled_window_path(hip, rows, c, q, n):
    """Long columns (>= 8192 rows) take the one-pass path: a window of keys
    around the quantile of every S-th row (S = 8 up to 65,536 rows, 9 and 25
    for the two longest cases), exact whenever both ranks land in it."""
    bits = workloads.bits(workloads.heavy_tailed_x(rows, c, seed=rows + c, outlier_channels=2))
    ld = ((c + 7) // 8) * 8 if c % 8 else None
    exact = run_pct_case(hip, bits, q, n, ld=ld)
    if 0.0 < q < 1.0:
        assert exact == 0  # the window resolved every channel of these columns


def test_percentile_sampled_window_misled_falls_back(hip):
    """Channels whose sampled rows (every 8th) are unrepresentative: the
    window misses the true ranks, the exact passes run for those channels,
    and every statistic still matches."""
    r = np.random.default_rng(61)
    rows, c = 16384, 192
    x = np.abs(r.standard_normal((rows, c))).astype(np.float32)
    x[0::8, :40] *= 1e-6           # the sample sees tiny values, the rest is large
    x[1::8, 40:80] *= 1e6          # the sample misses a block of huge values
    x[:, 80:100] = 0.0
    x[0::8, 80:100] = 3.0          # only the sampled rows are non-zero
    bits = uc.truncate_to_bits(x.astype(np.float64))
    for q in (0.999, 0.5, 0.05):
        assert run_pct_case(hip, bits, q, 9) >= 20  # at least the 20 zero columns fall back


def test_percentile_sample_pass_in_several_blocks(hip):
    """A wide activation: 16,448 channels, i.e. 257 blocks of 64, so one
    sample part per block. With 11,400 rows (1,425 sampled, every 8th) that
    part is longer than the 1,408 rows one single-buffered block of the sample
    pass reads. The pass takes two blocks, the second one 17 rows long, and
    every statistic still matches."""
    r = np.random.default_rng(71)
    rows, c = 11400, 16448
    scale = np.exp(r.standard_normal(c)).astype(np.float32)
    x = r.standard_normal((rows, c), dtype=np.float32) * scale
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)  # bf16 by truncation
    assert run_pct_case(hip, bits, 0.999, 40) == 0


def test_percentile_ties_across_many_channels(hip):
    """Most channels share one statistic: the protected ties are the lowest
    channel indices, counted across every thread of the mask kernel."""
    r = np.random.default_rng(57)
    c = 3000
    x = np.full((40, c), uc.to_bits([1.5])[0], dtype=np.uint16)
    x[:, r.choice(c, 9, replace=False)] = uc.to_bits([3.0])[0]   # 9 channels above the tie
    x[:, r.choice(c, 30, replace=False)] = uc.to_bits([0.5])[0]  # some below it
    for n in (9, 10, 700, 2500):
        run_pct_case(hip, x, 0.9, n)


def test_percentile_wide_magnitude_range(hip):
    """Values spanning subnormals to huge bf16, and rank boundaries that fall
    exactly at coarse-bin edges."""
    r = np.random.default_rng(41)
    a = r.integers(0, 0x7F7F, size=(2001, 136)).astype(np.uint16)
    a[:, :8] = r.integers(0, 0x0100, size=(2001, 8)).astype(np.uint16)  # subnormal/tiny
    run_pct_case(hip, a, 0.999, 5)
    run_pct_case(hip, a, 0.5, 5)
