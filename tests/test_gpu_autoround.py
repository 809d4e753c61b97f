"""GPU parity of hif4_quantize_offsets (the quantize step of HiAutoRound, the
HiFloat4 calibration article, section 3.2) against the oracle: codes and meta
bit for bit."""
import numpy as np
import pytest
import torch

import oracle
import unit_cases as uc
import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def hip():
    from bit_block_float_amd import hif4
    hif4.require_gpu()
    return hif4


def _dev_bits(bits, ld=None):
    rows, k = bits.shape
    t = torch.from_numpy(bits.astype(np.int16)).view(torch.bfloat16).cuda()
    if ld is None or ld == k:
        return t.contiguous()
    full = torch.zeros((rows, ld), dtype=torch.bfloat16, device="cuda")
    full[:, :k] = t
    return full[:, :k]


def _offsets(rows, k, seed, kscale=2.5, mscale=1.0):
    r = np.random.default_rng(seed)
    koff = r.uniform(-kscale, kscale, size=(rows, k // 4)).astype(np.float32)
    # exact whole numbers and values just inside them, where trunc changes
    pick = r.random(size=koff.shape)
    koff[pick < 0.1] = np.float32(1.0)
    koff[(pick >= 0.1) & (pick < 0.2)] = np.float32(-1.0)
    koff[(pick >= 0.2) & (pick < 0.25)] = np.nextafter(np.float32(1.0), np.float32(0.0))
    moff = r.uniform(-mscale, mscale, size=(rows, k)).astype(np.float32)
    pm = r.random(size=moff.shape)
    moff[pm < 0.05] = np.float32(0.5)
    moff[(pm >= 0.05) & (pm < 0.1)] = np.float32(-0.5)
    moff[(pm >= 0.1) & (pm < 0.15)] = np.float32(0.0)
    return koff, moff


def _run(hip, bits, koff, moff, ld=None):
    x = _dev_bits(bits, ld)
    codes, meta = hip.quantize_offsets(x, torch.from_numpy(koff).cuda(),
                                       torch.from_numpy(moff).cuda())
    return codes.cpu().numpy(), meta.cpu().numpy().view(np.uint32)


def _check(hip, bits, koff, moff, ld=None):
    c, m = _run(hip, bits, koff, moff, ld)
    rc, rm = oracle.quantize_offsets(bits, koff, moff)
    assert np.array_equal(m, rm), np.argwhere(m != rm)[:5]
    assert np.array_equal(c, rc), np.argwhere(c != rc)[:5]


def test_zero_offsets_equal_hif4_quantize(hip):
    bits = workloads.bits(workloads.heavy_tailed_x(37, 320, seed=3))
    rows, k = bits.shape
    z4, z = np.zeros((rows, k // 4), np.float32), np.zeros((rows, k), np.float32)
    c, m = _run(hip, bits, z4, z, ld=328)
    qc, qm, _ = hip.quantize(_dev_bits(bits, 328))
    assert np.array_equal(c, qc.cpu().numpy())
    assert np.array_equal(m, qm.cpu().numpy().view(np.uint32))
    _check(hip, bits, z4, z, ld=328)


@pytest.mark.parametrize("rows,k,ld,seed", [(1, 64, None, 1), (7, 192, 200, 2), (130, 640, None, 3),
                                            (513, 1024, 1032, 4), (64, 5120, None, 5)])
def test_random_offsets_match_oracle(hip, rows, k, ld, seed):
    bits = workloads.bits(workloads.heavy_tailed_x(rows, k, seed=seed + 100))
    koff, moff = _offsets(rows, k, seed)
    _check(hip, bits, koff, moff, ld)


def test_offsets_on_grid_midpoints_and_special_values(hip):
    bits = np.concatenate([uc.midpoint_bits(64, 7, oracle.e6m2_value),
                           uc.special_values_bits(9), uc.random_bits(64, 10)])
    rows, k = bits.shape
    for seed, ks, ms in ((11, 2.5, 1.0), (12, 100.0, 10.0), (13, 0.99, 0.49), (14, 3.0, 1e-6)):
        koff, moff = _offsets(rows, k, seed, ks, ms)
        _check(hip, bits, koff, moff)


def test_offsets_saturate_and_vanish(hip):
    """Large positive offsets saturate every code at 7; large negative ones
    take every code to 0 (and K pushes every level-3 bit to 1 or 0)."""
    bits = workloads.bits(workloads.heavy_tailed_x(16, 256, seed=21))
    rows, k = bits.shape
    for kv, mv in ((8.0, 20.0), (-8.0, -20.0)):
        koff = np.full((rows, k // 4), kv, np.float32)
        moff = np.full((rows, k), mv, np.float32)
        c, m = _run(hip, bits, koff, moff)
        rc, rm = oracle.quantize_offsets(bits, koff, moff)
        assert np.array_equal(c, rc) and np.array_equal(m, rm)
        e3 = (m >> 16) & 0xFFFF
        assert np.all(e3 == (0xFFFF if kv > 0 else 0))
        mags = np.concatenate([c & 7, (c >> 4) & 7], axis=1)
        assert np.all(mags == (7 if mv > 0 else 0))


def test_full_weight_sampled_rows(hip):
    """The FFN-up weight (13,824 x 5120) in one call, as timed by the
    benchmark; 64 evenly spaced rows and the last one against the oracle."""
    spec = workloads.WORKLOADS["ffn_up"]
    n, k = spec["N"], spec["K"]
    w = workloads.normal_bf16(n, k, 0.02, device="cuda", seed=spec["index"] + 1000)
    g = torch.Generator(device="cuda").manual_seed(77)
    koff = (torch.rand((n, k // 4), generator=g, device="cuda") * 5.0 - 2.5).contiguous()
    moff = (torch.rand((n, k), generator=g, device="cuda") * 2.0 - 1.0).contiguous()
    codes, meta = hip.quantize_offsets(w, koff, moff)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([np.linspace(0, n - 1, 64).astype(int), [n - 1]]))
    bits = workloads.bits(w[rows])
    rc, rm = oracle.quantize_offsets(bits, koff[rows].cpu().numpy(), moff[rows].cpu().numpy())
    assert np.array_equal(codes[rows].cpu().numpy(), rc)
    assert np.array_equal(meta[rows].cpu().numpy().view(np.uint32), rm)
