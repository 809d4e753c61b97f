"""GPU parity of the fp32 quantizer and of HiGPTQ scheme 1, through the C ABI.

HiGPTQ (the calibration article, section 3.1, scheme 1) quantizes one group
of 64 columns at once and then compensates the columns not yet quantized
(GPTQ's update with the upper factor U of H^-1). Each step is checked on the
GPU's own trajectory: the group's codes and meta must be exactly the oracle's
quantization of the weights the step started from, and the compensated
weights must match the oracle's fp64 step from the same start within
1e-5 * (sum_i |F_i||U_ic| + |W_c|) per entry (F = E U_SS^-1; the fp32
arithmetic's error measured on the CPU is below 4e-7 of that scale).
"""
import numpy as np
import pytest
import torch

import oracle
import unit_cases as uc
from test_oracle_pins import _gptq_problem

pytestmark = pytest.mark.gpu


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host_u32(t):
    return t.cpu().numpy().view(np.uint32)


def assert_same_f32_quant(hip, x, ld=None):
    xt = dev(x.astype(np.float32))
    if ld is not None:
        full = torch.zeros((x.shape[0], ld), dtype=torch.float32, device="cuda")
        full[:, :x.shape[1]] = xt
        xt = full[:, :x.shape[1]]
    codes, meta = hip.quantize_f32(xt)
    torch.cuda.synchronize()
    c_o, m_o = oracle.quantize_f32(x)
    assert np.array_equal(host_u32(meta), m_o)
    assert np.array_equal(codes.cpu().numpy(), c_o)


# ---------------------------------------------------------------- fp32 quantize

def test_quantize_f32_full_precision_random_and_ties(hip):
    r = np.random.default_rng(91)
    x = (r.standard_t(3, size=(3000, 64)) * np.exp(r.normal(0, 4, size=(3000, 1)))).astype(np.float32)
    x[r.random(size=x.shape) < 0.05] = 0.0
    for i in range(800):  # elements exactly on grid midpoints of their unit
        c = int(r.integers(0, 256))
        s = oracle.e6m2_value(c)
        x[i, :] = 0.0
        x[i, 0] = np.float32(7 * s)
        mids = (2 * r.integers(0, 7, size=56) + 1) * s / 8
        x[i, 8:] = (mids * np.where(r.random(56) < 0.5, -1, 1)).astype(np.float32)
    assert_same_f32_quant(hip, x.reshape(-1, 320))


def test_quantize_f32_special_values(hip):
    r = np.random.default_rng(92)
    x = np.zeros((64, 64), np.float32)
    tiny = np.float32(1e-45) * r.integers(1, 1000, size=(64, 64)).astype(np.float32)  # subnormals
    x[:16] = tiny[:16]
    x[16:32] = (r.standard_normal((16, 64)) * 1e30).astype(np.float32)  # level-1 saturation
    x[32:48] = -0.0
    x[48:] = np.float32(3.4e38) * np.sign(r.standard_normal((16, 64))).astype(np.float32)
    assert_same_f32_quant(hip, x)


def test_quantize_f32_on_bf16_values_equals_bf16_quantize(hip):
    bits = uc.random_bits(2000, seed=93).reshape(-1, 256)
    f = (bits.astype(np.uint32) << 16).view(np.float32)
    codes, meta = hip.quantize_f32(dev(f))
    codes_b, meta_b, _ = hip.quantize(dev(bits.view(np.int16)).view(torch.bfloat16))
    torch.cuda.synchronize()
    assert torch.equal(codes, codes_b) and torch.equal(meta, meta_b)


@pytest.mark.parametrize("rows,k,ld", [(1, 64, None), (3, 320, None), (257, 192, 196),
                                       (1000, 5120, None), (7, 13824, 13828)])
def test_quantize_f32_shapes(hip, rows, k, ld):
    r = np.random.default_rng(rows + k)
    x = (r.standard_normal((rows, k)) * np.exp(r.normal(0, 2, size=(rows, 1)))).astype(np.float32)
    assert_same_f32_quant(hip, x, ld)


# ---------------------------------------------------------------------- HiGPTQ

def _check_steps(hip, W, U, rows=None):
    """Run HiGPTQ on the GPU unit by unit; check every step (on `rows`, or all
    rows) against the oracle started from the GPU's own weights."""
    n, k = W.shape
    w = dev(W.astype(np.float32))
    u = dev(U.astype(np.float32))
    U64 = U.astype(np.float32).astype(np.float64)  # the values the GPU works with
    codes = torch.zeros((n, k // 2), dtype=torch.uint8, device="cuda")
    meta = torch.zeros((n, k // 64), dtype=torch.int32, device="cuda")
    ws = torch.empty((hip.higptq_workspace_bytes(n),), dtype=torch.uint8, device="cuda")
    sel = np.arange(n) if rows is None else rows
    seli = torch.from_numpy(sel).cuda()
    for unit in range(k // 64):
        s0, r0 = 64 * unit, 64 * unit + 64
        before = w[seli].cpu().numpy()
        hip.higptq_unit(w, u, unit, codes, meta, workspace=ws)
        torch.cuda.synchronize()
        after = w[seli].cpu().numpy()
        c_g = codes[seli].cpu().numpy()
        m_g = host_u32(meta[seli])
        # the group: exactly the quantization of the weights the step began with
        c_o, m_o = oracle.quantize_f32(before[:, s0:r0])
        assert np.array_equal(c_g[:, 32 * unit:32 * unit + 32], c_o), f"unit {unit} codes"
        assert np.array_equal(m_g[:, unit], m_o[:, 0]), f"unit {unit} meta"
        # columns up to the group's end are untouched
        assert np.array_equal(after[:, :r0], before[:, :r0])
        if r0 == k:
            continue
        # the compensation against the fp64 oracle step from the same start
        wo = before.astype(np.float64)
        co = np.zeros((len(sel), k // 2), np.uint8)
        mo = np.zeros((len(sel), k // 64), np.uint32)
        oracle.higptq_unit(wo, U64, unit, co, mo)
        E = before[:, s0:r0].astype(np.float64) - oracle.dequantize(c_o, m_o)
        F = np.linalg.solve(U64[s0:r0, s0:r0].T, E.T).T  # F U_SS = E
        scale = np.abs(F) @ np.abs(U64[s0:r0, r0:]) + np.abs(wo[:, r0:])
        err = np.abs(after[:, r0:].astype(np.float64) - wo[:, r0:])
        assert np.all(err <= 1e-5 * scale), f"unit {unit}: worst {np.max(err / scale):.3g}"
    return w, codes, meta


def test_higptq_steps_follow_the_oracle(hip):
    """200 rows (ragged against 64-row update tiles), 448 columns (7 groups;
    the column tiles of the updates end ragged)."""
    W, _, U = _gptq_problem(200, 448, 94)
    _check_steps(hip, W, U)


def test_higptq_identity_hessian_is_direct_quantization(hip):
    W, _, _ = _gptq_problem(96, 256, 95)
    w = dev(W)
    codes, meta = hip.higptq(w, dev(np.eye(256, dtype=np.float32)))
    torch.cuda.synchronize()
    c0, m0 = oracle.quantize_f32(W)
    assert np.array_equal(codes.cpu().numpy(), c0) and np.array_equal(host_u32(meta), m0)
    assert np.array_equal(w.cpu().numpy(), W)


def test_higptq_lowers_the_layer_output_error(hip):
    W, H, U = _gptq_problem(256, 512, 96)
    codes, meta = hip.higptq(dev(W), dev(U.astype(np.float32)))
    torch.cuda.synchronize()
    q = oracle.dequantize(codes.cpu().numpy(), host_u32(meta))
    c0, m0 = oracle.quantize_f32(W)
    E, E0 = W - q, W - oracle.dequantize(c0, m0)
    assert np.trace(E @ H @ E.T) < 0.8 * np.trace(E0 @ H @ E0.T)
