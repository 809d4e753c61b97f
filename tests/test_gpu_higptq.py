"""GPU parity of the fp32 quantizer and of HiGPTQ, through the C ABI.

HiGPTQ (the calibration article, section 3.1) quantizes groups of 64 columns
and compensates the columns not yet quantized (GPTQ's update with the upper
factor U of H^-1). Scheme 1 (a group at once) is checked on the GPU's own
trajectory: the group's codes and meta must be exactly the oracle's
quantization of the weights the step started from, and the compensated
weights must match the oracle's fp64 step from the same start within
1e-5 * (sum_i |F_i||U_ic| + |W_c|) per entry (F = E U_SS^-1; the fp32
arithmetic's error measured on the CPU is below 4e-7 of that scale).
Schemes 2 and 3 (8 or 4 columns at a time, with fp32 updates inside the
group) are checked against the oracle's step from the same starting rows:
identical codes and meta on every row whose decisions all lie farther than
1e-5 (relative) from their boundaries in the oracle's own values, F and the
later columns within tolerance; the rows inside that band are checked on the
GPU's own trajectory instead (see above those tests), and counted.
Whole passes in blocks of several groups (GPTQ's blocks, the same article,
sections 2.1 and 3.1) are checked against the oracle's run over all groups
on the rows whose decisions all lie outside that band, and every row on its
own trajectory (see above those tests).
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

def _padded(a, pad):
    """Device copy of a 2-D fp32 array as a view with row stride cols + pad."""
    rows, cols = a.shape
    t = torch.full((rows, cols + pad), float("nan"), dtype=torch.float32, device="cuda")
    t[:, :cols] = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t[:, :cols]


def _check_steps(hip, W, U, rows=None, pad_w=0, pad_u=0):
    """Run HiGPTQ on the GPU unit by unit; check every step (on `rows`, or all
    rows) against the oracle started from the GPU's own weights. pad_w / pad_u
    give W and U row strides beyond their widths (the padding holds NaN, so a
    read of it would show)."""
    n, k = W.shape
    w = _padded(W, pad_w) if pad_w else dev(W.astype(np.float32))
    u = _padded(U, pad_u) if pad_u else dev(U.astype(np.float32))
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
    """200 rows (ragged against the 64-row waves of the compensation and its
    256-row workgroups), 448 columns (7 groups)."""
    W, _, U = _gptq_problem(200, 448, 94)
    _check_steps(hip, W, U)


@pytest.mark.parametrize("n,k,pad_w,pad_u", [(1, 128, 0, 0), (3, 192, 12, 4), (63, 192, 0, 0),
                                             (65, 256, 4, 0), (130, 192, 0, 36)])
def test_higptq_small_and_strided(hip, n, k, pad_w, pad_u):
    """Row counts below, at and just past the compensation's 64-row waves
    (and quads of the group step that end inside a wave), and W / U row
    strides padded past their widths (32-bit buffer offsets are formed from
    the strides): every step against the oracle's fp64 step."""
    W, _, U = _gptq_problem(n, k, 97 + n)
    _check_steps(hip, W, U, pad_w=pad_w, pad_u=pad_u)


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


# ----------------------------------------------------- schemes 2 and 3 on the GPU
# Under schemes 2 and 3 the group's later columns are updated in fp32 inside
# the group before they are quantized, so a code can legitimately differ from
# the fp64 oracle only where a value lies within rounding of a decision
# boundary. Each step is checked against the oracle's step from the GPU's own
# starting rows (_check_scheme_step_oracle): the oracle reports, per row, the
# smallest distance of a decision on updated values to its boundary, relative
# to the size of the sums behind those values; rows farther than 1e-5 (two
# orders above fp32's rounding of such sums) must give the oracle's codes and
# meta exactly, F and the later columns within tolerance. Rows inside the
# band fall back to the trajectory check (_check_scheme_step), rebuilt from
# the F values the step leaves in its workspace: the level-1 code exactly;
# every exponent bit and element code against the rule applied to the rebuilt
# values, except within 1e-5 of the value's error scale from a boundary; F
# against the forward substitution of the rebuilt errors; and the later
# columns against W_R - F U_SR.

MARGIN = 1e-5


def _check_scheme_step_oracle(before, after, codes_u, meta_u, F, U64, unit, scheme):
    """One step of scheme 2/3 against the oracle started from `before`.
    Returns the number of rows that fell back to the trajectory check."""
    n, k = before.shape
    s0, r0 = 64 * unit, 64 * unit + 64
    span = 8 if scheme == 2 else 4
    wo = np.ascontiguousarray(before, dtype=np.float64)
    co = np.zeros((n, k // 2), np.uint8)
    mo = np.zeros((n, k // 64), np.uint32)
    mg = np.zeros(n, np.float64)
    oracle.higptq_unit(wo, U64, unit, co, mo, scheme, margin=mg)
    exact = mg > MARGIN
    co_u, mo_u = co[:, 32 * unit:32 * unit + 32], mo[:, unit]
    assert np.array_equal(codes_u[exact], co_u[exact]), f"scheme {scheme} unit {unit} codes"
    assert np.array_equal(meta_u[exact], mo_u[exact]), f"scheme {scheme} unit {unit} meta"
    # the oracle's F, span by span: F_T = E_T U_TT^-1 with E the oracle's own
    # quantization error (its group columns hold the values each span was
    # quantized from)
    E = wo[:, s0:r0] - oracle.dequantize(co_u, mo_u[:, None])
    F_o = np.zeros_like(E)
    sc = np.abs(before[:, s0:r0]).astype(np.float64)
    for t0 in range(0, 64, span):
        Ut = U64[s0 + t0:s0 + t0 + span, s0 + t0:s0 + t0 + span]
        F_o[:, t0:t0 + span] = np.linalg.solve(Ut.T, E[:, t0:t0 + span].T).T
        inv_norm = np.abs(np.linalg.inv(Ut)).sum(axis=0).max()
        bound = (1e-4 * np.abs(F_o[:, t0:t0 + span]).max(axis=1)
                 + inv_norm * MARGIN * sc[:, t0:t0 + span].max(axis=1))
        dF = np.abs(F[:, t0:t0 + span] - F_o[:, t0:t0 + span]).max(axis=1)
        assert np.all((dF <= bound) | ~exact), f"scheme {scheme} unit {unit} F, span {t0}"
        Ul = U64[s0 + t0:s0 + t0 + span, s0 + t0 + span:r0]
        sc[:, t0 + span:] += np.abs(F_o[:, t0:t0 + span]) @ np.abs(Ul)
    assert np.array_equal(after[:, :r0], before[:, :r0])
    if r0 < k:
        scale = np.abs(F_o) @ np.abs(U64[s0:r0, r0:]) + np.abs(before[:, r0:])
        err = np.abs(after[:, r0:].astype(np.float64) - wo[:, r0:])
        assert np.all((err <= 1e-5 * scale)[exact]), f"scheme {scheme} unit {unit} later columns"
    fb = np.nonzero(~exact)[0]
    if fb.size:
        _check_scheme_step(before[fb], after[fb], codes_u[fb], meta_u[fb], F[fb], U64, unit, scheme)
    return int(fb.size)

def _check_scheme_step(before, after, codes_u, meta_u, F, U64, unit, scheme):
    s0, r0 = 64 * unit, 64 * unit + 64
    _scheme_group_f(before[:, s0:r0], codes_u, meta_u, U64, unit, scheme, F)
    assert np.array_equal(after[:, :r0], before[:, :r0])
    if r0 < before.shape[1]:
        Us = U64[s0:r0, r0:]
        ref = before[:, r0:].astype(np.float64) - F @ Us
        scale = np.abs(F) @ np.abs(Us) + np.abs(before[:, r0:])
        assert np.all(np.abs(after[:, r0:] - ref) <= 1e-5 * scale)


def _scheme_group_f(start, codes_u, meta_u, U64, unit, scheme, F=None):
    """Scheme 2/3 group rebuilt in fp64 from the values it started from
    (start [n][64]) and its codes and meta: the level-1 code exactly; every
    exponent bit and element code against the rule applied to the rebuilt
    values, except within 1e-5 of the value's error scale from a boundary; F
    span by span against the forward substitution of the rebuilt errors
    (when F, the GPU's, is given: the rebuild then follows it). Returns the
    F the rebuild followed."""
    from fractions import Fraction

    n = start.shape[0]
    s0, r0 = 64 * unit, 64 * unit + 64
    span = 8 if scheme == 2 else 4
    follow = np.zeros((n, 64)) if F is None else F
    before = np.zeros((n, r0))
    before[:, s0:r0] = start
    v = before[:, s0:r0].astype(np.float64).copy()
    sc = np.abs(v).copy()  # error scale of each rebuilt value
    deq = oracle.dequantize(codes_u, meta_u[:, None])
    c = (meta_u & 255).astype(np.int64)
    e2b = (meta_u[:, None] >> (8 + np.arange(8))) & 1
    e3b = (meta_u[:, None] >> (16 + np.arange(16))) & 1
    for r in range(n):  # level-1 from the group before any update: exact
        A = Fraction(float(np.abs(before[r, s0:r0]).max()))
        assert 7 * Fraction(oracle.e6m2_value(int(c[r]))) >= A
        assert c[r] == 0 or 7 * Fraction(oracle.e6m2_value(int(c[r]) - 1)) < A
    s = np.array([oracle.e6m2_value(int(x)) for x in c])
    tol = 1e-5
    for t0 in range(0, 64, span):
        g = t0 // 8
        if t0 % 8 == 0:
            m8 = np.abs(v[:, 8 * g:8 * g + 8]).max(axis=1)
            near = np.abs(m8 - 3.5 * s) <= tol * sc[:, 8 * g:8 * g + 8].max(axis=1)
            assert np.all((e2b[:, g] == (m8 > 3.5 * s)) | near)
        for q in range(t0 // 4, (t0 + span) // 4):
            m4 = np.abs(v[:, 4 * q:4 * q + 4]).max(axis=1)
            t3 = 1.75 * 2.0 ** e2b[:, g] * s
            near = np.abs(m4 - t3) <= tol * sc[:, 4 * q:4 * q + 4].max(axis=1)
            assert np.all((e3b[:, q] == (m4 > t3)) | near)
            D = s * 2.0 ** (e2b[:, g] + e3b[:, q])
            for j in range(4 * q, 4 * q + 4):
                x = np.abs(v[:, j])
                k = np.rint(np.abs(deq[:, j]) / (D / 4)).astype(np.int64)
                assert np.all(np.abs(deq[:, j]) == k * D / 4)
                mids = (2 * np.arange(7) + 1)[None, :] * D[:, None] / 8
                k_rule = np.minimum((x[:, None] > mids).sum(axis=1) +
                                    ((x[:, None] == mids) & (np.arange(7)[None, :] % 2 == 1)).sum(axis=1), 7)
                near = np.min(np.abs(x[:, None] - mids), axis=1) <= tol * sc[:, j]
                assert np.all((k == k_rule) | near), f"scheme {scheme} unit {unit} element {j}"
        # F over the span from the rebuilt errors
        E = v[:, t0:t0 + span] - deq[:, t0:t0 + span]
        Uab = U64[s0 + t0:s0 + t0 + span, s0 + t0:s0 + t0 + span]
        F_ref = np.linalg.solve(Uab.T, E.T).T
        # row-wise: |dF| <= 1e-4 |F| + |U_tt^-1| * tol * (the rebuilt values' error
        # scale): E = v - deq cancels, so the values' own error carries into F
        inv_norm = np.abs(np.linalg.inv(Uab)).sum(axis=0).max()
        bound = 1e-4 * np.abs(F_ref).max(axis=1) + inv_norm * tol * sc[:, t0:t0 + span].max(axis=1)
        if F is None:
            follow[:, t0:t0 + span] = F_ref
        else:
            assert np.all(np.abs(F[:, t0:t0 + span] - F_ref).max(axis=1) <= bound)
        # follow the GPU's F (or the rebuilt one): update the group's later columns
        Ul = U64[s0 + t0:s0 + t0 + span, s0 + t0 + span:r0]
        v[:, t0 + span:] -= follow[:, t0:t0 + span] @ Ul
        sc[:, t0 + span:] += np.abs(follow[:, t0:t0 + span]) @ np.abs(Ul)
    return follow


@pytest.mark.parametrize("scheme", [2, 3])
def test_higptq_schemes_2_and_3_steps(hip, scheme, capsys):
    W, _, U = _gptq_problem(200, 448, 97 + scheme)
    n, k = W.shape
    w = dev(W)
    u = dev(U.astype(np.float32))
    U64 = U.astype(np.float32).astype(np.float64)
    codes = torch.zeros((n, k // 2), dtype=torch.uint8, device="cuda")
    meta = torch.zeros((n, k // 64), dtype=torch.int32, device="cuda")
    ws = torch.empty((hip.higptq_workspace_bytes(n),), dtype=torch.uint8, device="cuda")
    fallback = 0
    for unit in range(k // 64):
        before = w.cpu().numpy()
        hip.higptq_unit(w, u, unit, codes, meta, workspace=ws, scheme=scheme)
        torch.cuda.synchronize()
        F = ws[:n * 64 * 4].view(torch.float32).view(n, 64).cpu().numpy().astype(np.float64)
        fallback += _check_scheme_step_oracle(before, w.cpu().numpy(),
                                              codes[:, 32 * unit:32 * unit + 32].cpu().numpy(),
                                              host_u32(meta)[:, unit], F, U64, unit, scheme)
    with capsys.disabled():
        print(f"\n[higptq scheme {scheme}] row-steps checked on the trajectory instead of "
              f"exactly against the oracle: {fallback} of {n * (k // 64)}", flush=True)
    assert fallback < n * (k // 64) // 20


@pytest.mark.parametrize("scheme", [2, 3])
def test_higptq_schemes_2_and_3_identity_and_layer_error(hip, scheme):
    W, H, U = _gptq_problem(256, 512, 96)
    c0, m0 = oracle.quantize_f32(W)
    w = dev(W)
    codes, meta = hip.higptq(w, dev(np.eye(512, dtype=np.float32)), scheme=scheme)
    torch.cuda.synchronize()
    assert np.array_equal(codes.cpu().numpy(), c0) and np.array_equal(host_u32(meta), m0)
    codes, meta = hip.higptq(dev(W), dev(U.astype(np.float32)), scheme=scheme)
    torch.cuda.synchronize()
    E = W - oracle.dequantize(codes.cpu().numpy(), host_u32(meta))
    E0 = W - oracle.dequantize(c0, m0)
    assert np.trace(E @ H @ E.T) < 0.8 * np.trace(E0 @ H @ E0.T)


# ------------------------------------------------------------ HiGPTQ in blocks
# A block (hif4_higptq_block) runs its groups one after the other with the
# block's later columns updated after each, and the columns after the block
# once for the whole block: the weights a group starts from are not
# observable between its groups. Whole passes are therefore checked against
# the oracle's run over all groups (oracle.higptq_run, the group steps in
# order) from the same weights: codes and meta exactly on every row whose
# decisions on moved values -- moved inside a group or by any earlier group --
# all lie farther than 1e-5 from their boundaries, relative to the size of
# the sums behind them (|value| + the accumulated sum |F||U|); the final
# working weights on those rows within 1e-5 of that size per entry. Rows
# inside the band are counted (a decision there may go either way in fp32,
# and the rest of the row follows it).


def _block_pass(hip, W, U, scheme, units, pad_w=0, pad_u=0):
    n, k = W.shape
    w = _padded(W, pad_w) if pad_w else dev(W.astype(np.float32))
    u = _padded(U, pad_u) if pad_u else dev(U.astype(np.float32))
    codes = torch.zeros((n, k // 2), dtype=torch.uint8, device="cuda")
    meta = torch.zeros((n, k // 64), dtype=torch.int32, device="cuda")
    ws = torch.empty((hip.higptq_block_workspace_bytes(n, units),), dtype=torch.uint8,
                     device="cuda")
    for unit0 in range(0, k // 64, units):
        hip.higptq_block(w, u, unit0, min(units, k // 64 - unit0), codes, meta, workspace=ws,
                         scheme=scheme)
    torch.cuda.synchronize()
    return w.cpu().numpy(), codes.cpu().numpy(), host_u32(meta)


def _check_block_pass(hip, W, U, scheme, units, **pads):
    """Returns the number of rows inside the margin band."""
    n, k = W.shape
    wg, cg, mg = _block_pass(hip, W, U, scheme, units, **pads)
    U64 = U.astype(np.float32).astype(np.float64)  # the values the GPU works with
    wo = np.array(W, dtype=np.float64, order="C")
    co, mo = np.zeros((n, k // 2), np.uint8), np.zeros((n, k // 64), np.uint32)
    margin, accmag = np.full(n, np.inf), np.zeros((n, k))
    # a group's columns on the GPU end holding the values the group started
    # from (the oracle's end holding those its sets were quantized from under
    # schemes 2 and 3): record the oracle's at each group's start
    start = np.empty_like(wo)
    for unit in range(k // 64):
        start[:, 64 * unit:64 * unit + 64] = wo[:, 64 * unit:64 * unit + 64]
        oracle.higptq_run(wo, U64, unit, 1, co, mo, scheme, margin, accmag)
    wo = start
    exact = margin > MARGIN
    assert np.array_equal(cg[exact], co[exact]), f"scheme {scheme} blocks of {units}: codes"
    assert np.array_equal(mg[exact], mo[exact]), f"scheme {scheme} blocks of {units}: meta"
    scale = np.abs(W.astype(np.float64)) + accmag
    err = np.abs(wg.astype(np.float64) - wo)
    bad = (err > 1e-5 * scale) & exact[:, None]
    assert not bad.any(), (f"scheme {scheme} blocks of {units}: weights, worst "
                           f"{np.max((err / np.maximum(scale, 1e-300))[exact]):.3g}")
    return int(np.count_nonzero(~exact))


@pytest.mark.parametrize("scheme", [1, 2, 3])
def test_higptq_blocks_follow_the_oracle(hip, scheme, capsys):
    """200 rows (ragged against the 16-row workgroups of the group step and
    the 256-row workgroups of the updates), 640 columns (10 groups) in blocks
    of 4, 4 and 2. Over a whole pass every decision after the first group
    reads moved values (640 a row), so more rows fall inside the band than in
    a single step; every row, those included, is checked on its own
    trajectory below."""
    W, _, U = _gptq_problem(200, 640, 110 + scheme)
    inside = _check_block_pass(hip, W, U, scheme, 4)
    with capsys.disabled():
        print(f"\n[higptq blocks, scheme {scheme}] rows inside the margin band: {inside} of 200",
              flush=True)
    assert inside <= 200 // 4


@pytest.mark.parametrize("n,k,units,scheme,pad_w,pad_u", [
    (1, 128, 2, 1, 0, 0),      # one row, one block
    (17, 448, 4, 3, 12, 4),    # blocks of 4 and 3, strided W and U
    (65, 256, 3, 2, 4, 0),     # blocks of 3 and 1
    (257, 384, 16, 1, 0, 36),  # one block of 6 (units capped by the columns left)
    (300, 320, 1, 1, 0, 0),    # blocks of one group
])
def test_higptq_block_shapes(hip, n, k, units, scheme, pad_w, pad_u):
    W, _, U = _gptq_problem(n, k, 120 + n)
    inside = _check_block_pass(hip, W, U, scheme, units, pad_w=pad_w, pad_u=pad_u)
    assert inside <= max(1, n // 4)


def test_higptq_block_leaves_the_earlier_columns(hip):
    """One block of 3 groups in the middle of W: the columns before the block
    and those of its first group keep their values, the rest change; codes
    and meta are written for the block's groups only, the first from the
    weights as given."""
    W, _, U = _gptq_problem(70, 512, 130)
    w, u = dev(W), dev(U.astype(np.float32))
    codes = torch.zeros((70, 256), dtype=torch.uint8, device="cuda")
    meta = torch.zeros((70, 8), dtype=torch.int32, device="cuda")
    hip.higptq_block(w, u, 2, 3, codes, meta, scheme=1)
    torch.cuda.synchronize()
    after = w.cpu().numpy()
    assert np.array_equal(after[:, :192], W[:, :192])
    assert np.all(np.any(after[:, 192:256] != W[:, 192:256], axis=1))
    assert np.all(np.any(after[:, 320:] != W[:, 320:], axis=1))
    c, m = codes.cpu().numpy(), host_u32(meta)
    assert not c[:, :64].any() and not c[:, 160:].any()  # units 2..4 only
    assert not m[:, :2].any() and not m[:, 5:].any()
    c_o, m_o = oracle.quantize_f32(W[:, 128:192])
    assert np.array_equal(c[:, 64:96], c_o) and np.array_equal(m[:, 2], m_o[:, 0])


@pytest.mark.parametrize("scheme,units", [(1, 2), (1, 4), (1, 16), (2, 4), (3, 4), (3, 3)])
def test_higptq_blocks_on_their_own_trajectory(hip, scheme, units):
    """Every row of a pass in blocks, on its own trajectory. A group's columns
    end holding the values the group started from (the group step reads W
    and writes only later columns), so each group can be rebuilt in fp64 from
    the final weights: under scheme 1 its codes and meta must be exactly the
    quantization of those values; under schemes 2 and 3 the rebuild of
    _scheme_group_f (decisions against the rule outside the 1e-5 band, F span
    by span). Each group's starting values must be the initial weights minus
    the compensation of every earlier group, sum over u < v of F_u U_uv with
    the rebuilt F_u, within 1e-5 of the size of that sum per entry."""
    n, k = 160, 768
    W, _, U = _gptq_problem(n, k, 131 + scheme)
    wg, cg, mg = _block_pass(hip, W, U, scheme, units)
    U64 = U.astype(np.float32).astype(np.float64)
    if scheme == 1:
        c_o, m_o = oracle.quantize_f32(wg)
        assert np.array_equal(cg, c_o) and np.array_equal(mg, m_o)
    W64, G = W.astype(np.float64), wg.astype(np.float64)
    comp, size = np.zeros((n, k)), np.abs(W64).copy()
    for unit in range(k // 64):
        s0, r0 = 64 * unit, 64 * unit + 64
        want = W64[:, s0:r0] - comp[:, s0:r0]
        err = np.abs(G[:, s0:r0] - want)
        assert np.all(err <= 1e-5 * size[:, s0:r0]), \
            f"group {unit}: worst {np.max(err / size[:, s0:r0]):.3g}"
        cu, mu = cg[:, 32 * unit:32 * unit + 32], mg[:, unit]
        if scheme == 1:
            E = G[:, s0:r0] - oracle.dequantize(cu, mu[:, None])
            F = np.linalg.solve(U64[s0:r0, s0:r0].T, E.T).T
        else:
            F = _scheme_group_f(G[:, s0:r0], cu, mu, U64, unit, scheme)
        comp[:, r0:] += F @ U64[s0:r0, r0:]
        size[:, r0:] += np.abs(F) @ np.abs(U64[s0:r0, r0:])
