"""Pins of the CPU oracle against what the pages and the mathematics fix.

None of these checks re-runs the oracle's own formula: each compares it with a
fixed fact of the pages (golden fixtures under tests/golden/, cited there), a
hand-worked example, a closed form, an invariant, brute force on tiny inputs,
or a library routine (numpy) where the method reduces to one.

Pages: HiFloat4 calibration article (hwcomputing.csdn.net), section
"一：HiFloat4 (HiF4) 格式" and section 3.1 "HiGPTQ"; Tail-Aware HiFloat4 summary
(agents-report.net), sections "方法概述" and "尾部百分位統計的動機".
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest

import golden_io
import oracle

UNIT = 64


# ----------------------------------------------------------------- helpers

def to_bits(vals):
    """bf16 bit patterns of values that are exactly representable in bf16."""
    f = np.asarray(vals, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def bits_to_f64(bits):
    return oracle.bf16_bits_to_float(bits).astype(np.float64)


def nibble(codes_row, j):
    """Element j's nibble under the documented code layout (reading): byte
    4*(j//8) + j%4 of its unit, low nibble when j%8 < 4."""
    u, jj = divmod(j, UNIT)
    b = codes_row[u * 32 + 4 * (jj // 8) + jj % 4]
    return int(b >> 4) if jj % 8 >= 4 else int(b & 15)


def unit_fields(meta_word):
    c = meta_word & 255
    e2 = [(meta_word >> (8 + g)) & 1 for g in range(8)]
    e3 = [(meta_word >> (16 + q)) & 1 for q in range(16)]
    return int(c), e2, e3


# ------------------------------------------------- fixed facts of the pages

def test_s1p2_value_set_decodes_exactly():
    """All 16 nibbles decode to the S1P2 set of the format section (golden)."""
    mags = golden_io.s1p2_magnitudes()
    assert mags == [k / 4 for k in range(8)]
    codes = np.zeros((1, 32), np.uint8)
    for j in range(16):  # element j carries nibble j; e2 = e3 = 0
        b = 4 * (j // 8) + j % 4
        codes[0, b] |= (j << 4) if j % 8 >= 4 else j
    meta = np.array([[124]], np.uint32)  # level-1 scale 1.0 under the E6M2 reading
    x = oracle.dequantize(codes, meta)[0]
    for j in range(16):
        k, neg = j & 7, j >> 3
        assert abs(x[j]) == mags[k]
        if k:
            assert (x[j] < 0) == bool(neg)
    assert sorted(set(abs(v) for v in x[:16])) == mags


def test_metadata_budget():
    """4-bit elements + 32 metadata bits per 64 elements (golden budget)."""
    b = golden_io.unit_budget()
    assert b["level1_bits"] + b["level2_count"] * b["level2_bits_each"] + \
        b["level3_count"] * b["level3_bits_each"] == b["metadata_bits"]
    assert b["level1_exponent_bits"] + b["level1_mantissa_bits"] == b["level1_bits"]
    rows, k = 3, 256
    x = _random_bits(rows * k // UNIT, seed=3).reshape(rows, k)
    codes, meta, _ = oracle.quantize(x)
    assert codes.nbytes * 8 == rows * k * b["element_bits"]
    assert meta.nbytes * 8 == rows * (k // b["unit_elements"]) * b["metadata_bits"]
    assert (codes.nbytes + meta.nbytes) * 8 / (rows * k) == 4.5


def test_e6m2_scale_has_two_mantissa_bits_and_power_of_two_steps():
    """E6M2 (format section): 4 mantissa steps per binade, 64 binades.
    The bias (31) and "no specials" are readings: parity unpinned."""
    v = [oracle.e6m2_value(c) for c in range(256)]
    assert all(a < b for a, b in zip(v, v[1:]))
    for c in range(252):
        assert v[c + 4] == 2 * v[c]
    for c in range(256):
        m = v[c] / 2.0 ** math.floor(math.log2(v[c]))
        assert m in (1.0, 1.25, 1.5, 1.75)
    assert v[255] / v[0] == 1.75 * 2.0 ** 63


# --------------------------------------------------- hand-worked examples

@pytest.mark.parametrize("u", golden_io.hand_units(), ids=lambda u: u["name"])
def test_hand_units(u):
    x = golden_io.expand(u["x"], UNIT, 0.0)
    codes, meta, _ = oracle.quantize(to_bits(x).reshape(1, UNIT))
    assert int(meta[0, 0]) == u["meta"], hex(int(meta[0, 0]))
    nib = golden_io.expand(u["nib"], UNIT, 0)
    assert [nibble(codes[0], j) for j in range(UNIT)] == nib
    by = golden_io.expand(u["bytes"], 32, 0)
    assert list(codes[0]) == by
    deq = golden_io.expand(u["deq"], UNIT, 0.0)
    assert list(oracle.dequantize(codes, meta)[0]) == deq


# ------------------------------------------------ the level-1 rule, exact

def test_level1_code_is_minimal_for_every_bf16_magnitude():
    """For every positive finite bf16 A (alone in a unit): c is the smallest
    code with 7 v(c) >= A, or 255 when none reaches A (exact rationals)."""
    a_bits = np.arange(1, 0x7F80, dtype=np.uint16)
    x = np.zeros((a_bits.size, UNIT), np.uint16)
    x[:, 17] = a_bits
    _, meta, _ = oracle.quantize(x)
    v = [Fraction(oracle.e6m2_value(c)) for c in range(256)]
    top = 7 * v[255]
    for A_bits, m in zip(a_bits, meta[:, 0]):
        A = Fraction(float(bits_to_f64(np.array([A_bits]))[0]))
        c = int(m) & 255
        if A > top:
            assert c == 255
            continue
        assert 7 * v[c] >= A
        assert c == 0 or 7 * v[c - 1] < A


# ------------------------------------------ element rounding, exact rationals

def _check_unit_exact(xrow_bits, codes_row, meta_word, deq_row):
    """RNE onto S1P2 on exact rationals: |x - xhat| <= D/8, ties to even k,
    no element beyond 7D/4 unless the level-1 range saturated."""
    c, e2, e3 = unit_fields(int(meta_word))
    s = Fraction(oracle.e6m2_value(c))
    xs = bits_to_f64(xrow_bits)
    for j in range(UNIT):
        x = Fraction(float(xs[j]))
        D = s * 2 ** (e2[j // 8] + e3[j // 4])
        nib = nibble(codes_row, j)
        k = nib & 7
        xhat = Fraction(float(deq_row[j]))
        assert abs(xhat) == k * D / 4
        if k == 0:
            assert nib == 0  # canonical +0
        else:
            assert (xhat < 0) == (x < 0)
        err = abs(abs(x) - k * D / 4)
        if c == 255 and abs(x) > 7 * D / 4:
            assert k == 7
            continue
        assert abs(x) <= 7 * D / 4  # no clipping
        assert err <= D / 8
        if err == D / 8:
            assert k % 2 == 0, "tie must go to even k"


def _random_bits(n, seed, spread=3.0, zero_p=0.2):
    r = np.random.default_rng(seed)
    x = r.standard_t(3, size=(n, UNIT)) * np.exp(r.normal(0, spread, size=(n, 1)))
    x[r.random(size=x.shape) < zero_p] = 0.0
    u = np.float32(x).view(np.uint32) & np.uint32(0xFFFF0000)
    return (u >> 16).astype(np.uint16)


def _midpoint_bits(n, seed):
    """Units whose elements sit exactly on grid midpoints of their own unit."""
    r = np.random.default_rng(seed)
    rows = []
    while len(rows) < n:
        c = int(r.integers(20, 230))
        s = Fraction(oracle.e6m2_value(c))
        vals = [0.0] * UNIT
        vals[0] = float(7 * s)  # fixes c; group 0 gets e2 = e3 = 1
        for j in range(8, UNIT):
            D = s  # groups 1..7 stay at e2 = e3 = 0 if all |x| <= 1.75 s
            m = int(r.integers(0, 7))
            v = (2 * m + 1) * D / 8
            if v > Fraction(7, 4) * s:
                v = Fraction(7, 4) * s
            vals[j] = float(v) * (1 if r.random() < 0.5 else -1)
        f = np.float32(vals)
        if np.all((f.view(np.uint32) & 0xFFFF) == 0):
            rows.append((f.view(np.uint32) >> 16).astype(np.uint16))
    return np.stack(rows)


def test_element_rounding_is_exact_rne_random():
    x = _random_bits(1500, seed=11)
    codes, meta, _ = oracle.quantize(x)
    deq = oracle.dequantize(codes, meta)
    for i in range(x.shape[0]):
        _check_unit_exact(x[i], codes[i], meta[i, 0], deq[i])


def test_element_rounding_ties_go_to_even():
    x = _midpoint_bits(300, seed=12)
    codes, meta, _ = oracle.quantize(x)
    deq = oracle.dequantize(codes, meta)
    n_ties = 0
    for i in range(x.shape[0]):
        _check_unit_exact(x[i], codes[i], meta[i, 0], deq[i])
        c, e2, e3 = unit_fields(int(meta[i, 0]))
        assert e2[1:] == [0] * 7 and e3[2:] == [0] * 14
        n_ties += UNIT - 8
    assert n_ties > 10000


def test_element_rounding_every_bf16_against_each_grid():
    """Every positive finite bf16 magnitude, placed in a unit whose group has
    D = s (e2 = e3 = 0), for several level-1 codes with each mantissa."""
    allbits = np.arange(1, 0x7F80, dtype=np.uint16)
    vals = bits_to_f64(allbits)
    for c in (100, 101, 102, 103, 130, 131):
        s = oracle.e6m2_value(c)
        keep = allbits[(vals <= 1.75 * s)]
        n = keep.size
        x = np.zeros((n, UNIT), np.uint16)
        x[:, 0] = to_bits([7 * s])[0]
        x[:, 40] = keep
        codes, meta, _ = oracle.quantize(x)
        assert np.all(meta[:, 0] & 255 == c)
        deq = oracle.dequantize(codes, meta)[:, 40]
        S = Fraction(s)
        for b, xhat in zip(keep, deq):
            xv = Fraction(float(bits_to_f64(np.array([b]))[0]))
            k = Fraction(xhat) / (S / 4)
            assert k.denominator == 1 and 0 <= k <= 7
            err = abs(xv - k * S / 4)
            assert err <= S / 8
            if err == S / 8:
                assert k % 2 == 0


# -------------------------------------------- brute force over scale choices

def _rne_grid(x, D):
    """Nearest of {k D/4, k=0..7} to |x| (ties to even), exact rationals."""
    a = abs(x)
    best = None
    for k in range(8):
        e = abs(a - k * D / 4)
        if best is None or e < best[0] or (e == best[0] and k % 2 == 0):
            best = (e, k)
    return best[1] * D / 4 * (1 if x >= 0 else -1)


def _group_options(xs, s):
    """All 8 (e2, e3a, e3b) choices for a level-2 group of 8 exact values:
    returns list of (no_clip, [xhat]) ."""
    out = []
    for e2, ea, eb in itertools.product((0, 1), repeat=3):
        xh, ok = [], True
        for t, x in enumerate(xs):
            D = s * 2 ** (e2 + (ea if t < 4 else eb))
            if abs(x) > 7 * D / 4:
                ok = False
            xh.append(_rne_grid(x, D))
        out.append((ok, xh))
    return out


def test_micro_exponents_are_elementwise_optimal_among_no_clip_choices():
    """With the level-1 code fixed, the rule's level-2/3 bits give, element by
    element, the smallest error of all no-clip choices (brute force)."""
    x = _random_bits(120, seed=21, spread=1.0, zero_p=0.3)
    codes, meta, _ = oracle.quantize(x)
    deq = oracle.dequantize(codes, meta)
    xs = bits_to_f64(x)
    for i in range(x.shape[0]):
        c, e2, e3 = unit_fields(int(meta[i, 0]))
        if c == 255:
            continue
        s = Fraction(oracle.e6m2_value(c))
        for g in range(8):
            vals = [Fraction(float(v)) for v in xs[i, 8 * g:8 * g + 8]]
            mine = [Fraction(float(v)) for v in deq[i, 8 * g:8 * g + 8]]
            opts = [xh for ok, xh in _group_options(vals, s) if ok]
            assert opts, "some choice must avoid clipping"
            for t in range(8):
                best = min(abs(vals[t] - o[t]) for o in opts)
                assert abs(vals[t] - mine[t]) == best


def test_global_search_reports_rule_error_bound():
    """Brute force over level-1 codes (a window of 4 binades either side of
    the rule's code) x all micro choices on tiny units: the rule's per-element
    error obeys |x - xhat| <= 2^(E-3) s, and its max-abs error is compared
    (reported) with the searched optimum."""
    x = _random_bits(6, seed=31, spread=0.5, zero_p=0.5)
    codes, meta, _ = oracle.quantize(x)
    deq = oracle.dequantize(codes, meta)
    xs = bits_to_f64(x)
    worse = 0
    for i in range(x.shape[0]):
        c, e2, e3 = unit_fields(int(meta[i, 0]))
        s = Fraction(oracle.e6m2_value(c))
        vals = [Fraction(float(v)) for v in xs[i]]
        mine = [Fraction(float(v)) for v in deq[i]]
        for j in range(UNIT):
            E = e2[j // 8] + e3[j // 4]
            assert abs(vals[j] - mine[j]) <= s * 2 ** E / 8
        rule_max = max(abs(a - b) for a, b in zip(vals, mine))
        best_max = None
        for cc in range(max(0, c - 16), min(256, c + 17)):
            sc = Fraction(oracle.e6m2_value(cc))
            tot = Fraction(0)
            for g in range(8):
                grp = vals[8 * g:8 * g + 8]
                errs = [max(abs(a - b) for a, b in zip(grp, xh))
                        for _, xh in _group_options(grp, sc)]
                tot = max(tot, min(errs))
            best_max = tot if best_max is None else min(best_max, tot)
        assert best_max <= rule_max
        worse += best_max < rule_max
    print(f"units where a searched choice beats the no-clip rule on max error: {worse}/6")


# ----------------------------------------------------------- invariants

def _canonical_unit(r):
    """A random code unit that the rule reproduces: minimal bits, canonical
    zeros, and its decoded maximum equal to 7 v(c)."""
    c = int(r.integers(8, 248))
    e2 = [int(r.integers(0, 2)) for _ in range(8)]
    e3 = [int(r.integers(0, 2)) for _ in range(16)]
    k = [int(r.integers(0, 8)) for _ in range(UNIT)]
    e2[0], e3[0] = 1, 1
    k[int(r.integers(0, 4))] = 7  # decoded max 7 v(c) fixes c
    for g in range(8):
        if e2[g] and not (e3[2 * g] or e3[2 * g + 1]):
            e3[2 * g + int(r.integers(0, 2))] = 1
        if e2[g]:
            qs = [q for q in (2 * g, 2 * g + 1) if e3[q]]
            q = qs[int(r.integers(0, len(qs)))]
            j = 4 * q + int(r.integers(0, 4))
            k[j] = max(k[j], 4)
    for q in range(16):
        if e3[q] and max(k[4 * q:4 * q + 4]) < 4:
            k[4 * q + int(r.integers(0, 4))] = int(r.integers(4, 8))
    sign = [int(r.integers(0, 2)) if k[j] else 0 for j in range(UNIT)]
    codes = np.zeros(32, np.uint8)
    for j in range(UNIT):
        nib = k[j] | (sign[j] << 3)
        codes[4 * (j // 8) + j % 4] |= (nib << 4) if j % 8 >= 4 else nib
    meta = c | sum(e2[g] << (8 + g) for g in range(8)) | sum(e3[q] << (16 + q) for q in range(16))
    return codes, np.uint32(meta)


def test_round_trip_of_canonical_units():
    r = np.random.default_rng(41)
    units = [_canonical_unit(r) for _ in range(400)]
    codes = np.stack([u[0] for u in units])
    meta = np.array([[u[1]] for u in units], np.uint32)
    deq = oracle.dequantize(codes, meta)
    x = to_bits(deq.astype(np.float32)).reshape(deq.shape)  # exact in bf16
    assert np.array_equal(bits_to_f64(x), deq)
    c2, m2, _ = oracle.quantize(x)
    assert np.array_equal(m2, meta)
    assert np.array_equal(c2, codes)


def test_requantization_is_not_always_idempotent_but_settles():
    """Documented counterexample: s = 1, A = 6.25 -> 6 -> 6.125 -> 6.125."""
    x = np.zeros((1, UNIT), np.uint16)
    x[0, 0] = to_bits([6.25])[0]
    a = oracle.dequantize(*oracle.quantize(x)[:2])[0, 0]
    assert a == 6.0
    b = oracle.dequantize(*oracle.quantize(to_bits([[a] + [0.0] * 63]).reshape(1, UNIT))[:2])[0, 0]
    assert b == 6.125
    c = oracle.dequantize(*oracle.quantize(to_bits([[b] + [0.0] * 63]).reshape(1, UNIT))[:2])[0, 0]
    assert c == 6.125


def test_scale_equivariance():
    """Q(2^p x): same nibbles and E1 bits, level-1 code shifted by 4p."""
    x = _random_bits(200, seed=51, spread=0.5)
    c0, m0, _ = oracle.quantize(x)
    lv = m0[:, 0] & 255
    ok = (lv > 40) & (lv < 200)
    for p in (-5, -1, 1, 3, 7):
        xs = bits_to_f64(x) * 2.0 ** p
        xb = to_bits(xs.astype(np.float32)).reshape(x.shape)
        c1, m1, _ = oracle.quantize(xb)
        assert np.array_equal(c1[ok], c0[ok])
        assert np.array_equal(m1[ok] >> 8, m0[ok] >> 8)
        assert np.array_equal((m1[ok] & 255).astype(int), (m0[ok] & 255).astype(int) + 4 * p)


def test_sign_symmetry():
    x = _random_bits(300, seed=61)
    c0, m0, _ = oracle.quantize(x)
    c1, m1, _ = oracle.quantize(x ^ np.uint16(0x8000))
    assert np.array_equal(m0, m1)
    for i in range(x.shape[0]):
        for j in range(UNIT):
            a, b = nibble(c0[i], j), nibble(c1[i], j)
            if a & 7:
                assert b == a ^ 8
            else:
                assert a == b == 0


def test_grouping_locality_along_k():
    """Raising one element to the unit maximum changes only its own level-2
    group: its e2 bit, its two e3 bits and its own code word (format section:
    per-8 and per-4 sharing; HiGPTQ section: exponent order along K)."""
    r = np.random.default_rng(71)
    x = _random_bits(60, seed=72, spread=0.3)
    c0, m0, _ = oracle.quantize(x)
    xs = bits_to_f64(x)
    for i in range(x.shape[0]):
        j = int(r.integers(0, UNIT))
        amax = np.abs(xs[i]).max()
        y = x[i].copy()
        y[j] = to_bits([amax])[0]
        c1, m1, _ = oracle.quantize(y.reshape(1, UNIT))
        g = j // 8
        allowed = (1 << (8 + g)) | (1 << (16 + 2 * g)) | (1 << (17 + 2 * g))
        assert (int(m0[i, 0]) ^ int(m1[0, 0])) & ~allowed == 0
        diff = np.nonzero(c0[i] != c1[0])[0]
        assert all(4 * g <= b < 4 * g + 4 for b in diff)


def test_masked_channels_become_zero_and_are_kept():
    x = _random_bits(16, seed=81).reshape(4, 256)
    mask = np.zeros(256, np.uint8)
    mask[[3, 64, 65, 200, 255]] = 1
    c, m, kept = oracle.quantize(x, mask)
    y = x.copy()
    y[:, mask != 0] = 0
    c2, m2, _ = oracle.quantize(y)
    assert np.array_equal(c, c2) and np.array_equal(m, m2)
    assert np.array_equal(kept, x[:, [3, 64, 65, 200, 255]])


def test_nonfinite_input_is_out_of_contract():
    x = np.zeros((1, UNIT), np.uint16)
    x[0, 3] = 0x7FC0  # NaN
    with pytest.raises(oracle.OracleError):
        oracle.quantize(x)


# ------------------------------------------------------------------ linear

def test_linear_matches_numpy_fp64_matmul():
    import workloads
    t = workloads.workload("tiny")
    xb, wb = workloads.bits(t["x"]), workloads.bits(t["w"])
    xc, xm, _ = oracle.quantize(xb)
    wc, wm, _ = oracle.quantize(wb)
    a, b = oracle.dequantize(xc, xm), oracle.dequantize(wc, wm)
    y, s = oracle.linear(xc, xm, wc, wm)
    ref = a @ b.T
    assert np.all(np.abs(y - ref) <= 1e-12 * s)
    assert np.allclose(s, np.abs(a) @ np.abs(b).T, rtol=1e-14, atol=0)
    assert y.shape == (64, 128)


def test_linear_one_hot_weight_column_is_exact():
    """A W row with a single element 7 (decodes to exactly 7) gives column j
    of Y = 7 * deq(Q(X))[:, t], bit for bit."""
    import workloads
    xb = workloads.bits(workloads.tiny_x(16, 192, seed=5))
    xc, xm, _ = oracle.quantize(xb)
    a = oracle.dequantize(xc, xm)
    w = np.zeros((3, 192), np.uint16)
    cols = [5, 77, 190]
    for j, t in enumerate(cols):
        w[j, t] = to_bits([7.0])[0]
    wc, wm, _ = oracle.quantize(w)
    assert np.array_equal(oracle.dequantize(wc, wm)[np.arange(3), cols], [7.0] * 3)
    y = oracle.linear(xc, xm, wc, wm, with_mag=False)
    for j, t in enumerate(cols):
        assert np.array_equal(y[:, j], 7.0 * a[:, t])


def _dense_with_kept(codes, meta, kept, mask):
    """deq(codes) with the kept bf16 values written back at the masked
    channels (ascending channel order): the matrix the protected linear
    multiplies, built with numpy instead of the oracle's residual loop."""
    a = oracle.dequantize(codes, meta)
    chans = np.nonzero(mask)[0]
    if chans.size:
        a[:, chans] = (kept.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return a


@pytest.mark.parametrize("n_mask", [0, 1, 13, 64])
def test_linear_protected_equals_dense_product(n_mask):
    """[TA-method]: protected channels stay in high precision. The oracle's
    HiF4 product plus its bf16 residual equals numpy's fp64 product of the
    dense matrices in which the masked channels hold their original values;
    with no mask it is the plain linear."""
    import workloads
    k = 256
    r = np.random.default_rng(n_mask + 3)
    xb = workloads.bits(workloads.heavy_tailed_x(40, k, seed=n_mask + 1, outlier_channels=3))
    wb = workloads.bits(workloads.normal_bf16(24, k, 0.02, seed=n_mask + 2))
    mask = np.zeros(k, np.uint8)
    mask[r.choice(k, n_mask, replace=False)] = 1
    xc, xm, xk = oracle.quantize(xb, mask if n_mask else None)
    wc, wm, wk = oracle.quantize(wb, mask if n_mask else None)
    y, s = oracle.linear_protected(xc, xm, xk, wc, wm, wk)
    a = _dense_with_kept(xc, xm, xk, mask)
    b = _dense_with_kept(wc, wm, wk, mask)
    ref = a @ b.T
    assert np.all(np.abs(y - ref) <= 1e-12 * s)
    assert np.allclose(s, np.abs(a) @ np.abs(b).T, rtol=1e-13, atol=0)
    if n_mask == 0:
        y0, s0 = oracle.linear(xc, xm, wc, wm)
        assert np.array_equal(y, y0) and np.array_equal(s, s0)
    else:
        # the masked channels really are exact: their columns of a hold the inputs
        chans = np.nonzero(mask)[0]
        assert np.array_equal(a[:, chans], xb[:, chans].astype(np.uint32).__lshift__(16)
                              .view(np.float32).astype(np.float64))


def test_linear_protected_all_channels_masked_is_bf16_matmul():
    """Everything protected: the HiF4 part is all zeros and Y is the plain
    fp64 product of the bf16 inputs."""
    import workloads
    k = 64
    xb = workloads.bits(workloads.tiny_x(8, k, seed=11))
    wb = workloads.bits(workloads.normal_bf16(5, k, 0.02, seed=12))
    mask = np.ones(k, np.uint8)
    xc, xm, xk = oracle.quantize(xb, mask)
    wc, wm, wk = oracle.quantize(wb, mask)
    assert not xc.any() and not wc.any()
    y = oracle.linear_protected(xc, xm, xk, wc, wm, wk, with_mag=False)
    fx = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    fw = (wb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.allclose(y, fx @ fw.T, rtol=1e-13, atol=1e-300)


# -------------------------------------------------------------- percentile

@pytest.mark.parametrize("case", golden_io.percentile_cases())
def test_percentile_golden(case):
    q, vals, exp = case
    x = to_bits(vals).reshape(-1, 1)
    assert oracle.percentile(x, q)[0] == np.float32(exp)


def test_percentile_matches_numpy_linear():
    r = np.random.default_rng(91)
    x = r.standard_t(3, size=(257, 40)) * np.exp(r.normal(0, 1, size=(1, 40)))
    x[:, 7] = 2.5  # constant channel
    xb = to_bits((np.float32(x).view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32))
    xb = xb.reshape(x.shape)
    vals = np.abs(bits_to_f64(xb))
    for q in (0.0, 0.5, 0.75, 0.9, 0.99, 0.999, 1.0):
        mine = oracle.percentile(xb, q)
        ref = np.percentile(vals, q * 100.0, axis=0, method="linear").astype(np.float32)
        ulp = np.spacing(np.maximum(np.abs(ref), np.float32(1e-30)))
        assert np.all(np.abs(mine - ref) <= ulp), q
        assert mine[7] == np.float32(2.5)
        h = q * 256
        if h == int(h):  # an exact order statistic
            assert np.array_equal(mine, np.sort(vals, axis=0)[int(h)].astype(np.float32))


# -------------------------------------------------------------------- mask

def test_topn_mask_matches_stable_argsort():
    r = np.random.default_rng(101)
    for c, n in ((256, 13), (5120, 52), (7, 0), (7, 7)):
        s = np.float32(r.exponential(size=c))
        s[r.integers(0, c, size=c // 5)] = s[0]  # ties
        mine = oracle.topn_mask(s, n)
        order = np.argsort(-s.astype(np.float64), kind="stable")
        ref = np.zeros(c, np.uint8)
        ref[order[:n]] = 1
        assert np.array_equal(mine, ref)
        assert int(mine.sum()) == n


def test_topn_mask_ties_prefer_lower_index():
    s = np.float32([1, 3, 3, 2, 3, 0])
    assert list(oracle.topn_mask(s, 2)) == [0, 1, 1, 0, 0, 0]
    assert list(oracle.topn_mask(s, 3)) == [0, 1, 1, 0, 1, 0]


# ------------------------------------------------------------------- HiGPTQ
# [HiGPTQ] (the calibration article, section 3.1), scheme 1: every group of
# 64 columns (one HiF4 unit) is quantized at once with all its exponents
# fixed from it; the columns not yet quantized are then compensated, as in
# GPTQ. The working weights are real numbers, so the quantizer's fp32 entry
# is pinned first.

def _check_values_exact(xs, codes_row, meta_word, deq_row):
    """Exact-rational RNE check of one unit given its input values."""
    c, e2, e3 = unit_fields(int(meta_word))
    s = Fraction(oracle.e6m2_value(c))
    for j in range(UNIT):
        x = Fraction(float(xs[j]))
        D = s * 2 ** (e2[j // 8] + e3[j // 4])
        k = nibble(codes_row, j) & 7
        assert Fraction(float(deq_row[j])) == (k * D / 4) * (-1 if (x < 0 and k) else 1)
        err = abs(abs(x) - k * D / 4)
        assert abs(x) <= 7 * D / 4 and err <= D / 8
        if err == D / 8:
            assert k % 2 == 0
    # the rule's scales: the smallest level-1 code that covers the maximum
    A = max(abs(Fraction(float(v))) for v in xs)
    assert 7 * s >= A and (c == 0 or 7 * Fraction(oracle.e6m2_value(c - 1)) < A)


def test_quantize_f32_on_bf16_values_equals_bf16_quantize():
    bits = _random_bits(400, seed=71)
    f = (bits.astype(np.uint32) << 16).view(np.float32)
    c1, m1 = oracle.quantize_f32(f)
    c0, m0, _ = oracle.quantize(bits)
    assert np.array_equal(c1, c0) and np.array_equal(m1, m0)


def test_quantize_f32_is_exact_rne_on_full_precision_floats():
    r = np.random.default_rng(72)
    x = (r.standard_t(3, size=(600, UNIT)) * np.exp(r.normal(0, 3, size=(600, 1)))).astype(np.float32)
    # ties: fp32 elements exactly on grid midpoints (2m+1) D/8 of their unit
    for i in range(200):
        c = int(r.integers(20, 230))
        s = Fraction(oracle.e6m2_value(c))
        x[i, :] = 0
        x[i, 0] = float(7 * s)
        for j in range(8, UNIT):
            x[i, j] = float((2 * int(r.integers(0, 7)) + 1) * s / 8) * (1 if r.random() < 0.5 else -1)
    codes, meta = oracle.quantize_f32(x)
    deq = oracle.dequantize(codes, meta)
    for i in range(x.shape[0]):
        _check_values_exact(x[i], codes[i], meta[i, 0], deq[i])


def _gptq_problem(n, k, seed):
    """Correlated synthetic calibration inputs -> Hessian H = 2 X^T X / rows
    (+1% mean-diagonal damping) and the upper factor U of H^-1 = U^T U."""
    r = np.random.default_rng(seed)
    A = r.standard_normal((k, k)) / np.sqrt(k)
    X = r.standard_normal((4 * k, k)) @ (np.eye(k) + 0.8 * A)
    X *= np.exp(r.normal(0, 1, size=(1, k)))
    H = 2 * X.T @ X / X.shape[0]
    H += 0.01 * np.mean(np.diag(H)) * np.eye(k)
    U = np.linalg.cholesky(np.linalg.inv(H)).T
    W = (r.standard_normal((n, k)) * 0.02).astype(np.float32)
    return W, H, U


def test_higptq_step_is_the_obs_update_for_a_group():
    """Each step equals the closed-form optimal compensation when a set S of
    weights is fixed (the multi-weight form of the OBS/GPTQ update), computed
    with explicit inverses of the trailing Hessian block -- a route that does
    not use the Cholesky factor."""
    n, k = 24, 256
    W, H, U = _gptq_problem(n, k, 73)
    w = W.astype(np.float64)
    codes = np.zeros((n, k // 2), np.uint8)
    meta = np.zeros((n, k // 64), np.uint32)
    for unit in range(k // 64):
        s0, r0 = 64 * unit, 64 * unit + 64
        before = w.copy()
        oracle.higptq_unit(w, U, unit, codes, meta)
        # the group is the rule's quantization of the current weights
        c_ref, m_ref = oracle.quantize_f32(before[:, s0:r0].astype(np.float32))
        assert np.array_equal(codes[:, unit * 32:unit * 32 + 32], c_ref)
        assert np.array_equal(meta[:, unit], m_ref[:, 0])
        E = before[:, s0:r0] - oracle.dequantize(c_ref, m_ref)
        Hinv_rem = np.linalg.inv(H[s0:, s0:])
        S, R = slice(0, 64), slice(64, k - s0)
        delta = -E @ np.linalg.solve(Hinv_rem[S, S], Hinv_rem[S, R])
        assert np.allclose(w[:, r0:], before[:, r0:] + delta, rtol=0, atol=1e-9 * np.abs(before).max())
        assert np.array_equal(w[:, :r0], before[:, :r0])


def test_higptq_with_identity_hessian_is_direct_quantization():
    W, _, _ = _gptq_problem(32, 256, 74)
    codes, meta, wf = oracle.higptq(W, np.eye(256))
    c0, m0 = oracle.quantize_f32(W)
    assert np.array_equal(codes, c0) and np.array_equal(meta, m0)
    assert np.array_equal(wf, W.astype(np.float64))


def test_higptq_lowers_the_layer_output_error():
    """The point of the method: tr(E H E^T), the layer-output error on the
    calibration inputs, drops against direct quantization."""
    for seed in (75, 76):
        W, H, U = _gptq_problem(64, 256, seed)
        codes, meta, _ = oracle.higptq(W, U)
        c0, m0 = oracle.quantize_f32(W)
        E = W - oracle.dequantize(codes, meta)
        E0 = W - oracle.dequantize(c0, m0)
        assert np.trace(E @ H @ E.T) < 0.8 * np.trace(E0 @ H @ E0.T)


def _simulate_schemes(W, H, codes, meta, w_after, unit, scheme):
    """Re-derive one oracle step of scheme 2 or 3 with explicit inverses of
    the trailing Hessian blocks (no Cholesky factor), checking the scheme's
    exponent rules on the values each span was quantized from."""
    n, k = W.shape
    s0, r0 = 64 * unit, 64 * unit + 64
    span = 8 if scheme == 2 else 4
    state = W.astype(np.float64).copy()
    deq = oracle.dequantize(codes[:, 32 * unit:32 * unit + 32], meta[:, unit:unit + 1])
    for r in range(n):
        c, e2, e3 = unit_fields(int(meta[r, unit]))
        A = max(abs(Fraction(float(v))) for v in W[r, s0:r0])
        # level-1 fixed from the group before any update
        assert 7 * Fraction(oracle.e6m2_value(c)) >= A
        assert c == 0 or 7 * Fraction(oracle.e6m2_value(c - 1)) < A
    e2_seen = {}
    for t0 in range(0, 64, span):
        T = slice(s0 + t0, s0 + t0 + span)
        vals = state[:, T]
        # the span was quantized from exactly these values
        assert np.allclose(w_after[:, T], vals, rtol=0, atol=1e-12 * max(1.0, np.abs(W).max()))
        for r in range(n):
            c, e2, e3 = unit_fields(int(meta[r, unit]))
            s = oracle.e6m2_value(c)
            g = t0 // 8
            if t0 % 8 == 0:  # e2 fixed from the level-2 group's values at its first span
                m8 = np.abs(state[r, s0 + 8 * g:s0 + 8 * g + 8]).max()
                assert e2[g] == int(m8 > 3.5 * s)
            for q in range(t0 // 4, (t0 + span) // 4):
                m4 = np.abs(state[r, s0 + 4 * q:s0 + 4 * q + 4]).max()
                assert e3[q] == int(m4 > 1.75 * 2 ** e2[g] * s)
                D = s * 2 ** (e2[g] + e3[q])
                for j in range(4 * q, 4 * q + 4):
                    x = abs(state[r, s0 + j])
                    kk = abs(deq[r, j]) / (D / 4)
                    assert kk == int(kk) and 0 <= kk <= 7
                    err = abs(x - kk * D / 4)
                    if x > 7.5 * D / 4:
                        assert kk == 7  # fixed level-1 exponent: clipped
                    else:
                        assert err <= D / 8 + 1e-300
        E = vals - deq[:, t0:t0 + span]
        Hinv_rem = np.linalg.inv(H[s0 + t0:, s0 + t0:])
        S, R = slice(0, span), slice(span, None)
        state[:, s0 + t0 + span:] -= E @ np.linalg.solve(Hinv_rem[S, S], Hinv_rem[S, R])
    assert np.allclose(w_after[:, r0:], state[:, r0:], rtol=0, atol=1e-9 * np.abs(W).max())


@pytest.mark.parametrize("scheme", [2, 3])
def test_higptq_schemes_2_and_3_follow_their_rules_and_the_obs_update(scheme):
    n, k = 12, 192
    W, H, U = _gptq_problem(n, k, 77 + scheme)
    w = W.astype(np.float64)
    codes = np.zeros((n, k // 2), np.uint8)
    meta = np.zeros((n, k // 64), np.uint32)
    for unit in range(k // 64):
        before = w.copy()
        oracle.higptq_unit(w, U, unit, codes, meta, scheme)
        _simulate_schemes(before, H, codes, meta, w, unit, scheme)


@pytest.mark.parametrize("scheme", [2, 3])
def test_higptq_schemes_with_identity_hessian_are_direct_quantization(scheme):
    W, _, _ = _gptq_problem(32, 256, 78)
    codes, meta, wf = oracle.higptq(W, np.eye(256), scheme)
    c0, m0 = oracle.quantize_f32(W)
    assert np.array_equal(codes, c0) and np.array_equal(meta, m0)
    assert np.array_equal(wf, W.astype(np.float64))


def test_higptq_all_schemes_lower_the_layer_output_error():
    W, H, U = _gptq_problem(64, 256, 79)
    c0, m0 = oracle.quantize_f32(W)
    E0 = W - oracle.dequantize(c0, m0)
    base = np.trace(E0 @ H @ E0.T)
    for scheme in (1, 2, 3):
        codes, meta, _ = oracle.higptq(W, U, scheme)
        E = W - oracle.dequantize(codes, meta)
        assert np.trace(E @ H @ E.T) < 0.8 * base


@pytest.mark.parametrize("scheme", [1, 2, 3])
def test_higptq_decision_margin(scheme):
    """The decision margin the oracle reports (the distance of a decision on
    updated values to its boundary, relative to the size of the sums behind
    them): +inf under scheme 1 and with no update at all (identity Hessian:
    every decision reads the weights as given); 0 on a row where an updated
    value lands exactly on a rounding midpoint; unchanged when the problem is
    scaled by a power of two; positive on generic rows."""
    n, k = 16, 128
    W, _, U = _gptq_problem(n, k, 81)
    mg = np.zeros(n)
    w = W.astype(np.float64)
    codes = np.zeros((n, k // 2), np.uint8)
    meta = np.zeros((n, k // 64), np.uint32)
    oracle.higptq_unit(w.copy(), np.eye(k), 0, codes, meta, scheme, margin=mg)
    assert np.all(np.isinf(mg))
    oracle.higptq_unit(w.copy(), U, 0, codes, meta, scheme, margin=mg)
    if scheme == 1:
        assert np.all(np.isinf(mg))
        return
    assert np.all(np.isfinite(mg)) and np.all(mg > 0)
    mg2 = np.zeros(n)
    oracle.higptq_unit(4.0 * w, U, 0, codes, meta, scheme, margin=mg2)
    assert np.array_equal(mg, mg2)
    # A factor whose only off-diagonal entry moves column 8 by -F_1 U[1, 8]
    # once the first span is fixed; chosen so that column 8 lands exactly on
    # the midpoint 3 D / 8 of its grid. x_0 = 7 sets v(c) = 1 and, with
    # e2 = e3 = 1 (D = 4), quantizes exactly; x_1 = 0.25 rounds to 0 there,
    # so E_1 = F_1 = 0.25 and column 8 becomes 0.25 + 0.25 * 0.5 = 0.375. Its
    # own level-2 group then holds nothing larger: e2 = e3 = 0, D = 1, and
    # 0.375 is the tie between k = 1 and k = 2.
    x = np.zeros((1, k))
    x[0, 0] = 7.0
    x[0, 1] = 0.25
    x[0, 8] = 0.25
    uu = np.eye(k)
    uu[1, 8] = -0.5
    mg1 = np.zeros(1)
    c1 = np.zeros((1, k // 2), np.uint8)
    m1 = np.zeros((1, k // 64), np.uint32)
    w1 = x.copy()
    oracle.higptq_unit(w1, uu, 0, c1, m1, scheme, margin=mg1)
    assert w1[0, 8] == 0.375
    assert mg1[0] == 0.0
    assert (nibble(c1[0], 8) & 7) == 2  # the tie went to the even k


@pytest.mark.parametrize("scheme", [1, 2, 3])
def test_higptq_run_margin(scheme):
    """The oracle's run over several groups with margins across them: the
    same codes, meta and weights as its group steps one at a time (margins
    change no arithmetic); with the identity Hessian no update sizes and
    +inf; on generic rows finite and positive under every scheme (the later
    groups read values the earlier ones moved) and unchanged by a power-of-two
    scaling, with the update sizes scaled alike; under scheme 1 the update
    sizes are sum |F| |U| with F = E U_SS^-1 per group; and a tie planted
    across groups gives 0 where the per-group margin, which counts only moves
    inside a group, gives +inf."""
    n, k = 16, 256
    W, _, U = _gptq_problem(n, k, 82)
    w = W.astype(np.float64)
    wr, cr, mr = w.copy(), np.zeros((n, k // 2), np.uint8), np.zeros((n, k // 64), np.uint32)
    mg, am = np.full(n, np.inf), np.zeros((n, k))
    oracle.higptq_run(wr, U, 0, k // 64, cr, mr, scheme, mg, am)
    wu, cu, mu = w.copy(), np.zeros_like(cr), np.zeros_like(mr)
    for unit in range(k // 64):
        oracle.higptq_unit(wu, U, unit, cu, mu, scheme)
    assert np.array_equal(wr, wu) and np.array_equal(cr, cu) and np.array_equal(mr, mu)
    assert np.all(np.isfinite(mg)) and np.all(mg > 0)
    mg4, am4 = np.full(n, np.inf), np.zeros((n, k))
    oracle.higptq_run(4.0 * w, U, 0, k // 64, np.zeros_like(cr), np.zeros_like(mr), scheme, mg4,
                      am4)
    assert np.array_equal(mg, mg4) and np.array_equal(4.0 * am, am4)
    if scheme == 1:
        # update sizes from the F each group implies (E from the weights the
        # group started from, which the run leaves in the group's columns)
        ref = np.zeros((n, k))
        for unit in range(k // 64):
            s0, r0 = 64 * unit, 64 * unit + 64
            E = wr[:, s0:r0] - oracle.dequantize(cr[:, 32 * unit:32 * unit + 32],
                                                 mr[:, unit:unit + 1])
            F = np.linalg.solve(U[s0:r0, s0:r0].T, E.T).T
            ref[:, r0:] += np.abs(F) @ np.abs(U[s0:r0, r0:])
        assert np.allclose(am, ref, rtol=1e-12, atol=0)
        assert np.all(am[:, :64] == 0)
    mgi, ami = np.full(n, np.inf), np.zeros((n, k))
    oracle.higptq_run(w.copy(), np.eye(k), 0, k // 64, np.zeros_like(cr), np.zeros_like(mr),
                      scheme, mgi, ami)
    assert np.all(np.isinf(mgi)) and not ami.any()
    # Planted tie across groups. Group 0: x_0 = 7 sets v(c) = 1, e2 = e3 = 1
    # (D = 4) and quantizes exactly; x_1 = 0.25 rounds to 0, so F_1 = 0.25,
    # and U[1, 64] = 2 moves column 64 by -0.5: 2.6875 -> 2.1875. Group 1:
    # its largest value x_65 = 6 sets v(c) = 0.875 (7 v(c) = 6.125 >= 6),
    # e2 = e3 = 1 (6 > 3.0625), D = 3.5, and 2.1875 = 5 D / 8 is the tie
    # between k = 2 and k = 3; every other decision on column 64 is away
    # from its boundary.
    kk = 128
    x = np.zeros((1, kk))
    x[0, 0], x[0, 1], x[0, 64], x[0, 65] = 7.0, 0.25, 2.6875, 6.0
    uu = np.eye(kk)
    uu[1, 64] = 2.0
    c1, m1 = np.zeros((1, kk // 2), np.uint8), np.zeros((1, kk // 64), np.uint32)
    mg1, am1 = np.full(1, np.inf), np.zeros((1, kk))
    w1 = x.copy()
    oracle.higptq_run(w1, uu, 0, 2, c1, m1, scheme, mg1, am1)
    assert w1[0, 64] == 2.1875 and oracle.e6m2_value(int(m1[0, 1] & 255)) == 0.875
    assert mg1[0] == 0.0
    assert (nibble(c1[0], 64) & 7) == 2  # the tie went to the even k
    assert am1[0, 64] == 0.5 and np.count_nonzero(am1) == 1
    # the per-group margin of the same second step sees no move inside it
    w2 = x.copy()
    oracle.higptq_unit(w2, uu, 0, c1, m1, scheme)
    mg2 = np.zeros(1)
    oracle.higptq_unit(w2, uu, 1, c1, m1, scheme, margin=mg2)
    assert np.isinf(mg2[0])
