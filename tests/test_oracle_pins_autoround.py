"""Pins of the oracle's HiAutoRound quantize step (HiFloat4 calibration
article, section 3.2 "HiAutoRound": offsets K on the level-3 exponents,
E' = E + RZ(K), and mantissa offsets M, shifted M' = M >> RZ(K) before they
are added) against exact rational arithmetic, independently of the oracle's
binary32 path:

* K = 0 and M = 0 reproduce the plain quantize (pinned in test_oracle_pins);
* a mantissa offset just under +1/2 (-1/2) turns the rounding into ceil
  (floor) of the exact scaled magnitude t = 4|x| / D;
* K moves each level-3 bit to clamp(e3 + trunc(K), 0, 1), and then every
  element is the exact RNE of t on the new grid;
* with K moving the exponent by d, the mantissa offset acts as M 2^-d.

The oracle forms t = fl(|x| / (D/4)) and fl(t + M') in binary32 (reading
R16). |x| and D/4 are exact, so t carries at most 2^-24 t of error and the sum
at most 2^-24 |t + M'| more: with t <= 14 and |M'| <= 1 in these pins, less
than 2^-19 in all. Elements whose exact t + M' lies within 2^-18 of a
half-integer are therefore left out of the M checks, and every other
element must equal the exact-real round-to-nearest-even of t + M'. Exact
ties (t + M' = n + 1/2 with t and M' exact in binary32) are pinned
separately: they must go to the even n.
"""
from fractions import Fraction
import math

import numpy as np
import pytest

import oracle
import unit_cases as uc

UNIT = 64
BAND = Fraction(1, 2 ** 18)  # binary32 error of fl(t + M') is below 2^-19 here
pytestmark = pytest.mark.filterwarnings("ignore")


def _inputs(n, seed):
    return np.concatenate([uc.random_bits(n, seed), uc.midpoint_bits(max(1, n // 4), seed + 1,
                                                                      oracle.e6m2_value)])


def _bf16_value(b):
    return Fraction(float(np.array([np.uint32(b) << np.uint32(16)], np.uint32).view(np.float32)[0]))


def _element_steps(meta_row, e3_override=None):
    """Exact grid step D of each element of a row (D = v(c) 2^(e2 + e3))."""
    d = []
    for u, m in enumerate(meta_row):
        m = int(m)
        c = m & 255
        v = Fraction(2) ** ((c >> 2) - 31) * (1 + Fraction(c & 3, 4))
        for j in range(UNIT):
            e2 = (m >> (8 + j // 8)) & 1
            e3 = (m >> (16 + j // 4)) & 1 if e3_override is None else e3_override[u][j // 4]
            d.append(v * 2 ** (e2 + e3))
    return d


def _nibbles(codes_row):
    """Element nibbles of a row in element order (unit layout of hif4_quantize)."""
    out = []
    for u in range(codes_row.size // 32):
        b = codes_row[32 * u:32 * u + 32]
        for j in range(UNIT):
            byte = b[4 * (j // 8) + j % 4]
            out.append(int(byte >> (4 if j % 8 >= 4 else 0)) & 15)
    return out


def _rne(q):
    f = math.floor(q)
    r = q - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return f


def test_zero_offsets_are_the_plain_quantize():
    x = np.concatenate([_inputs(300, 11), uc.special_values_bits(7)[:, :UNIT]])
    x = x[:, :UNIT] if x.shape[1] > UNIT else x
    rows, k = x.shape
    c0, m0, _ = oracle.quantize(x)
    c1, m1 = oracle.quantize_offsets(x, np.zeros((rows, k // 4), np.float32),
                                     np.zeros((rows, k), np.float32))
    assert np.array_equal(c0, c1) and np.array_equal(m0, m1)


@pytest.mark.parametrize("sign", [1, -1])
def test_half_mantissa_offset_is_ceil_or_floor(sign):
    x = _inputs(120, 23 + sign)
    rows, k = x.shape
    delta = Fraction(1, 256)
    mval = sign * (Fraction(1, 2) - delta)
    _, meta0, _ = oracle.quantize(x)
    codes, meta = oracle.quantize_offsets(x, np.zeros((rows, k // 4), np.float32),
                                          np.full((rows, k), float(mval), np.float32))
    assert np.array_equal(meta, meta0)  # K = 0: exponents untouched
    checked = ceil_floor = 0
    for r in range(rows):
        steps = _element_steps(meta[r])
        nib = _nibbles(codes[r])
        for j in range(k):
            a = abs(_bf16_value(x[r, j]))
            t = 4 * a / steps[j]
            u = t + mval
            frac = u - math.floor(u)
            if abs(frac - Fraction(1, 2)) < BAND:
                continue  # within binary32's error of a rounding decision
            want = min(7, max(0, _rne(u)))
            assert nib[j] & 7 == want, (r, j, t, nib[j])
            neg = _bf16_value(x[r, j]) < 0
            assert (nib[j] >> 3) == (1 if (neg and want) else 0)
            checked += 1
            # the offset's purpose: ceil (floor) of t, except where the
            # fractional part of t lies within delta of the other side
            ft = t - math.floor(t)
            if ft == 0 or (ft > delta if sign > 0 else ft < 1 - delta):
                cf = min(7, max(0, math.ceil(t) if sign > 0 else math.floor(t)))
                assert want == cf
                ceil_floor += 1
    assert checked > rows * k * 99 // 100
    assert ceil_floor > rows * k * 9 // 10


def test_k_offset_moves_level3_exponent_then_exact_rne():
    x = _inputs(120, 31)
    rows, k = x.shape
    r = np.random.default_rng(5)
    choices = np.float32([-3.2, -1.5, -0.7, 0.0, 0.7, 1.5, 2.5])
    koff = r.choice(choices, size=(rows, k // 4)).astype(np.float32)
    _, meta0, _ = oracle.quantize(x)
    codes, meta = oracle.quantize_offsets(x, koff, np.zeros((rows, k), np.float32))
    for row in range(rows):
        e3new = []
        for u in range(k // UNIT):
            m0, m1 = int(meta0[row, u]), int(meta[row, u])
            assert (m0 & 0xFFFF) == (m1 & 0xFFFF)  # c and level-2 bits unchanged
            e3u = []
            for q in range(16):
                e3 = (m0 >> (16 + q)) & 1
                want = min(1, max(0, e3 + math.trunc(float(koff[row, 16 * u + q]))))
                assert (m1 >> (16 + q)) & 1 == want
                e3u.append(want)
            e3new.append(e3u)
        steps = _element_steps(meta0[row], e3new)
        nib = _nibbles(codes[row])
        for j in range(k):
            t = 4 * abs(_bf16_value(x[row, j])) / steps[j]
            want = min(7, _rne(t))
            assert nib[j] & 7 == want, (row, j, t)


def test_mantissa_offset_follows_the_exponent_change():
    """d = e3' - e3 = +1 halves the offset, d = -1 doubles it."""
    x = _inputs(80, 41)
    rows, k = x.shape
    _, meta0, _ = oracle.quantize(x)
    koff = np.zeros((rows, k // 4), np.float32)
    dsh = np.zeros((rows, k // 4), np.int64)
    for row in range(rows):
        for u in range(k // UNIT):
            for q in range(16):
                e3 = (int(meta0[row, u]) >> (16 + q)) & 1
                koff[row, 16 * u + q] = 1.5 if e3 == 0 else -1.5  # flips every level-3 bit
                dsh[row, 16 * u + q] = 1 if e3 == 0 else -1
    mval = Fraction(3, 8)
    codes, meta = oracle.quantize_offsets(x, koff, np.full((rows, k), float(mval), np.float32))
    checked = 0
    for row in range(rows):
        flipped = [[1 - ((int(meta0[row, u]) >> (16 + q)) & 1) for q in range(16)]
                   for u in range(k // UNIT)]
        steps = _element_steps(meta0[row], flipped)
        nib = _nibbles(codes[row])
        for j in range(k):
            d = int(dsh[row, j // 4])
            mp = mval / 2 if d > 0 else mval * 2
            t = 4 * abs(_bf16_value(x[row, j])) / steps[j]
            u = t + mp
            if abs((u - math.floor(u)) - Fraction(1, 2)) < BAND:
                continue
            want = min(7, max(0, _rne(u)))
            assert nib[j] & 7 == want, (row, j, t, d)
            checked += 1
    assert checked > rows * k * 99 // 100


def _tie_unit(r, with_d_minus):
    """One unit, as bf16 bits, whose grid steps are known in advance: element
    0 = 7 (v(c) = 1, c = 124; level-2 group 0 and level-3 group 0 get their
    bits set); with_d_minus: element 4 = 4 sets the level-3 bit of elements
    4..7 too (D = 4 there), else those elements stay small. Every other
    element is a multiple of 1/16 in [0, 1.75] with a random sign, so the
    groups 1..7 keep e2 = e3 = 0 (D = 1) and all t = 4|x| / D are exact."""
    v = np.zeros(UNIT, np.float32)
    v[0] = 7.0
    mags = r.integers(0, 29, size=UNIT) / 16.0
    v[1:] = (mags[1:] * np.where(r.random(UNIT - 1) < 0.5, -1.0, 1.0)).astype(np.float32)
    v[1:4] = r.integers(0, 8, size=3) / 2.0  # quad 0 (D = 4): t = |x| exact
    if with_d_minus:
        v[4] = 4.0
        v[5:8] = (r.integers(0, 8, size=3) / 8.0).astype(np.float32)
    return (v.view(np.uint32) >> 16).astype(np.uint16)


@pytest.mark.parametrize("kmode", ["none", "up", "down"])
def test_exact_ties_of_t_plus_offset_go_to_even(kmode):
    """t + M' = n + 1/2 exactly (t and M' exact in binary32): the element is
    the even neighbour, clamped to 0..7. kmode: level-3 offsets K = 0;
    K = +1.5 on every level-3 group whose bit is 0 (d = +1, M' = M / 2);
    K = -1.5 on the groups whose bit is 1 (d = -1, M' = 2 M). M is chosen per
    element to land exactly on a tie: M' = n + 1/2 - t."""
    r = np.random.default_rng({"none": 61, "up": 62, "down": 63}[kmode])
    rows = 40
    x = np.stack([_tie_unit(r, kmode == "down") for _ in range(rows)])
    _, meta0, _ = oracle.quantize(x)
    koff = np.zeros((rows, UNIT // 4), np.float32)
    moff = np.zeros((rows, UNIT), np.float32)
    want = np.zeros((rows, UNIT), np.int64)
    tied = 0
    for row in range(rows):
        m0 = int(meta0[row, 0])
        assert m0 & 255 == 124
        e3 = [(m0 >> (16 + q)) & 1 for q in range(16)]
        e3n = list(e3)
        for q in range(16):
            if kmode == "up" and e3[q] == 0:
                koff[row, q], e3n[q] = 1.5, 1
            if kmode == "down" and e3[q] == 1:
                koff[row, q], e3n[q] = -1.5, 0
        steps = _element_steps([m0], [e3n])
        for j in range(UNIT):
            t = 4 * abs(_bf16_value(x[row, j])) / steps[j]
            n = int(r.integers(max(0, math.floor(t) - 1), math.floor(t) + 2))
            mp = Fraction(2 * n + 1, 2) - t  # t is dyadic, so M' and M are exact
            d = e3n[j // 4] - e3[j // 4]
            m = mp * 2 ** d  # M' = M 2^-d
            moff[row, j] = float(m)
            assert Fraction(float(moff[row, j])) == m
            want[row, j] = min(7, max(0, n + (n % 2)))  # tie -> even neighbour
            tied += 1
    codes, meta = oracle.quantize_offsets(x, koff, moff)
    for row in range(rows):
        nib = _nibbles(codes[row])
        for j in range(UNIT):
            assert nib[j] & 7 == want[row, j], (kmode, row, j)
    assert tied == rows * UNIT


def test_offsets_reject_bad_shapes():
    x = uc.random_bits(2, 3)
    with pytest.raises(ValueError):
        oracle.quantize_offsets(x, np.zeros((2, 15), np.float32), np.zeros((2, 64), np.float32))
