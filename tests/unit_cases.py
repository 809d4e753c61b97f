"""Test inputs that stress the HiF4 encoder (bf16 bit patterns, numpy).

Random numbers and exact-value constructions only; no method arithmetic
beyond picking values on or between grid points of a chosen level-1 code.
"""
from fractions import Fraction

import numpy as np

UNIT = 64


def to_bits(vals):
    """bf16 bit patterns of values that are exactly representable in bf16."""
    f = np.asarray(vals, dtype=np.float32)
    u = f.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exact in bf16"
    return (u >> 16).astype(np.uint16)


def truncate_to_bits(x):
    """bf16 bit patterns of float values, truncated (any rounding will do)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32) & np.uint32(0xFFFF0000)
    return (u >> 16).astype(np.uint16)


def random_bits(n, seed, spread=3.0, zero_p=0.2):
    """n units of heavy-tailed values spread over many binades, some zeros."""
    r = np.random.default_rng(seed)
    x = r.standard_t(3, size=(n, UNIT)) * np.exp(r.normal(0, spread, size=(n, 1)))
    x[r.random(size=x.shape) < zero_p] = 0.0
    return truncate_to_bits(x)


def midpoint_bits(n, seed, e6m2_value):
    """Units whose groups 1..7 sit exactly on grid midpoints (ties)."""
    r = np.random.default_rng(seed)
    rows = []
    while len(rows) < n:
        c = int(r.integers(20, 230))
        s = Fraction(e6m2_value(c))
        vals = [0.0] * UNIT
        vals[0] = float(7 * s)  # fixes c; group 0 gets e2 = e3 = 1
        for j in range(8, UNIT):
            m = int(r.integers(0, 7))
            v = min((2 * m + 1) * s / 8, Fraction(7, 4) * s)
            vals[j] = float(v) * (1 if r.random() < 0.5 else -1)
        f = np.float32(vals)
        if np.all((f.view(np.uint32) & 0xFFFF) == 0):
            rows.append((f.view(np.uint32) >> 16).astype(np.uint16))
    return np.stack(rows)


def all_magnitudes_as_unit_max(position=17, negative=False):
    """One unit per positive finite bf16 value A, placed alone at `position`."""
    a = np.arange(1, 0x7F80, dtype=np.uint16)
    x = np.zeros((a.size, UNIT), np.uint16)
    x[:, position] = a | (np.uint16(0x8000) if negative else np.uint16(0))
    return x


def all_magnitudes_under_code(c, e6m2_value, position=40):
    """Every bf16 magnitude <= 1.75 v(c) at `position`, with 7 v(c) at
    element 0 so the level-1 code is c and the element's group has E = 0."""
    s = e6m2_value(c)
    a = np.arange(1, 0x7F80, dtype=np.uint16)
    vals = (a.astype(np.uint32) << 16).view(np.float32)
    keep = a[vals <= 1.75 * s]
    x = np.zeros((keep.size, UNIT), np.uint16)
    x[:, 0] = to_bits([7 * s])[0]
    x[:, position] = keep
    return x


def special_values_bits(seed=5):
    """Zeros of both signs, subnormals, huge values (level-1 saturation)."""
    r = np.random.default_rng(seed)
    rows = []
    for _ in range(64):
        u = np.zeros(UNIT, np.uint16)
        kind = r.integers(0, 4)
        if kind == 0:
            u[:] = r.choice([0x0000, 0x8000], size=UNIT)
        elif kind == 1:
            u[:] = r.integers(0, 0x80, size=UNIT).astype(np.uint16) | r.choice([0, 0x8000], size=UNIT).astype(np.uint16)
        elif kind == 2:
            u[:] = r.integers(0x5000, 0x7F7F, size=UNIT).astype(np.uint16)
        else:
            u[:] = r.integers(0, 0x7F7F, size=UNIT).astype(np.uint16) | r.choice([0, 0x8000], size=UNIT).astype(np.uint16)
        rows.append(u)
    return np.stack(rows)
