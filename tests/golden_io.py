"""Readers for the text fixtures under tests/golden/ (no method arithmetic)."""
import os

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _lines(name):
    with open(os.path.join(GOLDEN, name), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                yield line


def s1p2_magnitudes():
    return [float(v) for v in _lines("s1p2_values.txt")]


def unit_budget():
    out = {}
    for line in _lines("unit_budget.txt"):
        k, v = line.split()
        out[k] = int(v)
    return out


def _pairs(spec, conv):
    spec = spec.strip()
    if not spec:
        return {}
    if spec.startswith("all:"):
        return {"all": conv(spec[4:])}
    out = {}
    for item in spec.split(","):
        a, b = item.split(":")
        out[int(a)] = conv(b)
    return out


def hand_units():
    units = []
    for line in _lines("hand_units.txt"):
        fields = [f.strip() for f in line.split(";")]
        u = {"name": fields[0]}
        for f in fields[1:]:
            key, _, val = f.partition("=")
            if key == "x":
                u["x"] = _pairs(val, float)
            elif key == "meta":
                u["meta"] = int(val, 16)
            elif key == "nib":
                u["nib"] = _pairs(val, lambda s: int(s, 16))
            elif key == "bytes":
                u["bytes"] = _pairs(val, lambda s: int(s, 16))
            elif key == "deq":
                u["deq"] = _pairs(val, float)
        units.append(u)
    return units


def expand(d, n, default=0):
    """Dense list of length n from a {index: value} / {'all': value} map."""
    if "all" in d:
        return [d["all"]] * n
    out = [default] * n
    for i, v in d.items():
        out[i] = v
    return out


def percentile_cases():
    cases = []
    for line in _lines("percentile_type7.txt"):
        q, vals, exp = [f.strip() for f in line.split(";")]
        cases.append((float(q), [float(v) for v in vals.split(",")], float(exp)))
    return cases
