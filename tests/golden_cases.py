"""Reader for tests/golden/hand_cases.txt (hand-derived single-element cases)."""
import os
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_cases.txt")


def parse_value(text):
    """[-]<int> | [-]<int>*2^<int> | [-]2^<int>  ->  Fraction."""
    t = text.strip()
    sign = 1
    if t.startswith("-"):
        sign, t = -1, t[1:]
    if "*" in t:
        mant, pw = t.split("*")
        return sign * Fraction(int(mant)) * Fraction(2) ** int(pw.split("^")[1])
    if t.startswith("2^"):
        return sign * Fraction(2) ** int(t[2:])
    return sign * Fraction(int(t))


def bf16_bits_of(v):
    """Exact bf16 value (Fraction) -> bit pattern (asserts exactness)."""
    f = np.float32(float(v))
    assert Fraction(float(f)) == v, f"{v} is not exact in fp32"
    u = int(np.array([f], np.float32).view(np.uint32)[0])
    assert u & 0xFFFF == 0, f"{v} is not a bf16 value"
    return u >> 16


def load_cases():
    cases, cur = [], None
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.rstrip("\n")
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "case":
                cur = {"name": rest.strip(), "a": {}, "b": {}}
                cases.append(cur)
            elif key == "K":
                cur["K"] = int(rest)
            elif key in ("a", "b"):
                for item in rest.split():
                    idx, val = item.split(":")
                    cur[key][int(idx)] = parse_value(val)
            elif key == "expect":
                cur["expect"] = int(rest, 16)
            elif key == "why":
                cur["why"] = rest
            else:
                raise ValueError(f"bad line {line!r}")
    for c in cases:
        K = c["K"]
        a = np.zeros(K, np.uint16)
        b = np.full(K, 0x3F80, np.uint16)
        for i, v in c["a"].items():
            a[i] = bf16_bits_of(v)
        for i, v in c["b"].items():
            b[i] = bf16_bits_of(v)
        c["a_bits"], c["b_bits"] = a, b
    return cases
