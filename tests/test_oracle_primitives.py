"""Pins for the oracle's two scalar primitives (CPU only).

* fp32 -> bf16 rounding (page "Batch-Invariant Deterministic GEMM (det_gemm)",
  section "Ascend NPU backend": leaves are "rounded once to BF16
  (round-to-nearest-even)"): every one of the 2^32 fp32 bit patterns against
  torch's own float32 -> bfloat16 conversion, plus hand values.
* the tree's bf16 add (same bullet: leaves "merged with BF16 adds"): against
  the correctly rounded bf16 sum computed two independent ways -- exact rational
  arithmetic on a sample, and a float64 route rounded from the textbook
  definition on a large grid (all 2^32 pairs when DET_GEMM_EXHAUSTIVE=1).
"""
import os
import random
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from exact_reference import BF16, round_to, bf16_value, bf16_bits


def _torch_bf16_bits(f32):
    return torch.from_numpy(f32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _is_bf16_nan(h):
    return ((h & 0x7F80) == 0x7F80) & ((h & 0x007F) != 0)


def test_round_all_fp32_patterns_match_torch():
    step = 1 << 24
    base = np.arange(step, dtype=np.uint32)
    for start in range(0, 1 << 32, step):
        u = base + np.uint32(start)
        f = u.view(np.float32)
        ours = oracle.round_bf16(f)
        ref = _torch_bf16_bits(f)
        nan = np.isnan(f)
        bad = np.flatnonzero((ours != ref) & ~nan)
        assert bad.size == 0, f"mismatch at fp32 bits {u[bad[:5]]}: {ours[bad[:5]]} vs {ref[bad[:5]]}"
        assert _is_bf16_nan(ours[nan]).all()


@pytest.mark.parametrize("value, bits", [
    (1.0 + 2.0 ** -8, 0x3F80),          # halfway, 1.0 is even
    (1.0 + 3 * 2.0 ** -8, 0x3F82),      # halfway, 1 + 2^-6 is even
    (1.0 + 2.0 ** -8 + 2.0 ** -20, 0x3F81),  # just above halfway
    (-(1.0 + 2.0 ** -8 + 2.0 ** -20), 0xBF81),
    (float(np.finfo(np.float32).max), 0x7F80),  # rounds past the largest bf16
    (float("inf"), 0x7F80),
    (float("-inf"), 0xFF80),
    (-0.0, 0x8000),
    (0.0, 0x0000),
    (2.0 ** -149, 0x0000),              # smallest fp32 subnormal -> 0
    (3 * 2.0 ** -134, 0x0002),          # halfway between 2^-133 (odd) and 2^-132 (even)
])
def test_round_hand_values(value, bits):
    assert int(oracle.round_bf16(np.array([value], np.float32))[0]) == bits


def _f64_to_bf16_bits(s):
    """Nearest bf16 to each float64 (ties to even), from the definition: the
    spacing of bf16 numbers in [2^e, 2^(e+1)) is 2^(e-7), never below 2^-133;
    results at or above 2^128 overflow to infinity."""
    a = s.abs()
    _, e = torch.frexp(a)                  # a = m * 2^e with m in [0.5, 1)
    lead = torch.clamp(e.to(torch.int64) - 1, min=-126)
    ulp_exp = lead - 7
    q = a * torch.pow(2.0, (-ulp_exp).to(torch.float64))
    v = torch.round(q) * torch.pow(2.0, ulp_exp.to(torch.float64))
    v = torch.where(v >= 2.0 ** 128, torch.full_like(v, float("inf")), v)
    v = torch.copysign(v, s)
    return (v.to(torch.float32).view(torch.int32) >> 16).to(torch.int32).numpy().astype(np.uint16)


def _bits_to_f64(h):
    t = torch.from_numpy(h.astype(np.int32) << 16).view(torch.float32)
    return t.to(torch.float64)


def _check_add_block(a, b):
    ours = oracle.add_bf16(a, b)
    ref = _f64_to_bf16_bits(_bits_to_f64(a) + _bits_to_f64(b))
    nan = _is_bf16_nan(ref)
    bad = np.flatnonzero((ours != ref) & ~nan)
    assert bad.size == 0, (f"bf16 add mismatch: a={a[bad[:4]]} b={b[bad[:4]]} "
                           f"ours={ours[bad[:4]]} ref={ref[bad[:4]]}")
    assert _is_bf16_nan(ours[nan]).all()


def test_add_against_float64_definition():
    """All 2^16 left operands against a grid of right operands (every pattern when
    DET_GEMM_EXHAUSTIVE=1): every exponent, both signs, zeros, subnormals, inf."""
    a_all = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    if os.environ.get("DET_GEMM_EXHAUSTIVE") == "1":
        b_vals = a_all
    else:
        rng = np.random.default_rng(7)
        b_vals = np.unique(np.concatenate([
            np.arange(0, 1 << 16, 37, dtype=np.uint32).astype(np.uint16),
            rng.integers(0, 1 << 16, 1024).astype(np.uint16),
            np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x007F, 0x0080, 0x7F7F, 0xFF7F,
                      0x7F80, 0xFF80, 0x3F80, 0xBF80, 0x3B80, 0xBB80], np.uint16)]))
    block = 256
    for i in range(0, b_vals.size, block):
        bb = b_vals[i:i + block]
        a = np.tile(a_all, bb.size)
        b = np.repeat(bb, a_all.size)
        _check_add_block(a, b)


def test_add_against_exact_rationals():
    rng = random.Random(11)
    specials = [0x0000, 0x0001, 0x8001, 0x007F, 0x0080, 0x3F80, 0xBF80, 0x7F7F, 0xFF7F,
                0x3B80, 0x4B80, 0xCB80, 0x3F81, 0x3401]
    pairs = [(x, y) for x in specials for y in specials]
    for _ in range(20000):
        # keep exponents within reach of each other often, so ties and carries occur
        x = rng.randrange(1 << 16)
        if rng.random() < 0.7:
            y = (x & 0x8000) ^ rng.choice((0, 0x8000)) | max(0, min(0x7F7F, (x & 0x7FFF) + rng.randrange(-0x0C00, 0x0C00)))
        else:
            y = rng.randrange(1 << 16)
        pairs.append((x, y))
    finite = [(x, y) for x, y in pairs if (x & 0x7F80) != 0x7F80 and (y & 0x7F80) != 0x7F80]
    a = np.array([p[0] for p in finite], np.uint16)
    b = np.array([p[1] for p in finite], np.uint16)
    ours = oracle.add_bf16(a, b)
    for (x, y), got in zip(finite, ours):
        exact = bf16_value(x) + bf16_value(y)
        want = bf16_bits(round_to(exact, BF16))
        if exact == 0:
            # x + (-x) is +0 under round-to-nearest; -0 + -0 is -0
            want = 0x8000 if (x == 0x8000 and y == 0x8000) else 0x0000
        assert int(got) == want, f"{x:#06x} (+) {y:#06x}: got {int(got):#06x} want {want:#06x}"
