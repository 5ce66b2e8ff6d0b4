"""Pins of the batch-invariant RMSNorm oracle (summary page of "Defeating
Nondeterminism in LLM Inference", batch-invariant kernel design, RMSNorm: one
row per core, the same reduction whatever the batch size).

Definition (a reading; the page fixes only that the strategy is constant):
the squares x_i^2 (fp32) are summed by the mid-split tree of fp32 adds over
the row's H positions (a range of n splits into floor(n/2) on the left, the
rest on the right); rstd = 1/sqrt(ss/H + eps); y = bf16((x*rstd)*w).  The
order depends on H alone.

Pins: hand-derived sums of squares whose value depends on the tree shape
(pairwise rather than sequential, the split in the middle of the range, the
odd split taking floor(n/2) on the left), a closed form (constant rows of a
power of two), and float64 within the rounding bound of a depth-ceil(log2 H)
tree on random rows.
"""
import numpy as np
import pytest

import oracle


def bf(v):
    return (np.asarray(v, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def val(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _row(H, entries):
    x = np.zeros((1, H), np.uint16)
    for i, v in entries.items():
        x[0, i] = bf(v)
    return x


ONES = lambda H: np.full(H, bf(1.0), np.uint16)


# (H, {index: value}, expected sum of squares, why).  4096^2 = 2^24, where the
# fp32 spacing is 2: 2^24 + 1 is a tie that goes to the even 2^24.
CASES = [
    (4, {0: 4096.0, 2: 1.0, 3: 1.0}, 16777218.0,
     "squares (2^24, 0, 1, 1): the tree adds (2^24 + 0) + (1 + 1) = 2^24 + 2 exactly; "
     "a left-to-right sum would give ((2^24 + 0) + 1) + 1 = 2^24"),
    (3, {0: 4096.0, 1: 1.0, 2: 1.0}, 16777218.0,
     "squares (2^24, 1, 1), odd range: floor(3/2) = 1 on the left, so "
     "2^24 + (1 + 1) = 2^24 + 2; the other split, (2^24 + 1) + 1, gives 2^24"),
    (2048, {0: 4096.0, 1024: 1.0, 1536: 1.0}, 16777218.0,
     "the right half [1024, 2048) sums to 1 + 1 = 2 before meeting the left "
     "half's 2^24: 2^24 + 2; a sum in index order gives 2^24"),
    (2048, {0: 4096.0, 1023: 1.0, 1024: 1.0}, 16777216.0,
     "the two ones sit on either side of the root's split: the left half is "
     "2^24 + 1 -> 2^24 (tie to even), the right half 1, and 2^24 + 1 -> 2^24"),
]


@pytest.mark.parametrize("case", CASES, ids=[f"H{c[0]}_{i}" for i, c in enumerate(CASES)])
def test_sum_of_squares_tree_shape(case):
    H, e, want, why = case
    ss = oracle.rmsnorm(_row(H, e), ONES(H), 0.0)[2][0]
    assert ss == np.float32(want), why


def test_sum_of_squares_split_is_in_the_middle():
    """H = 6: splits 3 | 3, then 1 | 2.  Squares (2^24, 0, 0, 1, 0, 1): the
    right half (1 + (0 + 1)) = 2 meets the left half 2^24: 2^24 + 2.  A
    power-of-two split 4 | 2 would give (2^24 + 1) + 1 -> 2^24."""
    x = _row(6, {0: 4096.0, 3: 1.0, 5: 1.0})
    assert oracle.rmsnorm(x, ONES(6), 0.0)[2][0] == np.float32(16777218.0)


@pytest.mark.parametrize("H,k", [(64, 3), (4096, -2), (5000, 5)])
def test_constant_rows_closed_form(H, k):
    """x = 2^k everywhere, eps = 0: ss = H * 4^k exactly, the mean is 4^k,
    rstd = 2^-k exactly, and y = x * rstd * w = w bit for bit."""
    x = np.full((3, H), bf(2.0 ** k), np.uint16)
    rng = np.random.default_rng(H)
    w = bf(rng.standard_normal(H).astype(np.float32))
    y, rstd, ss = oracle.rmsnorm(x, w, 0.0)
    assert np.all(ss == np.float32(H * 4.0 ** k))
    assert np.all(rstd == np.float32(2.0 ** -k))
    assert np.array_equal(y, np.broadcast_to(w, y.shape))


@pytest.mark.parametrize("H", [1, 7, 4096, 5120])
def test_float64_bounds(H):
    rng = np.random.default_rng(7 + H)
    R = 16
    x = bf((rng.standard_normal((R, H)) * 3).astype(np.float32))
    w = bf((1 + 0.1 * rng.standard_normal(H)).astype(np.float32))
    eps = 1e-6
    y, rstd, ss = oracle.rmsnorm(x, w, eps)
    xv, wv = val(x).astype(np.float64), val(w).astype(np.float64)
    ss64 = (xv * xv).sum(axis=1)
    # fp32 tree of non-negative terms: relative error below (depth) * 2^-24
    depth = max(1, int(np.ceil(np.log2(H))))
    assert np.all(np.abs(ss - ss64) <= depth * 2.0 ** -24 * ss64)
    r64 = 1 / np.sqrt(ss64 / H + eps)
    assert np.all(np.abs(rstd - r64) <= (depth + 4) * 2.0 ** -24 * r64)
    y64 = xv * r64[:, None] * wv[None, :]
    spacing = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(y64), 2.0 ** -126))) - 7)
    assert np.all(np.abs(val(y) - y64) <= 0.5 * spacing + (depth + 8) * 2.0 ** -24 * np.abs(y64))


def test_zero_row_and_eps():
    H = 256
    x = np.zeros((1, H), np.uint16)
    w = ONES(H)
    y, rstd, ss = oracle.rmsnorm(x, w, 0.25)
    assert ss[0] == 0 and rstd[0] == np.float32(2.0) and np.all(y == 0)
