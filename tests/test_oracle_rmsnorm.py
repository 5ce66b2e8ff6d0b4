"""Pins of the batch-invariant RMSNorm oracle (summary page of "Defeating
Nondeterminism in LLM Inference", batch-invariant kernel design, RMSNorm: one
row per core, the same reduction whatever the batch size).

Definition (a reading; the page fixes only that the strategy is constant):
lane t of 256 sums, in fp32 and ascending order, the squares of the elements
of its 8-element chunks (chunk c belongs to lane c mod 256); the 256 lane sums
are joined by the pairwise tree; rstd = 1/sqrt(ss/H + eps); y = bf16((x*rstd)*w).

Pins: hand-derived sums of squares whose value depends on each part of the
order (in-lane sequential, chunk-to-lane assignment, pairwise across lanes),
a closed form (constant rows of a power of two), and float64 within the
rounding bounds on random rows.
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


# (H, {index: value}, expected sum of squares, why)
CASES = [
    (8, {0: 4096.0, 2: 1.0, 3: 1.0}, 16777216.0,
     "one chunk, one lane: 2^24 + 0 + 1 + 1 added in order; each + 1 is a tie "
     "between 2^24 and 2^24 + 2 and goes to the even 2^24 (a pairwise sum would "
     "give (2^24 + 0) + (1 + 1) = 2^24 + 2)"),
    (2048, {0: 4096.0, 1024: 1.0, 1536: 1.0}, 16777218.0,
     "chunks 0, 128, 192 sit in lanes 0, 128, 192; the pairwise tree over 256 "
     "lanes joins lanes 128..191 and 192..255 first (1 + 1 = 2), then adds 2^24: "
     "2^24 + 2 exactly (a single lane or lanes in sequence would give 2^24)"),
]


def test_sum_of_squares_in_lane_order():
    H, e, want, _ = CASES[0]
    assert oracle.rmsnorm(_row(H, e), ONES(H), 0.0)[2][0] == np.float32(want)


def test_sum_of_squares_across_lanes_pairwise():
    H, e, want, _ = CASES[1]
    assert oracle.rmsnorm(_row(H, e), ONES(H), 0.0)[2][0] == np.float32(want)


def test_chunk_to_lane_assignment_wraps_at_256():
    # element 2048 = chunk 256 belongs to lane 0 together with element 0: the
    # lane adds 2^24 + 1 -> 2^24 (tie to even), and the ones in lanes 128 and
    # 192 meet first (1 + 1 = 2): 2^24 + 2.  If chunk 256 had a lane of its own
    # (more than 256 lanes), the total would be 2^24 + 3 -> 2^24 + 4 (nearest).
    H = 4096
    x = _row(H, {0: 4096.0, 2048: 1.0, 1024: 1.0, 1536: 1.0})
    assert oracle.rmsnorm(x, ONES(H), 0.0)[2][0] == np.float32(16777218.0)


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
    # fp32 sums of non-negative terms: relative error below (depth) * 2^-24
    depth = 8 + int(np.ceil(H / (8 * 256))) * 8
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
