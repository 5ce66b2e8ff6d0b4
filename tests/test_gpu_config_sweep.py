"""Seeded sweep over shapes, strides, alignments and the six products: every
tile configuration the library accepts for a problem, and its automatic choice,
gives the bits of the general kernel.

Contract (RL-Kernel operator page "Batch-Invariant Deterministic GEMM
(det_gemm)", section "Guarantees"): the result of a product does not depend on
how the work is split; here the split is the tile configuration (tile shape,
wave count, copy scheme, the tree split over wave groups of the narrow tiles,
the decode kernel's split over waves), which the host picks from the shape.
The general kernel (configuration 2) is pinned to the oracle by the parity
tests; each problem here is computed by every configuration that takes it
(the others answer EINVAL) and compared with it bit for bit.
"""
import random

import numpy as np
import pytest
import torch

import det_workloads as W
import invariant_deterministic_gemm_det_amd as dg
from gpu_util import device, say

pytestmark = pytest.mark.gpu

GENERAL_CFG = 2
# Row counts around the decode limits (16, 32, 64, 128 rows) and the tile
# heights; column counts around the 16-, 32-, 64- and 128-column tiles,
# ragged ones included; reduction lengths with 1 to 192 leaves, powers of two,
# 3, 5 and 7 times 2^a and others, and two that are not whole leaves.
ROWS = [1, 2, 3, 15, 16, 17, 31, 32, 33, 48, 63, 64, 65, 96, 100, 127, 128, 129, 200, 256, 300]
COLS = [8, 16, 24, 40, 64, 100, 128, 136, 256, 392, 512, 1000, 1024, 2048, 2056, 6144]
REDS = [32, 64, 96, 160, 224, 256, 288, 512, 1024, 1536, 2048, 4096, 4128, 5120, 6144, 7168]
OPS = ["fwd", "fwd_rhs_transposed", "fwd_fp32", "da", "db", "db_transposed"]
PROBLEMS = 240


@pytest.fixture(scope="module")
def dev():
    d = device()
    dg.load_library()
    dg.det_gemm_debug_force_config(-1)
    return d


def _view(rows, cols, sigma, seed, pad, off, dev):
    """A [rows, cols] bf16 view with leading dimension cols + pad, starting
    `off` elements into its allocation (off = 1: rows not 16-byte aligned)."""
    ld = cols + pad
    flat = W.randn_bf16((rows * ld + off + 8,), sigma, seed).to(dev)
    return flat[off:off + rows * ld].view(rows, ld)[:, :cols]


def _problem(rng, i, dev):
    op = rng.choice(OPS)
    M, N, K = rng.choice(ROWS), rng.choice(COLS), rng.choice(REDS)
    pad = [rng.choice([0, 0, 8, 64, 3]) for _ in range(2)]
    off = [rng.choice([0, 0, 0, 8, 1]) for _ in range(2)]
    s = 9000 + 2 * i
    if op in ("fwd", "fwd_fp32"):
        P, Q = _view(M, K, 1.0, s, pad[0], off[0], dev), _view(K, N, 0.02, s + 1, pad[1], off[1], dev)
        f = dg.det_gemm_fwd if op == "fwd" else dg.det_gemm_fwd_fp32
    elif op == "fwd_rhs_transposed":
        P, Q = _view(M, K, 1.0, s, pad[0], off[0], dev), _view(N, K, 0.02, s + 1, pad[1], off[1], dev)
        f = dg.det_gemm_fwd_rhs_transposed
    elif op == "da":
        P, Q = _view(M, N, 1.0, s, pad[0], off[0], dev), _view(K, N, 0.02, s + 1, pad[1], off[1], dev)
        f = dg.det_gemm_da
    else:
        P, Q = _view(M, K, 1.0, s, pad[0], off[0], dev), _view(M, N, 0.5, s + 1, pad[1], off[1], dev)
        f = dg.det_gemm_db if op == "db" else dg.det_gemm_db_transposed
    return op, (M, N, K, pad, off), (lambda: f(P, Q))


def _bits(t):
    t = t.contiguous()
    return t.view(torch.int32 if t.dtype == torch.float32 else torch.int16).cpu().numpy()


def test_every_accepted_configuration_matches_the_general_kernel(dev):
    rng = random.Random(20261202)
    n = dg.det_gemm_debug_force_config(-1)
    taken = {c: 0 for c in range(-1, n)}
    try:
        for i in range(PROBLEMS):
            op, shape, call = _problem(rng, i, dev)
            say("config sweep", i, op, shape)
            dg.det_gemm_debug_force_config(GENERAL_CFG)
            ref = _bits(call())
            for cfg in range(-1, n):
                dg.det_gemm_debug_force_config(cfg)
                try:
                    got = _bits(call())
                except dg.DetGemmError as e:
                    # only a pinned configuration may refuse a problem
                    assert cfg >= 0 and e.code == dg.EINVAL, (i, op, shape, cfg)
                    continue
                taken[cfg] += 1
                assert np.array_equal(got, ref), (i, op, shape, cfg)
    finally:
        dg.det_gemm_debug_force_config(-1)
    say("configurations taken", taken)
    # the sweep reaches every kernel family: general, direct-to-LDS, wide,
    # decode and the narrow split tiles
    for cfg in (0, 3, 5, 8, 9, 10, 11, 12, 13, 14, 15, 16):
        assert taken[cfg] > 0, cfg
