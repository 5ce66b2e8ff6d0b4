"""GPU parity of the batch-invariant RMSNorm through the C-ABI
(include/det_norm.h): bitwise equal to the oracle (the reduction order, the
correctly rounded square root and division, and the bf16 rounding are the
same on both sides), and a row's bits independent of the batch.

Summary page of "Defeating Nondeterminism in LLM Inference", section on
batch-invariant kernel design, RMSNorm.
"""
import numpy as np
import pytest
import torch

import det_workloads as Wk
import oracle
import invariant_deterministic_gemm_det_amd as dg
from gpu_util import device, say, bits

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = device()
    dg.load_library()
    return d


def _check(x, w, eps):
    y, rstd = dg.det_rmsnorm(x, w, eps)
    yo, ro, _ = oracle.rmsnorm(bits(x), bits(w), eps)
    assert np.array_equal(bits(y), yo)
    assert np.array_equal(rstd.cpu().numpy().view(np.int32), ro.view(np.int32))
    return y, rstd


@pytest.mark.parametrize("R,H", [(1, 1), (3, 7), (5, 8), (64, 4096), (33, 5120), (9, 8200),
                                 (4, 20000), (2, 2049), (3, 256), (2, 768), (5, 3072),
                                 (3, 16384), (2, 7168), (4, 255), (3, 257)])
def test_rmsnorm_matches_oracle(dev, R, H):
    say("rmsnorm R", R, "H", H)
    x = Wk.randn_bf16((R, H), 2.0, 9000 + H, dev)
    w = Wk.randn_bf16((H,), 0.5, 9100 + H, dev)
    _check(x, w, 1e-6)


@pytest.mark.parametrize("H,ones", [(3, (1, 2)), (4, (2, 3)), (6, (3, 5)), (2048, (1024, 1536)),
                                    (2048, (1023, 1024)), (4096, (2048, 3072)), (4096, (5, 6))])
def test_rmsnorm_hand_order_cases(dev, H, ones):
    """The oracle's hand-derived tree shapes (4096^2 = 2^24 next to ones whose
    sum survives only if they meet first) reach rstd on the device; each H
    runs on the kernel it selects (a node per thread for H = 256 * M, the
    walk over computed node ranges otherwise)."""
    x = torch.zeros((1, H), dtype=torch.bfloat16)
    x[0, 0] = 4096.0
    x[0, ones[0]] = 1.0
    x[0, ones[1]] = 1.0
    w = torch.ones(H, dtype=torch.bfloat16)
    say("rmsnorm hand order case H", H, "ones at", ones)
    _check(x.to(dev), w.to(dev), 0.0)


def test_rmsnorm_strided_unaligned_and_edge_rows(dev):
    say("rmsnorm strided / unaligned / zero and non-finite rows")
    base = Wk.randn_bf16((40, 4104), 1.0, 9200, dev)
    _check(base[:, 8:4104], Wk.randn_bf16((4096,), 1.0, 9201, dev), 1e-5)      # ld 4104, aligned
    _check(base[:, 1:4097], Wk.randn_bf16((4096,), 1.0, 9202, dev), 1e-5)      # unaligned rows
    x = Wk.randn_bf16((6, 300), 1.0, 9203, dev)
    x[1] = 0
    x[2, 5] = float("inf")
    x[3, 7] = float("nan")
    w = Wk.randn_bf16((300,), 1.0, 9204, dev)
    y, rstd = dg.det_rmsnorm(x, w, 1e-6)
    yo, ro, _ = oracle.rmsnorm(bits(x), bits(w), 1e-6)
    g = bits(y)
    nan = (np.isnan((g.astype(np.uint32) << 16).view(np.float32)))
    assert np.array_equal(nan, np.isnan((yo.astype(np.uint32) << 16).view(np.float32)))
    assert np.array_equal(g[~nan], yo[~nan])
    r = rstd.cpu().numpy()
    assert np.array_equal(np.isnan(r), np.isnan(ro))
    assert np.array_equal(r[~np.isnan(r)].view(np.int32), ro[~np.isnan(ro)].view(np.int32))


@pytest.mark.parametrize("H", [4096, 5120])
def test_rmsnorm_batch_invariance(dev, H):
    """Token rows at full size: the rows of a batch of 8192 equal the same rows
    normalised alone, in chunks of 1, 7 and 1000, and inside a permuted batch."""
    say("rmsnorm batch invariance H", H)
    x = Wk.randn_bf16((8192, H), 1.0, 9300 + H, dev)
    w = Wk.randn_bf16((H,), 1.0, 9301 + H, dev)
    y, r = dg.det_rmsnorm(x, w)
    for a, b in ((0, 1), (4095, 4102), (7000, 8000)):
        yc, rc = dg.det_rmsnorm(x[a:b], w)
        assert torch.equal(yc.view(torch.int16), y[a:b].view(torch.int16))
        assert torch.equal(rc.view(torch.int32), r[a:b].view(torch.int32))
    perm = Wk.randperm(8192, 9302).to(dev)
    yp, rp = dg.det_rmsnorm(x[perm], w)
    assert torch.equal(yp.view(torch.int16), y[perm].view(torch.int16))
    rows = [0, 4096, 8191]
    yo, ro, _ = oracle.rmsnorm(bits(x[rows]), bits(w), 1e-6)
    assert np.array_equal(bits(y[rows]), yo)


@pytest.mark.parametrize("H", [1, 3, 5120])
def test_rstd_rounding_over_many_rows(dev, H):
    """rstd = 1/sqrt(ss/H + eps) with every step rounded to nearest: many short
    rows put many different values through the square root and the divisions."""
    R = 65536 if H < 100 else 512
    say("rstd rounding R", R, "H", H)
    x = Wk.randn_bf16((R, H), 3.0, 9400 + H, dev)
    w = torch.ones(H, dtype=torch.bfloat16, device=dev)
    _check(x, w, 1e-5)
