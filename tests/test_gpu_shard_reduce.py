"""GPU parity of the K-shard combination (include/det_gemm.h,
det_gemm_shard_reduce): RL-Kernel operator page "Batch-Invariant Deterministic
GEMM (det_gemm)", section "Ascend NPU backend", bullet "Reduction tree" -- a
contiguous half of the reduction is one child of the tree.  For TP = 2^j
contiguous equal shards the partial products are subtrees, so their fixed
rank-order tree equals the unsharded product bit for bit; this is the local
step of a deterministic reduce-scatter, shown here on one GPU."""
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


@pytest.mark.parametrize("nparts", list(range(1, 17)))
def test_tree_over_parts_matches_oracle(dev, nparts):
    say("shard reduce vs oracle tree, parts", nparts)
    M, N = 37, 333
    parts = [Wk.randn_bf16((M, N), 1.0, 300 + nparts * 17 + k, dev) for k in range(nparts)]
    got = bits(dg.det_gemm_shard_reduce(parts))
    stack = np.stack([bits(p) for p in parts], axis=-1)      # [M, N, nparts]
    want, _ = oracle.tree_from_leaves(stack)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("tp", [2, 4, 8, 16])
def test_tp_shards_equal_unsharded_product(dev, tp):
    """QKV shape, K = 4096 (L = 128) cut into TP contiguous shards."""
    say("simulated TP", tp, "at M=1024 K=4096 N=6144")
    X = Wk.randn_bf16((1024, 4096), 1.0, 2003, dev)
    W = Wk.qkv_weight(dev)
    full = dg.det_gemm_fwd(X, W)
    k = 4096 // tp
    parts = [dg.det_gemm_fwd(X[:, i * k:(i + 1) * k].contiguous(), W[i * k:(i + 1) * k])
             for i in range(tp)]
    assert torch.equal(dg.det_gemm_shard_reduce(parts).view(torch.int16), full.view(torch.int16))


def test_strided_and_unaligned(dev):
    say("shard reduce strided / unaligned")
    base = [Wk.randn_bf16((20, 70), 1.0, 400 + k, dev) for k in range(5)]
    parts = [b[:, 3:67] for b in base]                      # ld 70, unaligned rows
    got = bits(dg.det_gemm_shard_reduce(parts))
    want, _ = oracle.tree_from_leaves(np.stack([bits(p) for p in parts], axis=-1))
    assert np.array_equal(got, want)
