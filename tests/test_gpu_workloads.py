"""GPU checks at the full sizes of the transformer-shaped workloads, through
the C-ABI, in the tile configurations the library picks by itself (those the
benchmark times).

Contract (RL-Kernel operator page "Batch-Invariant Deterministic GEMM
(det_gemm)", section "Guarantees"): a row's bits never depend on the batch
size, on chunked prefill or on padding; a contiguous half of the reduction is
one child of the tree, so two half-K products merged with one bf16 add equal
the full product (TP = 2 equals TP = 1).

At these sizes the oracle computes sampled outputs only (probe rows, a few
rows or columns); everything else is checked through properties that hold at
any size: invariance to the batch, to chunking and to the order of unrelated
rows, the layout identities and the half-K / half-M identities.
"""
import numpy as np
import pytest
import torch

import det_workloads as Wk
import oracle
import invariant_deterministic_gemm_det_amd as dg
from gpu_util import device, say, bits, tolerance_report, ulp_distance, leaf_bound_ok

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = device()
    dg.load_library()
    dg.det_gemm_debug_force_config(-1)
    return d


def _same(a, b):
    """Bitwise equality of two device tensors (bf16 or fp32), on the device."""
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a.view(torch.int32), b.view(torch.int32))


def _oracle_check(got, A_rows, B):
    """Sampled outputs against the oracle: leaves structure is not available
    here, so the per-element bound of the MFMA path (within 2 bf16 spacings of
    the largest node of the oracle's tree for that element)."""
    c, _, big = oracle.fwd_detail(bits(A_rows), bits(B))
    hist, beyond, ratio = tolerance_report(bits(got), c, big)
    print("  sampled vs oracle: ulp histogram", hist, "beyond", beyond, "worst ratio",
          round(ratio, 3))
    assert beyond == 0
    return c


def test_qkv_probe_rows_across_batch_sizes(dev):
    say("QKV K=4096 N=6144: 16 probe rows bitwise across M in {1,16,128,1024,4096}")
    Wt = Wk.qkv_weight(dev)
    Wtt = Wt.t().contiguous()
    probes = Wk.qkv_probes(dev)
    ref = None
    for M in (1, 16, 128, 1024, 4096):
        if M == 1:   # one call per probe row
            rows = torch.cat([dg.det_gemm_fwd(probes[p:p + 1], Wt) for p in range(16)])
            rows_t = torch.cat([dg.det_gemm_fwd_rhs_transposed(probes[p:p + 1], Wtt)
                                for p in range(16)])
        else:
            b = Wk.qkv_batch(M, dev, probes)
            pos = b.positions.to(dev)
            rows = dg.det_gemm_fwd(b.x, Wt)[pos]
            rows_t = dg.det_gemm_fwd_rhs_transposed(b.x, Wtt)[pos]
        assert _same(rows, rows_t), M
        if ref is None:
            ref = rows
        assert _same(rows, ref), M
        print("  M =", M, "probe rows identical")
    # the strict kernel on the probes equals the oracle bit for bit
    c = _oracle_check(ref, probes, Wt)
    strict = dg.det_gemm_fwd(probes, Wt, strict=True)
    assert np.array_equal(bits(strict), c)


def _chunks(X, Wt, sizes):
    out, a = [], 0
    for s in sizes:
        out.append(dg.det_gemm_fwd(X[a:a + s], Wt))
        a += s
    assert a == X.shape[0]
    return torch.cat(out)


@pytest.mark.parametrize("which", ["gate_up", "down"])
def test_mlp_chunked_prefill(dev, which):
    X, Wgu, H, Wd = Wk.mlp_inputs(dev)
    A, Bm = (X, Wgu) if which == "gate_up" else (H, Wd)
    say("MLP", which, "M=8192: chunks of 512 and of 1000 vs unsplit", tuple(A.shape),
        tuple(Bm.shape))
    full = dg.det_gemm_fwd(A, Bm)
    assert _same(_chunks(A, Bm, [512] * 16), full)
    assert _same(_chunks(A, Bm, [1000] * 8 + [192]), full)
    rows = torch.tensor([0, 1000, 4097, 8191], device=dev)
    _oracle_check(full[rows], A[rows], Bm)


def test_backward_invariances(dev):
    A, B, dC = Wk.backward_inputs(dev)   # A[8192,4096] B[4096,4096] dC[8192,4096]
    M = A.shape[0]
    say("backward M=8192 K=N=4096: dA row order, dB columns, db_t, half-M")
    dA = dg.det_gemm_da(dC, B)
    dB = dg.det_gemm_db(A, dC)
    # dA rows follow their dC rows whatever the order of the other rows
    perm = Wk.randperm(M, 4099).to(dev)
    assert _same(dg.det_gemm_da(dC[perm], B), dA[perm])
    # a dB column depends on its dC column only
    cols = Wk.randperm(dC.shape[1], 4098)[:384].sort().values.to(dev)
    assert _same(dg.det_gemm_db(A, dC[:, cols].contiguous()), dB[:, cols])
    # the transposed store
    assert _same(dg.det_gemm_db_transposed(A, dC), dB.t().contiguous())
    # half-M identity: the two halves of the batch are the two children of the root
    h = M // 2
    lo = dg.det_gemm_db(A[:h], dC[:h])
    hi = dg.det_gemm_db(A[h:], dC[h:])
    assert _same(dg.det_gemm_debug_add(lo, hi), dB)
    # sampled against the oracle: rows of dA, columns of dB
    r = torch.tensor([0, 4095, 8191], device=dev)
    c_da = oracle.da(bits(dC[r]), bits(B))
    assert tolerance_report(bits(dA[r]), c_da, _big_da(dC[r], B))[1] == 0
    k = torch.tensor([3, 2048], device=dev)
    c_db = oracle.db(bits(A), bits(dC[:, k].contiguous()))
    got = bits(dB[:, k].contiguous())
    _, _, big = oracle.fwd_detail(bits(A.t().contiguous()), bits(dC[:, k].contiguous()))
    assert tolerance_report(got, c_db, big)[1] == 0


def _big_da(dCr, B):
    """Largest node magnitudes of the oracle's trees for rows of dA = dC B^T."""
    _, _, big = oracle.fwd_detail(bits(dCr), bits(B.t().contiguous()))
    return big


@pytest.mark.parametrize("M", [1, 256, 4096])
def test_lm_head_batch_and_fp32_out(dev, M):
    X, Wlm = Wk.lm_head_inputs(dev)   # X[4096,4096], Wlm[4096,151936]
    say("LM head K=4096 N=151936: rows of M =", M, "vs M = 4096, bf16 and fp32 out")
    ref = dg.det_gemm_fwd(X[:16], Wlm)
    C = dg.det_gemm_fwd(X[:M], Wlm)
    n = min(M, 16)
    assert _same(C[:n], ref[:n])
    F = dg.det_gemm_fwd_fp32(X[:M], Wlm)
    assert _same(F, C.float())
    if M == 1:
        _oracle_check(C, X[:1], Wlm)


@pytest.mark.parametrize("shape", ["lm_head", "deep"])
def test_simulated_tp2(dev, shape):
    if shape == "lm_head":
        X, Bm = Wk.lm_head_inputs(dev)
        X = X[:256]
    else:
        X, Bm = Wk.deep_inputs(dev)   # A[2048,32768] B[32768,4096]: the depth cap
    K = X.shape[1]
    h = K // 2
    say("simulated TP=2:", shape, tuple(X.shape), tuple(Bm.shape))
    full = dg.det_gemm_fwd(X, Bm)
    lo = dg.det_gemm_fwd(X[:, :h], Bm[:h])
    hi = dg.det_gemm_fwd(X[:, h:], Bm[h:])
    merged = dg.det_gemm_debug_add(lo, hi)
    assert _same(merged, full)
    assert _same(dg.det_gemm_fwd_fp32(X, Bm), merged.float())
    if shape == "deep":
        _oracle_check(full[:2], X[:2], Bm)


# ---------------------------------------------------------------- every element at the step shape

# Elements allowed beyond the literal 2-ulp bound, as a fraction of the
# product.  A leaf the matrix core sums in its own internal order can land one
# bf16 step (more for a leaf whose products cancel) from the sequential leaf;
# where the tree then cancels down to a root much smaller than that leaf, one
# step of the leaf is several steps of the root.  Each such element is checked
# structurally instead: the kernel's own leaves for it are within the rigorous
# leaf bound of the oracle's, and the oracle's tree over the kernel's leaves
# gives the kernel's output bit for bit -- the leaf-internal order is then the
# only difference.
BEYOND_2ULP_FRACTION = 1e-4


@pytest.mark.parametrize("op", ["fwd", "da", "db"])
def test_step_products_every_element(dev, op):
    """The three products of the benchmark step (M = K = 4096, N = 6144, the
    seeds and entry points the benchmark uses, so the same tile
    configurations), every output element against the oracle: within 2 bf16
    ulp of the oracle's element, except a counted few (at most a fraction
    1e-4) that cancellation pushes beyond it, each of which must be explained
    by its leaves alone (see BEYOND_2ULP_FRACTION)."""
    X, W, dC = Wk.step_inputs(dev)
    say("step product", op, "every element vs the oracle (M=K=4096, N=6144)")
    # the product as a forward contraction P[I,R] @ Q[R,J] (same products, same order)
    if op == "fwd":
        got = dg.det_gemm_fwd(X, W)
        P, Q = X, W
    elif op == "da":     # dX = dC W^T
        got = dg.det_gemm_da(dC, W)
        P, Q = dC, W.t().contiguous()
    else:                # dW = X^T dC
        got = dg.det_gemm_db(X, dC)
        P, Q = X.t().contiguous(), dC
    want, _, big = oracle.fwd_detail(bits(P), bits(Q), with_leaves=False)
    g = bits(got)
    hist, _, _ = tolerance_report(g, want, big)
    far = ulp_distance(g, want) > 2
    over = int(far.sum())
    print(f"  {op}: ulp histogram {hist}; beyond 2 ulp: {over} of {g.size} ({over / g.size:.2e})")
    assert over <= BEYOND_2ULP_FRACTION * g.size
    if over == 0:
        return
    ri, cj = np.nonzero(far)
    rows, cols = np.unique(ri), np.unique(cj)
    Pr = P[torch.as_tensor(rows, device=dev)].contiguous()
    Qc = Q[:, torch.as_tensor(cols, device=dev)].contiguous()
    lg = bits(dg.det_gemm_debug_leaves(Pr, Qc))
    _, lv, _ = oracle.fwd_detail(bits(Pr), bits(Qc))
    ok, worst = leaf_bound_ok(lg, lv, bits(Pr), bits(Qc))
    roots, _ = oracle.tree_from_leaves(lg)
    r_at = np.searchsorted(rows, ri)
    c_at = np.searchsorted(cols, cj)
    print(f"  {op}: leaves of those elements' rows and columns: within the leaf bound {ok}, "
          f"worst leaf distance {worst} ulp")
    assert ok
    assert np.array_equal(roots[r_at, c_at], g[ri, cj]), \
        "an element beyond 2 ulp is not the oracle's tree over the kernel's leaves"
