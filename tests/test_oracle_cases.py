"""Pins for the oracle's whole operations (CPU only).

Page: RL-Kernel operator page "Batch-Invariant Deterministic GEMM (det_gemm)".
  - section "Guarantees": C = A @ B, dA = dC B^T, dB = A^T dC; bf16 in, fp32
    accumulation, no split-K, fixed K order; a row's bits never depend on batch
    size, chunked prefill or padding.
  - section "Ascend NPU backend": 32-element fp32 leaves in ascending order,
    rounded once to bf16; mid-split tree of bf16 adds in ascending leaf order; a
    contiguous half-K product is one child of the tree (simulated TP=2 equals
    TP=1 bitwise); six entry points, db_transposed born in [N,K]; fp32 output
    from forward_fp32; reduction capped at 32768.

What pins what:
  * hand-derived golden cases (tests/golden/hand_cases.txt): leaf size, leaf
    order, rounding ties, overflow, tree shape and odd-split direction -- run
    through all six operations;
  * integer regime: with entries in {-1, 0, 1} and R <= 256 every partial sum is
    an exact small integer, so each operation must equal the int64 matrix
    product (indexing, operand roles, transposes, leading dimensions);
  * an exact-rational brute force on tiny random shapes (arithmetic);
  * the half-K identity, including leaf counts that are not powers of two (the
    split point of the tree);
  * a forward error bound against float64 (no gross loss of accuracy);
  * argument errors.
"""
import numpy as np
import pytest
import torch

import det_workloads as W
import oracle
from exact_reference import dot as exact_dot
from golden_cases import load_cases

CASES = load_cases()


def _np(t):
    return W.bits(t)


# --------------------------------------------------------------- golden cases

@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_golden_case_all_ops(case):
    a, b, K, want = case["a_bits"], case["b_bits"], case["K"], case["expect"]
    A = a.reshape(1, K)
    B = b.reshape(K, 1)
    got = {
        "fwd": oracle.fwd(A, B)[0, 0],
        "fwd_rhs_transposed": oracle.fwd_rhs_transposed(A, b.reshape(1, K))[0, 0],
        # dA[0,0] = sum_n dC[0,n] * Bw[0,n]   (reduction over N = K here)
        "da": oracle.da(A, b.reshape(1, K))[0, 0],
        # dB[0,0] = sum_m A[m,0] * dC[m,0]    (reduction over M = K here)
        "db": oracle.db(a.reshape(K, 1), b.reshape(K, 1))[0, 0],
        "db_transposed": oracle.db_transposed(a.reshape(K, 1), b.reshape(K, 1))[0, 0],
    }
    f32 = oracle.fwd_fp32(A, B)[0, 0]
    got["fwd_fp32"] = int(np.array([f32], np.float32).view(np.uint32)[0] >> 16)
    for op, v in got.items():
        assert int(v) == want, f"{op}: got {int(v):#06x}, hand-derived {want:#06x} ({case['why']})"
    assert exact_dot(list(a), list(b)) == want, "exact-rational brute force disagrees"


# --------------------------------------------------------------- integer regime

def _int_case(M, N, K, seed, pad=0):
    """A[M,K], B[K,N] in {-1,0,1}, stored with `pad` extra columns per row."""
    A = _np(W.int_bf16((M, K + pad), seed))[:, :K]
    B = _np(W.int_bf16((K, N + pad), seed + 1))[:, :N]
    return A, B


def _val(bits_):
    return (bits_.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@pytest.mark.parametrize("M,N,K,pad", [(1, 1, 1, 0), (3, 5, 7, 0), (7, 9, 33, 3), (5, 4, 64, 8),
                                       (16, 3, 95, 1), (4, 6, 256, 0), (2, 17, 200, 5)])
def test_integer_regime_equals_int64_product(M, N, K, pad):
    A, B = _int_case(M, N, K, 100 * M + N + K, pad)
    Ai, Bi = _val(A).astype(np.int64), _val(B).astype(np.int64)
    C = Ai @ Bi
    assert np.array_equal(_val(oracle.fwd(A, B)), C)
    assert np.array_equal(_val(oracle.fwd_rhs_transposed(A, np.ascontiguousarray(B.T))), C)
    assert np.array_equal(oracle.fwd_fp32(A, B).astype(np.float64), C)
    # backward shapes: treat A as [M,K] activations and B as [K,N] weights
    dC = _np(W.int_bf16((M, N + pad), 900 + K))[:, :N]
    dCi = _val(dC).astype(np.int64)
    assert np.array_equal(_val(oracle.da(dC, np.ascontiguousarray(B))), dCi @ Bi.T)
    assert np.array_equal(_val(oracle.db(A, dC)), Ai.T @ dCi)
    assert np.array_equal(_val(oracle.db_transposed(A, dC)), (Ai.T @ dCi).T)


# --------------------------------------------------------------- brute force

@pytest.mark.parametrize("seed", range(6))
def test_exact_rational_brute_force(seed):
    rng = np.random.default_rng(seed)
    M, N = int(rng.integers(1, 4)), int(rng.integers(1, 4))
    K = int(rng.choice([1, 5, 31, 32, 33, 64, 95, 96, 160, 224, 385]))
    A = _np(W.randn_bf16((M, K), 1.0, 7000 + seed))
    B = _np(W.randn_bf16((K, N), 1.0, 7100 + seed))
    want = [[exact_dot(list(A[i]), list(B[:, j])) for j in range(N)] for i in range(M)]
    assert oracle.fwd(A, B).tolist() == want


# --------------------------------------------------------------- half-K identity

@pytest.mark.parametrize("K", [64, 192, 320, 1024, 12288])
def test_half_k_is_one_child_of_the_tree(K):
    """fwd(A, B) == fwd(A[:, :K/2], B[:K/2]) (+) fwd(A[:, K/2:], B[K/2:]).
    K = 192 (6 leaves), 320 (10) and 12288 (384) are not powers of two: a
    power-of-two or left-to-right tree would fail them."""
    A = _np(W.randn_bf16((3, K), 1.0, 8000 + K))
    B = _np(W.randn_bf16((K, 5), 0.02, 8100 + K))
    h = K // 2
    lo = oracle.fwd(A[:, :h], B[:h])
    hi = oracle.fwd(A[:, h:], B[h:])
    assert np.array_equal(oracle.fwd(A, B), oracle.add_bf16(lo, hi))


def test_half_k_breaks_for_a_misaligned_split():
    """Sanity of the test above: splitting K=192 at 80 (not a tree child) must
    change at least one bit on random data."""
    K = 192
    A = _np(W.randn_bf16((8, K), 1.0, 8300))
    B = _np(W.randn_bf16((K, 8), 1.0, 8301))
    full = oracle.fwd(A, B)
    mis = oracle.add_bf16(oracle.fwd(A[:, :80], B[:80]), oracle.fwd(A[:, 80:], B[80:]))
    assert not np.array_equal(full, mis)


# --------------------------------------------------------------- invariances

def test_rows_independent_of_batch_padding_and_chunks():
    A, B = W.small_forward()
    A, B = _np(A), _np(B)
    full = oracle.fwd(A, B)
    for M in (1, 7, 64):
        assert np.array_equal(oracle.fwd(A[:M], B), full[:M])
    padded = np.concatenate([A[:7], np.zeros((16, A.shape[1]), np.uint16)])
    assert np.array_equal(oracle.fwd(padded, B)[:7], full[:7])
    wide = np.zeros((64, 300), np.uint16)
    wide[:, :256] = A
    assert np.array_equal(oracle.fwd(wide[:, :256], B), full)   # lda = 300
    chunks = [oracle.fwd(A[i:i + 10], B) for i in range(0, 64, 10)]
    assert np.array_equal(np.concatenate(chunks), full)


def test_layout_identities():
    A = _np(W.randn_bf16((9, 100), 1.0, 9001))
    B = _np(W.randn_bf16((100, 11), 1.0, 9002))
    dC = _np(W.randn_bf16((9, 11), 1.0, 9003))
    C = oracle.fwd(A, B)
    assert np.array_equal(oracle.fwd_rhs_transposed(A, np.ascontiguousarray(B.T)), C)
    assert np.array_equal(oracle.fwd_fp32(A, B), _val(C).astype(np.float32))
    assert np.array_equal(oracle.da(dC, np.ascontiguousarray(B)),
                          oracle.fwd_rhs_transposed(dC, np.ascontiguousarray(B)))
    assert np.array_equal(oracle.db(A, dC), oracle.fwd(np.ascontiguousarray(A.T), dC))
    assert np.array_equal(oracle.db_transposed(A, dC), oracle.db(A, dC).T)


def test_tree_from_leaves_matches_detail():
    A = _np(W.randn_bf16((4, 416), 1.0, 9101))
    B = _np(W.randn_bf16((416, 6), 1.0, 9102))
    C, leaves, big = oracle.fwd_detail(A, B)
    roots, big2 = oracle.tree_from_leaves(leaves)
    assert np.array_equal(roots, C) and np.array_equal(big, big2)
    assert leaves.shape == (4, 6, 13)
    assert (big >= np.abs(_val(C))).all()


# --------------------------------------------------------------- error bound

def test_forward_error_bound_against_float64():
    """|c - sum x*y| <= ((ceil(log2 L) + 1) * 2^-8 + 32 * 2^-24) * 1.01 * sum |x*y|:
    one bf16 rounding per tree level plus the leaf rounding, and at most 31 fp32
    roundings inside a leaf."""
    for K in (32, 96, 1000, 4096):
        A = _np(W.randn_bf16((6, K), 1.0, 9200 + K))
        B = _np(W.randn_bf16((K, 7), 1.0, 9300 + K))
        x, y = _val(A), _val(B)
        exact = x @ y
        mag = np.abs(x) @ np.abs(y)
        L = (K + 31) // 32
        depth = int(np.ceil(np.log2(L))) if L > 1 else 0
        bound = ((depth + 1) * 2.0 ** -8 + 32 * 2.0 ** -24) * 1.01 * mag
        err = np.abs(_val(oracle.fwd(A, B)) - exact)
        assert (err <= bound).all()


# --------------------------------------------------------------- argument errors

def test_reduction_cap_and_empty_shapes():
    A = np.zeros((2, 32769), np.uint16)
    B = np.zeros((32769, 2), np.uint16)
    with pytest.raises(oracle.OracleError) as e:
        oracle.fwd(A, B)
    assert e.value.code == -2
    with pytest.raises(oracle.OracleError):
        oracle.fwd(np.zeros((2, 0), np.uint16), np.zeros((0, 2), np.uint16))
    assert oracle.fwd(np.zeros((0, 8), np.uint16), np.zeros((8, 3), np.uint16)).shape == (0, 3)
    # the cap itself is accepted
    out = oracle.fwd(np.zeros((1, 32768), np.uint16), np.zeros((32768, 1), np.uint16))
    assert out.tolist() == [[0]]
