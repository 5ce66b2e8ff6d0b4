"""Pins of the oracle for the MoE grouped GEMM and its per-token reduction
epilogue (reading notes "Bitwise-Deterministic Pretraining at Scale: How
Megatron Core Finds and Removes Every Flipped Bit", section "Kernel redesign:
the grouped-GEMM epilogue": private per-N-tile slots combined by a fixed
reduction tree instead of atomic adds).

Each pin checks the oracle against something other than itself:
  * hand-derived single-row cases (tests/golden/moe_cases.txt): tree shapes,
    the odd-split direction across slots, signed zeros of the padding;
  * the integer regime: with entries in {-1, 0, 1} every product, partial sum
    and output is an exact integer, so Y equals the int64 product with the
    row's own expert weight and dprob / the slots equal int64 dot products;
  * float64: dprob lies within the pairwise-summation error bound of the exact
    dot product (a dropped term, a wrong sign or a wrong column fails it).
"""
import os

import numpy as np
import pytest

import oracle
from golden_cases import parse_value

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "moe_cases.txt")


def _bf16(v):
    """Exact value (Fraction or -0 marker) -> bf16 bits."""
    if v == "-0":
        return 0x8000
    f = np.float32(float(v))
    u = int(np.array([f], np.float32).view(np.uint32)[0])
    assert u & 0xFFFF == 0 and float(f) == float(v)
    return u >> 16


def _load_cases():
    cases, cur = [], None
    with open(GOLDEN) as fh:
        for line in fh:
            line = line.rstrip("\n")
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "case":
                cur = {"name": rest.strip(), "y": {}, "g": {}, "slot": {}}
                cases.append(cur)
            elif key == "N":
                cur["N"] = int(rest)
            elif key in ("y", "g"):
                for item in rest.split():
                    idx, val = item.split(":")
                    cur[key][idx] = "-0" if val == "-0" else parse_value(val)
            elif key == "slot":
                for item in rest.split():
                    j, bits = item.split(":")
                    cur["slot"][int(j)] = int(bits, 16)
            elif key == "expect":
                cur["expect"] = int(rest, 16)
    return cases


CASES = _load_cases()


def _row(entries, N):
    r = np.zeros((1, N), np.uint16)
    for idx, v in entries.items():
        if idx == "all":
            r[0, :] = _bf16(v)
        else:
            r[0, int(idx)] = _bf16(v)
    return r


def _f32_bits(x):
    return int(np.array([x], np.float32).view(np.uint32)[0])


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_golden_epilogue_cases(case):
    Y, G = _row(case["y"], case["N"]), _row(case["g"], case["N"])
    slots, dprob = oracle.moe_dprob(Y, G)
    assert slots.shape == ((case["N"] + 127) // 128, 1)
    for j, bits in case["slot"].items():
        assert _f32_bits(slots[j, 0]) == bits, (case["name"], j)
    assert _f32_bits(dprob[0]) == case["expect"], case["name"]


def test_golden_file_covers_the_readings():
    names = {c["name"] for c in CASES}
    assert {"slot_pairwise_tree", "slots_odd_split_floor_left",
            "padding_positions_are_plus_zero"} <= names


def _int_bits(a):
    """Small integers -> bf16 bits (exact)."""
    return (np.asarray(a, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _bits_val(b):
    return (b.astype(np.uint32) << 16).view(np.float32)


def _offsets(sizes):
    return np.concatenate([[0], np.cumsum(sizes)]).astype(np.int64)


@pytest.mark.parametrize("sizes,N,K", [
    ([5, 0, 1, 9], 300, 96),      # an empty expert, a one-row expert, a ragged last slot
    ([16], 128, 64),              # one expert, one full slot
    ([3, 7], 1, 33),              # one column, a partial leaf
])
def test_integer_regime_exact(sizes, N, K):
    rng = np.random.default_rng(11 + N + K)
    E, T = len(sizes), int(sum(sizes))
    X = rng.integers(-1, 2, (T, K))
    W = rng.integers(-1, 2, (E, K, N))
    G = rng.integers(-1, 2, (T, N))
    off = _offsets(sizes)
    Yb, slots, dprob = oracle.moe_fwd_dprob(_int_bits(X), _int_bits(W), off, _int_bits(G))
    # every row is multiplied by its own expert's weight
    Yexp = np.zeros((T, N), np.int64)
    for e in range(E):
        Yexp[off[e]:off[e + 1]] = X[off[e]:off[e + 1]] @ W[e]
    assert np.array_equal(_bits_val(Yb).astype(np.int64), Yexp)
    P = Yexp * G
    assert np.array_equal(dprob.astype(np.int64), P.sum(axis=1))
    J = (N + 127) // 128
    for j in range(J):
        assert np.array_equal(slots[j].astype(np.int64), P[:, 128 * j:128 * j + 128].sum(axis=1))


def test_rows_with_another_expert_weight_differ():
    """The routing pin has teeth: the same rows under a neighbouring expert's
    weight give different outputs."""
    rng = np.random.default_rng(5)
    X = rng.integers(-1, 2, (4, 64))
    W = rng.integers(-1, 2, (2, 64, 128))
    Yb, _, _ = oracle.moe_fwd_dprob(_int_bits(X), _int_bits(W), [0, 2, 4], _int_bits(np.ones((4, 128))))
    assert np.array_equal(_bits_val(Yb[:2]).astype(np.int64), X[:2] @ W[0])
    assert not np.array_equal(_bits_val(Yb[:2]).astype(np.int64), X[:2] @ W[1])


@pytest.mark.parametrize("N", [128, 1000, 4096 + 64])
def test_dprob_within_pairwise_bound_of_float64(N):
    rng = np.random.default_rng(N)
    T = 64
    Y = oracle.round_bf16(rng.standard_normal((T, N)).astype(np.float32))
    G = oracle.round_bf16((rng.standard_normal((T, N)) * 1e-3).astype(np.float32))
    slots, dprob = oracle.moe_dprob(Y, G)
    P = _bits_val(Y).astype(np.float64) * _bits_val(G).astype(np.float64)
    J = (N + 127) // 128
    h = 7 + int(np.ceil(np.log2(J))) if J > 1 else 7
    u = 2.0 ** -24
    gamma = h * u / (1 - h * u)
    err = np.abs(dprob.astype(np.float64) - P.sum(axis=1))
    assert np.all(err <= gamma * np.abs(P).sum(axis=1))
    for j in range(J):
        blk = P[:, 128 * j:128 * j + 128]
        g7 = 7 * u / (1 - 7 * u)
        assert np.all(np.abs(slots[j] - blk.sum(axis=1)) <= g7 * np.abs(blk).sum(axis=1))
    # the bound is tight enough to see a dropped column
    P2 = P.copy()
    P2[:, N // 2] = 0
    assert np.any(np.abs(dprob.astype(np.float64) - P2.sum(axis=1)) > gamma * np.abs(P).sum(axis=1))


def test_empty_columns_and_rows():
    slots, dprob = oracle.moe_dprob(np.zeros((3, 0), np.uint16), np.zeros((3, 0), np.uint16))
    assert slots.shape == (0, 3) and np.array_equal(dprob.view(np.uint32), np.zeros(3, np.uint32))
    slots, dprob = oracle.moe_dprob(np.zeros((0, 5), np.uint16), np.zeros((0, 5), np.uint16))
    assert dprob.shape == (0,)


def test_offsets_validated():
    X = np.zeros((4, 32), np.uint16)
    W = np.zeros((2, 32, 16), np.uint16)
    G = np.zeros((4, 16), np.uint16)
    for bad in ([0, 3, 2], [1, 2, 4], [0, 2, 5]):
        with pytest.raises(oracle.OracleError):
            oracle.moe_fwd_dprob(X, W, bad, G)
