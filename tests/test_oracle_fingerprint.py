"""Pins of the oracle for tensor fingerprints and the first-mismatch comparator
(reading notes "Bitwise-Deterministic Pretraining at Scale", sections
"5. Fingerprinting Tensors on the GPU" and "Reading the first mismatch").

The digest (a reading; the pages name no hash): S = sum over the little-endian
64-bit words w_i of mix(w_i + GAMMA*(i+1)) mod 2^64, digest = mix(S + n), mix =
SplitMix64's finalizer.  Pins, each independent of the oracle's code:
  * mix is the bijection its published constants define: an inverse written
    here from the algebra (xor-shift inversion, modular inverses of the
    multipliers) undoes it on random inputs; SplitMix64 seeded with 0 yields
    mix(GAMMA) = 0xE220A8397B1DCDAF as its first output;
  * inverting the final mix recovers S, which checks the word assembly
    (little endian, zero fill past n), the position term and the length term;
  * row digests are the digests of each row's bytes;
  * the first mismatch equals a brute-force scan.
"""
import numpy as np
import pytest

import oracle

M64 = 2**64 - 1
GAMMA = 0x9E3779B97F4A7C15
C1, C2 = 0xBF58476D1CE4E5B9, 0x94D049BB133111EB


def _unxorshift(y, s):
    x = y
    for _ in range(64 // s + 1):
        x = y ^ (x >> s)
    return x


def mix_inverse(z):
    z = _unxorshift(z, 31)
    z = (z * pow(C2, -1, 2**64)) & M64
    z = _unxorshift(z, 27)
    z = (z * pow(C1, -1, 2**64)) & M64
    return _unxorshift(z, 30)


def test_mix_is_the_published_bijection():
    rng = np.random.default_rng(1)
    for x in [0, 1, 2**63, M64] + [int(v) for v in rng.integers(0, 2**63, 200, dtype=np.int64)]:
        assert mix_inverse(oracle.mix64(x)) == x
    assert oracle.mix64(0) == 0
    # SplitMix64 from state 0: state += GAMMA, output mix(state)
    assert oracle.mix64(GAMMA) == 0xE220A8397B1DCDAF


def _S(buf):
    n = np.asarray(buf).nbytes
    return (mix_inverse(oracle.fingerprint(buf)) - n) & M64


def _term(w, i):
    return oracle.mix64((w + GAMMA * (i + 1)) & M64)


def test_digest_structure():
    assert oracle.fingerprint(np.zeros(0, np.uint8)) == 0          # mix(0 + 0)
    # little-endian words, position term i + 1
    b = np.zeros(16, np.uint8)
    b[0] = 1
    assert _S(b) == (_term(1, 0) + _term(0, 1)) & M64
    b = np.zeros(16, np.uint8)
    b[15] = 1
    assert _S(b) == (_term(0, 0) + _term(1 << 56, 1)) & M64
    # bytes past n read as 0: the same words, only the length term differs
    x = np.arange(1, 12, dtype=np.uint8)
    y = np.concatenate([x, np.zeros(1, np.uint8)])
    assert _S(x) == _S(y) and oracle.fingerprint(x) != oracle.fingerprint(y)


def test_digest_is_a_sum_of_position_terms():
    rng = np.random.default_rng(2)
    a = rng.integers(0, 256, 8 * 37 + 5, dtype=np.uint8)
    W = (a.size + 7) // 8
    padded = np.zeros(8 * W, np.uint8)
    padded[:a.size] = a
    words = padded.view("<u8")
    assert _S(a) == sum(_term(int(w), i) for i, w in enumerate(words)) & M64
    # changing one word changes exactly its term
    j = 11
    b = a.copy()
    b[8 * j:8 * j + 8] ^= 0x5A
    wj = int(words[j])
    wj2 = int(b[8 * j:8 * j + 8].view("<u8")[0])
    assert (_S(b) - _S(a)) & M64 == (_term(wj2, j) - _term(wj, j)) & M64


def test_order_sensitivity():
    rng = np.random.default_rng(3)
    t = rng.standard_normal((64, 32)).astype(np.float32)
    p = t[::-1].copy()                           # rows permuted
    assert oracle.fingerprint(t) != oracle.fingerprint(p)
    w = t.copy().reshape(-1).view(np.uint64)
    w[[0, 1]] = w[[1, 0]]                        # two 8-byte words swapped
    assert oracle.fingerprint(t) != oracle.fingerprint(w)
    assert oracle.fingerprint(t) == oracle.fingerprint(t.copy())


def test_rows_are_digests_of_row_bytes():
    rng = np.random.default_rng(4)
    a = rng.integers(0, 2**16, (9, 13), dtype=np.uint16)   # 26-byte rows: a partial word
    d = oracle.fingerprint_rows(a)
    for r in range(a.shape[0]):
        assert int(d[r]) == oracle.fingerprint(a[r])
    # equal rows, equal digests, wherever they sit
    a[7] = a[2]
    d = oracle.fingerprint_rows(a)
    assert d[7] == d[2]


@pytest.mark.parametrize("n", [0, 1, 7, 8, 4097])
def test_first_mismatch_brute_force(n):
    rng = np.random.default_rng(n)
    a = rng.integers(0, 256, n, dtype=np.uint8)
    assert oracle.first_mismatch(a, a.copy()) == -1
    for k in ([n - 1, 0, n // 2] if n else []):
        b = a.copy()
        b[k] ^= 1
        b[min(n - 1, k + 3)] ^= 2 if k + 3 < n else 0
        assert oracle.first_mismatch(a, b) == int(np.nonzero(a != b)[0][0])
