"""Pins of the float64 decode-attention oracle against closed forms (summary
page of "Defeating Nondeterminism in LLM Inference", batch-invariant kernel
design, attention)."""
import numpy as np

from oracle.attention import attention_decode, attention_prefill


def bf(x):
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def val(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _inputs(B, Hq, Hkv, S, D, seed):
    rng = np.random.default_rng(seed)
    return (bf(rng.standard_normal((B, Hq, D)).astype(np.float32)),
            bf(rng.standard_normal((B, Hkv, S, D)).astype(np.float32)),
            bf(rng.standard_normal((B, Hkv, S, D)).astype(np.float32)))


def test_equal_keys_give_the_mean_of_values():
    q, k, v = _inputs(2, 4, 2, 9, 8, 1)
    k[:] = k[:, :, :1]                       # every key equal: uniform weights
    lens = [9, 5]
    o = attention_decode(q, k, v, lens, 0.3)
    for b in range(2):
        for h in range(4):
            assert np.allclose(o[b, h], val(v[b, h // 2, :lens[b]]).mean(axis=0), rtol=0, atol=1e-12)


def test_dominant_key_selects_its_value():
    q, k, v = _inputs(1, 2, 1, 6, 8, 2)
    q[:] = bf(np.ones((1, 2, 8), np.float32))
    k[:] = bf(np.zeros((1, 1, 6, 8), np.float32))
    k[0, 0, 4] = bf(np.full(8, 8.0, np.float32))      # score 64 * scale, the others 0
    o = attention_decode(q, k, v, [6], 1.0)
    assert np.allclose(o[0, 0], val(v[0, 0, 4]), atol=1e-20 + 1e-25)
    # with a small scale the weights follow exp(score): exact two-key mixture
    k2 = bf(np.zeros((1, 1, 2, 8), np.float32))
    k2[0, 0, 1] = bf(np.full(8, 0.125, np.float32))   # score 1 for q = ones
    v2 = bf(np.array([[[[1.0] * 8, [3.0] * 8]]], np.float32))
    o2 = attention_decode(q, k2, v2, [2], 1.0)
    w1 = np.e / (1 + np.e)
    assert np.allclose(o2[0, 0], (1 - w1) * 1.0 + w1 * 3.0, rtol=1e-14)


def test_permuting_keys_and_values_together():
    q, k, v = _inputs(1, 8, 2, 40, 16, 3)
    p = np.random.default_rng(4).permutation(40)
    o = attention_decode(q, k, v, [40], 0.25)
    op = attention_decode(q, k[:, :, p], v[:, :, p], [40], 0.25)
    assert np.allclose(o, op, rtol=1e-12, atol=1e-14)


def test_length_masks_the_tail_and_zero_length():
    q, k, v = _inputs(2, 2, 1, 10, 4, 5)
    o = attention_decode(q, k, v, [7, 0], 0.5)
    k2, v2 = k.copy(), v.copy()
    k2[0, :, 7:] = bf(np.full((1, 3, 4), 30.0, np.float32))   # garbage past the length
    v2[0, :, 7:] = bf(np.full((1, 3, 4), 1e3, np.float32))
    assert np.array_equal(attention_decode(q, k2, v2, [7, 0], 0.5), o)
    assert np.all(o[1] == 0)


def test_prefill_rows_each_attend_their_own_prefix():
    """Equal keys give uniform weights, so row r's output is the mean of the
    first lens[r] values of its sequence, whatever the other rows."""
    rng = np.random.default_rng(11)
    B, Hkv, G, Smax, D = 2, 2, 2, 9, 8
    k = np.zeros((B, Hkv, Smax, D), np.uint16)                   # all keys +0: equal scores
    v = bf(rng.standard_normal((B, Hkv, Smax, D)).astype(np.float32))
    offsets = [0, 3, 7]
    lens = [1, 4, 9, 2, 5, 5, 7]
    q = bf(rng.standard_normal((7, Hkv * G, D)).astype(np.float32))
    o = attention_prefill(q, k, v, offsets, lens, 0.3)
    V = val(v)
    for b in range(B):
        for r in range(offsets[b], offsets[b + 1]):
            for h in range(Hkv * G):
                np.testing.assert_allclose(o[r, h], V[b, h // G, :lens[r]].mean(axis=0), rtol=1e-12,
                                           atol=1e-12)
