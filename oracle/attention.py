"""CPU oracle for decode attention with a fixed split-KV size -- TEST
INFRASTRUCTURE ONLY (only the test suite, the smoke check and the benchmark's
CPU-baseline leg may use it; it shares no code with the HIP library).

Summary page of "Defeating Nondeterminism in LLM Inference", section on
batch-invariant kernel design, attention: a split-KV (FlashDecoding)
reduction stays batch-invariant when the split size is fixed, and the
cached keys and values of a sequence keep one consistent layout.

The method computes, up to the rounding order of its fixed splits, plain
scaled dot-product attention, so the oracle is that definition in float64:
for sequence b, query head h (sharing key/value head h // G, G = Hq / Hkv) and
its first len[b] cached positions,
    o[b, h] = softmax(scale * K[b, h//G, :len] @ q[b, h]) @ V[b, h//G, :len];
an empty sequence (len 0) gives o = 0.
"""
import numpy as np


def _val(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def attention_decode(q, k, v, lens, scale):
    """q [B, Hq, D], k and v [B, Hkv, Smax, D] (bf16 bit patterns), lens [B]:
    returns o [B, Hq, D] float64."""
    Q, K, V = _val(q), _val(k), _val(v)
    B, Hq, D = Q.shape
    Hkv = K.shape[1]
    G = Hq // Hkv
    o = np.zeros((B, Hq, D))
    for b in range(B):
        n = int(lens[b])
        if n == 0:
            continue
        for h in range(Hq):
            kk, vv = K[b, h // G, :n], V[b, h // G, :n]
            s = scale * (kk @ Q[b, h])
            w = np.exp(s - s.max())
            o[b, h] = (w / w.sum()) @ vv
    return o


def attention_prefill(q, k, v, row_offsets, lens, scale):
    """Query rows q [NQ, Hq, D] grouped by sequence (row_offsets, B + 1
    entries), k and v [B, Hkv, Smax, D], lens [NQ]: row r attends the first
    lens[r] positions of its sequence.  Returns o [NQ, Hq, D] float64 (the
    same definition, one query row at a time)."""
    NQ = q.shape[0]
    o = np.zeros(q.shape)
    for b in range(len(row_offsets) - 1):
        for r in range(int(row_offsets[b]), int(row_offsets[b + 1])):
            o[r] = attention_decode(q[r:r + 1], k[b:b + 1], v[b:b + 1], [lens[r]], scale)[0]
    return o
