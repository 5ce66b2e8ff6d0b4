"""GPU parity of the tensor fingerprints and the first-mismatch comparator,
through the C-ABI (include/det_fingerprint.h), against the oracle: integer
work, compared bit for bit.

Reading notes "Bitwise-Deterministic Pretraining at Scale", sections
"5. Fingerprinting Tensors on the GPU" and "Reading the first mismatch".
"""
import numpy as np
import pytest
import torch

import det_workloads as Wk
import oracle
import invariant_deterministic_gemm_det_amd as dg
from invariant_deterministic_gemm_det_amd.trace import Trace, first_divergence
from gpu_util import device, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = device()
    dg.load_library()
    return d


def _rand_bytes(n, seed, dev):
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return torch.randint(0, 256, (n,), generator=g, dtype=torch.uint8).to(dev)


def _host(t):
    return t.cpu().numpy()


@pytest.mark.parametrize("n", [0, 1, 7, 8, 15, 16, 17, 4096, 65536 + 13, (1 << 22) + 5])
@pytest.mark.parametrize("offset", [0, 3])
def test_digest_matches_oracle(dev, n, offset):
    say("fingerprint n", n, "offset", offset)
    buf = _rand_bytes(n + offset, 100 + n, dev)
    t = buf[offset:]
    got = dg.digest_value(dg.det_fingerprint(t))
    assert got == oracle.fingerprint(_host(t))


def test_digest_of_tensors_and_determinism(dev):
    x = Wk.randn_bf16((513, 300), 1.0, 7, dev)
    say("fingerprint bf16 tensor", tuple(x.shape))
    d1 = dg.digest_value(dg.det_fingerprint(x))
    assert d1 == oracle.fingerprint(Wk.bits(x))
    assert d1 == dg.digest_value(dg.det_fingerprint(x.clone()))
    y = x.clone()
    y.view(torch.int16)[200, 17] ^= 1          # one bit
    assert dg.digest_value(dg.det_fingerprint(y)) != d1
    z = x[torch.arange(512, -1, -1, device=dev)].contiguous()   # rows reversed
    assert dg.digest_value(dg.det_fingerprint(z)) != d1


def test_large_buffer(dev):
    n = (256 << 20) + 24
    say("fingerprint", n, "bytes")
    t = _rand_bytes(n, 5, dev)
    assert dg.digest_value(dg.det_fingerprint(t)) == oracle.fingerprint(_host(t))


@pytest.mark.parametrize("rows,cols,wide", [(1, 5, 5), (37, 13, 13), (64, 4096, 4096),
                                            (100, 300, 320), (9, 1000, 1003)])
def test_row_digests_match_oracle(dev, rows, cols, wide):
    say("row fingerprints", rows, cols, "ld", wide)
    base = Wk.randn_bf16((rows, wide), 1.0, rows + cols, dev)
    t = base[:, :cols]
    got = dg.det_fingerprint_rows(t).cpu().numpy().view(np.uint64)
    want = oracle.fingerprint_rows(Wk.bits(t.contiguous()))
    assert np.array_equal(got, want)
    # equal rows give equal digests wherever they sit (per-row hashing sees
    # a permutation as a permutation of the digests)
    perm = torch.randperm(rows, generator=torch.Generator().manual_seed(1)).to(dev)
    got_p = dg.det_fingerprint_rows(t[perm]).cpu().numpy().view(np.uint64)
    assert np.array_equal(got_p, got[perm.cpu().numpy()])


@pytest.mark.parametrize("n", [0, 1, 16, 17, 4096 + 7, (8 << 20) + 3])
def test_first_mismatch(dev, n):
    say("first mismatch", n)
    a = _rand_bytes(n, 300 + n, dev)
    assert int(dg.det_first_mismatch(a, a.clone()).item()) == -1
    for k in sorted({0, n // 3, n - 1} if n else set()):
        b = a.clone()
        b[k] ^= 0x10
        if k + 5 < n:
            b[k + 5] ^= 1
        got = int(dg.det_first_mismatch(a, b).item())
        assert got == oracle.first_mismatch(_host(a), _host(b)) == k
    if n > 2:  # unaligned views
        b = a.clone()
        b[n - 1] ^= 4
        got = int(dg.det_first_mismatch(a[1:], b[1:]).item())
        assert got == n - 2


def test_trace_finds_the_perturbed_op(dev):
    """Two runs of a chain of det_gemm products; run B flips one bit of one
    intermediate (a stand-in for a nondeterministic kernel).  The localiser
    names that op as the origin and the comparator the flipped byte."""
    say("trace of a det_gemm chain")
    X = Wk.randn_bf16((64, 256), 1.0, 11, dev)
    Ws = [Wk.randn_bf16((256, 256), 0.05, 20 + i, dev) for i in range(4)]

    def run(flip_at):
        t = Trace()
        h = X
        outs = []
        for i, W in enumerate(Ws):
            y = dg.det_gemm_fwd(h, W)
            if i == flip_at:
                y.view(torch.int16)[5, 7] ^= 0x0100
            t.log("det_gemm_fwd", f"layer{i}", [h, W], [y])
            outs.append(y)
            h = y
        return t.events, outs

    ev_a, out_a = run(None)
    ev_b, out_b = run(2)
    d = first_divergence(ev_a, ev_b)
    assert d.kind == "origin" and d.event["scope"] == "layer2"
    assert int(dg.det_first_mismatch(out_a[2], out_b[2]).item()) == (5 * 256 + 7) * 2 + 1
    ev_c, _ = run(None)
    assert first_divergence(ev_a, ev_c).kind == "identical"
