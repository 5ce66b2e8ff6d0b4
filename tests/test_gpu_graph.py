"""Entry points captured in a HIP graph (torch.cuda.CUDAGraph) replay the bits
of an eager call: the graph is replayed three times, with the program's own
eager calls and synchronisations between the replays, and every replay is
compared bitwise with the eager result.  Nothing in these paths records a
memset into the graph (the fingerprint's accumulator is cleared by a kernel),
so the replays must hold.  Covers the decode kernel, the split 32-column
tiles, the wide kernel, RMSNorm, decode attention (work buffer and the
allocation-free entry point), the tensor digest and the MoE grouped GEMM."""
import pytest
import torch

import det_workloads as W
import invariant_deterministic_gemm_det_amd as dg
from gpu_util import device, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = device()
    dg.load_library()
    dg.det_gemm_debug_force_config(-1)
    return d


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32) \
        if t.dtype == torch.float32 else t


def _replays_match(fn, eager_again):
    """fn() -> tuple of output tensors.  Capture fn in a graph, replay it three
    times with eager work between, compare every replay with an eager call."""
    torch.cuda.synchronize()
    ref = [x.clone() for x in fn()]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                      # warm the caching allocator on the side stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn()
    for r in range(3):
        for o in outs:
            o.fill_(0)            # the replay must rewrite every output
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, ref):
            assert torch.equal(_bits(o), _bits(e)), f"replay {r}"
        eager_again()             # the program's own eager work between replays
        torch.cuda.synchronize()


@pytest.mark.parametrize("M,N,K", [(1, 6144, 4096), (128, 6144, 4096), (256, 512, 4096)])
def test_det_gemm_in_a_graph(dev, M, N, K):
    say("det_gemm_fwd in a graph", M, N, K)
    A = W.randn_bf16((M, K), 1.0, 8100 + M, dev)
    B = W.randn_bf16((K, N), 0.02, 8101, dev)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    other = W.randn_bf16((64, K), 1.0, 8102, dev)
    _replays_match(lambda: (dg.det_gemm_fwd(A, B, out=C),),
                   lambda: dg.det_gemm_fwd(other, B))


def test_rmsnorm_in_a_graph(dev):
    say("det_rmsnorm in a graph")
    x = W.randn_bf16((64, 4096), 1.0, 8110, dev)
    w = W.randn_bf16((4096,), 1.0, 8111, dev)
    y = torch.empty_like(x)
    rstd = torch.empty(64, dtype=torch.float32, device=dev)
    _replays_match(lambda: dg.det_rmsnorm(x, w, 1e-6, out=y, rstd=rstd),
                   lambda: dg.det_rmsnorm(x[:7], w))


def test_attention_decode_in_a_graph(dev):
    say("det_attention_decode (work buffer and allocation-free) in a graph")
    B, Hq, Hkv, S, D = 4, 32, 8, 1100, 128
    q = W.randn_bf16((B, Hq, D), 1.0, 8120, dev)
    k = W.randn_bf16((B, Hkv, S, D), 1.0, 8121, dev)
    v = W.randn_bf16((B, Hkv, S, D), 1.0, 8122, dev)
    lens = torch.tensor([1100, 257, 1, 700], dtype=torch.int32, device=dev)
    o1 = torch.empty((B, Hq, D), dtype=torch.bfloat16, device=dev)
    o2 = torch.empty_like(o1)
    work = torch.empty(B * Hq * ((S + 255) // 256) * (D + 2), dtype=torch.float32, device=dev)
    scale = D ** -0.5
    _replays_match(lambda: (dg.det_attention_decode(q, k, v, lens, scale, out=o1, work=work),
                            dg.det_attention_decode_noalloc(q, k, v, lens, scale, o2)),
                   lambda: dg.det_attention_decode(q[:1], k[:1], v[:1], lens[:1], scale))
    assert torch.equal(_bits(o1), _bits(o2))


def test_fingerprint_in_a_graph(dev):
    say("det_fingerprint in a graph")
    t = torch.randint(0, 256, (1 << 20,), dtype=torch.uint8, device=dev,
                      generator=torch.Generator(device=dev).manual_seed(8130))
    out = torch.empty(1, dtype=torch.int64, device=dev)
    _replays_match(lambda: (dg.det_fingerprint(t, out=out),),
                   lambda: dg.det_fingerprint(t[:4096]))


def test_moe_in_a_graph(dev):
    say("det_moe_fwd_dprob in a graph")
    T, E, K, N = 512, 4, 1024, 512
    X = W.randn_bf16((T, K), 1.0, 8140, dev)
    Wt = W.randn_bf16((E, K, N), 0.02, 8141, dev)
    G = W.randn_bf16((T, N), 1e-3, 8142, dev)
    offsets = [0, 200, 201, 390, T]
    Y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    slots = torch.empty(((N + 127) // 128, T), dtype=torch.float32, device=dev)
    dprob = torch.empty(T, dtype=torch.float32, device=dev)
    _replays_match(lambda: dg.det_moe_fwd_dprob(X, Wt, offsets, G, Y=Y, slots=slots, dprob=dprob),
                   lambda: dg.det_moe_fwd_dprob(X[:200], Wt[:1], [0, 200], G[:200]))
