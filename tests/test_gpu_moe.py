"""GPU parity of the MoE grouped GEMM with the per-token slot epilogue, through
the C-ABI (include/det_moe.h).

Source: reading notes "Bitwise-Deterministic Pretraining at Scale: How
Megatron Core Finds and Removes Every Flipped Bit", section "Kernel redesign:
the grouped-GEMM epilogue": each N-tile writes a private slot, and the slots
are combined by a fixed tree, so the per-token value has the same bits on
every run.

Checks:
  * Y: bitwise equal to det_gemm_fwd of each expert's rows (the grouped launch
    computes the same leaves and tree), and within the det_gemm MFMA tolerance
    of the oracle; in the integer regime bitwise equal to the oracle;
  * slots and dprob: bitwise equal to the oracle's epilogue applied to the
    device's Y (the epilogue's arithmetic is fixed completely);
  * the fused epilogue of the grouped kernel equals the slot kernel of its own
    (the path taken when the grouped kernel does not apply), bitwise;
  * a row's results do not depend on the other experts' rows.
"""
import numpy as np
import pytest
import torch

import det_workloads as Wk
import oracle
import invariant_deterministic_gemm_det_amd as dg
from gpu_util import device, say, bits, tolerance_report

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = device()
    dg.load_library()
    dg.det_gemm_debug_force_config(-1)
    yield d
    dg.det_gemm_debug_force_config(-1)


def _fbits(t):
    return t.detach().contiguous().view(torch.int32).cpu().numpy()


def _np_fbits(a):
    return np.ascontiguousarray(a, np.float32).view(np.int32)


def _case(sizes, K, N, seed, dev, integer=False):
    E = len(sizes)
    off = [0] + list(np.cumsum(sizes).astype(int))
    T = off[-1]
    if integer:
        X = Wk.int_bf16((T, K), seed, device=dev)
        W = Wk.int_bf16((E, K, N), seed + 1, device=dev)
        G = Wk.int_bf16((T, N), seed + 2, device=dev)
    else:
        X = Wk.randn_bf16((T, K), 1.0, seed, dev)
        W = Wk.randn_bf16((E, K, N), 0.02, seed + 1, dev)
        G = Wk.randn_bf16((T, N), 1e-3, seed + 2, dev)
    return X, W, G, off


def _per_expert_fwd(X, W, off):
    Y = torch.empty((X.shape[0], W.shape[2]), dtype=torch.bfloat16, device=X.device)
    for e in range(W.shape[0]):
        if off[e + 1] > off[e]:
            dg.det_gemm_fwd(X[off[e]:off[e + 1]], W[e], out=Y[off[e]:off[e + 1]])
    return Y


def _check_epilogue(Y, G, slots, dprob):
    s_or, d_or = oracle.moe_dprob(bits(Y), bits(G))
    assert np.array_equal(_fbits(slots), _np_fbits(s_or))
    assert np.array_equal(_fbits(dprob), _np_fbits(d_or))


# (sizes per expert, K, N): grouped wide kernel (K = 2048, L = 64; K = 1536,
# L = 48 three-leaf units), an empty expert, a one-row expert, ragged N, and a
# leaf count the wide kernels do not take (per-expert products + slot kernel).
SHAPES = [
    ([200, 0, 1, 300, 57], 2048, 640, "grouped wide, empty and one-row experts"),
    ([129, 256], 1536, 384, "grouped three-leaf units"),
    ([130, 70, 5], 1024, 328, "ragged N (last slot 72 columns)"),
    ([64, 96], 1000, 256, "per-expert products, slot kernel"),
    ([17], 4096, 128, "one expert, one slot"),
]


@pytest.mark.parametrize("sizes,K,N,what", SHAPES, ids=[s[3] for s in SHAPES])
def test_moe_against_oracle(dev, sizes, K, N, what):
    say("MoE", what, "sizes", sizes, "K", K, "N", N)
    X, W, G, off = _case(sizes, K, N, 7000 + K + N, dev)
    Y, dprob, slots = dg.det_moe_fwd_dprob(X, W, off, G)
    torch.cuda.synchronize()
    # the grouped product has the bits of the per-expert products
    assert torch.equal(Y.view(torch.int16), _per_expert_fwd(X, W, off).view(torch.int16))
    # the epilogue is exact: the oracle's slots and trees on the device's Y
    _check_epilogue(Y, G, slots, dprob)
    # Y within the det_gemm MFMA tolerance of the oracle, expert by expert
    Xb, Wb = bits(X), bits(W)
    for e in range(len(sizes)):
        if off[e + 1] == off[e]:
            continue
        rows = slice(off[e], min(off[e + 1], off[e] + 64))
        c, _, big = oracle.fwd_detail(Xb[rows], Wb[e])
        assert tolerance_report(bits(Y[rows]), c, big)[1] == 0


@pytest.mark.parametrize("sizes,K,N", [([40, 0, 130, 3], 1024, 256), ([128, 128], 192, 300)])
def test_moe_integer_regime_equals_oracle(dev, sizes, K, N):
    """Entries in {-1, 0, 1}: every leaf and node is an exact integer, so the
    device's Y, slots and dprob equal the oracle's bit for bit."""
    say("MoE integer regime", sizes, K, N)
    X, W, G, off = _case(sizes, K, N, 7100 + K, dev, integer=True)
    Y, dprob, slots = dg.det_moe_fwd_dprob(X, W, off, G)
    Yo, So, Do = oracle.moe_fwd_dprob(bits(X), bits(W), off, bits(G))
    assert np.array_equal(bits(Y), Yo)
    assert np.array_equal(_fbits(slots), _np_fbits(So))
    assert np.array_equal(_fbits(dprob), _np_fbits(Do))


def test_no_columns_and_no_rows(dev):
    say("MoE N = 0 and T = 0")
    X, W, G, off = _case([3, 5], 64, 0, 7050, dev)
    Y, dprob, slots = dg.det_moe_fwd_dprob(X, W, off, G)
    assert slots.shape == (0, 8)
    assert torch.equal(dprob.view(torch.int32), torch.zeros(8, dtype=torch.int32, device=dev))
    X, W, G, off = _case([0, 0], 64, 128, 7051, dev)
    Y, dprob, slots = dg.det_moe_fwd_dprob(X, W, off, G)
    assert Y.shape == (0, 128) and dprob.shape == (0,)


def test_fused_epilogue_equals_slot_kernel(dev):
    say("MoE fused slots vs the slot kernel, and forced per-expert products")
    X, W, G, off = _case([300, 150, 0, 90], 2048, 512, 7200, dev)
    Y, dprob, slots = dg.det_moe_fwd_dprob(X, W, off, G)
    sep = dg.det_moe_debug_slots(Y, G)
    assert torch.equal(sep.view(torch.int32), slots.view(torch.int32))
    # per-expert products on the direct-to-LDS kernel, slots from the slot kernel
    dg.det_gemm_debug_force_config(3)
    try:
        Y3, d3, s3 = dg.det_moe_fwd_dprob(X, W, off, G)
    finally:
        dg.det_gemm_debug_force_config(-1)
    assert torch.equal(Y3.view(torch.int16), Y.view(torch.int16))
    assert torch.equal(s3.view(torch.int32), slots.view(torch.int32))
    assert torch.equal(d3.view(torch.int32), dprob.view(torch.int32))
    # G rows not 16-byte aligned: the grouped kernel leaves the slots to the slot kernel
    Gpad = torch.zeros((G.shape[0], G.shape[1] + 1), dtype=G.dtype, device=dev)
    Gpad[:, 1:] = G
    Yu, du, su = dg.det_moe_fwd_dprob(X, W, off, Gpad[:, 1:])
    assert torch.equal(su.view(torch.int32), slots.view(torch.int32))
    assert torch.equal(du.view(torch.int32), dprob.view(torch.int32))


def test_rows_independent_of_other_experts(dev):
    """Expert blocks in another order, with other experts' rows dropped or added:
    every surviving row keeps its Y, slots and dprob bits."""
    say("MoE row invariance to the other experts")
    X, W, G, off = _case([180, 77, 260], 1024, 384, 7300, dev)
    Y, dprob, slots = dg.det_moe_fwd_dprob(X, W, off, G)
    # experts (2, 0) only, in that order; expert 1's rows dropped
    r2, r0 = slice(off[2], off[3]), slice(off[0], off[1])
    X2 = torch.cat([X[r2], X[r0]])
    G2 = torch.cat([G[r2], G[r0]])
    W2 = torch.stack([W[2], W[0]])
    n2 = off[3] - off[2]
    Yb, db, sb = dg.det_moe_fwd_dprob(X2, W2, [0, n2, X2.shape[0]], G2)
    assert torch.equal(Yb[:n2].view(torch.int16), Y[r2].view(torch.int16))
    assert torch.equal(Yb[n2:].view(torch.int16), Y[r0].view(torch.int16))
    assert torch.equal(db[:n2].view(torch.int32), dprob[r2].view(torch.int32))
    assert torch.equal(db[n2:].view(torch.int32), dprob[r0].view(torch.int32))
    assert torch.equal(sb[:, :n2].view(torch.int32), slots[:, r2].view(torch.int32))


def test_nonfinite_rows(dev):
    """A row with inf/NaN inputs takes the element-wise recomputation of its
    tile; the epilogue still matches the oracle on the device's Y."""
    say("MoE non-finite inputs")
    X, W, G, off = _case([140, 120], 2048, 256, 7400, dev)
    X[3, 5] = float("inf")
    X[200, 17] = float("nan")
    G[7, 9] = float("inf")
    Y, dprob, slots = dg.det_moe_fwd_dprob(X, W, off, G)
    assert torch.equal(Y.view(torch.int16), _per_expert_fwd(X, W, off).view(torch.int16))
    s_or, d_or = oracle.moe_dprob(bits(Y), bits(G))
    got = slots.cpu().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(s_or))
    ok = ~np.isnan(s_or)
    assert np.array_equal(_fbits(slots)[ok], _np_fbits(s_or)[ok])
    dg_ = dprob.cpu().numpy()
    assert np.array_equal(np.isnan(dg_), np.isnan(d_or))
    ok = ~np.isnan(d_or)
    assert np.array_equal(_fbits(dprob)[ok], _np_fbits(d_or)[ok])
    assert np.isnan(d_or).any()


def test_moe_full_size_workload(dev):
    """The benchmark's workload: 4096 tokens, top-2 of 8 experts (8192 rows),
    K = 2048, N = 4096.  Two runs agree bitwise; sampled rows against the
    oracle; two experts against det_gemm_fwd (the last one's final row tiles
    run as half-height tail tiles)."""
    inp = Wk.moe_inputs(dev)
    say("MoE full size: rows", inp.offsets[-1], "segments", np.diff(inp.offsets).tolist())
    Y, dprob, slots = dg.det_moe_fwd_dprob(inp.x, inp.w, inp.offsets, inp.g)
    Y2, d2, s2 = dg.det_moe_fwd_dprob(inp.x, inp.w, inp.offsets, inp.g)
    assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16))
    assert torch.equal(dprob.view(torch.int32), d2.view(torch.int32))
    assert torch.equal(slots.view(torch.int32), s2.view(torch.int32))
    # expert 3, and expert 7, whose last row tiles run as half-height tiles
    # (2176 tiles: the 128 past the eighth round of 256 are split)
    for e in (3, 7):
        r = slice(inp.offsets[e], inp.offsets[e + 1])
        assert torch.equal(dg.det_gemm_fwd(inp.x[r], inp.w[e]).view(torch.int16),
                           Y[r].view(torch.int16))
    # sampled rows: Y within tolerance of the oracle, epilogue exact
    off = inp.offsets
    rows = [0, off[1] - 1, off[4] + 5, off[-1] - 1]
    for row in rows:
        ex = int(np.searchsorted(off, row, side="right") - 1)
        c, _, big = oracle.fwd_detail(bits(inp.x[row:row + 1]), bits(inp.w[ex]))
        assert tolerance_report(bits(Y[row:row + 1]), c, big)[1] == 0
    s_or, d_or = oracle.moe_dprob(bits(Y[rows]), bits(inp.g[rows]))
    assert np.array_equal(_fbits(dprob[rows]), _np_fbits(d_or))
    assert np.array_equal(_fbits(slots[:, rows]), _np_fbits(s_or))
    # the whole epilogue on the device's Y
    _check_epilogue(Y, inp.g, slots, dprob)


def test_tail_tiles_split_in_half(dev):
    """11 row tiles x 32 column tiles = 352 tiles on 256 compute units: the 96
    past the last full round run as half-height tiles whose tree is split over
    two wave groups (an expert of 60 rows: its lower half holds no rows; one of
    100: a ragged half).  Y equals det_gemm_fwd per expert bitwise, the
    epilogue equals the oracle's on the device's Y, and both equal the
    per-expert products with the slot kernel; a non-finite input inside a half
    tile takes the element-wise recomputation."""
    say("MoE tail tiles split in half")
    X, W, G, off = _case([300, 200, 500, 100, 60], 2048, 4096, 7500, dev)
    Y, dprob, slots = dg.det_moe_fwd_dprob(X, W, off, G)
    assert torch.equal(Y.view(torch.int16), _per_expert_fwd(X, W, off).view(torch.int16))
    _check_epilogue(Y, G, slots, dprob)
    dg.det_gemm_debug_force_config(3)
    try:
        Y3, d3, s3 = dg.det_moe_fwd_dprob(X, W, off, G)
    finally:
        dg.det_gemm_debug_force_config(-1)
    assert torch.equal(Y3.view(torch.int16), Y.view(torch.int16))
    assert torch.equal(s3.view(torch.int32), slots.view(torch.int32))
    assert torch.equal(d3.view(torch.int32), dprob.view(torch.int32))
    # a non-finite input in the lower half of expert 3's only row tile
    X[off[3] + 70, 11] = float("inf")
    Yn, dn, sn = dg.det_moe_fwd_dprob(X, W, off, G)
    assert torch.equal(Yn.view(torch.int16), _per_expert_fwd(X, W, off).view(torch.int16))
    s_or, d_or = oracle.moe_dprob(bits(Yn), bits(G))
    got = sn.cpu().numpy()
    assert np.array_equal(np.isnan(got), np.isnan(s_or))
    ok = ~np.isnan(s_or)
    assert np.array_equal(_fbits(sn)[ok], _np_fbits(s_or)[ok])
    assert np.isnan(s_or).any()
