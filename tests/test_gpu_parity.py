"""GPU parity of the HIP library against the CPU oracle, through the C-ABI.

Contract (RL-Kernel operator page "Batch-Invariant Deterministic GEMM
(det_gemm)", sections "Guarantees" and "Ascend NPU backend"):
  * 32-element fp32 leaves in ascending order, rounded once to bf16 (RNE);
    mid-split tree of bf16 adds; reduction capped at 32768;
  * a row's bits never depend on batch size, padding or chunking;
  * a contiguous half-K product is one child of the tree (TP=2 == TP=1);
  * the Ascend bullet on the fixed MAC order inside a leaf: a backend whose
    leaf-internal order differs is not bit-exact to the sequential definition.

Bars (see the tolerance note in tolerance_report):
  * strict kernel vs oracle: bit-exact, every element;
  * MFMA kernel: bit-exact wherever the oracle is exact (integer regime),
    bitwise invariant to batch/padding/chunking/tile configuration, half-K
    exact; its leaves within 1 bf16 ulp of the oracle's and the oracle's tree
    applied to its leaves reproduces its output bit for bit; each output within
    2 bf16 spacings of the largest node of the oracle's tree for that element.
"""
import numpy as np
import pytest
import torch

import det_workloads as W
import oracle
import invariant_deterministic_gemm_det_amd as dg
from gpu_util import (device, say, bits, tolerance_report, ulp_distance, bf16_value,
                      bf16_spacing)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    d = device()
    dg.load_library()  # raises when the library is missing: no fallback exists
    dg.det_gemm_debug_force_config(-1)
    return d


def _sync():
    torch.cuda.synchronize()


def _to(t, dev):
    return t.to(dev)


# ---------------------------------------------------------------- device primitives

def test_device_rounding_all_fp32_patterns(dev):
    say("debug_round: all 2^32 fp32 bit patterns vs torch's bf16 conversion")
    step = 1 << 26
    base = torch.arange(step, dtype=torch.int64, device=dev)
    sub_diff = 0
    for start in range(0, 1 << 32, step):
        u = base + start
        u32 = torch.where(u >= 2 ** 31, u - 2 ** 32, u).to(torch.int32)
        x = u32.view(torch.float32)
        ours = dg.det_gemm_debug_round(x).view(torch.int16)
        ref = x.to(torch.bfloat16).view(torch.int16)
        nan = torch.isnan(x)
        sub = (x != 0) & (x.abs() < 2.0 ** -126)
        bad = (ours != ref) & ~nan
        assert not bool((bad & ~sub).any()), f"normal-range rounding differs near {start:#x}"
        sub_diff += int((bad & sub).sum())
        o = ours.to(torch.int32) & 0xFFFF
        assert bool((((o[nan] & 0x7F80) == 0x7F80) & ((o[nan] & 0x7F) != 0)).all())
    print(f"subnormal fp32 inputs rounded differently: {sub_diff}")


def test_device_add_all_bf16_pairs(dev):
    """Every pair of bf16 values through the kernel's add (v_cvt_pk + v_dot2),
    against the fp32 sum rounded to bf16.  Pairs whose operands or exact sum are
    subnormal are counted, not asserted (subnormals are outside the promise)."""
    say("debug_add: all 2^32 bf16 pairs vs fp32 add + bf16 rounding")
    a_all = torch.arange(65536, dtype=torch.int32, device=dev).to(torch.int16)
    sub_diff = 0
    for b0 in range(0, 65536, 256):
        bb = torch.arange(b0, b0 + 256, dtype=torch.int32, device=dev).to(torch.int16)
        a = a_all.repeat(256).view(torch.bfloat16)
        b = bb.repeat_interleave(65536).view(torch.bfloat16)
        ours = dg.det_gemm_debug_add(a, b).view(torch.int16)
        exact = a.double() + b.double()
        ref = exact.float().to(torch.bfloat16).view(torch.int16)
        nan = torch.isnan(exact)
        tiny = lambda v: (v != 0) & (v.abs() < 2.0 ** -126)
        sub = tiny(a.double()) | tiny(b.double()) | tiny(exact)
        bad = (ours != ref) & ~nan & ~sub
        # v_dot2 returns +0 for (-0) + (-0); no tree node is ever -0 (leaves start
        # from +0 and x + (-x) is +0), so this one pair cannot reach an output.
        both_neg_zero = (a.view(torch.int16) == -32768) & (b.view(torch.int16) == -32768)
        assert not bool((bad & both_neg_zero & (ours != 0)).any())
        bad &= ~both_neg_zero
        if bool(bad.any()):
            idx = torch.nonzero(bad).flatten()[:8]
            pairs = [(hex(int(a.view(torch.int16)[i]) & 0xFFFF), hex(int(b.view(torch.int16)[i]) & 0xFFFF),
                      hex(int(ours[i]) & 0xFFFF), hex(int(ref[i]) & 0xFFFF)) for i in idx]
            raise AssertionError(f"bf16 add differs (a, b, ours, ref): {pairs}")
        sub_diff += int(((ours != ref) & ~nan & sub).sum())
    print(f"pairs involving subnormals added differently: {sub_diff}")
    nz = torch.tensor([-0.0], dtype=torch.bfloat16, device=dev)
    print("(-0) (+) (-0) ->", hex(int(dg.det_gemm_debug_add(nz, nz).view(torch.int16)[0]) & 0xFFFF),
          "(the only normal-range pair that differs)")


@pytest.mark.parametrize("selector", [0, 1])
def test_device_matrix_add_all_bf16_pairs(dev, selector):
    """Every pair of bf16 values through the tree add the matrix-core kernels
    run (det_gemm_debug_matrix_add: one bf16 MFMA against a 0/1 selector per
    block of 256 pairs, rounded by v_cvt_pk; a block with a non-finite sum
    redone element-wise), against the oracle's bf16 add.  Pairs whose sum is
    finite are sent in blocks of their own, so every one of them goes through
    the matrix core; the rest (non-finite operands, overflowing sums) go
    through the element-wise redo, as a tile with a non-finite root does.
    Subnormal operands or sums are counted, not asserted (outside the promise);
    NaN results are compared as NaN; (-0) + (-0) is excluded as in the VALU
    add's test (no tree node is ever -0)."""
    say(f"debug_matrix_add selector {selector}: all 2^32 bf16 pairs vs oracle.add_bf16")
    a_host = np.tile(np.arange(65536, dtype=np.uint16), 256)
    a_dev = torch.from_numpy(a_host.view(np.int16)).to(dev)
    a_bf = a_dev.view(torch.bfloat16)
    a_f = a_bf.float()
    tiny = lambda v: (v != 0) & (v.abs() < 2.0 ** -126)
    sub_a = tiny(a_f)
    sub_diff = 0
    mfma_pairs = 0
    for b0 in range(0, 65536, 256):
        b_host = np.repeat(np.arange(b0, b0 + 256, dtype=np.uint16), 65536)
        b_dev = torch.from_numpy(b_host.view(np.int16)).to(dev)
        b_bf = b_dev.view(torch.bfloat16)
        b_f = b_bf.float()
        fin = torch.isfinite(a_f + b_f)         # partition only; the expectation is the oracle's
        res = torch.empty_like(a_dev)
        for part in (fin, ~fin):
            idx = torch.nonzero(part).flatten()
            if idx.numel():
                res[idx] = dg.det_gemm_debug_matrix_add(a_bf[idx], b_bf[idx], selector).view(torch.int16)
        mfma_pairs += int(fin.sum())
        ref = torch.from_numpy(oracle.add_bf16(a_host, b_host).view(np.int16)).to(dev)
        ri, oi = ref.to(torch.int32) & 0xFFFF, res.to(torch.int32) & 0xFFFF
        ref_nan = ((ri & 0x7F80) == 0x7F80) & ((ri & 0x7F) != 0)
        our_nan = ((oi & 0x7F80) == 0x7F80) & ((oi & 0x7F) != 0)
        exact = a_bf.double() + b_bf.double()
        sub = sub_a | tiny(b_f) | tiny(exact)
        both_neg_zero = (a_dev == -32768) & (b_dev == -32768)
        assert bool((ref_nan == our_nan).all()), f"NaN-ness differs near b0={b0:#x}"
        bad = (res != ref) & ~ref_nan & ~sub & ~both_neg_zero
        if bool(bad.any()):
            idx = torch.nonzero(bad).flatten()[:8]
            pairs = [(hex(int(a_dev[i]) & 0xFFFF), hex(int(b_dev[i]) & 0xFFFF),
                      hex(int(res[i]) & 0xFFFF), hex(int(ref[i]) & 0xFFFF)) for i in idx]
            raise AssertionError(f"matrix-core add differs from the oracle (a, b, ours, oracle): {pairs}")
        sub_diff += int(((res != ref) & ~ref_nan & sub).sum())
    print(f"pairs through the matrix core: {mfma_pairs}; pairs involving subnormals added "
          f"differently: {sub_diff}")


# ---------------------------------------------------------------- helpers

def _inputs(M, N, K, seed, sigma=1.0):
    A = W.randn_bf16((M, K), 1.0, seed)
    B = W.randn_bf16((K, N), sigma, seed + 1)
    dC = W.randn_bf16((M, N), 1.0, seed + 2)
    return A, B, dC


def _six_gpu(A, B, dC, strict):
    Bt = B.t().contiguous()
    return {
        "fwd": dg.det_gemm_fwd(A, B, strict=strict),
        "fwd_rhs_transposed": dg.det_gemm_fwd_rhs_transposed(A, Bt, strict=strict),
        "fwd_fp32": dg.det_gemm_fwd_fp32(A, B, strict=strict),
        "da": dg.det_gemm_da(dC, B, strict=strict),
        "db": dg.det_gemm_db(A, dC, strict=strict),
        "db_transposed": dg.det_gemm_db_transposed(A, dC, strict=strict),
    }


def _six_oracle(A, B, dC):
    a, b, d = bits(A), bits(B), bits(dC)
    return {
        "fwd": oracle.fwd(a, b),
        "fwd_rhs_transposed": oracle.fwd_rhs_transposed(a, np.ascontiguousarray(b.T)),
        "fwd_fp32": oracle.fwd_fp32(a, b),
        "da": oracle.da(d, b),
        "db": oracle.db(a, d),
        "db_transposed": oracle.db_transposed(a, d),
    }


def _as_bits(t):
    if t.dtype == torch.float32:
        return (t.detach().cpu().numpy().view(np.uint32) >> 16).astype(np.uint16)
    return bits(t)


def _oracle_bits(o):
    if o.dtype == np.float32:
        return (o.view(np.uint32) >> 16).astype(np.uint16)
    return o


SMALL_SHAPES = [(1, 128, 256), (7, 128, 256), (64, 128, 256), (37, 53, 1), (37, 53, 31),
                (37, 53, 33), (19, 70, 95), (33, 17, 160), (45, 29, 1000), (130, 66, 384)]


# ---------------------------------------------------------------- strict kernel

@pytest.mark.parametrize("M,N,K", SMALL_SHAPES)
def test_strict_bit_exact_all_ops(dev, M, N, K):
    say("strict vs oracle, six ops", M, N, K)
    A, B, dC = _inputs(M, N, K, 100 + M + N + K)
    got = _six_gpu(A.to(dev), B.to(dev), dC.to(dev), strict=True)
    want = _six_oracle(A, B, dC)
    _sync()
    for op in got:
        if got[op].dtype == torch.float32:
            g = got[op].cpu().numpy().view(np.uint32)
            assert np.array_equal(g, want[op].view(np.uint32)), op
        else:
            assert np.array_equal(bits(got[op]), want[op]), op


def test_strict_padded_and_unaligned_operands(dev):
    say("strict vs oracle with padded / unaligned leading dimensions")
    M, N, K = 21, 35, 200
    A_wide = W.randn_bf16((M, K + 5), 1.0, 501)   # lda = K + 5: not 16-byte aligned
    B_wide = W.randn_bf16((K, N + 8), 1.0, 502)   # ldb = N + 8
    A, B = A_wide[:, :K], B_wide[:, :N]
    got = dg.det_gemm_fwd(A_wide.to(dev)[:, :K], B_wide.to(dev)[:, :N], strict=True)
    _sync()
    assert np.array_equal(bits(got), oracle.fwd(bits(A.contiguous()), bits(B.contiguous())))


# ---------------------------------------------------------------- MFMA kernel

INT_SHAPES = [(200, 150, 256), (130, 70, 96), (16, 300, 64), (5, 129, 200), (300, 17, 33),
              (64, 64, 7)]


@pytest.mark.parametrize("M,N,K", INT_SHAPES)
def test_mfma_integer_regime_bit_exact_all_ops(dev, M, N, K):
    """Entries in {-1,0,1}, R <= 256: every leaf and node is a small exact integer,
    whatever the order inside a leaf, so all six ops equal the oracle bit for bit."""
    say("mfma integer regime, six ops", M, N, K)
    A = W.int_bf16((M, K), 10 + K)
    B = W.int_bf16((K, N), 20 + K)
    dC = W.int_bf16((M, N), 30 + K)
    got = _six_gpu(A.to(dev), B.to(dev), dC.to(dev), strict=False)
    want = _six_oracle(A, B, dC)
    _sync()
    for op in got:
        assert np.array_equal(_as_bits(got[op]), _oracle_bits(want[op])), op


def test_mfma_unaligned_operands_integer_regime(dev):
    say("mfma with non-16-byte-aligned leading dimensions")
    M, N, K = 70, 90, 120
    A_wide = W.int_bf16((M, K + 3), 601)      # lda = 123
    B_wide = W.int_bf16((K, N + 5), 602)      # ldb = 95
    dC_wide = W.int_bf16((M, N + 5), 603)     # lddc = 95
    A, B, dC = A_wide[:, :K], B_wide[:, :N], dC_wide[:, :N]
    Ad, Bd, dCd = A_wide.to(dev)[:, :K], B_wide.to(dev)[:, :N], dC_wide.to(dev)[:, :N]
    got = dg.det_gemm_fwd(Ad, Bd)
    got_db = dg.det_gemm_db(Ad, dCd)
    got_da = dg.det_gemm_da(dCd, B_wide.to(dev)[:, :N])
    _sync()
    a, b, d = bits(A.contiguous()), bits(B.contiguous()), bits(dC.contiguous())
    assert np.array_equal(bits(got), oracle.fwd(a, b))
    assert np.array_equal(bits(got_db), oracle.db(a, d))
    assert np.array_equal(bits(got_da), oracle.da(d, b))


TREE_K = [32, 64, 96, 128, 160, 256, 416, 512, 768, 1000, 1024, 1536, 2048, 3200, 4096,
          12288, 32000, 32768]


@pytest.mark.parametrize("K", TREE_K)
def test_mfma_leaves_and_tree_structure(dev, K):
    """Leaves within 1 bf16 ulp of the oracle's; the oracle's tree applied to the
    kernel's own leaves reproduces the kernel's output bit for bit.  K spans
    every tree evaluator: static blocks of 8 and 32 leaves, blocks of 3*16, and
    the LDS stack for other leaf counts (1..5, 13, 100, 1000 leaves)."""
    M, N = (24, 40) if K > 4096 else (40, 72)
    say("mfma leaves + tree", M, N, K)
    A = W.randn_bf16((M, K), 1.0, 40 + K)
    B = W.randn_bf16((K, N), 0.02, 50 + K)
    Ad, Bd = A.to(dev), B.to(dev)
    leaves = dg.det_gemm_debug_leaves(Ad, Bd)
    out = dg.det_gemm_fwd(Ad, Bd)
    _sync()
    c, lv, big = oracle.fwd_detail(bits(A), bits(B))
    lg = bits(leaves)
    assert lg.shape == lv.shape
    # |leaf_gpu - leaf_oracle| <= spacing(max |leaf|) + 64 * 2^-24 * sum_r |x_r y_r|:
    # each side is the exact leaf sum plus at most 31 (sequential) or 32 (any
    # order) fp32 roundings of partial sums, then one bf16 rounding.
    Lk = (K + 31) // 32
    x = np.zeros((M, Lk * 32)); x[:, :K] = bf16_value(bits(A))
    y = np.zeros((Lk * 32, N)); y[:K] = bf16_value(bits(B))
    x, y = x.reshape(M, Lk, 32), y.reshape(Lk, 32, N)
    mag = np.einsum("mlk,lkn->mnl", np.abs(x), np.abs(y))
    lgv, lvv = bf16_value(lg), bf16_value(lv)
    lim = bf16_spacing(np.maximum(np.abs(lgv), np.abs(lvv))) + 64 * 2.0 ** -24 * mag
    d = ulp_distance(lg, lv)
    worst = np.unravel_index(np.argmax(d), d.shape)
    print("leaf ulp distances: max", int(d.max()), "count>1", int((d > 1).sum()),
          "worst leaf", lgv[worst], lvv[worst], "sum|p|", mag[worst])
    assert (np.abs(lgv - lvv) <= lim).all()
    roots, _ = oracle.tree_from_leaves(lg)
    assert np.array_equal(roots, bits(out))
    hist, beyond, ratio = tolerance_report(bits(out), c, big)
    print("ulp histogram vs oracle", hist, "beyond 2 spacings of largest node:", beyond)
    assert beyond == 0


def test_mfma_zero_products_give_positive_zero(dev):
    """A leaf whose products are all -0 is +0 in the definition (the fp32 sum
    starts at +0); check the MFMA leaf and the output agree."""
    say("mfma signed-zero leaves")
    A = torch.zeros((16, 64), dtype=torch.bfloat16)
    A[1] = -0.0
    B = -torch.ones((64, 16), dtype=torch.bfloat16)
    lv = bits(dg.det_gemm_debug_leaves(A.to(dev), B.to(dev)))
    out = bits(dg.det_gemm_fwd(A.to(dev), B.to(dev)))
    assert (lv == 0).all() and (out == 0).all()


def test_mfma_tolerance_random(dev):
    say("mfma vs oracle tolerance, K=4096")
    M, N, K = 64, 256, 4096
    A = W.randn_bf16((M, K), 1.0, 61)
    B = W.randn_bf16((K, N), 0.02, 62)
    out = dg.det_gemm_fwd(A.to(dev), B.to(dev))
    _sync()
    c, _, big = oracle.fwd_detail(bits(A), bits(B))
    hist, beyond, ratio = tolerance_report(bits(out), c, big)
    print("ulp histogram", hist, "beyond", beyond, "worst ratio", ratio)
    assert beyond == 0


def test_mfma_small_forward_batch_and_padding(dev):
    say("mfma rows invariant to M and padding (A[64,256], B[256,128])")
    A, B = W.small_forward()
    Ad, Bd = A.to(dev), B.to(dev)
    full = bits(dg.det_gemm_fwd(Ad, Bd))
    for M in (1, 7, 64):
        assert np.array_equal(bits(dg.det_gemm_fwd(Ad[:M], Bd)), full[:M]), M
    padded = torch.cat([Ad[:7], torch.zeros((16, 256), dtype=torch.bfloat16, device=dev)])
    assert np.array_equal(bits(dg.det_gemm_fwd(padded, Bd))[:7], full[:7])
    wide = torch.zeros((64, 264), dtype=torch.bfloat16, device=dev)
    wide[:, :256] = Ad
    assert np.array_equal(bits(dg.det_gemm_fwd(wide[:, :256], Bd)), full)
    # every row's position inside a 16-row block: rotate rows
    rot = torch.roll(Ad, shifts=5, dims=0)
    assert np.array_equal(bits(dg.det_gemm_fwd(rot, Bd)), np.roll(full, 5, axis=0))
    # strict kernel: bit-exact to the oracle on the same inputs
    assert np.array_equal(bits(dg.det_gemm_fwd(Ad, Bd, strict=True)), oracle.fwd(bits(A), bits(B)))


@pytest.mark.parametrize("K", [256, 4096, 160, 12288])
def test_mfma_tile_configs_identical(dev, K):
    say("mfma: every tile configuration gives the same bits", K)
    M, N = 80, 200
    A = W.randn_bf16((M, K), 1.0, 70 + K).to(dev)
    B = W.randn_bf16((K, N), 0.02, 71 + K).to(dev)
    n = dg.det_gemm_debug_force_config(-1)
    ref = bits(dg.det_gemm_fwd(A, B))
    try:
        for cfg in range(n):
            dg.det_gemm_debug_force_config(cfg)
            try:
                got = bits(dg.det_gemm_fwd(A, B))
            except dg.DetGemmError as e:   # configuration without room for this tree depth
                assert e.code == dg.EINVAL
                continue
            assert np.array_equal(got, ref), cfg
            assert np.array_equal(bits(dg.det_gemm_fwd(A, B)), ref), "repeat run"
    finally:
        dg.det_gemm_debug_force_config(-1)


# Tile configurations 3 and 4 are the direct-to-LDS kernels (whole 64-index
# stages, 16-byte aligned rows, 8-row chunks of operands whose row index is
# contiguous), 5 to 9 and 13 to 16 the wide kernels (the same, and leaf counts
# 2^a or 3 * 2^a; 13 to 16 are the 32- and 64-column tiles that split the tree
# over two or four wave groups, X K-major only); 2 is the general kernel they must
# reproduce bit for bit.
FAST_SHAPES = [(200, 192, 256), (256, 136, 768), (320, 256, 4096), (128, 64, 12288),
               (72, 64, 32768), (512, 512, 1024), (264, 392, 8192), (768, 384, 1536),
               (384, 768, 6144)]
GENERAL_CFG, FAST_CFGS = 2, (3, 4, 5, 6, 7, 8, 9, 13, 14, 15, 16, 17) + tuple(range(18, 30))


def _six_forced(cfg, A, B, dC):
    """The six ops with the tile configuration pinned; None where the pinned
    kernel does not take the problem (EINVAL)."""
    dg.det_gemm_debug_force_config(cfg)
    out = {}
    try:
        Bt = B.t().contiguous()
        calls = {
            "fwd": lambda: dg.det_gemm_fwd(A, B),
            "fwd_rhs_transposed": lambda: dg.det_gemm_fwd_rhs_transposed(A, Bt),
            "fwd_fp32": lambda: dg.det_gemm_fwd_fp32(A, B),
            "da": lambda: dg.det_gemm_da(dC, B),
            "db": lambda: dg.det_gemm_db(A, dC),
            "db_transposed": lambda: dg.det_gemm_db_transposed(A, dC),
        }
        for op, f in calls.items():
            try:
                out[op] = _as_bits(f())
            except dg.DetGemmError as e:
                assert e.code == dg.EINVAL, (op, e.code)
                out[op] = None
    finally:
        dg.det_gemm_debug_force_config(-1)
    return out


@pytest.mark.parametrize("M,N,K", FAST_SHAPES)
def test_fast_path_matches_general_kernel(dev, M, N, K):
    say("direct-to-LDS kernels vs general kernel, six ops", M, N, K)
    A, B, dC = _inputs(M, N, K, 900 + K, sigma=0.02)
    Ad, Bd, dCd = A.to(dev), B.to(dev), dC.to(dev)
    ref = _six_forced(GENERAL_CFG, Ad, Bd, dCd)
    assert all(v is not None for v in ref.values())
    ran = 0
    for cfg in FAST_CFGS:
        got = _six_forced(cfg, Ad, Bd, dCd)
        for op, g in got.items():
            if g is None:
                continue
            ran += 1
            assert np.array_equal(g, ref[op]), (cfg, op)
    print("fast-path (config, op) runs compared:", ran)
    assert ran >= 3


@pytest.mark.parametrize("M,N,K", [(200, 192, 256), (256, 136, 256), (256, 256, 256), (512, 256, 1024),
                                   (768, 192, 1536)])
def test_fast_path_integer_regime_bit_exact(dev, M, N, K):
    say("direct-to-LDS kernels, integer regime vs oracle", M, N, K)
    A = W.int_bf16((M, K), 910 + K)
    B = W.int_bf16((K, N), 920 + K)
    dC = W.int_bf16((M, N), 930 + K)
    want = _six_oracle(A, B, dC)
    ran = 0
    for cfg in FAST_CFGS:
        got = _six_forced(cfg, A.to(dev), B.to(dev), dC.to(dev))
        for op, g in got.items():
            if g is not None:
                ran += 1
                assert np.array_equal(g, _oracle_bits(want[op])), (cfg, op)
    assert ran >= 4


@pytest.mark.parametrize("K", [4096, 12288, 32768, 192])
def test_mfma_half_k_identity(dev, K):
    say("mfma half-K identity", K)
    M, N = 48, 96
    A = W.randn_bf16((M, K), 1.0, 80 + K).to(dev)
    B = W.randn_bf16((K, N), 0.02, 81 + K).to(dev)
    h = K // 2
    full = dg.det_gemm_fwd(A, B)
    lo = dg.det_gemm_fwd(A[:, :h], B[:h])
    hi = dg.det_gemm_fwd(A[:, h:], B[h:])
    assert torch.equal(full.view(torch.int16), dg.det_gemm_debug_add(lo, hi).view(torch.int16))
    f32 = dg.det_gemm_fwd_fp32(A, B)
    assert torch.equal(f32, full.float())


@pytest.mark.parametrize("K", [160, 4096])
def test_mfma_layout_identities(dev, K):
    say("mfma layout identities", K)
    M, N = 96, 80
    A, B, dC = [t.to(dev) for t in _inputs(M, N, K, 90 + K)]
    C = dg.det_gemm_fwd(A, B)
    eq = lambda x, y: torch.equal(x.view(torch.int16), y.view(torch.int16))
    assert eq(dg.det_gemm_fwd_rhs_transposed(A, B.t().contiguous()), C)
    assert torch.equal(dg.det_gemm_fwd_fp32(A, B), C.float())
    Bn = W.randn_bf16((K, N), 1.0, 95 + K).to(dev)   # da: B is [K,N], reduction over N
    assert eq(dg.det_gemm_da(dC, Bn), dg.det_gemm_fwd_rhs_transposed(dC, Bn))
    Am = W.randn_bf16((N, K), 1.0, 96 + K).to(dev)   # db with M = N rows
    dCm = W.randn_bf16((N, M), 1.0, 97 + K).to(dev)
    db = dg.det_gemm_db(Am, dCm)
    assert eq(db, dg.det_gemm_fwd(Am.t().contiguous(), dCm))
    assert eq(dg.det_gemm_db_transposed(Am, dCm), db.t().contiguous())


def test_errors_leave_output_untouched(dev):
    say("argument errors and empty shapes")
    A = torch.ones((4, 32769), dtype=torch.bfloat16, device=dev)
    B = torch.ones((32769, 8), dtype=torch.bfloat16, device=dev)
    C = torch.full((4, 8), 7.0, dtype=torch.bfloat16, device=dev)
    with pytest.raises(dg.DetGemmError) as e:
        dg.det_gemm_fwd(A, B, out=C)
    assert e.value.code == dg.EKCAP
    _sync()
    assert bool((C == 7.0).all())
    empty = dg.det_gemm_fwd(torch.ones((0, 16), dtype=torch.bfloat16, device=dev),
                            torch.ones((16, 8), dtype=torch.bfloat16, device=dev))
    assert empty.shape == (0, 8)
    # the cap itself is accepted
    A = W.int_bf16((2, 32768), 3).to(dev)
    B = W.int_bf16((32768, 3), 4).to(dev)
    got = dg.det_gemm_fwd(A, B)
    leaves = dg.det_gemm_debug_leaves(A, B)
    _sync()
    roots, _ = oracle.tree_from_leaves(bits(leaves))
    assert np.array_equal(roots, bits(got))


# Leaf counts L = m * 2^a for m = 5, 7, 11, 17, 19, 25, 27, 35, 37, 43: the
# mid-split tree is the perfect tree over units of m leaves, which the wide
# kernel evaluates in configurations 18 to 29 (m stages per pair of units; from
# m = 11 on, each unit's tree walked with a stack of static register slots).  Each
# reduction (K for the forward family, N for da, M for db) with such a leaf
# count, ragged tiles included, against the general kernel, bit for bit.
@pytest.mark.parametrize("M,N,K", [
    (256, 384, 5120),     # L = 160 over K
    (200, 136, 7168),     # L = 224 over K, ragged rows and columns
    (384, 256, 14336),    # L = 448
    (256, 256, 20480),    # L = 640: upper levels parked in LDS
    (128, 256, 28672),    # L = 896: two stage buffers (configuration 20)
    (256, 7168, 320),     # da: L = 224 over N
    (5120, 256, 384),     # db: L = 160 over M
    (256, 10240, 320),    # da: L = 320 over N
    (256, 384, 11008),    # L = 344 = 43 * 8: units of 43 leaves (configuration 21)
    (200, 136, 13824),    # L = 432 = 27 * 16: units of 27 leaves (configuration 22)
    (256, 256, 22016),    # L = 688 = 43 * 16: upper levels parked in LDS
    (256, 11008, 320),    # da: L = 344 over N
    (11008, 256, 384),    # db: L = 344 over M
    (128, 256, 27648),    # L = 864 = 27 * 32: two stage buffers (configuration 23)
    (256, 200, 18944),    # L = 592 = 37 * 16: units of 37 leaves (configuration 24)
    (256, 136, 5632),     # L = 176 = 11 * 16 (configuration 25)
    (128, 256, 17408),    # L = 544 = 17 * 32, two stage buffers (26)
    (200, 256, 9728),     # L = 304 = 19 * 16 (27)
    (128, 128, 25600),    # L = 800 = 25 * 32, two stage buffers (28)
    (256, 256, 8960),     # L = 280 = 35 * 8 (29)
])
def test_wide_kernel_five_and_seven_leaf_units(dev, M, N, K):
    say("wide kernel, units of five and seven leaves vs general kernel", M, N, K)
    A, B, dC = [t.to(dev) for t in _inputs(M, N, K, 970 + K + M, sigma=0.02)]
    ref = _six_forced(GENERAL_CFG, A, B, dC)
    ran = 0
    for cfg in range(18, 30):
        got = _six_forced(cfg, A, B, dC)
        for op, g in got.items():
            if g is None:
                continue
            ran += 1
            assert np.array_equal(g, ref[op]), (cfg, op)
    assert ran >= 1
    # the library picks these configurations by itself
    auto = _six_forced(-1, A, B, dC)
    for op in auto:
        assert np.array_equal(auto[op], ref[op]), op


# The wide kernels' tree adds run on the matrix core, where one non-finite node
# spoils the other sums of its row; such tiles are recomputed with element-wise
# adds.  Inf and NaN inputs must give the general kernel's bits.
@pytest.mark.parametrize("K", [1024, 1536, 5120, 7168, 11008, 13824, 18944, 5632, 8960])
def test_wide_kernel_nonfinite_inputs(dev, K):
    say("wide kernels, non-finite inputs vs general kernel", K)
    M, N = 1024, 768
    A, B, dC = _inputs(M, N, K, 950 + K, sigma=0.02)
    A[3, 100] = float("inf")
    A[130, 7] = float("nan")
    B[K - 12, 77] = float("-inf")
    dC[517, 5] = float("inf")
    Ad, Bd, dCd = A.to(dev), B.to(dev), dC.to(dev)
    ref = _six_forced(GENERAL_CFG, Ad, Bd, dCd)
    ran = 0
    for cfg in (5, 6, 7, 8, 9, 13, 14, 15, 16, 17) + tuple(range(18, 30)):
        got = _six_forced(cfg, Ad, Bd, dCd)
        for op, g in got.items():
            if g is None:
                continue
            ran += 1
            assert np.array_equal(g, ref[op]), (cfg, op)
    assert ran >= 6


# The batch-invariance guarantee across the kernels that the automatic choice
# picks for one weight as M grows (decode kernel, split tiles, the wide
# kernel's unit schedules): a row's bits do not depend on how many rows are
# computed with it.
@pytest.mark.parametrize("K", [5120, 7168, 11008, 13824])
def test_rows_invariant_across_batch_sizes_with_unit_schedules(dev, K):
    say("rows across batch sizes, unit schedules", K)
    N = 384
    X = W.randn_bf16((1024, K), 1.0, 990 + K).to(dev)
    Wt = W.randn_bf16((K, N), 0.02, 991 + K).to(dev)
    full = dg.det_gemm_fwd(X, Wt).view(torch.int16)
    full_t = dg.det_gemm_fwd_rhs_transposed(X, Wt.t().contiguous()).view(torch.int16)
    assert torch.equal(full, full_t)
    for m in (1, 16, 40, 100, 300):
        part = dg.det_gemm_fwd(X[:m].contiguous(), Wt).view(torch.int16)
        assert torch.equal(part, full[:m]), m
    off = dg.det_gemm_fwd(X[517:517 + 200].contiguous(), Wt).view(torch.int16)
    assert torch.equal(off, full[517:717])
