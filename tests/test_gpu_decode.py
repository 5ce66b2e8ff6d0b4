"""GPU parity of the decode kernel (tile configurations 10 to 12: at most 128,
16 or 64 rows of X on 16-, 64- or 32-column tiles, the reduction split over the
8 or 16 subtrees of the mid-split tree at depth 3 or 4, tree adds on the matrix
core with an element-wise recomputation of tiles whose root is not finite),
through the C-ABI.

Contract (RL-Kernel operator page "Batch-Invariant Deterministic GEMM
(det_gemm)", sections "Guarantees" and "Ascend NPU backend"): the same leaves
and the same tree as every other configuration, so the bits must equal those
of the general kernel (configuration 1, itself checked against the oracle in
test_gpu_parity.py) on every shape, equal the oracle exactly wherever the
oracle is exact, and a row's bits must not depend on how many rows share the
call.
"""
import numpy as np
import pytest
import torch

import det_workloads as W
import oracle
import invariant_deterministic_gemm_det_amd as dg
from gpu_util import device, say, bits

pytestmark = pytest.mark.gpu

DECODE_CFGS, GENERAL_CFG = (10, 11, 12), 1


@pytest.fixture(scope="module")
def dev():
    d = device()
    dg.load_library()
    dg.det_gemm_debug_force_config(-1)
    return d


def _forced(cfg, f):
    dg.det_gemm_debug_force_config(cfg)
    try:
        return f()
    finally:
        dg.det_gemm_debug_force_config(-1)


def _ops(A, B, dC):
    """The four products whose X operand has the row count M."""
    Bt = B.t().contiguous()
    return {
        "fwd": lambda: dg.det_gemm_fwd(A, B),
        "fwd_rhs_transposed": lambda: dg.det_gemm_fwd_rhs_transposed(A, Bt),
        "fwd_fp32": lambda: dg.det_gemm_fwd_fp32(A, B),
        "da": lambda: dg.det_gemm_da(dC, B),   # X = dC [M, N], reduction over N
    }


def _as_bits(t):
    if t.dtype == torch.float32:
        return t.cpu().numpy().view(np.uint32)
    return bits(t)


# M, N, K: leaf counts 8 (one leaf per wave), 9, 128, 129, 130, 1000 and 1024
# (the deepest per-wave trees); N ragged against the 16-column blocks.  A
# K-major Y with an even leaf count is copied two leaves at a time (waves whose
# range starts or ends inside such a unit: L = 130); odd counts one at a time.
SHAPES = [(1, 6144, 4096), (16, 6144, 4096), (5, 200, 4096), (3, 136, 288), (1, 64, 256),
          (2, 48, 32768), (16, 40, 4160), (7, 24, 32000), (1, 8, 1024), (2, 64, 4128),
          (1, 72, 4128)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_decode_matches_general_kernel(dev, M, N, K):
    say("decode kernel vs general kernel", M, N, K)
    A = W.randn_bf16((M, K), 1.0, 1000 + M + K).to(dev)
    B = W.randn_bf16((K, N), 0.02, 1001 + N + K).to(dev)
    dC = W.randn_bf16((M, N), 1.0, 1002 + N).to(dev)
    ops = _ops(A, B, dC)
    ran = 0
    for op, f in ops.items():
        ref = _as_bits(_forced(GENERAL_CFG, f))
        auto = _as_bits(f())
        assert np.array_equal(auto, ref), op
        da_fits = op != "da" or (N % 32 == 0 and N // 32 >= 8)
        for cfg in DECODE_CFGS:
            if not da_fits:
                with pytest.raises(dg.DetGemmError):
                    _forced(cfg, f)
                continue
            got = _as_bits(_forced(cfg, f))
            assert np.array_equal(got, ref), (op, cfg)
            assert np.array_equal(_as_bits(_forced(cfg, f)), ref), (op, cfg, "repeat")
            ran += 1
    assert ran >= 6


@pytest.mark.parametrize("M,N,K", [(3, 200, 4096), (1, 64, 256), (16, 48, 1024), (1, 24, 8192)])
def test_decode_integer_regime_bit_exact(dev, M, N, K):
    """Inputs in {-1, 0, 1}: every leaf and tree add is exact, so the kernel
    must reproduce the oracle bit for bit."""
    say("decode kernel, integer regime vs oracle", M, N, K)
    A = W.int_bf16((M, K), 1100 + K)
    B = W.int_bf16((K, N), 1101 + N)
    want = oracle.fwd(bits(A), bits(B))
    Bt = B.t().contiguous()
    for cfg in DECODE_CFGS:
        got = _forced(cfg, lambda: dg.det_gemm_fwd(A.to(dev), B.to(dev)))
        assert np.array_equal(bits(got), want), cfg
        got_t = _forced(cfg, lambda: dg.det_gemm_fwd_rhs_transposed(A.to(dev), Bt.to(dev)))
        assert np.array_equal(bits(got_t), want), cfg


def test_decode_rows_invariant_to_batch(dev):
    """QKV projection (K = 4096, N = 6144): each row of a 16-row call (decode
    kernel, 16 staged rows), the same row alone (decode kernel, one staged
    row) and the same row inside a 256-row batch (wide kernel) agree bit for
    bit."""
    say("decode rows vs single-row and 256-row calls")
    K, N = 4096, 6144
    B = W.randn_bf16((K, N), 0.02, 1200).to(dev)
    big = W.randn_bf16((256, K), 1.0, 1201).to(dev)
    X16 = big[100:116].contiguous()
    c16 = bits(dg.det_gemm_fwd(X16, B))
    c256 = bits(dg.det_gemm_fwd(big, B))
    assert np.array_equal(c16, c256[100:116])
    for i in (0, 7, 15):
        c1 = bits(dg.det_gemm_fwd(X16[i:i + 1].contiguous(), B))
        assert np.array_equal(c1[0], c16[i]), i
    for m in (2, 9):
        cm = bits(dg.det_gemm_fwd(X16[:m].contiguous(), B))
        assert np.array_equal(cm, c16[:m]), m
    for m in (17, 24, 32, 40, 64, 65, 100, 128):   # two, four or eight staged row blocks
        cm = bits(dg.det_gemm_fwd(big[100:100 + m].contiguous(), B))
        assert np.array_equal(cm, c256[100:100 + m]), m


def test_decode_lm_head_row(dev):
    """LM head (K = 4096, N = 151936), one and 16 rows: both decode tile
    widths against the general kernel over the whole vocabulary."""
    say("decode kernel, LM head rows")
    A = W.randn_bf16((16, 4096), 1.0, 1300).to(dev)
    B = W.randn_bf16((4096, 151936), 0.02, 1301, device=dev)
    for m in (1, 16):
        ref = bits(_forced(GENERAL_CFG, lambda: dg.det_gemm_fwd(A[:m], B)))
        assert np.array_equal(bits(dg.det_gemm_fwd(A[:m], B)), ref), m
        for cfg in DECODE_CFGS:
            assert np.array_equal(bits(_forced(cfg, lambda: dg.det_gemm_fwd(A[:m], B))), ref), (m, cfg)


def test_lm_head_transposed_weight_rows_across_kernels(dev):
    """LM head in the nn.Linear layout (W [N][K], 1.2 GB: the decode kernel's
    weight copies are non-temporal): 1, 16, 17 and 32 rows run on the decode
    kernel, 33 and 256 rows on the wide kernel; every row equals the same row
    of the 256-row call, and the 32-row call equals the general kernel."""
    say("LM head W [N][K] rows across the decode and wide kernels")
    A = W.randn_bf16((256, 4096), 1.0, 1310).to(dev)
    Bt = W.randn_bf16((151936, 4096), 0.02, 1311, device=dev)
    full = bits(dg.det_gemm_fwd_rhs_transposed(A, Bt))
    for m in (1, 16, 17, 32, 33):
        assert np.array_equal(bits(dg.det_gemm_fwd_rhs_transposed(A[:m], Bt)), full[:m]), m
    ref = bits(_forced(GENERAL_CFG, lambda: dg.det_gemm_fwd_rhs_transposed(A[:32], Bt)))
    assert np.array_equal(full[:32], ref)


@pytest.mark.parametrize("case", ["rows129", "leaves7", "ragged_k", "unaligned", "n_not_8"])
def test_decode_rejects_unsupported(dev, case):
    """Forcing configuration 10, 11 or 12 on a problem it does not take is EINVAL;
    the automatic choice runs another kernel with the same bits."""
    say("decode kernel rejects", case)
    M, N, K = {"rows129": (129, 64, 1024), "leaves7": (4, 64, 224), "ragged_k": (4, 64, 1040 + 8),
               "unaligned": (4, 64, 1024), "n_not_8": (4, 13, 1024)}[case]
    A = W.randn_bf16((M, K + 8), 1.0, 1400).to(dev)
    A = A[:, 1:K + 1] if case == "unaligned" else A[:, :K].contiguous()
    B = W.randn_bf16((K, N), 0.02, 1401).to(dev)
    for cfg in DECODE_CFGS:
        with pytest.raises(dg.DetGemmError) as e:
            _forced(cfg, lambda: dg.det_gemm_fwd(A, B))
        assert e.value.code == dg.EINVAL
    auto = bits(dg.det_gemm_fwd(A, B))
    ref = bits(_forced(GENERAL_CFG, lambda: dg.det_gemm_fwd(A, B)))
    assert np.array_equal(auto, ref)


def test_decode_zero_products_give_positive_zero(dev):
    """Leaves whose products are all -0 (or +0) are +0 in the definition (the
    fp32 sum starts at +0), and so is every node above them: the decode
    kernel stores +0."""
    say("decode kernel, signed-zero leaves")
    A = torch.zeros((3, 512), dtype=torch.bfloat16)
    A[1] = -0.0
    B = -torch.ones((512, 48), dtype=torch.bfloat16)
    for cfg in DECODE_CFGS:
        out = bits(_forced(cfg, lambda: dg.det_gemm_fwd(A.to(dev), B.to(dev))))
        assert (out == 0).all(), cfg
        out_t = bits(_forced(cfg, lambda: dg.det_gemm_fwd_rhs_transposed(
            A.to(dev), B.t().contiguous().to(dev))))
        assert (out_t == 0).all(), cfg


ROW_LIMITS = ((10, 128), (12, 64), (11, 16))
# 32- and 64-column wide tiles with the tree split over wave groups, and the least
# leaf count each takes (a group of 8 stages of 2 leaves per wave group)
NARROW_WIDE_CFGS = {13: 32, 14: 32, 15: 64, 16: 64}


@pytest.mark.parametrize("M,K", [(1, 4096), (5, 1024), (16, 4128), (40, 4096), (128, 1024),
                                 (100, 4128)])
def test_decode_nonfinite_inputs(dev, M, K):
    """Inf and NaN in X or the weight: every decode configuration that takes M
    rows gives the general kernel's bits (both layouts of the weight)."""
    say("decode kernel, non-finite inputs", M, K)
    N = 200
    A = W.randn_bf16((M, K), 1.0, 1500 + K)
    B = W.randn_bf16((K, N), 0.02, 1501 + K)
    A[0, 17] = float("inf")
    A[M - 1, K - 3] = float("nan")
    B[40, 33] = float("-inf")
    B[K // 2, 150] = float("nan")
    Ad, Bd, Btd = A.to(dev), B.to(dev), B.t().contiguous().to(dev)
    ref = bits(_forced(GENERAL_CFG, lambda: dg.det_gemm_fwd(Ad, Bd)))
    ref_t = bits(_forced(GENERAL_CFG, lambda: dg.det_gemm_fwd_rhs_transposed(Ad, Btd)))
    assert np.array_equal(ref, ref_t)
    for cfg, rows in ROW_LIMITS:
        if M > rows:
            continue
        assert np.array_equal(bits(_forced(cfg, lambda: dg.det_gemm_fwd(Ad, Bd))), ref), cfg
        assert np.array_equal(bits(_forced(cfg, lambda: dg.det_gemm_fwd_rhs_transposed(Ad, Btd))),
                              ref), cfg


@pytest.mark.parametrize("M", [1, 16, 64, 128])
def test_decode_tree_overflow(dev, M):
    """Finite leaves whose tree adds overflow: in columns 5 and 37 every leaf
    is 32 * 2^122 = 2^127 (exact), so the first add of two leaves is 2^128,
    +Inf in fp32 and bf16, and so is the root; the other columns stay finite.
    The decode configurations give the general kernel's bits, and those
    columns are +Inf."""
    say("decode kernel, overflow in the tree adds", M)
    K, N = 1024, 72
    A = torch.ones((M, K), dtype=torch.bfloat16)
    B = W.randn_bf16((K, N), 0.02, 1510 + M)
    B[:, 5] = 2.0 ** 122
    B[:, 37] = 2.0 ** 122
    Ad, Bd, Btd = A.to(dev), B.to(dev), B.t().contiguous().to(dev)
    ref = bits(_forced(GENERAL_CFG, lambda: dg.det_gemm_fwd(Ad, Bd)))
    assert (ref[:, [5, 37]] == 0x7F80).all()
    assert ((ref[:, [c for c in range(N) if c not in (5, 37)]] & 0x7F80) != 0x7F80).all()
    for cfg, rows in ROW_LIMITS:
        if M > rows:
            continue
        assert np.array_equal(bits(_forced(cfg, lambda: dg.det_gemm_fwd(Ad, Bd))), ref), cfg
        assert np.array_equal(bits(_forced(cfg, lambda: dg.det_gemm_fwd_rhs_transposed(Ad, Btd))),
                              ref), cfg


# The last four reach past the decode kernel's range of choice: N = 28672 at
# 17 and 64 rows runs on 128x128 wide tiles, N = 14336 at 64 rows on 128x64
# wide tiles, and K = 1536 (48 leaves, not a power of two, which the wide
# kernels need) at N = 28672 stays on the decode kernel.
@pytest.mark.parametrize("M,N,K", [(17, 200, 4096), (24, 6144, 4096), (32, 136, 1024), (20, 48, 4128),
                                   (32, 40, 32768), (33, 200, 4096), (48, 6144, 4096), (64, 72, 4128),
                                   (61, 40, 1024), (65, 200, 4096), (80, 6144, 4096),
                                   (100, 40, 1024), (128, 72, 4128), (128, 6144, 4096),
                                   (17, 28672, 4096), (64, 28672, 4096),
                                   (64, 14336, 4096), (40, 28672, 1536)])
def test_row_blocks_match_general_kernel(dev, M, N, K):
    """17 to 128 rows: the decode kernel stages 2 or 4 blocks of 16 rows of X on
    16- and 32-column tiles, and 8 blocks on 16-column tiles (wider tiles
    refuse what they do not take); the automatic choice
    moves wide products to the wide kernel.  Every path gives the general
    kernel's bits on the four X-row products."""
    say("17..128 rows on the decode kernel vs general kernel", M, N, K)
    A = W.randn_bf16((M, K), 1.0, 1600 + M + K).to(dev)
    B = W.randn_bf16((K, N), 0.02, 1601 + N + K).to(dev)
    dC = W.randn_bf16((M, N), 1.0, 1602 + N).to(dev)
    for op, f in _ops(A, B, dC).items():
        ref = _as_bits(_forced(GENERAL_CFG, f))
        assert np.array_equal(_as_bits(f()), ref), op
        da_fits = op != "da" or (N % 32 == 0 and N // 32 >= 8)
        for cfg, rows in ROW_LIMITS:
            if not da_fits:
                continue
            if M <= rows:
                assert np.array_equal(_as_bits(_forced(cfg, f)), ref), (op, cfg)
            else:
                with pytest.raises(dg.DetGemmError) as e:
                    _forced(cfg, f)
                assert e.value.code == dg.EINVAL
        # narrow split wide tiles: power-of-two leaf counts from the least each
        # takes, whose parked levels fit the LDS (the reduction runs over K, or
        # over N for da); up to 128 leaves they all run
        R = N if op == "da" else K
        pow2 = R % 64 == 0 and (R // 32) & (R // 32 - 1) == 0
        for cfg, least in NARROW_WIDE_CFGS.items():
            runs = pow2 and least <= R // 32 <= 128
            try:
                got = _as_bits(_forced(cfg, f))
            except dg.DetGemmError as err:
                assert err.code == dg.EINVAL and not runs, (op, cfg)
                continue
            assert pow2 and np.array_equal(got, ref), (op, cfg)
