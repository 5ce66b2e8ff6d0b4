"""Tile-configuration selection, pinned on the host (no device).

Every configuration computes the same leaves and the same mid-split tree, so
the choice never changes bits (the GPU tests compare them); these tests pin
which kernel each problem class runs on, through det_gemm_debug_config, which
applies the entry point's argument checks and the selection to shape,
alignment and leaf count without touching memory.  Configurations: 5 to 9
wide kernels (6: 128x64 tiles; 8: 128x128 two-leaf units; 9: three-leaf
units), 10 to 12 decode kernels with 16, 64 and 32 columns per workgroup, 13
and 14 the 128x32 and 64x32 wide tiles whose tree is split at its root over
two wave groups, 15 and 16 the 64x32 and 64x64 tiles on four wave groups,
17 the 128x128 tiles with two register levels for the deepest trees, 18 to
29 the 128x128 tiles over units of 5, 7, 43, 27, 37, 11, 17, 19, 25 and 35
leaves.
"""
import pytest

import invariant_deterministic_gemm_det_amd as dg

A_ADDR, B_ADDR, C_ADDR = 0x100000000, 0x200000000, 0x300000000  # disjoint, 256-byte aligned


def cfg(op, M, N, K, transposed_rhs=False):
    """Configuration of a contiguous product: fwd family C[M][N] = A[M][K] B,
    da dA[M][K] = dC[M][N] B^T, db dB[K][N] = A^T dC."""
    if op == dg.OP_FWD_RHS_TRANSPOSED:
        return dg.det_gemm_debug_config(op, A_ADDR, K, B_ADDR, K, C_ADDR, N, M, N, K)
    if op in (dg.OP_FWD, dg.OP_FWD_FP32):
        return dg.det_gemm_debug_config(op, A_ADDR, K, B_ADDR, N, C_ADDR, N, M, N, K)
    if op == dg.OP_DA:
        return dg.det_gemm_debug_config(op, A_ADDR, N, B_ADDR, N, C_ADDR, K, M, N, K)
    if op == dg.OP_DB:
        return dg.det_gemm_debug_config(op, A_ADDR, K, B_ADDR, N, C_ADDR, N, M, N, K)
    raise ValueError(op)


@pytest.fixture(autouse=True)
def automatic():
    dg.det_gemm_debug_force_config(-1)
    yield
    dg.det_gemm_debug_force_config(-1)


def test_step_products_run_on_the_wide_kernel():
    # M = K = 4096, N = 6144: fwd and db have 128 leaves (two-leaf units),
    # da reduces over N = 6144, 192 leaves (three-leaf units).
    assert cfg(dg.OP_FWD, 4096, 6144, 4096) == 8
    assert cfg(dg.OP_DA, 4096, 6144, 4096) == 9
    assert cfg(dg.OP_DB, 4096, 6144, 4096) == 8
    # fewer than four waves of 128x128 workgroups: 128x64 tiles
    assert cfg(dg.OP_FWD, 1024, 6144, 4096) == 6


@pytest.mark.parametrize("M,N,want", [
    (1, 4096, 10),     # at most 128 tiles of 32 columns
    (1, 6144, 12),     # QKV: 192 tiles of 32 columns
    (16, 6144, 12),
    (1, 8192, 12),     # 128 tiles of 64 columns: still 32 columns
    (1, 11008, 11),    # 172 tiles of 64 columns
    (16, 151936, 11),  # LM head
    (32, 6144, 12),    # two row blocks, 384 (tiles x blocks)
    (64, 11008, 16),   # 172 tiles of 64x64 on four wave groups
    (17, 14336, 16),   # 224 tiles of 64x64
    (17, 16384, 16),   # 256 tiles of 64x64: still one round
    (17, 18432, 12),   # 288 tiles of 64x64: more than one round; decode
    (64, 18432, 8),    # 576 x 4 = 2304: wide, 144 tiles of 128 columns
    (17, 28672, 8),    # 896 x 2: wide, 224 tiles of 128 columns
    (48, 151936, 8),
])
def test_small_m_row_major_weight(M, N, want):
    assert cfg(dg.OP_FWD, M, N, 4096) == want
    assert cfg(dg.OP_FWD_FP32, M, N, 4096) == want


def test_small_m_leaf_count_the_wide_kernel_refuses():
    # K = 1536: 48 leaves, not a power of two, so 40 rows at N = 28672 stay on
    # the decode kernel although the wide kernel would be chosen for K = 4096
    assert cfg(dg.OP_FWD, 40, 28672, 4096) == 8
    assert cfg(dg.OP_FWD, 40, 28672, 1536) == 12


@pytest.mark.parametrize("M,N,want_t", [
    (17, 151936, 12),   # a K-major weight read in whole lines: the decode kernel up to 32 rows
    (32, 151936, 12),
    (32, 40960, 12),
    (33, 151936, 8),    # more rows: the wide kernel
])
def test_small_m_transposed_weight_stays_on_decode_up_to_32_rows(M, N, want_t):
    assert cfg(dg.OP_FWD_RHS_TRANSPOSED, M, N, 4096) == want_t
    assert cfg(dg.OP_FWD, M, N, 4096) == 8          # a [K][N] weight: the wide kernel


def test_small_m_transposed_weight():
    # W [N][K] with an even leaf count is read in two-leaf lines at any width:
    # 32 columns even for the LM head; an odd leaf count takes 64 columns
    assert cfg(dg.OP_FWD_RHS_TRANSPOSED, 1, 151936, 4096) == 12
    assert cfg(dg.OP_FWD_RHS_TRANSPOSED, 1, 151936, 4128) == 11
    assert cfg(dg.OP_FWD_RHS_TRANSPOSED, 1, 6144, 4096) == 12


def test_decode_limits():
    assert cfg(dg.OP_FWD, 129, 6144, 4096) not in (10, 11, 12)  # more than 128 rows
    assert cfg(dg.OP_FWD, 1, 6144, 224) not in (10, 11, 12)     # 7 leaves
    assert cfg(dg.OP_FWD, 1, 4096, 32768) == 10   # 1024 leaves, the reduction cap
    assert cfg(dg.OP_FWD, 1, 6143, 4096) not in (10, 11, 12)    # N not whole 8-column chunks


def test_pinned_configuration_is_reported():
    dg.det_gemm_debug_force_config(3)
    assert cfg(dg.OP_FWD, 1, 6144, 4096) == 3


def test_argument_errors():
    with pytest.raises(dg.DetGemmError) as e:
        dg.det_gemm_debug_config(6, A_ADDR, 64, B_ADDR, 64, C_ADDR, 64, 64, 64, 64)
    assert e.value.code == dg.EINVAL
    with pytest.raises(dg.DetGemmError) as e:   # empty product: nothing is launched
        cfg(dg.OP_FWD, 0, 64, 64)
    assert e.value.code == dg.EINVAL
    with pytest.raises(dg.DetGemmError) as e:   # reduction past the cap
        cfg(dg.OP_FWD, 4, 64, 32768 + 32)
    assert e.value.code == dg.EKCAP
    with pytest.raises(dg.DetGemmError) as e:   # output overlapping an input
        dg.det_gemm_debug_config(dg.OP_FWD, A_ADDR, 64, B_ADDR, 64, A_ADDR, 64, 64, 64, 64)
    assert e.value.code == dg.EINVAL


@pytest.mark.parametrize("M,N,want,want_t", [
    (128, 6144, 16, 13),   # QKV at 128 rows: 192 tiles of 64x64 (W [K][N]) or 128x32
    (65, 6144, 16, 13),
    (128, 8192, 16, 13),
    (96, 8192, 16, 13),
    (128, 10240, 6, 6),    # 320 column tiles of 32: more than one round; 128x64 wide
    (64, 6144, 14, 15),    # 192 tiles of 64x32; a K-major weight on four wave groups
    (48, 6144, 14, 15),
    (40, 6144, 14, 15),
    (32, 6144, 12, 15),    # up to 32 rows: the decode kernel for W [K][N]
    (128, 2048, 14, 15),   # 2 x 64 tiles of 64x32
    (128, 4096, 14, 15),   # 2 x 128 = 256 tiles: one round over the compute units
    (64, 2048, 10, 15),    # at most 128 column tiles: the decode kernel for W [K][N]
    (48, 8192, 14, 15),    # 256 column tiles of 64x32 ([K][N]: tiles 2u, 2u + 1 on one XCD)
    (48, 10240, 16, 16),   # 160 tiles of 64x64 on four wave groups
    (48, 18432, 8, 8),     # 288 tiles of 64x64: the wide kernel
    (128, 14336, 6, 6),    # 448 tiles of 128x32: the 128x64 wide kernel
])
def test_narrow_split_tiles(M, N, want, want_t):
    assert cfg(dg.OP_FWD, M, N, 4096) == want
    assert cfg(dg.OP_FWD_FP32, M, N, 4096) == want
    assert cfg(dg.OP_FWD_RHS_TRANSPOSED, M, N, 4096) == want_t


@pytest.mark.parametrize("M,N,want_t", [
    (32, 6144, 15),    # 17 to 32 rows, 192 column tiles of 32: four wave groups
    (17, 6144, 15),
    (24, 8192, 15),    # 256 column tiles
    (16, 6144, 12),    # at most 16 rows: the decode kernel
    (32, 4096, 10),    # at most 128 column tiles: the decode kernel
    (32, 10240, 12),   # more than one round of 64x32 tiles: the decode kernel
])
def test_split_tiles_for_17_to_32_rows_of_a_k_major_weight(M, N, want_t):
    assert cfg(dg.OP_FWD_RHS_TRANSPOSED, M, N, 4096) == want_t


@pytest.mark.parametrize("M,N,want", [
    (17, 6144, 12),    # 192 column tiles of 32: the decode kernel
    (32, 6144, 12),
    (24, 8192, 15),    # 193 to 256 column tiles: 64x32 on four wave groups
    (32, 8192, 15),
    (32, 4096, 10),    # at most 128 column tiles: the decode kernel
    (32, 10240, 16),   # 160 tiles of 64x64 on four wave groups
    (16, 10240, 11),   # at most 16 rows: the decode kernel
])
def test_split_tiles_for_17_to_32_rows_of_a_row_major_weight(M, N, want):
    assert cfg(dg.OP_FWD, M, N, 4096) == want


def test_narrow_split_tiles_need_a_power_of_two_leaf_count():
    # K = 4128: 129 leaves; neither the split tiles nor the wide kernel take it
    assert cfg(dg.OP_FWD, 128, 6144, 4128) == 10
    # da at 128 rows reduces over N = 4096 (128 leaves) into 6144 columns
    assert cfg(dg.OP_DA, 128, 4096, 6144) == 13


@pytest.mark.parametrize("M,N,K,want", [
    (512, 4096, 4096, 6),      # 128 tiles of 128x128: 128x64 tiles, one round
    (1024, 6144, 4096, 6),     # 384 tiles: 128x64, two workgroups per compute unit
    (2048, 4096, 4096, 8),     # 512 tiles: two rounds of 128x128
    (512, 4096, 8192, 6),      # 256 leaves, 128x64 tiles still one round
    (1024, 4096, 8192, 8),     # 256 leaves: 128x64 would hold one workgroup per unit
    (2048, 4096, 16384, 5),    # 512 leaves: two stage buffers (three do not fit the LDS)
    (2048, 4096, 32768, 17),   # 1024 leaves: 128x128 with a second register level
    (512, 4096, 32768, 6),     # ... unless 128x64 tiles fit one round
])
def test_mid_size_products_by_leaves_and_tiles(M, N, K, want):
    assert cfg(dg.OP_FWD, M, N, K) == want


@pytest.mark.parametrize("K,want", [
    (5120, 18),     # L = 160 = 5 * 32: five-leaf units
    (10240, 18),
    (7168, 19),     # L = 224 = 7 * 32: seven-leaf units
    (14336, 19),
    (28672, 20),    # L = 896: seven-leaf units on two stage buffers
    (11008, 21),    # L = 344 = 43 * 8: 43-leaf units
    (22016, 21),
    (13824, 22),    # L = 432 = 27 * 16: 27-leaf units
    (27648, 23),    # L = 864 = 27 * 32: 27-leaf units on two stage buffers
    (18944, 24),    # L = 592 = 37 * 16: 37-leaf units
    (5632, 25),     # L = 176 = 11 * 16
    (17408, 26),    # L = 544 = 17 * 32, two stage buffers
    (9728, 27),     # L = 304 = 19 * 16
    (25600, 28),    # L = 800 = 25 * 32, two stage buffers
    (8960, 29),     # L = 280 = 35 * 8
    (4128, 2),      # L = 129: no unit schedule
])
def test_unit_schedules_by_leaf_count(K, want):
    assert cfg(dg.OP_FWD, 4096, 4096, K) == want
