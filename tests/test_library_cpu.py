"""The C-ABI library without a GPU: it loads, it exports every entry point the
header declares, and argument errors are reported before anything touches a
device (RL-Kernel det_gemm page, "Ascend NPU backend": reduction capped at
32768; unsupported inputs are rejected, never run another way)."""
import ctypes
import os
import re

import pytest

import invariant_deterministic_gemm_det_amd as dg

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "det_gemm.h")

FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: every call below fails validation
NULL = ctypes.c_void_p(0)


@pytest.fixture(scope="module")
def lib():
    from invariant_deterministic_gemm_det_amd import build
    build.build(force=False)
    return dg.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|const char \*)\s*(det_gemm_\w+)\s*\(", text, re.M)))


def test_header_declares_the_six_operations():
    names = declared_functions()
    for op in ("fwd", "fwd_rhs_transposed", "fwd_fp32", "da", "db", "db_transposed"):
        assert f"det_gemm_{op}" in names
        assert f"det_gemm_strict_{op}" in names


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert set(names) == set(dg.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in (dg.OK, dg.EINVAL, dg.EKCAP, dg.EHIP):
        assert lib.det_gemm_status_string(code)
    assert b"32768" in lib.det_gemm_status_string(dg.EKCAP)


def _fwd(lib, M, N, K, A=FAKE, B=FAKE, C=FAKE, lda=None, ldb=None, ldc=None, name="det_gemm_fwd"):
    lda = K if lda is None else lda
    ldb = N if ldb is None else ldb
    ldc = N if ldc is None else ldc
    return getattr(lib, name)(A, lda, B, ldb, C, ldc, M, N, K, NULL)


@pytest.mark.parametrize("strict", [False, True])
def test_argument_errors_without_device(lib, strict):
    name = "det_gemm_strict_fwd" if strict else "det_gemm_fwd"
    assert _fwd(lib, 4, 4, 32769, name=name) == dg.EKCAP
    assert _fwd(lib, 4, 4, 0, name=name) == dg.EKCAP
    assert _fwd(lib, -1, 4, 8, name=name) == dg.EINVAL
    assert _fwd(lib, 4, 4, 8, A=NULL, name=name) == dg.EINVAL
    assert _fwd(lib, 4, 4, 8, lda=7, name=name) == dg.EINVAL          # lda < K
    assert _fwd(lib, 4, 4, 8, ldc=3, name=name) == dg.EINVAL          # ldc < N
    # output overlapping an input
    assert _fwd(lib, 4, 4, 8, A=FAKE, C=ctypes.c_void_p(0x10000 + 8), name=name) == dg.EINVAL
    # empty outputs are successful no-ops, whatever the pointers
    assert _fwd(lib, 0, 4, 8, A=NULL, B=NULL, C=NULL, name=name) == dg.OK
    assert _fwd(lib, 4, 0, 8, A=NULL, B=NULL, C=NULL, name=name) == dg.OK


def test_backward_caps_apply_to_their_reduction(lib):
    # da reduces over N, db over M: the cap follows the reduction, not K
    assert lib.det_gemm_da(FAKE, 40000, FAKE, 40000, ctypes.c_void_p(0x900000000), 8,
                           4, 40000, 8, NULL) == dg.EKCAP
    assert lib.det_gemm_db(FAKE, 8, ctypes.c_void_p(0x900000000), 8, ctypes.c_void_p(0x990000000),
                           8, 40000, 8, 8, NULL) == dg.EKCAP
    assert lib.det_gemm_db_transposed(FAKE, 8, FAKE, 8, FAKE, 8, 0, 8, 8, NULL) == dg.EKCAP
    # db output [K,N] empty -> no-op even with M over the cap
    assert lib.det_gemm_db(FAKE, 8, FAKE, 8, FAKE, 8, 40000, 8, 0, NULL) == dg.OK


def test_force_config_bounds(lib):
    n = lib.det_gemm_debug_force_config(-1)
    assert n >= 2
    assert lib.det_gemm_debug_force_config(n) == dg.EINVAL
    assert lib.det_gemm_debug_force_config(-2) == dg.EINVAL
    assert lib.det_gemm_debug_force_config(0) == n
    assert lib.det_gemm_debug_force_config(-1) == n
