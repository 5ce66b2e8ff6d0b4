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
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

FAKE = ctypes.c_void_p(0x10000)   # never dereferenced: every call below fails validation
NULL = ctypes.c_void_p(0)


@pytest.fixture(scope="module")
def lib():
    from invariant_deterministic_gemm_det_amd import build
    build.build(force=False)
    return dg.load_library()


def declared_functions():
    names = set()
    for h in HEADERS:
        text = open(h).read()
        names |= set(re.findall(r"^\s*(?:int|const char \*)\s*(det_\w+)\s*\(", text, re.M))
    return sorted(names)


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


# ---------------------------------------------------------------- det_moe.h

def _moe(lib, T, N, K, offsets, E=None, slot_ld=None, X=FAKE, W=FAKE, G=FAKE, Y=FAKE,
         slots=ctypes.c_void_p(0x900000000), dprob=ctypes.c_void_p(0xA00000000), w_stride=None):
    E = len(offsets) - 1 if E is None else E
    off = (ctypes.c_int64 * max(len(offsets), 1))(*offsets)
    return lib.det_moe_fwd_dprob(X, K, W, N, K * N if w_stride is None else w_stride, off, E,
                                 G, N, Y, N, slots, T if slot_ld is None else slot_ld, dprob,
                                 T, N, K, NULL)


def test_moe_argument_errors_without_device(lib):
    """Section "Kernel redesign: the grouped-GEMM epilogue" of the Megatron Core
    reading notes; every error is reported before any device work."""
    assert _moe(lib, 0, 128, 64, [0, 0]) == dg.OK                 # no rows: no-op
    assert _moe(lib, 4, 128, 0, [0, 4]) == dg.EKCAP
    assert _moe(lib, 4, 128, 32769, [0, 4]) == dg.EKCAP
    assert _moe(lib, 4, 128, 64, [0, 3, 2, 4]) == dg.EINVAL       # decreasing offsets
    assert _moe(lib, 4, 128, 64, [1, 4]) == dg.EINVAL             # offsets[0] != 0
    assert _moe(lib, 4, 128, 64, [0, 5]) == dg.EINVAL             # offsets[E] != T
    assert _moe(lib, 4, 128, 64, [0, 4], E=0) == dg.EINVAL
    assert _moe(lib, 4, 128, 64, [0] * 129 + [4]) == dg.EINVAL    # more than 128 experts
    assert _moe(lib, 4, 128, 64, [0, 4], slot_ld=3) == dg.EINVAL  # slot rows shorter than T
    assert _moe(lib, -1, 128, 64, [0, -1]) == dg.EINVAL
    assert _moe(lib, 4, 128, 64, [0, 4], w_stride=-1) == dg.EINVAL
    # the output Y over the input X
    assert _moe(lib, 4, 128, 64, [0, 4], Y=FAKE, X=FAKE) == dg.EINVAL
    # dprob over the slots
    assert _moe(lib, 4, 128, 64, [0, 4], Y=ctypes.c_void_p(0x700000000),
                dprob=ctypes.c_void_p(0x900000000)) == dg.EINVAL


def test_moe_debug_slots_argument_errors(lib):
    s = ctypes.c_void_p(0x900000000)
    assert lib.det_moe_debug_slots(FAKE, 128, FAKE, 128, s, 3, 4, 128, NULL) == dg.EINVAL
    assert lib.det_moe_debug_slots(FAKE, 128, FAKE, 128, s, 4, -1, 128, NULL) == dg.EINVAL
    assert lib.det_moe_debug_slots(FAKE, 128, FAKE, 128, s, 4, 0, 128, NULL) == dg.OK


# ---------------------------------------------------------------- det_fingerprint.h

def test_fingerprint_argument_errors_without_device(lib):
    """Reading notes on bitwise-deterministic pretraining, section "5.
    Fingerprinting Tensors on the GPU"; errors are reported before any device
    work."""
    out = ctypes.c_void_p(0x900000000)
    assert lib.det_fingerprint(FAKE, -1, out, NULL) == dg.EINVAL
    assert lib.det_fingerprint(NULL, 16, out, NULL) == dg.EINVAL
    assert lib.det_fingerprint(FAKE, 16, NULL, NULL) == dg.EINVAL
    assert lib.det_fingerprint(FAKE, 64, ctypes.c_void_p(0x10008), NULL) == dg.EINVAL  # overlap
    assert lib.det_fingerprint_rows(FAKE, 4, 32, 16, out, NULL) == dg.EINVAL          # ld < row
    assert lib.det_fingerprint_rows(FAKE, -1, 32, 32, out, NULL) == dg.EINVAL
    assert lib.det_fingerprint_rows(FAKE, 0, 32, 32, out, NULL) == dg.OK               # no rows
    assert lib.det_fingerprint_rows(FAKE, 4, 32, 32, ctypes.c_void_p(0x10040), NULL) == dg.EINVAL
    assert lib.det_first_mismatch(FAKE, FAKE, -1, out, NULL) == dg.EINVAL
    assert lib.det_first_mismatch(FAKE, NULL, 8, out, NULL) == dg.EINVAL
    assert lib.det_first_mismatch(FAKE, FAKE, 8, NULL, NULL) == dg.EINVAL


# ---------------------------------------------------------------- det_norm.h

def test_rmsnorm_argument_errors_without_device(lib):
    """Summary of "Defeating Nondeterminism in LLM Inference", batch-invariant
    RMSNorm; errors before any device work."""
    y, r = ctypes.c_void_p(0x900000000), ctypes.c_void_p(0xA00000000)
    eps = ctypes.c_float(1e-6)
    assert lib.det_rmsnorm(FAKE, 64, FAKE, eps, y, 64, r, -1, 64, NULL) == dg.EINVAL
    assert lib.det_rmsnorm(FAKE, 64, FAKE, eps, y, 64, r, 4, 0, NULL) == dg.EINVAL
    assert lib.det_rmsnorm(FAKE, 64, FAKE, eps, y, 64, r, 4, (1 << 20) + 1, NULL) == dg.EINVAL
    assert lib.det_rmsnorm(FAKE, 32, FAKE, eps, y, 64, r, 4, 64, NULL) == dg.EINVAL   # ldx < H
    assert lib.det_rmsnorm(NULL, 64, FAKE, eps, y, 64, r, 4, 64, NULL) == dg.EINVAL
    assert lib.det_rmsnorm(FAKE, 64, FAKE, eps, FAKE, 64, r, 4, 64, NULL) == dg.EINVAL  # y over x
    assert lib.det_rmsnorm(FAKE, 64, FAKE, eps, y, 64, y, 4, 64, NULL) == dg.EINVAL    # rstd over y
    assert lib.det_rmsnorm(FAKE, 64, FAKE, eps, y, 64, r, 0, 64, NULL) == dg.OK        # no rows


# ---------------------------------------------------------------- det_attention.h

def test_attention_argument_errors_without_device(lib):
    """Summary of "Defeating Nondeterminism in LLM Inference", attention with a
    fixed split-KV size; errors before any device work."""
    f = lib.det_attention_decode
    o, w = ctypes.c_void_p(0x900000000), ctypes.c_void_p(0xA00000000)
    s = ctypes.c_float(0.1)
    A = ctypes.c_void_p(0x100000000)
    assert f(FAKE, A, A, FAKE, 2, 8, 2, 64, 64, s, w, o, NULL) == dg.EINVAL    # D != 128
    assert f(FAKE, A, A, FAKE, 2, 8, 3, 64, 128, s, w, o, NULL) == dg.EINVAL   # Hq % Hkv
    assert f(FAKE, A, A, FAKE, 2, 32, 2, 64, 128, s, w, o, NULL) == dg.EINVAL  # G > 8
    assert f(FAKE, A, A, FAKE, -1, 8, 2, 64, 128, s, w, o, NULL) == dg.EINVAL
    assert f(FAKE, A, A, NULL, 2, 8, 2, 64, 128, s, w, o, NULL) == dg.EINVAL   # no lens
    assert f(FAKE, A, A, FAKE, 2, 8, 2, 64, 128, s, w, A, NULL) == dg.EINVAL   # O over K
    assert f(FAKE, A, A, FAKE, 0, 8, 2, 64, 128, s, w, o, NULL) == dg.OK       # no sequences


def test_shard_reduce_argument_errors_without_device(lib):
    """det_gemm.h, combination of K-shard partials: errors before any device work."""
    parts = (ctypes.c_void_p * 3)(0x100000000, 0x200000000, 0x300000000)
    f = lib.det_gemm_shard_reduce
    out = ctypes.c_void_p(0x900000000)
    assert f(parts, 0, 64, out, 64, 4, 64, NULL) == dg.EINVAL           # no parts
    assert f(parts, 17, 64, out, 64, 4, 64, NULL) == dg.EINVAL          # too many
    assert f(parts, 3, 32, out, 64, 4, 64, NULL) == dg.EINVAL           # ld < N
    assert f(parts, 3, 64, ctypes.c_void_p(0x200000000), 64, 4, 64, NULL) == dg.EINVAL  # overlap
    assert f(parts, 3, 64, out, 64, 0, 64, NULL) == dg.OK               # empty
    assert f(None, 3, 64, out, 64, 4, 64, NULL) == dg.EINVAL


def test_leading_dimension_limit(lib):
    """Leading dimensions above DET_GEMM_MAX_LD = 2^23 are refused before any
    device work (the tile byte offsets must stay below 2^31)."""
    big = (1 << 23) + 8
    far = ctypes.c_void_p(0x40000000000)
    assert _fwd(lib, 4, 4, 8, lda=big, C=far) == dg.EINVAL
    assert _fwd(lib, 4, 4, 8, ldb=big, C=far) == dg.EINVAL
    assert _fwd(lib, 4, 4, 8, ldc=big, C=far) == dg.EINVAL
    hdr = open(HEADER).read()
    assert "DET_GEMM_MAX_LD" in hdr and "(INT64_C(1) << 23)" in hdr


def test_debug_matrix_add_argument_errors(lib):
    out = ctypes.c_void_p(0x900000000)
    f = lib.det_gemm_debug_matrix_add
    assert f(FAKE, FAKE, out, -1, 0, NULL) == dg.EINVAL
    assert f(FAKE, FAKE, out, 16, 2, NULL) == dg.EINVAL      # unknown selector
    assert f(NULL, FAKE, out, 16, 0, NULL) == dg.EINVAL
    assert f(FAKE, FAKE, out, 0, 1, NULL) == dg.OK


def test_issue_probe_argument_errors(lib):
    sink = ctypes.c_void_p(0x900000000)
    f = lib.det_gemm_debug_issue_probe
    assert f(2, 10, 256, sink, NULL) == dg.EINVAL      # unknown mode
    assert f(-1, 10, 256, sink, NULL) == dg.EINVAL
    assert f(0, 0, 256, sink, NULL) == dg.EINVAL       # no iterations
    assert f(1, 10, 0, sink, NULL) == dg.EINVAL        # no workgroups
    assert f(1, 10, 256, NULL, NULL) == dg.EINVAL


# ---------------------------------------------------------------- the Python binding

def _t(shape, dtype):
    import torch
    return torch.zeros(shape, dtype=dtype)


def test_binding_checks_caller_outputs_before_any_launch():
    """A caller's output must have the dtype, shape and layout the C call
    writes: a bf16 buffer for an fp32 product (half the bytes) or a float32
    buffer for a bf16 product is refused, as are outputs on another device,
    undersized work buffers and non-contiguous vectors."""
    import torch
    A, B = _t((4, 64), torch.bfloat16), _t((64, 8), torch.bfloat16)
    with pytest.raises(TypeError, match="dtype"):
        dg.det_gemm_fwd_fp32(A, B, out=_t((4, 8), torch.bfloat16))
    with pytest.raises(TypeError, match="dtype"):
        dg.det_gemm_fwd(A, B, out=_t((4, 8), torch.float32))
    with pytest.raises(ValueError, match="shape"):
        dg.det_gemm_fwd(A, B, out=_t((4, 9), torch.bfloat16))
    with pytest.raises(TypeError, match="must be on"):          # CPU tensor output
        dg.det_gemm_fwd(A, B, out=_t((4, 8), torch.bfloat16))
    with pytest.raises(TypeError, match="torch tensor"):
        dg.det_gemm_fwd(A, B, out=[0] * 32)
    x, w = _t((4, 64), torch.bfloat16), _t((64,), torch.bfloat16)
    with pytest.raises(TypeError, match="dtype"):
        dg.det_rmsnorm(x, w, rstd=_t((4,), torch.float16))
    with pytest.raises(ValueError, match="contiguous"):
        dg.det_rmsnorm(x, w, rstd=_t((8,), torch.float32)[::2])
    with pytest.raises(TypeError, match="dtype"):
        dg._out(_t((4,), torch.int32), (4,), x, torch.int64, contiguous=True)


def test_binding_refuses_host_tensors():
    """No CPU fallback: host tensors never reach the library."""
    import torch
    q = _t((2, 8, 128), torch.bfloat16)
    k = _t((2, 2, 64, 128), torch.bfloat16)
    lens = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(TypeError):
        dg.det_attention_decode(q, k, k, lens, 0.1)
    with pytest.raises(TypeError):
        dg.det_gemm_fwd(_t((4, 64), torch.bfloat16), _t((64, 8), torch.bfloat16))


def test_attention_noalloc_refuses_oversize_without_device(lib):
    """det_attention_decode_noalloc: a problem whose per-split partials exceed
    the fixed device array is refused before any device work."""
    f = lib.det_attention_decode_noalloc
    A = ctypes.c_void_p(0x100000000)
    s = ctypes.c_float(0.1)
    o = ctypes.c_void_p(0x900000000)
    assert f(FAKE, A, A, FAKE, 65535, 32, 8, 4096, 128, s, o, NULL) == dg.ESCRATCH
    assert f(FAKE, A, A, FAKE, 2, 8, 2, 64, 64, s, o, NULL) == dg.EINVAL   # D != 128
    assert f(FAKE, A, A, FAKE, 0, 8, 2, 64, 128, s, o, NULL) == dg.OK      # no sequences
    assert b"scratch" in lib.det_gemm_status_string(dg.ESCRATCH)


def test_attention_prefill_argument_errors_without_device(lib):
    """det_attention_prefill: grouping and shape errors before any device work."""
    f = lib.det_attention_prefill
    A = ctypes.c_void_p(0x100000000)
    o, w = ctypes.c_void_p(0x900000000), ctypes.c_void_p(0xA00000000)
    s = ctypes.c_float(0.1)
    off = lambda *v: (ctypes.c_int64 * len(v))(*v)
    assert f(FAKE, A, A, off(0, 3, 4), FAKE, 5, 2, 8, 2, 64, 128, s, w, o, NULL) == dg.EINVAL  # last != NQ
    assert f(FAKE, A, A, off(1, 3, 5), FAKE, 5, 2, 8, 2, 64, 128, s, w, o, NULL) == dg.EINVAL  # first != 0
    assert f(FAKE, A, A, off(0, 4, 3), FAKE, 3, 2, 8, 2, 64, 128, s, w, o, NULL) == dg.EINVAL  # decreasing
    assert f(FAKE, A, A, off(0, 3, 5), FAKE, 5, 2, 8, 2, 64, 64, s, w, o, NULL) == dg.EINVAL   # D != 128
    assert f(FAKE, A, A, None, FAKE, 5, 2, 8, 2, 64, 128, s, w, o, NULL) == dg.EINVAL          # no offsets
    assert f(FAKE, A, A, off(0, 0), FAKE, 0, 1, 8, 2, 64, 128, s, w, o, NULL) == dg.OK         # no rows


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU; --gpus N > 1 exits with status 2 and says so
    before touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_no_long_branch_through_a_return_address(tmp_path):
    """The library's device code (built here from its sources) has no long
    branch that goes through s[30:31]: in a called function those registers
    hold the return address, and a long branch that reuses them makes the
    function jump back into its own body when it returns (a recomputation
    of non-finite tiles whose unrolled code outgrew the range of a short
    branch never returned).  Each translation unit's offload bundle is
    unbundled and disassembled with the ROCm LLVM tools."""
    import re
    import shutil
    import subprocess
    llvm = "/opt/rocm/llvm/bin"
    tools = [os.path.join(llvm, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-objdump")]
    if not all(os.path.exists(t) for t in tools) or not os.path.exists(dg.LIB_PATH):
        pytest.skip("ROCm LLVM tools or the built library not present")
    objcopy, bundler, objdump = tools
    fatbin = tmp_path / "fatbin.bin"
    subprocess.run([objcopy, "--dump-section", f".hip_fatbin={fatbin}", dg.LIB_PATH,
                    str(tmp_path / "lib_copy.so")], check=True, capture_output=True)
    data = fatbin.read_bytes()
    magic = b"__CLANG_OFFLOAD_BUNDLE__"
    starts = [m.start() for m in re.finditer(re.escape(magic), data)]
    assert starts, "no offload bundles in the library"
    scanned = 0
    for i, o in enumerate(starts):
        chunk = tmp_path / f"b{i}.bin"
        chunk.write_bytes(data[o:starts[i + 1] if i + 1 < len(starts) else len(data)])
        co = tmp_path / f"b{i}.co"
        subprocess.run([bundler, "--type=o", "--targets=hipv4-amdgcn-amd-amdhsa--gfx950",
                        f"--input={chunk}", f"--output={co}", "--unbundle"],
                       check=True, capture_output=True)
        if co.stat().st_size == 0:
            continue
        dis = subprocess.run([objdump, "-d", "--mcpu=gfx950", str(co)], check=True,
                             capture_output=True, text=True).stdout
        scanned += 1
        assert not re.search(r"s_getpc_b64 s\[30:31\]", dis), f"translation unit {i}"
    assert scanned >= 8
    shutil.rmtree(tmp_path, ignore_errors=True)
