"""Python binding of the det_gemm C-ABI library (libdet_gemm.so, gfx950).

Argument marshalling only: every function takes torch tensors on a gfx950
device, checks dtype/shape/stride, allocates the output if none is given and
calls the entry point of the same name in ``include/det_gemm.h`` on torch's
current stream.  All arithmetic runs in the library's HIP kernels; there is no
fallback of any kind -- if the library is missing or the device is not a
gfx950, the call raises.

The operation (RL-Kernel operator page "Batch-Invariant Deterministic GEMM
(det_gemm)", sections "Guarantees" and "Ascend NPU backend"): bf16 inputs,
32-element fp32 leaves rounded once to bf16, leaves merged by the mid-split
tree of bf16 adds, reduction length capped at 32768.
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdet_gemm.so")

OK, EINVAL, EKCAP, EHIP, ESCRATCH = 0, -1, -2, -3, -4
MAX_REDUCTION = 32768
LEAF = 32

_SIX = ("det_gemm_fwd", "det_gemm_fwd_rhs_transposed", "det_gemm_fwd_fp32", "det_gemm_da",
        "det_gemm_db", "det_gemm_db_transposed")
EXPORTS = _SIX + tuple(n.replace("det_gemm_", "det_gemm_strict_") for n in _SIX) + (
    "det_gemm_debug_leaves", "det_gemm_debug_round", "det_gemm_debug_add",
    "det_gemm_debug_matrix_add", "det_gemm_debug_issue_probe",
    "det_gemm_debug_force_config", "det_gemm_debug_config", "det_gemm_status_string",
    "det_moe_fwd_dprob",
    "det_moe_debug_slots", "det_fingerprint", "det_fingerprint_rows", "det_first_mismatch",
    "det_rmsnorm", "det_attention_decode", "det_attention_decode_noalloc", "det_attention_prefill",
    "det_gemm_shard_reduce")
ATTN_SCRATCH_FLOATS = 8 << 20
MAX_PARTS = 16
ATTN_SPLIT = 256
MOE_SLOT = 128
MOE_MAX_EXPERTS = 128


class DetGemmError(RuntimeError):
    def __init__(self, code, what=""):
        msg = _status_string(code)
        super().__init__(f"{what}: det_gemm status {code} ({msg})" if what else
                         f"det_gemm status {code} ({msg})")
        self.code = code


_lib = None


def library_loaded():
    return _lib is not None


def load_library(path=LIB_PATH):
    """Load libdet_gemm.so (raises if it is not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run __graft_entry__.build() "
                          "(or python -m invariant_deterministic_gemm_det_amd.build)")
    lib = ctypes.CDLL(path)
    p, i64 = ctypes.c_void_p, ctypes.c_int64
    for name in _SIX:
        for n in (name, name.replace("det_gemm_", "det_gemm_strict_")):
            f = getattr(lib, n)
            f.argtypes = [p, i64, p, i64, p, i64, i64, i64, i64, p]
            f.restype = ctypes.c_int
    lib.det_gemm_debug_leaves.argtypes = [p, i64, p, i64, p, i64, i64, i64, p]
    lib.det_gemm_debug_leaves.restype = ctypes.c_int
    lib.det_gemm_debug_round.argtypes = [p, p, i64, p]
    lib.det_gemm_debug_round.restype = ctypes.c_int
    lib.det_gemm_debug_add.argtypes = [p, p, p, i64, p]
    lib.det_gemm_debug_add.restype = ctypes.c_int
    lib.det_gemm_debug_matrix_add.argtypes = [p, p, p, i64, ctypes.c_int, p]
    lib.det_gemm_debug_matrix_add.restype = ctypes.c_int
    lib.det_gemm_debug_issue_probe.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, p, p]
    lib.det_gemm_debug_issue_probe.restype = ctypes.c_int
    lib.det_gemm_debug_force_config.argtypes = [ctypes.c_int]
    lib.det_gemm_debug_force_config.restype = ctypes.c_int
    lib.det_gemm_debug_config.argtypes = [ctypes.c_int, p, i64, p, i64, p, i64, i64, i64, i64]
    lib.det_gemm_debug_config.restype = ctypes.c_int
    lib.det_moe_fwd_dprob.argtypes = [p, i64, p, i64, i64, p, i64, p, i64, p, i64, p, i64, p,
                                      i64, i64, i64, p]
    lib.det_moe_fwd_dprob.restype = ctypes.c_int
    lib.det_moe_debug_slots.argtypes = [p, i64, p, i64, p, i64, i64, i64, p]
    lib.det_moe_debug_slots.restype = ctypes.c_int
    lib.det_fingerprint.argtypes = [p, i64, p, p]
    lib.det_fingerprint.restype = ctypes.c_int
    lib.det_fingerprint_rows.argtypes = [p, i64, i64, i64, p, p]
    lib.det_fingerprint_rows.restype = ctypes.c_int
    lib.det_first_mismatch.argtypes = [p, p, i64, p, p]
    lib.det_first_mismatch.restype = ctypes.c_int
    lib.det_rmsnorm.argtypes = [p, i64, p, ctypes.c_float, p, i64, p, i64, i64, p]
    lib.det_rmsnorm.restype = ctypes.c_int
    lib.det_attention_decode.argtypes = [p, p, p, p, i64, i64, i64, i64, i64, ctypes.c_float, p,
                                         p, p]
    lib.det_attention_decode.restype = ctypes.c_int
    lib.det_attention_prefill.argtypes = [p, p, p, p, p, i64, i64, i64, i64, i64, i64,
                                          ctypes.c_float, p, p, p]
    lib.det_attention_prefill.restype = ctypes.c_int
    lib.det_attention_decode_noalloc.argtypes = [p, p, p, p, i64, i64, i64, i64, i64,
                                                 ctypes.c_float, p, p]
    lib.det_attention_decode_noalloc.restype = ctypes.c_int
    lib.det_gemm_shard_reduce.argtypes = [p, i64, i64, p, i64, i64, i64, p]
    lib.det_gemm_shard_reduce.restype = ctypes.c_int
    lib.det_gemm_status_string.argtypes = [ctypes.c_int]
    lib.det_gemm_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _status_string(code):
    try:
        return load_library().det_gemm_status_string(code).decode()
    except Exception:  # library unavailable: still report the number
        return "unknown"


def _check(rc, what):
    if rc != OK:
        raise DetGemmError(rc, what)


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _mat(t, name, dtype=torch.bfloat16):
    """(pointer, leading dimension) of a 2-D tensor with unit column stride."""
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or t.dim() != 2:
        raise TypeError(f"{name} must be a 2-D {dtype} tensor")
    if not t.is_cuda:
        raise TypeError(f"{name} must be on a GPU device")
    rows, cols = t.shape
    if cols > 1 and t.stride(1) != 1:
        raise ValueError(f"{name} needs unit stride along its last dimension")
    ld = t.stride(0) if rows > 1 else max(cols, 1)
    return ctypes.c_void_p(t.data_ptr()), ld


def _same_device(*ts):
    devs = {t.device for t in ts}
    if len(devs) != 1:
        raise ValueError(f"tensors are on different devices: {sorted(map(str, devs))}")


def _out(out, shape, like, dtype, contiguous=False, name="output"):
    """A caller's output tensor, checked against what the C call will write:
    dtype, device (that of `like`), shape and, for `contiguous`, a dense
    layout (the C call then writes numel elements from its data pointer).  A
    2-D output may carry a row stride; its unit column stride is checked where
    its leading dimension is taken.  None allocates a fresh tensor."""
    if out is None:
        return torch.empty(shape, dtype=dtype, device=like.device)
    if not isinstance(out, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if out.dtype != dtype:
        raise TypeError(f"{name} must have dtype {dtype}, not {out.dtype}")
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}")
    if contiguous and not out.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if not out.is_cuda or out.device != like.device:
        raise TypeError(f"{name} must be on {like.device}")
    return out


def _call(name, P, Q, out, M, N, K, what):
    _same_device(P, Q, out)
    pp, ldp = _mat(P, "first operand")
    qp, ldq = _mat(Q, "second operand")
    op, ldo = _mat(out, "output", out.dtype)
    with torch.cuda.device(out.device):
        rc = getattr(load_library(), name)(pp, ldp, qp, ldq, op, ldo, M, N, K, _stream(out))
    _check(rc, what)
    return out


# ---------------------------------------------------------------- the six operations

def det_gemm_fwd(A, B, out=None, strict=False):
    """C[M,N] = A[M,K] @ B[K,N] (bf16 out)."""
    M, K = A.shape
    N = B.shape[1]
    if B.shape[0] != K:
        raise ValueError("A and B disagree on K")
    out = _out(out, (M, N), A, torch.bfloat16)
    return _call("det_gemm_strict_fwd" if strict else "det_gemm_fwd", A, B, out, M, N, K,
                 "det_gemm_fwd")


def det_gemm_fwd_rhs_transposed(A, Bt, out=None, strict=False):
    """C[M,N] = A[M,K] @ Bt[N,K]^T (weight in nn.Linear layout)."""
    M, K = A.shape
    N = Bt.shape[0]
    if Bt.shape[1] != K:
        raise ValueError("A and Bt disagree on K")
    out = _out(out, (M, N), A, torch.bfloat16)
    return _call("det_gemm_strict_fwd_rhs_transposed" if strict else
                 "det_gemm_fwd_rhs_transposed", A, Bt, out, M, N, K, "det_gemm_fwd_rhs_transposed")


def det_gemm_fwd_fp32(A, B, out=None, strict=False):
    """As det_gemm_fwd with the bf16 root widened to float32."""
    M, K = A.shape
    N = B.shape[1]
    if B.shape[0] != K:
        raise ValueError("A and B disagree on K")
    out = _out(out, (M, N), A, torch.float32)
    return _call("det_gemm_strict_fwd_fp32" if strict else "det_gemm_fwd_fp32", A, B, out,
                 M, N, K, "det_gemm_fwd_fp32")


def det_gemm_da(dC, B, out=None, strict=False):
    """dA[M,K] = dC[M,N] @ B[K,N]^T."""
    M, N = dC.shape
    K = B.shape[0]
    if B.shape[1] != N:
        raise ValueError("dC and B disagree on N")
    out = _out(out, (M, K), dC, torch.bfloat16)
    return _call("det_gemm_strict_da" if strict else "det_gemm_da", dC, B, out, M, N, K,
                 "det_gemm_da")


def det_gemm_db(A, dC, out=None, strict=False):
    """dB[K,N] = A[M,K]^T @ dC[M,N]."""
    M, K = A.shape
    N = dC.shape[1]
    if dC.shape[0] != M:
        raise ValueError("A and dC disagree on M")
    out = _out(out, (K, N), A, torch.bfloat16)
    return _call("det_gemm_strict_db" if strict else "det_gemm_db", A, dC, out, M, N, K,
                 "det_gemm_db")


def det_gemm_db_transposed(A, dC, out=None, strict=False):
    """dBt[N,K] = (A[M,K]^T @ dC[M,N])^T, written directly in [N,K]."""
    M, K = A.shape
    N = dC.shape[1]
    if dC.shape[0] != M:
        raise ValueError("A and dC disagree on M")
    out = _out(out, (N, K), A, torch.bfloat16)
    return _call("det_gemm_strict_db_transposed" if strict else "det_gemm_db_transposed", A, dC,
                 out, M, N, K, "det_gemm_db_transposed")


# ---------------------------------------------------------------- K-shard combination

def det_gemm_shard_reduce(parts, out=None):
    """The mid-split tree of bf16 adds over K-shard partial products in rank
    order (include/det_gemm.h): parts is a list of [M,N] bf16 GPU tensors with
    one common leading dimension."""
    if not 1 <= len(parts) <= MAX_PARTS:
        raise ValueError(f"between 1 and {MAX_PARTS} parts")
    M, N = parts[0].shape
    lds = set()
    ptrs = []
    for t in parts:
        if tuple(t.shape) != (M, N):
            raise ValueError("parts differ in shape")
        pp, ld = _mat(t, "part")
        lds.add(ld)
        ptrs.append(pp.value or 0)
    if len(lds) != 1:
        raise ValueError("parts must share one leading dimension")
    _same_device(*parts)
    out = _out(out, (M, N), parts[0], torch.bfloat16)
    op, ldo = _mat(out, "out")
    arr = (ctypes.c_void_p * len(parts))(*ptrs)
    with torch.cuda.device(out.device):
        rc = load_library().det_gemm_shard_reduce(arr, len(parts), lds.pop(), op, ldo, M, N,
                                                  _stream(out))
    _check(rc, "det_gemm_shard_reduce")
    return out


# ---------------------------------------------------------------- MoE grouped GEMM

def det_moe_fwd_dprob(X, W, offsets, G, Y=None, slots=None, dprob=None):
    """MoE grouped GEMM with the per-token slot epilogue (include/det_moe.h).

    X [T,K] bf16, rows grouped by expert (expert e owns rows offsets[e] ..
    offsets[e+1]-1); W [E,K,N] bf16 (unit stride along N); G [T,N] bf16;
    offsets: E + 1 host integers.  Returns (Y [T,N] bf16, dprob [T] float32,
    slots [ceil(N/128), T] float32): Y row r = det_gemm_fwd(X[r], W[e(r)]);
    slot j of row r and dprob[r] are fixed fp32 trees over Y[r]*G[r]."""
    T, K = X.shape
    if W.dim() != 3 or W.dtype != torch.bfloat16 or not W.is_cuda:
        raise TypeError("W must be a 3-D bfloat16 GPU tensor [E,K,N]")
    E, K2, N = W.shape
    if K2 != K or tuple(G.shape) != (T, N):
        raise ValueError("X, W and G disagree in shape")
    if N > 1 and W.stride(2) != 1:
        raise ValueError("W needs unit stride along N")
    off = [int(v) for v in offsets]
    if len(off) != E + 1:
        raise ValueError("offsets must hold E + 1 entries")
    J = (N + MOE_SLOT - 1) // MOE_SLOT
    _same_device(X, W, G)
    Y = _out(Y, (T, N), X, torch.bfloat16, name="Y")
    dprob = _out(dprob, (T,), X, torch.float32, contiguous=True, name="dprob")
    if slots is None:
        slots = torch.empty((J, T), dtype=torch.float32, device=X.device)
    if not isinstance(slots, torch.Tensor) or not slots.is_cuda or slots.device != X.device:
        raise TypeError(f"slots must be a tensor on {X.device}")
    if slots.dtype != torch.float32 or slots.dim() != 2 or slots.shape[0] != J or \
            slots.shape[1] < T or (J > 0 and T > 1 and slots.stride(1) != 1) or \
            (J > 1 and slots.stride(0) < T):
        raise ValueError("slots must be float32 [ceil(N/128), >= T] with unit column stride")
    xp, ldx = _mat(X, "X")
    gp, ldg = _mat(G, "G")
    yp, ldy = _mat(Y, "Y")
    ldw = W.stride(1) if K > 1 else max(N, 1)
    slot_ld = slots.stride(0) if J > 1 else max(T, 1)
    if not dprob.is_contiguous():
        raise ValueError("dprob must be contiguous")
    off_arr = (ctypes.c_int64 * (E + 1))(*off)
    with torch.cuda.device(X.device):
        rc = load_library().det_moe_fwd_dprob(
            xp, ldx, ctypes.c_void_p(W.data_ptr()), ldw, W.stride(0) if E > 1 else K * ldw,
            off_arr, E, gp, ldg, yp, ldy, ctypes.c_void_p(slots.data_ptr()), slot_ld,
            ctypes.c_void_p(dprob.data_ptr()), T, N, K, _stream(X))
    _check(rc, "det_moe_fwd_dprob")
    return Y, dprob, slots


def det_moe_debug_slots(Y, G, slots=None):
    """The slot writer as a kernel of its own over given Y and G: [ceil(N/128), T]."""
    T, N = Y.shape
    J = (N + MOE_SLOT - 1) // MOE_SLOT
    _same_device(Y, G)
    if slots is None:
        slots = torch.empty((J, T), dtype=torch.float32, device=Y.device)
    if not isinstance(slots, torch.Tensor) or not slots.is_cuda or slots.device != Y.device:
        raise TypeError(f"slots must be a tensor on {Y.device}")
    if slots.dtype != torch.float32 or slots.dim() != 2 or slots.shape[0] != J or \
            slots.shape[1] < T or (J > 0 and T > 1 and slots.stride(1) != 1) or \
            (J > 1 and slots.stride(0) < T):
        raise ValueError("slots must be float32 [ceil(N/128), >= T] with unit column stride")
    yp, ldy = _mat(Y, "Y")
    gp, ldg = _mat(G, "G")
    slot_ld = slots.stride(0) if J > 1 else max(T, 1)
    with torch.cuda.device(Y.device):
        rc = load_library().det_moe_debug_slots(yp, ldy, gp, ldg,
                                                ctypes.c_void_p(slots.data_ptr()), slot_ld, T, N,
                                                _stream(Y))
    _check(rc, "det_moe_debug_slots")
    return slots


# ---------------------------------------------------------------- RMSNorm

def det_rmsnorm(x, w, eps=1e-6, out=None, rstd=None):
    """Batch-invariant RMSNorm (include/det_norm.h): x [R,H] bf16, w [H] bf16.
    Returns (y [R,H] bf16, rstd [R] float32)."""
    R, H = x.shape
    if w.dim() != 1 or w.shape[0] != H or w.dtype != torch.bfloat16 or not w.is_contiguous():
        raise ValueError("w must be a contiguous bf16 vector of H entries")
    _same_device(x, w)
    out = _out(out, (R, H), x, torch.bfloat16, name="out")
    rstd = _out(rstd, (R,), x, torch.float32, contiguous=True, name="rstd")
    xp, ldx = _mat(x, "x")
    yp, ldy = _mat(out, "y")
    with torch.cuda.device(x.device):
        rc = load_library().det_rmsnorm(xp, ldx, ctypes.c_void_p(w.data_ptr()), ctypes.c_float(eps),
                                        yp, ldy, ctypes.c_void_p(rstd.data_ptr() if R else 0), R,
                                        H, _stream(x))
    _check(rc, "det_rmsnorm")
    return out, rstd


# ---------------------------------------------------------------- decode attention

def det_attention_decode(q, k, v, lens, scale, out=None, work=None):
    """Decode attention with fixed 256-position splits (include/det_attention.h):
    q [B,Hq,128], k and v [B,Hkv,Smax,128] bf16 (contiguous), lens [B] int32 on
    the device.  Returns o [B,Hq,128] bf16."""
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous bf16 GPU tensor")
    B, Hq, D = q.shape
    _, Hkv, Smax, D2 = k.shape
    if tuple(v.shape) != tuple(k.shape) or D2 != D or k.shape[0] != B:
        raise ValueError("q, k, v disagree in shape")
    if lens.dtype != torch.int32 or not lens.is_cuda or tuple(lens.shape) != (B,):
        raise TypeError("lens must be an int32 GPU tensor [B]")
    NS = (Smax + ATTN_SPLIT - 1) // ATTN_SPLIT
    _same_device(q, k, v, lens)
    out = _out(out, (B, Hq, D), q, torch.bfloat16, contiguous=True, name="out")
    need = B * Hq * NS * (D + 2)
    if work is None:
        work = torch.empty((max(need, 1),), dtype=torch.float32, device=q.device)
    if not isinstance(work, torch.Tensor) or work.dtype != torch.float32 or not work.is_cuda or \
            work.device != q.device or not work.is_contiguous():
        raise TypeError(f"work must be a contiguous float32 tensor on {q.device}")
    if work.numel() < need:
        raise ValueError(f"work must hold at least {need} floats")
    ptr = lambda t: ctypes.c_void_p(t.data_ptr() if t.numel() else 0)
    with torch.cuda.device(q.device):
        rc = load_library().det_attention_decode(ptr(q), ptr(k), ptr(v), ptr(lens), B, Hq, Hkv,
                                                 Smax, D, ctypes.c_float(scale), ptr(work),
                                                 ptr(out), _stream(q))
    _check(rc, "det_attention_decode")
    return out


def det_attention_prefill(q, k, v, row_offsets, lens, scale, out=None, work=None):
    """Chunked prefill with the decode arithmetic (include/det_attention.h):
    q [NQ,Hq,128] query rows grouped by sequence (rows of sequence b:
    row_offsets[b] .. row_offsets[b+1]-1, host integers), k and v
    [B,Hkv,Smax,128] bf16 (contiguous), lens [NQ] int32 on the device (keys
    each row attends).  Returns o [NQ,Hq,128] bf16: row r equals what
    det_attention_decode returns for its query with length lens[r]."""
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous bf16 GPU tensor")
    NQ, Hq, D = q.shape
    B, Hkv, Smax, D2 = k.shape
    if tuple(v.shape) != tuple(k.shape) or D2 != D:
        raise ValueError("q, k, v disagree in shape")
    off = [int(x) for x in row_offsets]
    if len(off) != B + 1:
        raise ValueError("row_offsets must hold B + 1 entries")
    if lens.dtype != torch.int32 or not lens.is_cuda or tuple(lens.shape) != (NQ,):
        raise TypeError("lens must be an int32 GPU tensor [NQ]")
    _same_device(q, k, v, lens)
    NS = (Smax + ATTN_SPLIT - 1) // ATTN_SPLIT
    out = _out(out, (NQ, Hq, D), q, torch.bfloat16, contiguous=True, name="out")
    need = NQ * Hq * NS * (D + 2)
    if work is None:
        work = torch.empty((max(need, 1),), dtype=torch.float32, device=q.device)
    if not isinstance(work, torch.Tensor) or work.dtype != torch.float32 or not work.is_cuda or \
            work.device != q.device or not work.is_contiguous():
        raise TypeError(f"work must be a contiguous float32 tensor on {q.device}")
    if work.numel() < need:
        raise ValueError(f"work must hold at least {need} floats")
    ptr = lambda t: ctypes.c_void_p(t.data_ptr() if t.numel() else 0)
    off_arr = (ctypes.c_int64 * (B + 1))(*off)
    with torch.cuda.device(q.device):
        rc = load_library().det_attention_prefill(ptr(q), ptr(k), ptr(v), off_arr, ptr(lens), NQ,
                                                  B, Hq, Hkv, Smax, D, ctypes.c_float(scale),
                                                  ptr(work), ptr(out), _stream(q))
    _check(rc, "det_attention_prefill")
    return out


def det_attention_decode_noalloc(q, k, v, lens, scale, out):
    """det_attention_decode without a work buffer (include/det_attention.h):
    the library keeps the per-split partials in a fixed device array, so the C
    call allocates nothing.  `out` [B,Hq,128] bf16 is required; calls that can
    overlap on one device race on the shared array."""
    for t, name in ((q, "q"), (k, "k"), (v, "v")):
        if t.dtype != torch.bfloat16 or not t.is_cuda or not t.is_contiguous():
            raise TypeError(f"{name} must be a contiguous bf16 GPU tensor")
    B, Hq, D = q.shape
    _, Hkv, Smax, D2 = k.shape
    if tuple(v.shape) != tuple(k.shape) or D2 != D or k.shape[0] != B:
        raise ValueError("q, k, v disagree in shape")
    if lens.dtype != torch.int32 or not lens.is_cuda or tuple(lens.shape) != (B,):
        raise TypeError("lens must be an int32 GPU tensor [B]")
    if out is None:
        raise ValueError("out is required: this entry point allocates nothing")
    _same_device(q, k, v, lens)
    out = _out(out, (B, Hq, D), q, torch.bfloat16, contiguous=True, name="out")
    ptr = lambda t: ctypes.c_void_p(t.data_ptr() if t.numel() else 0)
    with torch.cuda.device(q.device):
        rc = load_library().det_attention_decode_noalloc(ptr(q), ptr(k), ptr(v), ptr(lens), B, Hq,
                                                         Hkv, Smax, D, ctypes.c_float(scale),
                                                         ptr(out), _stream(q))
    _check(rc, "det_attention_decode_noalloc")
    return out


# ---------------------------------------------------------------- fingerprints

def _bytes_of(t, name):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (its bytes are hashed in order)")
    return ctypes.c_void_p(t.data_ptr() if t.numel() else 0), t.numel() * t.element_size()


def det_fingerprint(t, out=None):
    """64-bit digest of the bytes of a contiguous GPU tensor (include/
    det_fingerprint.h); returned in an int64 device tensor [1] holding its bits."""
    p, n = _bytes_of(t, "t")
    out = _out(out, (1,), t, torch.int64, contiguous=True)
    with torch.cuda.device(t.device):
        rc = load_library().det_fingerprint(p, n, ctypes.c_void_p(out.data_ptr()), _stream(t))
    _check(rc, "det_fingerprint")
    return out


def det_fingerprint_rows(t, out=None):
    """One digest per row of a 2-D GPU tensor with unit column stride (row r =
    the bytes of t[r]); int64 device tensor [rows] holding the digest bits."""
    if not isinstance(t, torch.Tensor) or t.dim() != 2 or not t.is_cuda:
        raise TypeError("t must be a 2-D GPU tensor")
    rows, cols = t.shape
    if cols > 1 and t.stride(1) != 1:
        raise ValueError("t needs unit stride along its last dimension")
    es = t.element_size()
    ld = t.stride(0) * es if rows > 1 else cols * es
    out = _out(out, (rows,), t, torch.int64, contiguous=True)
    with torch.cuda.device(t.device):
        rc = load_library().det_fingerprint_rows(
            ctypes.c_void_p(t.data_ptr() if t.numel() else 0), rows, cols * es, ld,
            ctypes.c_void_p(out.data_ptr() if rows else 0), _stream(t))
    _check(rc, "det_fingerprint_rows")
    return out


def det_first_mismatch(a, b, out=None):
    """Smallest byte index where the bytes of two contiguous GPU tensors differ,
    or -1; int64 device tensor [1]."""
    pa, na = _bytes_of(a, "a")
    pb, nb = _bytes_of(b, "b")
    if na != nb:
        raise ValueError("a and b differ in byte length")
    _same_device(a, b)
    out = _out(out, (1,), a, torch.int64, contiguous=True)
    with torch.cuda.device(a.device):
        rc = load_library().det_first_mismatch(pa, pb, na, ctypes.c_void_p(out.data_ptr()),
                                               _stream(a))
    _check(rc, "det_first_mismatch")
    return out


def digest_value(d):
    """The unsigned 64-bit digest held in an int64 tensor element."""
    return int(d.reshape(-1)[0].item()) & (2**64 - 1)


# ---------------------------------------------------------------- inspection

def det_gemm_debug_leaves(A, B):
    """The MFMA forward kernel's bf16 leaves, [M, N, ceil(K/32)]."""
    M, K = A.shape
    N = B.shape[1]
    L = (K + LEAF - 1) // LEAF
    out = torch.empty((M, N, L), dtype=torch.bfloat16, device=A.device)
    ap, lda = _mat(A, "A")
    bp, ldb = _mat(B, "B")
    with torch.cuda.device(A.device):
        rc = load_library().det_gemm_debug_leaves(ap, lda, bp, ldb, ctypes.c_void_p(out.data_ptr()),
                                                  M, N, K, _stream(A))
    _check(rc, "det_gemm_debug_leaves")
    return out


def det_gemm_debug_round(x):
    """Device bf16 rounding of a float32 tensor (as the MFMA kernel rounds)."""
    x = x.contiguous()
    out = torch.empty(x.shape, dtype=torch.bfloat16, device=x.device)
    with torch.cuda.device(x.device):
        rc = load_library().det_gemm_debug_round(ctypes.c_void_p(x.data_ptr()),
                                                 ctypes.c_void_p(out.data_ptr()), x.numel(),
                                                 _stream(x))
    _check(rc, "det_gemm_debug_round")
    return out


def det_gemm_debug_add(a, b):
    """Device bf16 add of two bf16 tensors (as the MFMA kernel merges nodes)."""
    a, b = a.contiguous(), b.contiguous()
    if a.shape != b.shape or a.dtype != torch.bfloat16 or b.dtype != torch.bfloat16:
        raise TypeError("a and b must be bf16 tensors of one shape")
    out = torch.empty_like(a)
    with torch.cuda.device(a.device):
        rc = load_library().det_gemm_debug_add(ctypes.c_void_p(a.data_ptr()),
                                               ctypes.c_void_p(b.data_ptr()),
                                               ctypes.c_void_p(out.data_ptr()), a.numel(),
                                               _stream(a))
    _check(rc, "det_gemm_debug_add")
    return out


def det_gemm_debug_matrix_add(a, b, selector=0):
    """Device bf16 add of two bf16 tensors as the matrix-core kernels merge
    tree nodes (selector 0: wide and direct-to-LDS kernels; 1: general kernel)."""
    a, b = a.contiguous(), b.contiguous()
    if a.shape != b.shape or a.dtype != torch.bfloat16 or b.dtype != torch.bfloat16:
        raise TypeError("a and b must be bf16 tensors of one shape")
    _same_device(a, b)
    out = torch.empty_like(a)
    with torch.cuda.device(a.device):
        rc = load_library().det_gemm_debug_matrix_add(ctypes.c_void_p(a.data_ptr()),
                                                      ctypes.c_void_p(b.data_ptr()),
                                                      ctypes.c_void_p(out.data_ptr()), a.numel(),
                                                      int(selector), _stream(a))
    _check(rc, "det_gemm_debug_matrix_add")
    return out


def det_gemm_debug_issue_probe(mode, iters, sink):
    """Launch the issue-rate probe on the current stream of sink's device:
    mode 0 the MFMAs of one wide-kernel stage alone, 1 the stage's MFMAs and
    conversions; one workgroup per 512 elements of `sink` (contiguous float32,
    overwritten)."""
    if sink.dtype != torch.float32 or not sink.is_contiguous() or sink.numel() < 512:
        raise TypeError("sink must be a contiguous float32 tensor of at least 512 elements")
    if sink.device.type != "cuda":
        raise ValueError("sink must be a device tensor")
    with torch.cuda.device(sink.device):
        rc = load_library().det_gemm_debug_issue_probe(int(mode), int(iters), sink.numel() // 512,
                                                       ctypes.c_void_p(sink.data_ptr()), _stream(sink))
    _check(rc, "det_gemm_debug_issue_probe")


OP_FWD, OP_FWD_RHS_TRANSPOSED, OP_FWD_FP32, OP_DA, OP_DB, OP_DB_TRANSPOSED = range(6)


def det_gemm_debug_config(op, p, ldp, q, ldq, out, ldo, M, N, K):
    """The tile configuration the MFMA entry point of `op` (OP_FWD ...) would
    run for these arguments (addresses as integers, never dereferenced; no
    device needed)."""
    rc = load_library().det_gemm_debug_config(int(op), ctypes.c_void_p(p), ldp, ctypes.c_void_p(q),
                                               ldq, ctypes.c_void_p(out), ldo, M, N, K)
    if rc < 0:
        raise DetGemmError(rc, "det_gemm_debug_config")
    return rc


def det_gemm_debug_force_config(config):
    """Pin the MFMA tile configuration (-1 restores automatic selection).
    Returns the number of configurations."""
    rc = load_library().det_gemm_debug_force_config(int(config))
    if rc < 0:
        raise DetGemmError(rc, "det_gemm_debug_force_config")
    return rc
