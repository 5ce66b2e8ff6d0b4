"""CPU oracle for det_gemm -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct implementation of what the RL-Kernel operator
page "Batch-Invariant Deterministic GEMM (det_gemm)" specifies (sections
"Guarantees" and "Ascend NPU backend"): 32-element fp32 leaves summed in
ascending order and rounded once to bf16 (round-to-nearest-even), merged by the
mid-split tree of bf16 adds, reduction length capped at 32768.  The arithmetic
lives in ``det_gemm_oracle.c``; this module only marshals numpy arrays.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
and never imports it.

bf16 data are numpy ``uint16`` arrays holding the bit patterns.  2-D operands
need a unit stride along their last axis; any row stride is accepted and is
passed on as the leading dimension.

Pins (see ``tests/test_oracle_*.py``): exhaustive fp32->bf16 rounding against
torch's conversion; the bf16 add against exact rational arithmetic; hand-derived
leaf-order and tree-shape cases in ``tests/golden/``; exact equality with int64
matrix products in the integer regime, for all six operations; an independent
exact-rational brute force on tiny shapes; the half-K identity; a forward error
bound against float64.  Parity unpinned (fixed by reading, locked by tests):
the odd-split direction, the fp32-output reading, the backward invariance
reading.

The MoE grouped GEMM's per-token epilogue (reading notes on bitwise-
deterministic pretraining in Megatron Core, section "Kernel redesign: the
grouped-GEMM epilogue") is pinned in ``tests/test_oracle_moe.py``: exact
integer dot products and expert routing, hand-derived tree-shape and
signed-zero cases in ``tests/golden/moe_cases.txt``, and the float64 sum within
the pairwise-summation error bound.  Parity unpinned (fixed by reading): the
slot width of 128 columns, fp32 adds, the two tree shapes.
"""
import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

MAX_R = 32768
LEAF = 32

_ERRORS = {-1: "invalid argument", -2: "reduction length must be in [1, 32768]",
           -4: "out of host memory"}


class OracleError(RuntimeError):
    def __init__(self, code):
        super().__init__(f"oracle error {code}: {_ERRORS.get(code, 'unknown')}")
        self.code = code


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            from . import build as _b
            _b.build(force=False)
        lib = ctypes.CDLL(_LIB_PATH)
        p, i64 = ctypes.c_void_p, ctypes.c_int64
        for name in ("oracle_det_gemm_fwd", "oracle_det_gemm_fwd_rhs_transposed",
                     "oracle_det_gemm_fwd_fp32", "oracle_det_gemm_da", "oracle_det_gemm_db",
                     "oracle_det_gemm_db_transposed"):
            f = getattr(lib, name)
            f.argtypes = [p, i64, p, i64, p, i64, i64, i64, i64]
            f.restype = ctypes.c_int
        lib.oracle_det_gemm_fwd_detail.argtypes = [p, i64, p, i64, p, i64, i64, i64, i64, p, p]
        lib.oracle_det_gemm_fwd_detail.restype = ctypes.c_int
        lib.oracle_tree_from_leaves.argtypes = [p, i64, i64, p, p]
        lib.oracle_tree_from_leaves.restype = ctypes.c_int
        lib.oracle_round_bf16_array.argtypes = [p, p, i64]
        lib.oracle_round_bf16_array.restype = None
        lib.oracle_add_bf16_array.argtypes = [p, p, p, i64]
        lib.oracle_add_bf16_array.restype = None
        lib.oracle_moe_dprob.argtypes = [p, i64, p, i64, i64, i64, p, i64, p]
        lib.oracle_moe_dprob.restype = ctypes.c_int
        lib.oracle_moe_fwd_dprob.argtypes = [p, i64, p, i64, i64, p, i64, p, i64, p, i64, p, i64,
                                             p, i64, i64, i64]
        lib.oracle_moe_fwd_dprob.restype = ctypes.c_int
        u64 = ctypes.c_uint64
        lib.oracle_mix64.argtypes = [u64]
        lib.oracle_mix64.restype = u64
        lib.oracle_fingerprint.argtypes = [p, i64, p]
        lib.oracle_fingerprint.restype = ctypes.c_int
        lib.oracle_fingerprint_rows.argtypes = [p, i64, i64, i64, p]
        lib.oracle_fingerprint_rows.restype = ctypes.c_int
        lib.oracle_first_mismatch.argtypes = [p, p, i64]
        lib.oracle_first_mismatch.restype = i64
        lib.oracle_rmsnorm.argtypes = [p, i64, p, ctypes.c_float, p, i64, p, p, i64, i64]
        lib.oracle_rmsnorm.restype = ctypes.c_int
        lib.oracle_num_threads.argtypes = []
        lib.oracle_num_threads.restype = ctypes.c_int
        _lib = lib
    return _lib


def _mat(a, name):
    a = np.asarray(a)
    if a.dtype != np.uint16 or a.ndim != 2:
        raise TypeError(f"{name} must be a 2-D uint16 (bf16 bit pattern) array")
    if a.shape[1] > 1 and a.strides[1] != 2:
        a = np.ascontiguousarray(a)
    if a.shape[0] > 1 and (a.strides[0] <= 0 or a.strides[0] % 2):
        a = np.ascontiguousarray(a)
    ld = a.strides[0] // 2 if a.shape[0] > 1 else max(a.shape[1], 1)
    return a, ld


def _ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc):
    if rc != 0:
        raise OracleError(rc)


def fwd(A, B):
    """C[M,N] = A[M,K] @ B[K,N] under the leaf/tree contract (bf16 out)."""
    A, lda = _mat(A, "A")
    B, ldb = _mat(B, "B")
    (M, K), (K2, N) = A.shape, B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    C = np.zeros((M, N), np.uint16)
    _check(_load().oracle_det_gemm_fwd(_ptr(A), lda, _ptr(B), ldb, _ptr(C), max(N, 1), M, N, K))
    return C


def fwd_rhs_transposed(A, Bt):
    """C[M,N] = A[M,K] @ Bt[N,K]^T (weight in [N,K] layout)."""
    A, lda = _mat(A, "A")
    Bt, ldbt = _mat(Bt, "Bt")
    (M, K), (N, K2) = A.shape, Bt.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    C = np.zeros((M, N), np.uint16)
    _check(_load().oracle_det_gemm_fwd_rhs_transposed(_ptr(A), lda, _ptr(Bt), ldbt, _ptr(C),
                                                      max(N, 1), M, N, K))
    return C


def fwd_fp32(A, B):
    """As :func:`fwd`, returning the bf16 root widened to float32."""
    A, lda = _mat(A, "A")
    B, ldb = _mat(B, "B")
    (M, K), (K2, N) = A.shape, B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    C = np.zeros((M, N), np.float32)
    _check(_load().oracle_det_gemm_fwd_fp32(_ptr(A), lda, _ptr(B), ldb, _ptr(C), max(N, 1),
                                            M, N, K))
    return C


def da(dC, B):
    """dA[M,K] = dC[M,N] @ B[K,N]^T (reduction over N)."""
    dC, lddc = _mat(dC, "dC")
    B, ldb = _mat(B, "B")
    (M, N), (K, N2) = dC.shape, B.shape
    if N != N2:
        raise ValueError("dC and B disagree on N")
    dA = np.zeros((M, K), np.uint16)
    _check(_load().oracle_det_gemm_da(_ptr(dC), lddc, _ptr(B), ldb, _ptr(dA), max(K, 1),
                                      M, N, K))
    return dA


def db(A, dC):
    """dB[K,N] = A[M,K]^T @ dC[M,N] (reduction over M)."""
    A, lda = _mat(A, "A")
    dC, lddc = _mat(dC, "dC")
    (M, K), (M2, N) = A.shape, dC.shape
    if M != M2:
        raise ValueError("A and dC disagree on M")
    dB = np.zeros((K, N), np.uint16)
    _check(_load().oracle_det_gemm_db(_ptr(A), lda, _ptr(dC), lddc, _ptr(dB), max(N, 1),
                                      M, N, K))
    return dB


def db_transposed(A, dC):
    """dBt[N,K] = (A[M,K]^T @ dC[M,N])^T, written in [N,K] layout."""
    A, lda = _mat(A, "A")
    dC, lddc = _mat(dC, "dC")
    (M, K), (M2, N) = A.shape, dC.shape
    if M != M2:
        raise ValueError("A and dC disagree on M")
    dBt = np.zeros((N, K), np.uint16)
    _check(_load().oracle_det_gemm_db_transposed(_ptr(A), lda, _ptr(dC), lddc, _ptr(dBt),
                                                 max(K, 1), M, N, K))
    return dBt


def fwd_detail(A, B, with_leaves=True):
    """Forward product plus every element's leaves [M,N,L] (None when
    with_leaves is false, for products too large to keep them) and the largest
    node magnitude of its tree [M,N] (float32)."""
    A, lda = _mat(A, "A")
    B, ldb = _mat(B, "B")
    (M, K), (K2, N) = A.shape, B.shape
    if K != K2:
        raise ValueError("inner dimensions differ")
    L = max((K + LEAF - 1) // LEAF, 1)
    C = np.zeros((M, N), np.uint16)
    leaves = np.zeros((M, N, L), np.uint16) if with_leaves else None
    big = np.zeros((M, N), np.float32)
    _check(_load().oracle_det_gemm_fwd_detail(_ptr(A), lda, _ptr(B), ldb, _ptr(C), max(N, 1),
                                              M, N, K, _ptr(leaves) if with_leaves else None,
                                              _ptr(big)))
    return C, leaves, big


def tree_from_leaves(leaves):
    """Applies the mid-split bf16 tree to the last axis of ``leaves``; returns
    (roots, largest node magnitude) with the leading shape of ``leaves``."""
    lv = np.ascontiguousarray(np.asarray(leaves, dtype=np.uint16))
    L = lv.shape[-1]
    flat = lv.reshape(-1, L)
    out = np.zeros(flat.shape[0], np.uint16)
    big = np.zeros(flat.shape[0], np.float32)
    _check(_load().oracle_tree_from_leaves(_ptr(flat), flat.shape[0], L, _ptr(out), _ptr(big)))
    return out.reshape(lv.shape[:-1]), big.reshape(lv.shape[:-1])


def round_bf16(x):
    """fp32 -> bf16 bit patterns, round to nearest even (element-wise)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    out = np.empty(x.shape, np.uint16)
    _load().oracle_round_bf16_array(_ptr(x), _ptr(out), x.size)
    return out


def add_bf16(a, b):
    """The tree's bf16 add, element-wise over bit-pattern arrays."""
    a = np.ascontiguousarray(np.asarray(a, dtype=np.uint16))
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    if a.shape != b.shape:
        raise ValueError("shape mismatch")
    out = np.empty(a.shape, np.uint16)
    _load().oracle_add_bf16_array(_ptr(a), _ptr(b), _ptr(out), a.size)
    return out


SLOT = 128


def moe_dprob(Y, G):
    """Per-token reduction epilogue of the MoE grouped GEMM: for Y, G [T,N]
    (bf16 bit patterns) returns (slots [J,T] float32, dprob [T] float32) with
    J = ceil(N/128): slot j of row r is the mid-split fp32 tree over the 128
    column positions of columns [128j, 128j+128) of Y[r]*G[r] (+0 past N), and
    dprob[r] the mid-split fp32 tree over the J slots of row r."""
    Y, ldy = _mat(Y, "Y")
    G, ldg = _mat(G, "G")
    if Y.shape != G.shape:
        raise ValueError("Y and G differ in shape")
    T, N = Y.shape
    J = (N + SLOT - 1) // SLOT
    slots = np.zeros((J, T), np.float32)
    dprob = np.zeros(T, np.float32)
    _check(_load().oracle_moe_dprob(_ptr(Y), ldy, _ptr(G), ldg, T, N, _ptr(slots), max(T, 1),
                                    _ptr(dprob)))
    return slots, dprob


def moe_fwd_dprob(X, W, offsets, G):
    """The MoE grouped GEMM with its per-token epilogue: X [T,K] with rows grouped
    by expert (expert e owns rows offsets[e]..offsets[e+1]), W [E,K,N], G [T,N].
    Returns (Y [T,N] bf16 bits, slots [J,T], dprob [T])."""
    X, ldx = _mat(X, "X")
    G, ldg = _mat(G, "G")
    W = np.ascontiguousarray(np.asarray(W))
    if W.dtype != np.uint16 or W.ndim != 3:
        raise TypeError("W must be a 3-D uint16 array [E,K,N]")
    E, K, N = W.shape
    T = X.shape[0]
    off = np.ascontiguousarray(np.asarray(offsets, dtype=np.int64))
    if off.shape != (E + 1,) or X.shape[1] != K or G.shape != (T, N):
        raise ValueError("shape mismatch")
    J = (N + SLOT - 1) // SLOT
    Y = np.zeros((T, N), np.uint16)
    slots = np.zeros((J, T), np.float32)
    dprob = np.zeros(T, np.float32)
    _check(_load().oracle_moe_fwd_dprob(_ptr(X), ldx, _ptr(W), max(N, 1), K * N, _ptr(off), E,
                                        _ptr(G), ldg, _ptr(Y), max(N, 1), _ptr(slots), max(T, 1),
                                        _ptr(dprob), T, N, K))
    return Y, slots, dprob


def _bytes(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint8).reshape(-1)


def mix64(z):
    """SplitMix64's 64-bit finalizer (the digest's mixer)."""
    return int(_load().oracle_mix64(ctypes.c_uint64(int(z) & (2**64 - 1))))


def fingerprint(a):
    """64-bit digest of the bytes of array ``a`` (C order): mix(S + n) with
    S = sum of mix(w_i + GAMMA*(i+1)) over its little-endian 64-bit words."""
    b = _bytes(a)
    out = np.zeros(1, np.uint64)
    _check(_load().oracle_fingerprint(_ptr(b), b.size, _ptr(out)))
    return int(out[0])


def fingerprint_rows(a):
    """One digest per row of a 2-D array (the bytes of each row)."""
    a = np.ascontiguousarray(a)
    if a.ndim != 2:
        raise ValueError("2-D array expected")
    rows, row_bytes = a.shape[0], a.shape[1] * a.itemsize
    out = np.zeros(rows, np.uint64)
    _check(_load().oracle_fingerprint_rows(_ptr(a), rows, row_bytes, max(row_bytes, 1), _ptr(out)))
    return out


def first_mismatch(a, b):
    """Smallest byte index where the bytes of a and b differ, or -1."""
    x, y = _bytes(a), _bytes(b)
    if x.size != y.size:
        raise ValueError("byte lengths differ")
    return int(_load().oracle_first_mismatch(_ptr(x), _ptr(y), x.size))


def rmsnorm(x, w, eps):
    """Batch-invariant RMSNorm of the rows of x [R,H] (bf16 bits) with weight w
    [H]: returns (y [R,H] bf16 bits, rstd [R] float32, sum of squares [R]
    float32).  Lane t of 256 sums the squares of its 8-element chunks (chunk c
    belongs to lane c mod 256) in ascending order; the lanes are joined by the
    pairwise tree; rstd = 1/sqrt(ss/H + eps); y = bf16((x*rstd)*w)."""
    x, ldx = _mat(x, "x")
    w = np.ascontiguousarray(np.asarray(w, dtype=np.uint16)).reshape(-1)
    R, H = x.shape
    if w.size != H:
        raise ValueError("w must have H entries")
    y = np.zeros((R, H), np.uint16)
    rstd = np.zeros(R, np.float32)
    ss = np.zeros(R, np.float32)
    _check(_load().oracle_rmsnorm(_ptr(x), ldx, _ptr(w), ctypes.c_float(eps), _ptr(y), max(H, 1),
                                  _ptr(rstd), _ptr(ss), R, H))
    return y, rstd, ss


def num_threads():
    """Host threads the oracle's parallel loops use."""
    return int(_load().oracle_num_threads())
