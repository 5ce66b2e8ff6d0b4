"""Independent brute force for tiny det_gemm cases, in exact rational arithmetic.

Used only to pin the C oracle.  It does not use hardware floating point at all:
every value is a ``fractions.Fraction`` and every rounding is done here from
the definition of a binary floating-point format (precision p, minimum normal
exponent, overflow to infinity, round to nearest with ties to even).

Contract followed (RL-Kernel operator page "Batch-Invariant Deterministic GEMM
(det_gemm)", section "Ascend NPU backend", bullet "Reduction tree"): fp32 leaves
of 32 products added in ascending order, each leaf rounded once to bf16, leaves
joined by the mid-split tree of bf16 adds.  Here a tree add is the *exact* sum
rounded once to bf16 (the correctly rounded bf16 add), not fp32-then-bf16 as in
the oracle; the two agree because fp32 carries more than 2*8+2 bits (double
rounding is then innocuous), so agreement also checks that claim.
"""
from fractions import Fraction
import struct

INF = float("inf")


class Fmt:
    def __init__(self, p, emin, emax):
        self.p, self.emin, self.emax = p, emin, emax


FP32 = Fmt(24, -126, 127)
BF16 = Fmt(8, -126, 127)


def _floor_log2(q):
    """floor(log2(q)) for a positive Fraction."""
    n, d = q.numerator, q.denominator
    e = n.bit_length() - d.bit_length()
    # adjust so that 2^e <= q < 2^(e+1)
    if e >= 0:
        if n < (d << e):
            e -= 1
    else:
        if (n << -e) < d:
            e -= 1
    return e


def round_to(q, fmt):
    """Round an exact value (Fraction, or +-inf) to ``fmt``, nearest-even.

    Returns a Fraction or +-inf.  Zero keeps no sign here (callers that need a
    signed zero track it themselves)."""
    if q in (INF, -INF):
        return q
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = -q if q < 0 else q
    e = max(_floor_log2(a), fmt.emin)
    ulp = Fraction(2) ** (e - fmt.p + 1)
    m = a / ulp
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    if r >= Fraction(2) ** (fmt.emax + 1):
        return sign * INF
    return sign * r


def bf16_value(h):
    """bf16 bit pattern -> Fraction (finite) or +-inf; NaN is not supported."""
    f = struct.unpack("<f", struct.pack("<I", (int(h) & 0xFFFF) << 16))[0]
    if f != f:
        raise ValueError("NaN input")
    if f in (INF, -INF):
        return f
    return Fraction(f)


def bf16_bits(v):
    """Fraction/inf that is exactly a bf16 value -> its bit pattern (+0 for zero)."""
    if v == INF:
        return 0x7F80
    if v == -INF:
        return 0xFF80
    f = float(v)
    u = struct.unpack("<I", struct.pack("<f", f))[0]
    assert u & 0xFFFF == 0, "value is not a bf16"
    return u >> 16


def _add(a, b):
    """Exact sum; an infinite operand wins (inf - inf is not supported)."""
    if a in (INF, -INF) or b in (INF, -INF):
        if a in (INF, -INF) and b in (INF, -INF) and a != b:
            raise ValueError("inf - inf")
        return a if a in (INF, -INF) else b
    return a + b


def leaf(xs, ys):
    """One leaf: exact products (finite inputs) added in order into an fp32 sum
    that starts at 0, then rounded once to bf16."""
    s = Fraction(0)
    for x, y in zip(xs, ys):
        s = round_to(_add(s, x * y), FP32)
    return round_to(s, BF16)


def tree(leaves, lo, hi):
    if hi - lo == 1:
        return leaves[lo]
    mid = lo + (hi - lo) // 2
    return round_to(_add(tree(leaves, lo, mid), tree(leaves, mid, hi)), BF16)


def dot(xbits, ybits):
    """det_gemm value of one output element from its two length-R bf16 vectors."""
    R = len(xbits)
    xs = [bf16_value(h) for h in xbits]
    ys = [bf16_value(h) for h in ybits]
    leaves = [leaf(xs[r:r + 32], ys[r:r + 32]) for r in range(0, R, 32)]
    return bf16_bits(tree(leaves, 0, len(leaves)))


def matmul(Abits, Bbits):
    """C[M,N] = A[M,K] @ B[K,N] on nested lists/arrays of bf16 bit patterns."""
    M, K = len(Abits), len(Abits[0])
    N = len(Bbits[0])
    return [[dot([Abits[i][r] for r in range(K)], [Bbits[r][j] for r in range(K)])
             for j in range(N)] for i in range(M)]
