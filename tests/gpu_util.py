"""Helpers shared by the GPU tests: device handles, bit views and the
bf16 distance measures used by the tolerance checks."""
import sys

import numpy as np
import pytest
import torch

import det_workloads as W


def device():
    if not torch.cuda.is_available():
        pytest.skip("no GPU device")
    return torch.device("cuda:0")


def say(*args):
    """Name the case before GPU work, flushed, so a failed run still shows it."""
    print("[case]", *args, flush=True)
    sys.stdout.flush()


def bits(t):
    return W.bits(t)


def dev_bits(a, dev):
    return W.from_bits(a, dev)


def bf16_value(h):
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ordinal(h):
    """Monotone integer image of bf16 patterns (+0 and -0 both map to 0)."""
    h = np.asarray(h, np.int64)
    mag = h & 0x7FFF
    return np.where(h & 0x8000, -mag, mag)


def ulp_distance(a, b):
    return np.abs(ordinal(a) - ordinal(b))


def bf16_spacing(x):
    """Distance between consecutive bf16 numbers at magnitude x (fp64)."""
    x = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(x, 2.0 ** -126)))
    return 2.0 ** (e - 7)


def tolerance_report(got, want, big):
    """Compare MFMA-path output bits with the oracle's.

    got, want: bf16 bit patterns; big: the oracle's largest node magnitude per
    element.  Returns (histogram of ulp distances {0,1,2,>2}, count of elements
    beyond 2 bf16 spacings of the largest node, worst ratio)."""
    d = ulp_distance(got, want)
    hist = {0: int((d == 0).sum()), 1: int((d == 1).sum()), 2: int((d == 2).sum()),
            ">2": int((d > 2).sum())}
    err = np.abs(bf16_value(got) - bf16_value(want))
    lim = 2.0 * bf16_spacing(big)
    beyond = int((err > lim).sum())
    ratio = float(np.max(err / lim)) if err.size else 0.0
    return hist, beyond, ratio


def leaf_bound_ok(lg, lv, x_bits, y_bits):
    """Device leaves lg against the oracle's lv ([M, N, L] bf16 patterns) for
    operands x [M, K], y [K, N] (bf16 patterns): each side is the exact leaf
    sum plus at most 31 (sequential) or 32 (any order) fp32 roundings of
    partial sums, then one bf16 rounding, so
    |leaf_gpu - leaf_oracle| <= spacing(max |leaf|) + 64 * 2^-24 * sum_r |x_r y_r|.
    Returns (all within the bound, max ulp distance)."""
    M, K = x_bits.shape
    N = y_bits.shape[1]
    Lk = (K + 31) // 32
    x = np.zeros((M, Lk * 32))
    x[:, :K] = bf16_value(x_bits)
    y = np.zeros((Lk * 32, N))
    y[:K] = bf16_value(y_bits)
    x, y = x.reshape(M, Lk, 32), y.reshape(Lk, 32, N)
    mag = np.einsum("mlk,lkn->mnl", np.abs(x), np.abs(y))
    lgv, lvv = bf16_value(lg), bf16_value(lv)
    lim = bf16_spacing(np.maximum(np.abs(lgv), np.abs(lvv))) + 64 * 2.0 ** -24 * mag
    return bool((np.abs(lgv - lvv) <= lim).all()), int(ulp_distance(lg, lv).max())
