"""The allocation-free entry point det_attention_decode_noalloc
(include/det_attention.h), through the C-ABI: the same bits as
det_attention_decode with a caller's work buffer, on two calls in a row (the
second smaller, so the shared device array holds the first call's partials
when it starts), and the refusal of a problem larger than the array.

Decode attention with a fixed split size: summary page of "Defeating
Nondeterminism in LLM Inference", section on batch-invariant kernel design,
attention.
"""
import ctypes

import numpy as np
import pytest
import torch

import det_workloads as Wk
import invariant_deterministic_gemm_det_amd as dg
from gpu_util import device, say

pytestmark = pytest.mark.gpu

D = 128
SCALE = 1.0 / np.sqrt(D)


@pytest.fixture(scope="module")
def dev():
    d = device()
    dg.load_library()
    return d


def _case(B, Hq, Hkv, Smax, lens, seed, dev):
    q = Wk.randn_bf16((B, Hq, D), 1.0, seed, dev)
    k = Wk.randn_bf16((B, Hkv, Smax, D), 1.0, seed + 1, dev)
    v = Wk.randn_bf16((B, Hkv, Smax, D), 1.0, seed + 2, dev)
    return q, k, v, torch.tensor(lens, dtype=torch.int32, device=dev)


def test_noalloc_matches_work_buffer_entry_twice(dev):
    lens1 = (1024 + Wk.randperm(3073, 2100)[:64]).tolist()
    cases = [(64, 32, 8, 4096, lens1, 2200),            # the decode batch: 4.3 M partials
             (5, 16, 2, 900, [900, 1, 0, 256, 513], 2300)]  # then a smaller one
    for B, Hq, Hkv, Smax, lens, seed in cases:
        say("attention noalloc vs work buffer", B, Hq, Hkv, Smax)
        q, k, v, L = _case(B, Hq, Hkv, Smax, lens, seed, dev)
        want = dg.det_attention_decode(q, k, v, L, SCALE)
        out = torch.empty_like(want)
        got = dg.det_attention_decode_noalloc(q, k, v, L, SCALE, out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(got.view(torch.int16), want.view(torch.int16)), (B, Hq, Smax)


def test_noalloc_refuses_problems_beyond_the_array(dev):
    say("attention noalloc: too large for the scratch array")
    lib = dg.load_library()
    B, Hq, Hkv, Smax = 1024, 64, 8, 4096          # 1024*64*16*130 floats > 8 M
    assert B * Hq * (Smax // 256) * (D + 2) > dg.ATTN_SCRATCH_FLOATS
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device=dev)
    kv = torch.zeros((1, 16), dtype=torch.bfloat16, device=dev)  # never read: refused first
    o = torch.empty_like(q)
    L = torch.zeros(B, dtype=torch.int32, device=dev)
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    rc = lib.det_attention_decode_noalloc(p(q), p(kv), p(kv), p(L), B, Hq, Hkv, Smax, D,
                                          ctypes.c_float(SCALE), p(o), None)
    assert rc == dg.ESCRATCH
    assert b"scratch" in lib.det_gemm_status_string(rc)
