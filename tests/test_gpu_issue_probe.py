"""The issue-rate probe behind the roofline ceiling of the wide kernel
(det_gemm_debug_issue_probe), through the C-ABI: one stage's mix of MFMAs and
conversions takes at least the time of its MFMAs alone, and the clock the
MFMAs alone imply (two waves per SIMD of 32 MFMAs of 16 cycles per stage) is a
plausible shader clock."""
import pytest
import torch

import invariant_deterministic_gemm_det_amd as dg
from gpu_util import device, say

pytestmark = pytest.mark.gpu


def _stage_us(mode, sink, iters=1000):
    dg.det_gemm_debug_issue_probe(mode, 20, sink)   # warm
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    dg.det_gemm_debug_issue_probe(mode, iters, sink)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / iters


def test_issue_probe_mix_and_clock():
    dev = device()
    dg.load_library()
    say("issue-rate probe: MFMAs alone and the stage mix")
    sink = torch.empty(256 * 512, dtype=torch.float32, device=dev)
    mfma = _stage_us(0, sink)
    mix = _stage_us(1, sink)
    mhz = 2 * 32 * 16 / mfma
    print("us per stage: MFMAs alone %.4f, stage mix %.4f; implied clock %.0f MHz" % (mfma, mix, mhz))
    assert 800 < mhz < 2600, mhz
    assert mix >= 0.98 * mfma


def test_issue_probe_rejects_bad_arguments():
    dev = device()
    sink = torch.empty(512, dtype=torch.float32, device=dev)
    with pytest.raises(TypeError):
        dg.det_gemm_debug_issue_probe(0, 10, sink[:100])
    with pytest.raises(dg.DetGemmError) as e:
        dg.det_gemm_debug_issue_probe(3, 10, sink)
    assert e.value.code == dg.EINVAL
