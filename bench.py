"""Benchmark of the det_gemm hot path on one MI355X.

One step = one pass of the whole path at the QKV-projection shape
(M=4096, K=4096, N=6144, bf16 inputs, synthetic): the forward product
C = X W (det_gemm_fwd, W given as [K,N]) and the two backward products of that
layer, dX = dC W^T (det_gemm_da, reduction over N) and dW = X^T dC (det_gemm_db,
reduction over M).  Inputs are generated on the device from fixed seeds and are
resident in HBM before timing starts.

Prints one JSON line: throughput of the step in TFLOP/s (2*M*N*K per product),
per-product timings from HIP events on the launch stream, the roofline record
of the dominant kernel against MI355X's dense bf16 MFMA peak, and the CPU
oracle timed on a bounded slice of the same products on the host cores.
"""
import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
M, K, N = 4096, 4096, 6144
COPY_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles",
                            "hbm_traffic_per_launch.md")
ISSUE_FILE = os.path.join(ROOT, "profiles", "det_gemm_step_M4096_K4096_N6144_sq_counters.md")
CLOCK_MHZ_PEAK = 2400.0     # the clock the published peak assumes
CSRC = os.path.join(ROOT, "invariant_deterministic_gemm_det_amd", "csrc")


def kernel_source_hash():
    """sha256 over the kernel sources, to tell whether recorded counters are current."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name.endswith((".h", ".hip")):
            with open(os.path.join(CSRC, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def profile_fields(path):
    """The machine-readable `- key: value` lines of a rocprofv3 summary under
    profiles/, or {} when the file is missing or was taken on other kernel
    sources (its kernel_source_sha256 differs from the current sources)."""
    try:
        with open(path) as f:
            lines = f.read().splitlines()
    except OSError:
        return {}
    fields = {}
    for ln in lines:
        if ln.startswith("- ") and ": " in ln:
            k, v = ln[2:].split(": ", 1)
            fields[k.strip()] = v.strip().strip("`")
    if fields.get("kernel_source_sha256") != kernel_source_hash():
        return {}
    return fields


def recorded_traffic(op):
    """HBM bytes per launch of `op` from the rocprofv3 counter summary, or None when
    the summary is missing or was taken on different kernel sources."""
    v = profile_fields(TRAFFIC_FILE).get(f"hbm_bytes_per_launch_{op}")
    return int(v) if v else None


def recorded_issue(op):
    """From the matrix-core / VALU counter pass of the step kernels: the shader
    clock under load (SQ_BUSY_CYCLES per shader engine / kernel duration, MHz)
    and the non-MFMA VALU instructions per 16x16 block and leaf, or {}."""
    f = profile_fields(ISSUE_FILE)
    out = {}
    if f.get(f"sclk_mhz_{op}"):
        out["sclk_mhz"] = float(f[f"sclk_mhz_{op}"])
    if f.get(f"valu_per_block_leaf_{op}"):
        out["valu_per_block_leaf"] = float(f[f"valu_per_block_leaf_{op}"])
    return out


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target host time of the oracle sample")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle leg")
    ap.add_argument("--no-moe", action="store_true", help="skip the MoE grouped GEMM leg")
    ap.add_argument("--no-fingerprint", action="store_true", help="skip the fingerprint leg")
    ap.add_argument("--no-rmsnorm", action="store_true", help="skip the RMSNorm leg")
    ap.add_argument("--no-attention", action="store_true", help="skip the decode attention leg")
    ap.add_argument("--no-shard", action="store_true", help="skip the K-shard combination leg")
    ap.add_argument("--no-small-m", action="store_true", help="skip the decode-shaped products")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the other transformer-shaped products (MLP, backward, LM head, depth cap)")
    ap.add_argument("--profile-only", action="store_true",
                    help="run only the GPU steps (for rocprofv3 runs)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="with --profile-only: also run a plain device copy of known size, "
                         "the reference for the HBM byte counters")
    return ap.parse_args()


def cpu_baseline(X, W, dC, target_s):
    """The oracle, untuned, on a row slice of each of the three products."""
    import numpy as np
    import oracle
    import det_workloads as Wk

    x, w, d = Wk.bits(X), Wk.bits(W), Wk.bits(dC)
    threads = oracle.num_threads()
    # calibrate: one slice of `threads` rows of the forward product
    rows = max(1, threads)
    t0 = time.perf_counter()
    oracle.fwd(x[:rows], w)
    t_cal = time.perf_counter() - t0
    per_row = t_cal / rows  # seconds per forward row (all threads busy)
    rows = max(threads, int(target_s / 3.0 / max(per_row, 1e-9)) // threads * threads)
    rows = min(rows, 512)
    t0 = time.perf_counter()
    oracle.fwd(x[:rows], w)                                 # C[:rows]      2*rows*N*K
    oracle.da(d[:rows], w)                                  # dX[:rows]     2*rows*K*N
    oracle.db(np.ascontiguousarray(x[:, :rows]), d)         # dW[:rows]     2*rows*N*M
    dt = time.perf_counter() - t0
    flops = 2.0 * rows * N * K + 2.0 * rows * K * N + 2.0 * rows * N * M
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "seconds": round(dt, 3), "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "sample": f"CPU oracle on {rows} output rows of each product: fwd C[:{rows}], "
                      f"da dX[:{rows}], db dW[:{rows}] of the M=4096 K=4096 N=6144 step"}


def moe_leg(dev, steps, warmup, with_cpu, context=True):
    """The MoE grouped GEMM with its per-token slot epilogue (det_moe_fwd_dprob) on
    the expert down projection of a top-2-of-8 MoE layer: 4096 tokens -> 8192
    rows grouped by expert, K = 2048, N = 4096.  Also times the same products
    as one det_gemm_fwd launch per expert (no epilogue), as context."""
    import torch
    import det_workloads as Wk
    import invariant_deterministic_gemm_det_amd as dg

    inp = Wk.moe_inputs(dev)
    T, K, N, E = inp.x.shape[0], Wk.MOE_K, Wk.MOE_N, Wk.MOE_E
    off = inp.offsets
    Y = torch.empty((T, N), dtype=torch.bfloat16, device=dev)
    dprob = torch.empty((T,), dtype=torch.float32, device=dev)
    slots = torch.empty(((N + 127) // 128, T), dtype=torch.float32, device=dev)

    def call():
        dg.det_moe_fwd_dprob(inp.x, inp.w, off, inp.g, Y=Y, slots=slots, dprob=dprob)

    def per_expert():
        for e in range(E):
            dg.det_gemm_fwd(inp.x[off[e]:off[e + 1]], inp.w[e], out=Y[off[e]:off[e + 1]])

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            ts.append((e0, e1))
        torch.cuda.synchronize()
        return [a.elapsed_time(b) for a, b in ts]

    flop = 2.0 * T * K * N
    # This leg runs first after the host-only oracle leg: calls for a quarter
    # second first, so that the timed calls see the device's loaded clocks
    # (as the headline step does), not its ramp from idle.
    t_end = time.perf_counter() + 0.25
    while time.perf_counter() < t_end:
        for _ in range(20):
            call()
        torch.cuda.synchronize()
    t = timed(call)
    avg = sum(t) / len(t)
    out = {"workload": "MoE expert down projection: 4096 tokens, top-2 of 8 experts "
                       "(skewed routing), rows grouped by expert, K=2048, N=4096, "
                       "epilogue dprob[r] = fixed trees over 128-column slots of Y*G",
           "rows": T, "segments": [off[e + 1] - off[e] for e in range(E)],
           "ms": round(avg, 4), "min_ms": round(min(t), 4), "max_ms": round(max(t), 4),
           "tflops": round(flop / (avg * 1e-3) / 1e12, 2),
           "roofline": {"bound": "mfma",
                        "kernel": "mfma_wide_grouped_kernel<2-leaf units> + slot tree combine",
                        "achieved": round(flop / (avg * 1e-3) / 1e12, 2),
                        "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(flop / (avg * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                        "traffic": None}}
    out["roofline"]["traffic"] = recorded_traffic("moe")
    if context:
        tp = timed(per_expert)
        out["per_expert_det_gemm_fwd_ms"] = round(sum(tp) / len(tp), 4)
    if with_cpu:
        import numpy as np
        import oracle
        rows = [np.arange(off[e], min(off[e + 1], off[e] + 32)) for e in range(E)]
        idx = np.concatenate(rows)
        sub_off = [0] + list(np.cumsum([len(r) for r in rows]))
        x = Wk.bits(inp.x[torch.as_tensor(idx, device=dev)])
        g = Wk.bits(inp.g[torch.as_tensor(idx, device=dev)])
        w = Wk.bits(inp.w)
        t0 = time.perf_counter()
        oracle.moe_fwd_dprob(x, w, sub_off, g)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": 2.0 * len(idx) * K * N / dt / 1e12, "unit": "TFLOP/s",
                               "cores": oracle.num_threads(), "kind": "oracle",
                               "seconds": round(dt, 3),
                               "sample": f"CPU oracle on the first 32 rows of each expert "
                                         f"({len(idx)} rows) of the same workload"}
    return out


PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, published
COLD_COPIES = 13            # 13 x 50 MB QKV weights: 650 MB, beyond the 256 MB Infinity Cache
FP_BYTES = 1 << 30
FP_ROWS, FP_ROW_BYTES = 16384, 32768


def fingerprint_leg(dev, steps, warmup, with_cpu):
    """Tensor fingerprints and the byte comparator (det_fingerprint.h) on
    seeded random bytes resident in HBM: the digest of a 1 GiB buffer, per-row
    digests of a [16384, 32 KiB] layout (512 MiB), and the first mismatch of two
    equal 1 GiB buffers (the whole of both is read)."""
    import torch
    import invariant_deterministic_gemm_det_amd as dg

    def draw():  # the same bytes each time (no copy kernel: the counter runs
        g = torch.Generator(device=dev)  # calibrate on the only device copy)
        g.manual_seed(7001)
        return torch.randint(0, 256, (FP_BYTES,), generator=g, dtype=torch.uint8, device=dev)

    a, b = draw(), draw()
    rows = a[:FP_ROWS * FP_ROW_BYTES].view(FP_ROWS, FP_ROW_BYTES)
    d = torch.empty(1, dtype=torch.int64, device=dev)
    dr = torch.empty(FP_ROWS, dtype=torch.int64, device=dev)
    mm = torch.empty(1, dtype=torch.int64, device=dev)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            ts.append((e0, e1))
        torch.cuda.synchronize()
        t = [x.elapsed_time(y) for x, y in ts]
        return sum(t) / len(t)

    t_d = timed(lambda: dg.det_fingerprint(a, out=d))
    t_r = timed(lambda: dg.det_fingerprint_rows(rows, out=dr))
    t_m = timed(lambda: dg.det_first_mismatch(a, b, out=mm))
    gbs = lambda nbytes, ms: round(nbytes / (ms * 1e-3) / 1e9, 1)
    out = {"workload": "digest of 1 GiB, row digests of 16384 x 32 KiB, first mismatch of two "
                       "equal 1 GiB buffers; seeded random bytes in HBM",
           "digest": {"ms": round(t_d, 4), "GB/s": gbs(FP_BYTES, t_d)},
           "rows": {"ms": round(t_r, 4), "GB/s": gbs(FP_ROWS * FP_ROW_BYTES, t_r)},
           "first_mismatch": {"ms": round(t_m, 4), "GB/s": gbs(2 * FP_BYTES, t_m)},
           "roofline": {"bound": "hbm", "kernel": "digest_sum_kernel (1 GiB digest)",
                        "achieved": gbs(FP_BYTES, t_d), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs(FP_BYTES, t_d) / PEAK_HBM_GBS, 4),
                        "traffic": recorded_traffic("fp")}}
    if with_cpu:
        import oracle
        n = 64 << 20
        host = a[:n].cpu().numpy()
        t0 = time.perf_counter()
        oracle.fingerprint(host)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(n / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
                               "kind": "oracle", "seconds": round(dt, 3),
                               "sample": "CPU oracle digest of the first 64 MiB of the buffer"}
    return out


NORM_R, NORM_H = 8192, 4096


def graph_time(fn, out, steps, rotate=None):
    """Per-call time of `fn` (which writes `out`) from `steps` calls replayed
    back to back out of a captured graph: the GPU time of calls shorter than
    the host's launch path.  Every replay must reproduce the eager bits.
    `rotate`: calls equal to `fn` on copies of its operands, taken in turn."""
    import torch
    fn()
    torch.cuda.synchronize()
    ref = out.clone()
    calls = rotate or [fn]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            calls[i % len(calls)]()
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), ref.view(torch.uint8)), "graph replay differs"
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), ref.view(torch.uint8)), "graph replay differs"
    del graph
    return e0.elapsed_time(e1) / steps


def rmsnorm_leg(dev, steps, warmup, with_cpu, decode=True):
    """Batch-invariant RMSNorm (det_norm.h) over 8192 token rows of width 4096
    (the MLP input of the workloads), and a 64-row decode batch."""
    import torch
    import det_workloads as Wk
    import invariant_deterministic_gemm_det_amd as dg

    x = Wk.randn_bf16((NORM_R, NORM_H), 1.0, 9500, dev)
    w = Wk.randn_bf16((NORM_H,), 1.0, 9501, dev)
    y = torch.empty_like(x)
    r = torch.empty(NORM_R, dtype=torch.float32, device=dev)

    def timed(fn):
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(steps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            ts.append((e0, e1))
        torch.cuda.synchronize()
        t = [a.elapsed_time(b) for a, b in ts]
        return sum(t) / len(t)

    t_full = timed(lambda: dg.det_rmsnorm(x, w, out=y, rstd=r))
    t_dec = graph_time(lambda: dg.det_rmsnorm(x[:64], w, out=y[:64], rstd=r[:64]), y[:64], steps) \
        if decode else 0.0
    nbytes = NORM_R * NORM_H * 4 + NORM_H * 2 + NORM_R * 4
    gbs = nbytes / (t_full * 1e-3) / 1e9
    out = {"workload": "RMSNorm of 8192 x 4096 bf16 rows (read x, write y and rstd); "
                       "decode: 64 rows, per call from graph replays of back-to-back calls",
           "ms": round(t_full, 4), "GB/s": round(gbs, 1), "decode_64_rows_us": round(t_dec * 1e3, 2),
           "roofline": {"bound": "hbm", "kernel": "rmsnorm_fixed_kernel<16> (8192 x 4096)",
                        "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": recorded_traffic("norm")}}
    if with_cpu:
        import oracle
        rows = 1024
        xb, wb = Wk.bits(x[:rows]), Wk.bits(w)
        t0 = time.perf_counter()
        oracle.rmsnorm(xb, wb, 1e-6)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(rows * NORM_H * 4 / dt / 1e9, 3), "unit": "GB/s",
                               "cores": oracle.num_threads(), "kind": "oracle",
                               "seconds": round(dt, 3),
                               "sample": f"CPU oracle on the first {rows} rows"}
    return out


ATT_B, ATT_HQ, ATT_HKV, ATT_S, ATT_D = 64, 32, 8, 4096, 128


def attention_leg(dev, steps, warmup, with_cpu):
    """Decode attention with fixed 256-position splits (det_attention.h): 64
    sequences with seeded lengths in [1024, 4096], 32 query heads on 8
    key/value heads, head dimension 128 (the shape of an 8B-class GQA model)."""
    import numpy as np
    import torch
    import det_workloads as Wk
    import invariant_deterministic_gemm_det_amd as dg

    lens = (1024 + Wk.randperm(3073, 2100)[:ATT_B]).tolist()
    q = Wk.randn_bf16((ATT_B, ATT_HQ, ATT_D), 1.0, 2200, dev)
    k = Wk.randn_bf16((ATT_B, ATT_HKV, ATT_S, ATT_D), 1.0, 2201, dev)
    v = Wk.randn_bf16((ATT_B, ATT_HKV, ATT_S, ATT_D), 1.0, 2202, dev)
    L = torch.tensor(lens, dtype=torch.int32, device=dev)
    o = torch.empty((ATT_B, ATT_HQ, ATT_D), dtype=torch.bfloat16, device=dev)
    ns = (ATT_S + 255) // 256
    work = torch.empty(ATT_B * ATT_HQ * ns * (ATT_D + 2), dtype=torch.float32, device=dev)
    scale = 1.0 / np.sqrt(ATT_D)
    fn = lambda: dg.det_attention_decode(q, k, v, L, scale, out=o, work=work)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        ts.append((e0, e1))
    torch.cuda.synchronize()
    t = sum(a.elapsed_time(b) for a, b in ts) / len(ts)
    kv_bytes = sum(lens) * ATT_HKV * ATT_D * 2 * 2
    gbs = kv_bytes / (t * 1e-3) / 1e9
    out = {"workload": "decode attention: 64 sequences, lengths 1024..4096 (seeded), 32 query "
                       "heads on 8 key/value heads, head dim 128, fixed 256-position splits",
           "ms": round(t, 4), "kv_bytes": kv_bytes, "GB/s": round(gbs, 1),
           "roofline": {"bound": "hbm", "kernel": "attn_split_kernel + attn_combine_kernel",
                        "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                        "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": recorded_traffic("attn")}}
    # chunked prefill with the decode arithmetic: 4 sequences of 4096 cached
    # positions, the last 512 of each as the chunk (causal rows)
    PB, PC = 4, 512
    pq = Wk.randn_bf16((PB * PC, ATT_HQ, ATT_D), 1.0, 2203, dev)
    plens = torch.arange(ATT_S - PC + 1, ATT_S + 1, dtype=torch.int32, device=dev).repeat(PB)
    poff = [i * PC for i in range(PB + 1)]
    pk, pv = k[:PB].contiguous(), v[:PB].contiguous()
    pwork = torch.empty(PB * PC * ATT_HQ * ns * (ATT_D + 2), dtype=torch.float32, device=dev)
    po = torch.empty((PB * PC, ATT_HQ, ATT_D), dtype=torch.bfloat16, device=dev)
    pfn = lambda: dg.det_attention_prefill(pq, pk, pv, poff, plens, scale, out=po, work=pwork)
    for _ in range(max(1, warmup // 2)):
        pfn()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        pfn()
    e1.record()
    torch.cuda.synchronize()
    tp = e0.elapsed_time(e1) / 5
    flops = 4.0 * float(plens.sum().item()) * ATT_HQ * ATT_D
    out["prefill"] = {"workload": f"{PB} sequences x {PC}-row causal chunks at positions "
                                  f"{ATT_S - PC}..{ATT_S - 1}, 32/8 heads, head dim 128, the "
                                  "decode arithmetic per row",
                      "ms": round(tp, 4), "tflops": round(flops / (tp * 1e-3) / 1e12, 2)}
    if with_cpu:
        from oracle.attention import attention_decode
        sel = [0, 1]
        t0 = time.perf_counter()
        attention_decode(Wk.bits(q[sel]), Wk.bits(k[sel]), Wk.bits(v[sel]),
                         np.array([lens[i] for i in sel]), scale)
        dt = time.perf_counter() - t0
        nb = sum(lens[i] for i in sel) * ATT_HKV * ATT_D * 4
        out["cpu_baseline"] = {"value": round(nb / dt / 1e9, 3), "unit": "GB/s", "cores": 1,
                               "kind": "oracle", "seconds": round(dt, 3),
                               "sample": "float64 oracle on 2 of the 64 sequences"}
    return out


def shard_leg(dev, steps, warmup):
    """Combination of TP = 8 K-shard partial products of the step shape's
    forward ([4096, 6144] bf16 each) by the fixed rank-order tree."""
    import torch
    import det_workloads as Wk
    import invariant_deterministic_gemm_det_amd as dg

    parts = [Wk.randn_bf16((M, N), 1.0, 9600 + k, dev) for k in range(8)]
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    fn = lambda: dg.det_gemm_shard_reduce(parts, out=out)
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        fn()
        e1.record()
        ts.append((e0, e1))
    torch.cuda.synchronize()
    t = sum(a.elapsed_time(b) for a, b in ts) / len(ts)
    nbytes = 9 * M * N * 2
    gbs = nbytes / (t * 1e-3) / 1e9
    return {"workload": "TP = 8 partial products [4096, 6144] bf16 -> fixed rank-order tree of "
                        "bf16 adds (the local step of a deterministic reduce-scatter)",
            "ms": round(t, 4), "GB/s": round(gbs, 1),
            "roofline": {"bound": "hbm", "kernel": "shard_reduce_kernel<8>", "achieved": round(gbs, 1),
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                         "traffic": recorded_traffic("shard")}}


def small_m_leg(dev, steps, warmup, decode_only=False):
    """Decode-shaped forward products (few rows against a full weight), which
    stream the weight once: time per call and HBM GB/s of the algorithmic bytes
    (X, W and C once each) against the 8 TB/s roofline.  QKV projection K =
    4096, N = 6144 with the weight stored [K][N] and [N][K]; LM head K = 4096,
    N = 151936."""
    import torch
    import det_workloads as Wk
    import invariant_deterministic_gemm_det_amd as dg

    Wq = Wk.qkv_weight(dev)
    Wqt = Wk.qkv_weight(dev, transposed=True)
    Xl, Wl = Wk.lm_head_inputs(dev, M=256)
    Xq = Wk.randn_bf16((128, Wk.QKV_K), 1.0, 9700, dev)
    cases = [("qkv", "W[K][N]", 1), ("qkv", "W[K][N]", 16), ("qkv", "W[K][N]", 32),
             ("qkv", "W[K][N]", 64), ("qkv", "W[K][N]", 128),
             ("qkv", "W[N][K]", 1), ("qkv", "W[N][K]", 16), ("qkv", "W[N][K]", 32),
             ("qkv", "W[N][K]", 64),
             ("qkv", "W[N][K]", 128), ("lm_head", "W[K][N]", 1),
             ("lm_head", "W[K][N]", 32), ("lm_head", "W[K][N]", 256)]
    if decode_only:  # the rows on the decode kernel and the split 32-column tiles, one
        # kernel instance each (the LM head at 32 rows is wide enough in N to run on the
        # wide kernel)
        cases = [c for c in cases if c[2] <= 16 or (c[0] == "qkv" and c[2] <= 128)]
    rows = []
    cold_copies = {}
    for name, layout, m in cases:
        if name == "qkv":
            x, k, n = Xq[:m], Wk.QKV_K, Wk.QKV_N
            fn = (lambda: dg.det_gemm_fwd(x, Wq)) if layout == "W[K][N]" else \
                 (lambda: dg.det_gemm_fwd_rhs_transposed(x, Wqt))
        else:
            x, k, n = Xl[:m], Xl.shape[1], Wl.shape[1]
            fn = lambda: dg.det_gemm_fwd(x, Wl)
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        # A call of a few microseconds is shorter than the host's launch path:
        # time calls replayed from a captured graph, and the eager calls beside it.
        out = fn()
        run = (lambda: dg.det_gemm_fwd(x, Wq, out=out)) if name == "qkv" and layout == "W[K][N]" else \
              (lambda: dg.det_gemm_fwd_rhs_transposed(x, Wqt, out=out)) if name == "qkv" else \
              (lambda: dg.det_gemm_fwd(x, Wl, out=out))
        t = graph_time(run, out, steps)
        # The same calls, each on another copy of the weight, the copies
        # together well beyond the 256 MB Infinity Cache: what a model's
        # decode step sees, each layer's weight read once per token.  The LM
        # head's weight alone exceeds the cache.
        if name == "qkv":
            if layout not in cold_copies:
                base = Wq if layout == "W[K][N]" else Wqt
                cold_copies[layout] = [base] + [base.clone() for _ in range(COLD_COPIES - 1)]
            copies = cold_copies[layout]
            rot = [(lambda w=w: dg.det_gemm_fwd(x, w, out=out)) if layout == "W[K][N]" else
                   (lambda w=w: dg.det_gemm_fwd_rhs_transposed(x, w, out=out)) for w in copies]
            t_cold = graph_time(run, out, steps, rotate=rot)
        else:
            t_cold = t
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        t_eager = e0.elapsed_time(e1) / steps
        # the tile configuration the library chose for this call
        transposed = name == "qkv" and layout == "W[N][K]"
        w = Wqt if transposed else (Wq if name == "qkv" else Wl)
        cfg = dg.det_gemm_debug_config(dg.OP_FWD_RHS_TRANSPOSED if transposed else dg.OP_FWD,
                                       x.data_ptr(), x.stride(0), w.data_ptr(), w.stride(0),
                                       out.data_ptr(), out.stride(0), m, n, k)
        kernel = ("mfma_wide_split_kernel" if cfg >= 13 else "mfma_decode_kernel" if cfg >= 10
                  else "mfma_wide_kernel" if cfg >= 5 else "mfma_kernel")
        nbytes = (m * k + k * n + m * n) * 2
        gbs = nbytes / (t * 1e-3) / 1e9
        gbs_cold = nbytes / (t_cold * 1e-3) / 1e9
        rows.append({"op": name, "weight": layout, "M": m, "K": k, "N": n, "us": round(t * 1e3, 2),
                     "us_eager_calls": round(t_eager * 1e3, 2),
                     "GB/s": round(gbs, 1), "frac_of_hbm": round(gbs / PEAK_HBM_GBS, 4),
                     "us_cold_weight": round(t_cold * 1e3, 2),
                     "frac_of_hbm_cold_weight": round(gbs_cold / PEAK_HBM_GBS, 4),
                     "kernel": kernel, "config": cfg})
    return {"workload": "forward products with 1..256 rows: the weight read once per call "
                        "(the decode kernel; from 33 to 128 rows, narrow wide tiles whose tree is "
                        "split over two or four wave groups; the wide kernel when wide in N)",
            "timing": "us: per call, calls replayed from a captured graph (the QKV weight, "
                      "50 MB, stays in the 256 MB Infinity Cache from call to call); "
                      "us_cold_weight: the same, each call on another of "
                      f"{COLD_COPIES} copies of the weight (as a model's layers: the weight "
                      "comes from HBM); us_eager_calls: back-to-back calls through the "
                      "binding (host launch path included)",
            "roofline": "hbm, 8000 GB/s", "rows": rows}


def configs_leg(dev, reps=5):
    """TFLOP/s of the other transformer-shaped products, one launch each per
    rep (median of `reps` after one warm-up call): the MLP of an 8B-class
    model at 8192 rows (gate+up K = 4096, N = 24576; down K = 12288, N = 4096,
    384 leaves), the backward at M = 8192, K = N = 4096 (dA; dB and its
    [N,K] form, reduction depth 8192), the LM head at 4096 rows (N = 151936,
    bf16 and fp32 out), two MLP down projections with other leaf counts
    (K = 14336 and 11008) and the depth cap (K = 32768, N = 4096, 2048 rows)."""
    import torch
    import det_workloads as Wk
    import invariant_deterministic_gemm_det_amd as dg

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return statistics.median(ts), min(ts), max(ts)

    rows = []

    def add(name, shape, flop, fn, cfg):
        med, lo, hi = timed(fn)
        tf = flop / (med * 1e-3) / 1e12
        rows.append({"product": name, "M,N,K": shape, "median_ms": round(med, 4),
                     "min_ms": round(lo, 4), "max_ms": round(hi, 4), "tflops": round(tf, 1),
                     "pct_of_bf16_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2), "config": cfg})

    def cfg_of(op, a, lda, b, ldb, c, ldc, M, N, K):
        return dg.det_gemm_debug_config(op, a.data_ptr(), lda, b.data_ptr(), ldb, c.data_ptr(), ldc,
                                        M, N, K)

    X, Wgu, H, Wd = Wk.mlp_inputs(dev)
    M, K, N = X.shape[0], X.shape[1], Wgu.shape[1]
    out = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    add("MLP gate+up fwd", [M, N, K], 2.0 * M * N * K, lambda: dg.det_gemm_fwd(X, Wgu, out=out),
        cfg_of(dg.OP_FWD, X, K, Wgu, N, out, N, M, N, K))
    M, K, N = H.shape[0], H.shape[1], Wd.shape[1]
    out2 = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    add("MLP down fwd (L = 384)", [M, N, K], 2.0 * M * N * K,
        lambda: dg.det_gemm_fwd(H, Wd, out=out2), cfg_of(dg.OP_FWD, H, K, Wd, N, out2, N, M, N, K))
    del X, Wgu, H, Wd, out, out2

    A, B, dC = Wk.backward_inputs(dev)
    M, K, N = A.shape[0], A.shape[1], B.shape[1]
    dA = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dB = torch.empty((K, N), dtype=torch.bfloat16, device=dev)
    dBt = torch.empty((N, K), dtype=torch.bfloat16, device=dev)
    add("backward da (R = 4096)", [M, N, K], 2.0 * M * N * K, lambda: dg.det_gemm_da(dC, B, out=dA),
        cfg_of(dg.OP_DA, dC, N, B, N, dA, K, M, N, K))
    add("backward db (R = 8192)", [M, N, K], 2.0 * M * N * K, lambda: dg.det_gemm_db(A, dC, out=dB),
        cfg_of(dg.OP_DB, A, K, dC, N, dB, N, M, N, K))
    add("backward db_transposed (R = 8192)", [M, N, K], 2.0 * M * N * K,
        lambda: dg.det_gemm_db_transposed(A, dC, out=dBt), cfg_of(dg.OP_DB_TRANSPOSED, A, K, dC, N, dBt, K, M, N, K))
    del A, B, dC, dA, dB, dBt

    Xl, Wl = Wk.lm_head_inputs(dev, M=4096)
    M, K, N = Xl.shape[0], Xl.shape[1], Wl.shape[1]
    ol = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    add("LM head fwd, bf16 out", [M, N, K], 2.0 * M * N * K, lambda: dg.det_gemm_fwd(Xl, Wl, out=ol),
        cfg_of(dg.OP_FWD, Xl, K, Wl, N, ol, N, M, N, K))
    del ol
    of = torch.empty((M, N), dtype=torch.float32, device=dev)
    add("LM head fwd, fp32 out", [M, N, K], 2.0 * M * N * K, lambda: dg.det_gemm_fwd_fp32(Xl, Wl, out=of),
        cfg_of(dg.OP_FWD_FP32, Xl, K, Wl, N, of, N, M, N, K))
    del Xl, Wl, of

    # MLP down projections whose leaf counts are not 2^a or 3 * 2^a: an
    # 8B-class model's (K = 14336, L = 448 = 7 * 64: units of seven leaves) and
    # a 7B-class one's (K = 11008, L = 344 = 43 * 8: units of 43 leaves)
    for kd, name in ((14336, "MLP down, K = 14336 (L = 448, seven-leaf units)"),
                     (11008, "MLP down, K = 11008 (L = 344, 43-leaf units)")):
        Hd = Wk.randn_bf16((8192, kd), 1.0, 3005, dev)
        Wdd = Wk.randn_bf16((kd, 4096), 0.02, 3006, dev)
        od = torch.empty((8192, 4096), dtype=torch.bfloat16, device=dev)
        add(name, [8192, 4096, kd], 2.0 * 8192 * 4096 * kd,
            lambda: dg.det_gemm_fwd(Hd, Wdd, out=od), cfg_of(dg.OP_FWD, Hd, kd, Wdd, 4096, od, 4096, 8192, 4096, kd))
        del Hd, Wdd, od

    Ad, Bd = Wk.deep_inputs(dev)
    M, K, N = Ad.shape[0], Ad.shape[1], Bd.shape[1]
    od = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    add("depth cap fwd (K = 32768, L = 1024)", [M, N, K], 2.0 * M * N * K,
        lambda: dg.det_gemm_fwd(Ad, Bd, out=od), cfg_of(dg.OP_FWD, Ad, K, Bd, N, od, N, M, N, K))
    del Ad, Bd, od
    torch.cuda.empty_cache()
    return {"workload": "the other transformer-shaped products, inputs seeded as the parity "
                        "tests' (MLP 3001-3004, backward 4001-4003, LM head 5001-5002, depth cap "
                        "5003-5004; the two other MLP down projections 3005-3006), resident in HBM",
            "timing": f"median of {reps} launches after one warm-up, HIP events", "rows": rows}


def issue_probe_leg(iters=4000):
    """The instruction mix of one pipeline stage of the 128x128 wide kernel
    (per wave: 32 MFMAs, 64 bf16 conversions, each conversion feeding the next
    MFMA; 8 waves per compute unit), without memory traffic, on all 256
    compute units: its time per stage bounds the kernel's main loop from
    below.  The MFMAs alone give the matrix-core rate at the clock the chip
    holds under this load: 2 waves x 32 MFMAs of 16 cycles (the published
    bf16 peak over 1024 SIMDs at 2.4 GHz) per SIMD and stage."""
    import torch
    import invariant_deterministic_gemm_det_amd as dg
    dev = torch.device("cuda:0")
    sink = torch.empty(256 * 512, dtype=torch.float32, device=dev)
    dg.det_gemm_debug_issue_probe(1, 100, sink)
    torch.cuda.synchronize()
    out = {}
    for mode, name in ((0, "mfma_only"), (1, "stage_mix")):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dg.det_gemm_debug_issue_probe(mode, iters, sink)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        out[name] = {"ms": round(ms, 4), "ns_per_stage": round(ms * 1e6 / iters, 2)}
    mhz = 2 * 32 * 16 / (out["mfma_only"]["ns_per_stage"] * 1e-3)
    out["sclk_mhz_implied"] = round(mhz, 1)
    out["stage_mix_cycles"] = round(out["stage_mix"]["ns_per_stage"] * mhz * 1e-3, 1)
    return out


def cold_fwd_leg(X, W, C, flop, reps=10):
    """The forward with cold caches: 512 MiB written between calls (twice the
    256 MB Infinity Cache, far beyond the L2s), so every operand comes from
    HBM.  Median and range over `reps` calls, each timed alone."""
    import torch
    import invariant_deterministic_gemm_det_amd as dg
    flush = torch.empty(256 << 20, dtype=torch.bfloat16, device=X.device)
    ts = []
    for _ in range(reps):
        flush.zero_()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dg.det_gemm_fwd(X, W, out=C)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del flush
    med = statistics.median(ts)
    return {"median_ms": round(med, 4), "min_ms": round(min(ts), 4), "max_ms": round(max(ts), 4),
            "tflops": round(flop / (med * 1e-3) / 1e12, 2), "reps": reps,
            "flush": "512 MiB written before each call"}


def strict_leg(X, W, rows):
    """The strict-order kernel (det_gemm_strict_fwd: one scalar fp32 FMA chain
    per leaf, bit-exact to the oracle) on a row slice of the forward product,
    timed with HIP events on the launch stream."""
    import torch
    import invariant_deterministic_gemm_det_amd as dg
    x = X[:rows]
    out = dg.det_gemm_fwd(x, W, strict=True)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        dg.det_gemm_fwd(x, W, out=out, strict=True)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / 3
    flop = 2.0 * rows * N * K
    return {"kernel": "strict_kernel (K1)", "sample": f"fwd on {rows} rows of the step shape "
            f"(M={rows}, K={K}, N={N})", "ms": round(ms, 4),
            "tflops": round(flop / (ms * 1e-3) / 1e12, 3)}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(det_gemm shards by rows/columns without communication; see the design notes)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import det_workloads as Wk
    import invariant_deterministic_gemm_det_amd as dg

    dev = torch.device("cuda:0")
    dg.load_library()
    X, W, dC = Wk.step_inputs(dev)
    assert tuple(X.shape) == (M, K) and tuple(W.shape) == (K, N) and tuple(dC.shape) == (M, N)
    C = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    dX = torch.empty((M, K), dtype=torch.bfloat16, device=dev)
    dW = torch.empty((K, N), dtype=torch.bfloat16, device=dev)
    flop = 2.0 * M * N * K

    def step(ev=None):
        if ev:
            ev[0].record()
        dg.det_gemm_fwd(X, W, out=C)
        if ev:
            ev[1].record()
        dg.det_gemm_da(dC, W, out=dX)
        if ev:
            ev[2].record()
        dg.det_gemm_db(X, dC, out=dW)
        if ev:
            ev[3].record()

    def timed_step_loop():
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)]
                  for _ in range(args.steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.steps):
            step(events[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        per_op = {"fwd": [], "da": [], "db": []}
        for ev in events:
            per_op["fwd"].append(ev[0].elapsed_time(ev[1]))
            per_op["da"].append(ev[1].elapsed_time(ev[2]))
            per_op["db"].append(ev[2].elapsed_time(ev[3]))
        ops = {}
        for name, ts in per_op.items():
            avg = sum(ts) / len(ts)
            med = statistics.median(ts)
            ops[name] = {"ms": round(avg, 4), "tflops": round(flop / (avg * 1e-3) / 1e12, 2),
                         "median_ms": round(med, 4), "min_ms": round(min(ts), 4),
                         "max_ms": round(max(ts), 4)}
        return wall, ops

    if args.profile_only:
        _, ops = timed_step_loop()
        if not args.no_moe:
            moe_leg(dev, args.steps, args.warmup, False, context=False)
        if not args.no_fingerprint:
            fingerprint_leg(dev, args.steps, args.warmup, False)
        if not args.no_rmsnorm:
            rmsnorm_leg(dev, args.steps, args.warmup, False, decode=False)
        if not args.no_attention:
            attention_leg(dev, args.steps, args.warmup, False)
        if not args.no_shard:
            shard_leg(dev, args.steps, args.warmup)
        if not args.no_small_m:
            small_m_leg(dev, args.steps, args.warmup, decode_only=True)
        if args.copy_calibration:
            # 256 MiB read + 256 MiB written per launch, far beyond the caches
            src = torch.ones(COPY_BYTES // 2, dtype=torch.bfloat16, device=dev)
            dst = torch.empty_like(src)
            for _ in range(3):
                dst.copy_(src)
            torch.cuda.synchronize()
        print(json.dumps({"profile_only": True, "ops": ops}))
        return

    # The CPU oracle first, then the other GPU legs, then the headline step: the
    # step is timed once the device has been under load for a while (its clocks
    # at their loaded level), not straight after the host-bound oracle leg.
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(X, W, dC, args.cpu_seconds)
    moe = None if args.no_moe else moe_leg(dev, args.steps, args.warmup, not args.no_cpu)
    fp = None if args.no_fingerprint else fingerprint_leg(dev, args.steps, args.warmup,
                                                          not args.no_cpu)
    norm = None if args.no_rmsnorm else rmsnorm_leg(dev, args.steps, args.warmup, not args.no_cpu)
    attn = None if args.no_attention else attention_leg(dev, args.steps, args.warmup,
                                                        not args.no_cpu)
    shard = None if args.no_shard else shard_leg(dev, args.steps, args.warmup)
    small = None if args.no_small_m else small_m_leg(dev, args.steps, args.warmup)
    others = None if args.no_configs else configs_leg(dev)
    strict = strict_leg(X, W, 256)

    wall, ops = timed_step_loop()
    ms_step = wall * 1e3 / args.steps
    cold = cold_fwd_leg(X, W, C, flop)
    value = 3 * flop / (ms_step * 1e-3) / 1e12
    dom = max(ops, key=lambda k: ops[k]["ms"])
    achieved = ops[dom]["tflops"]
    # the kernels the library selects for these shapes (wide kernel, 128x128 tiles):
    # L = 128 for fwd (R = K) and db (R = M), L = 192 = 3 * 64 for da (R = N)
    kernel_names = {"fwd": "mfma_wide_kernel<K-major X, MN-major Y, bf16 out, 2-leaf units>",
                    "da": "mfma_wide_kernel<K-major X, K-major Y, bf16 out, 3-leaf units>",
                    "db": "mfma_wide_kernel<MN-major X, MN-major Y, bf16 out, 2-leaf units>"}

    # context, not the metric: the nondeterministic library GEMM on the forward shape
    ctx = {}
    try:
        for _ in range(3):
            torch.matmul(X, W)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            torch.matmul(X, W)
        e1.record()
        torch.cuda.synchronize()
        t_mm = e0.elapsed_time(e1) / 10
        ctx = {"torch_matmul_fwd_tflops": round(flop / (t_mm * 1e-3) / 1e12, 1),
               "determinism_tax_fwd_pct": round((ops["fwd"]["ms"] / t_mm - 1) * 100, 1)}
    except Exception as e:  # context only
        ctx = {"torch_matmul_error": str(e)[:120]}

    # Ceilings of the dominant kernel (from the committed counter pass of the
    # same kernels): the clock the chip held under this load, the share of the
    # published peak at that clock, and the two issue ceilings per 16x16 block
    # and leaf -- the matrix core (a leaf MFMA and a tree-add MFMA of 16 cycles
    # each: at most half of its cycles are leaf products) and the VALU issue
    # port (v non-MFMA VALU instructions plus the two MFMA issues, 4 cycles
    # each, against the 16 cycles of the leaf MFMA).
    issue = recorded_issue(dom)
    ceilings = {"mfma_leaf_share": 0.5}
    at_clock = None
    # The issue probe (live, this run): the stage's instruction mix alone, in
    # TFLOP/s of the whole chip at 2 * 128 * 128 * 64 flops per compute unit
    # and stage, at the clock the probe held.
    try:
        probe = issue_probe_leg()
        flops_stage = 2.0 * 128 * 128 * 64 * 256   # leaf flops of one stage on every compute unit
        ceil = flops_stage / (probe["stage_mix"]["ns_per_stage"] * 1e-9) / 1e12
        probe["stage_mix_ceiling_tflops"] = round(ceil, 1)
        probe["mfma_only_ceiling_tflops"] = round(
            flops_stage / (probe["mfma_only"]["ns_per_stage"] * 1e-9) / 1e12, 1)
        probe["frac_of_stage_mix_ceiling"] = round(achieved / ceil, 4)
        ceilings["issue_probe"] = probe
    except Exception as e:  # a ceiling, not the measurement
        ceilings["issue_probe_error"] = str(e)[:120]
    if "sclk_mhz" in issue:
        peak_at_clock = PEAK_BF16_TFLOPS * issue["sclk_mhz"] / CLOCK_MHZ_PEAK
        at_clock = {"sclk_mhz": issue["sclk_mhz"], "source": "counter pass under profiles/",
                    "peak_tflops": round(peak_at_clock, 1),
                    "pct_of_peak_at_measured_clock": round(100 * achieved / peak_at_clock, 2)}
    elif "issue_probe" in ceilings:
        mhz = ceilings["issue_probe"]["sclk_mhz_implied"]
        peak_at_clock = PEAK_BF16_TFLOPS * mhz / CLOCK_MHZ_PEAK
        at_clock = {"sclk_mhz": mhz, "source": "MFMA rate of the issue probe, this run",
                    "peak_tflops": round(peak_at_clock, 1),
                    "pct_of_peak_at_measured_clock": round(100 * achieved / peak_at_clock, 2)}
    if "valu_per_block_leaf" in issue:
        v = issue["valu_per_block_leaf"]
        ceilings["valu_issue"] = round(16.0 / (4.0 * (v + 2.0)), 4)
        ceilings["valu_per_block_leaf"] = v

    line = {
        "metric": "det_gemm TFLOP/s and % of bf16 MFMA peak at M=4096,K=4096,N=6144 (1 GPU)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "det_gemm linear layer step: fwd C=XW, da dX=dC W^T, db dW=X^T dC",
                   "M": M, "K": K, "N": N,
                   "inputs": "X~N(0,1), W~N(0,0.02), dC~N(0,1e-3), bf16, seeded, resident in HBM"},
        "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
        "fwd_tflops": ops["fwd"]["tflops"],
        "ops": ops,
        "fwd_cold_caches": cold,
        "roofline": {"bound": "mfma", "kernel": f"{dom}: {kernel_names[dom]}",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": recorded_traffic(dom),
                     "at_measured_clock": at_clock, "ceilings": ceilings},
        "strict_k1": strict,
        "cpu_baseline": cpu,
        "context": ctx,
        "moe_grouped_gemm": moe,
        "fingerprint": fp,
        "rmsnorm": norm,
        "attention_decode": attn,
        "shard_reduce": shard,
        "small_m": small,
        "other_configs": others,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
