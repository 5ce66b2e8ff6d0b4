"""Seeded synthetic inputs for det_gemm -- shared by tests and the benchmark.

Holds no det_gemm arithmetic: it only draws bf16 tensors from seeds.  Every
tensor is ``torch.randn(shape) * sigma`` in float32 from a seeded
``torch.Generator`` on the requested device, rounded to bfloat16 by torch's
round-to-nearest-even conversion.  CPU and GPU generators give different
numbers for the same seed; within one run both the HIP path and the oracle see
the same tensor.

The shapes stand in for the transformer GEMMs the det_gemm page motivates
(QKV projection, MLP, LM head; section "Why"): activations ~N(0, 1),
weights ~N(0, 0.02), upstream gradients ~N(0, 1e-3).
"""
from dataclasses import dataclass

import numpy as np
import torch

# Headline: QKV projection, hidden 4096 -> Q 4096 + K 1024 + V 1024.
QKV_K = 4096
QKV_N = 6144
HEADLINE_M = 4096

# MLP: gate+up 4096 -> 2*12288, down 12288 -> 4096.
MLP_M = 8192
MLP_H = 4096
MLP_I = 12288

# Backward shapes.
BWD_M, BWD_K, BWD_N = 8192, 4096, 4096

# LM head.
LM_K, LM_N = 4096, 151936
# Deepest reduction the contract allows.
DEEP_M, DEEP_K, DEEP_N = 2048, 32768, 4096


def randn_bf16(shape, sigma, seed, device="cpu"):
    """bf16 tensor of N(0, sigma^2) samples drawn from ``seed``."""
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    x = torch.randn(tuple(shape), generator=g, device=device, dtype=torch.float32)
    if sigma != 1.0:
        x.mul_(sigma)
    return x.to(torch.bfloat16)


def int_bf16(shape, seed, values=(-1, 0, 1), device="cpu"):
    """bf16 tensor with entries drawn uniformly from the small integers ``values``."""
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    v = torch.tensor(values, dtype=torch.float32)
    idx = torch.randint(0, len(values), tuple(shape), generator=g)
    return v[idx].to(torch.bfloat16).to(device)


def randperm(n, seed):
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return torch.randperm(n, generator=g)


def bits(t):
    """bf16 torch tensor (any device) -> numpy uint16 bit patterns (host copy)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def from_bits(a, device="cpu"):
    """numpy uint16 bit patterns -> bf16 torch tensor."""
    a = np.ascontiguousarray(a, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)


# ---------------------------------------------------------------- recipes


def small_forward(device="cpu"):
    """A[64,256] and B[256,128], both ~N(0,1)."""
    return randn_bf16((64, 256), 1.0, 1001, device), randn_bf16((256, 128), 1.0, 1002, device)


@dataclass
class QKVBatch:
    x: torch.Tensor          # [M, 4096] activations with the probe rows embedded
    positions: torch.Tensor  # where probe p sits in x (int64, length <= 16)


def qkv_weight(device="cpu", transposed=False):
    """QKV weight [4096, 6144] ~N(0, 0.02) (or its [6144, 4096] transpose, same values)."""
    w = randn_bf16((QKV_K, QKV_N), 0.02, 2001, device)
    return w.t().contiguous() if transposed else w


def qkv_probes(device="cpu"):
    """The 16 probe rows [16, 4096] ~N(0,1) that are checked across batch sizes."""
    return randn_bf16((16, QKV_K), 1.0, 2002, device)


def qkv_batch(M, device="cpu", probes=None):
    """An [M, 4096] activation batch holding the probes at seeded positions.

    M >= 16: filler rows ~N(0,1) (seed 2003+M) with probe p at row
    ``randperm(M, 2099+M)[p]``.  M < 16: the first M probes in order."""
    if probes is None:
        probes = qkv_probes(device)
    if M < 16:
        return QKVBatch(probes[:M].clone(), torch.arange(M))
    x = randn_bf16((M, QKV_K), 1.0, 2003 + M, device)
    pos = randperm(M, 2099 + M)[:16]
    x[pos.to(x.device)] = probes
    return QKVBatch(x, pos)


def mlp_inputs(device="cpu"):
    """(X[8192,4096], Wgu[4096,24576], H[8192,12288], Wd[12288,4096])."""
    return (randn_bf16((MLP_M, MLP_H), 1.0, 3001, device),
            randn_bf16((MLP_H, 2 * MLP_I), 0.02, 3002, device),
            randn_bf16((MLP_M, MLP_I), 1.0, 3003, device),
            randn_bf16((MLP_I, MLP_H), 0.02, 3004, device))


def backward_inputs(device="cpu", M=BWD_M, K=BWD_K, N=BWD_N):
    """(A[M,K] ~N(0,1), B[K,N] ~N(0,0.02), dC[M,N] ~N(0,1e-3))."""
    return (randn_bf16((M, K), 1.0, 4001, device),
            randn_bf16((K, N), 0.02, 4002, device),
            randn_bf16((M, N), 1e-3, 4003, device))


def step_inputs(device="cpu"):
    """The linear-layer step the benchmark times, at the QKV shape:
    (X[4096,4096] ~N(0,1), W[4096,6144] ~N(0,0.02), dC[4096,6144] ~N(0,1e-3));
    fwd C = X W, da dX = dC W^T, db dW = X^T dC."""
    return (randn_bf16((HEADLINE_M, QKV_K), 1.0, 4001, device),
            randn_bf16((QKV_K, QKV_N), 0.02, 2001, device),
            randn_bf16((HEADLINE_M, QKV_N), 1e-3, 4003, device))


def lm_head_inputs(device="cpu", M=4096):
    """(X[M,4096] ~N(0,1), Wlm[4096,151936] ~N(0,0.02))."""
    return (randn_bf16((M, LM_K), 1.0, 5001, device),
            randn_bf16((LM_K, LM_N), 0.02, 5002, device))


def deep_inputs(device="cpu"):
    """(A[2048,32768] ~N(0,1), B[32768,4096] ~N(0,0.02)): the 32768 depth cap."""
    return (randn_bf16((DEEP_M, DEEP_K), 1.0, 5003, device),
            randn_bf16((DEEP_K, DEEP_N), 0.02, 5004, device))


# ---------------------------------------------------------------- MoE grouped GEMM
# Expert down projection of a top-2 MoE layer: 4096 tokens routed to 2 of 8
# experts give 8192 rows grouped by expert; expert width 2048 -> model width
# 4096.  The routing is skewed (expert e drawn with weight (e+1)^-1/2), as a
# learned router's load is uneven.
MOE_TOKENS, MOE_TOPK, MOE_E = 4096, 2, 8
MOE_K, MOE_N = 2048, 4096


@dataclass
class MoEInputs:
    x: torch.Tensor       # [T, K] expert inputs, rows grouped by expert
    w: torch.Tensor       # [E, K, N] expert weights
    g: torch.Tensor       # [T, N] gradient of each row's expert output (its token's)
    offsets: list         # E + 1 row offsets
    token: torch.Tensor   # token of each grouped row (int64, CPU)


def moe_routing(tokens, topk, E, seed, skew=0.5):
    """Seeded top-k routing: each token draws topk distinct experts with weights
    (e+1)^-skew.  Returns (offsets [E+1], token of each row, expert of each row)
    with rows sorted by expert (stable: ascending token within an expert)."""
    gen = torch.Generator(device="cpu")
    gen.manual_seed(int(seed))
    w = torch.arange(1, E + 1, dtype=torch.float64).pow(-skew)
    picks = torch.multinomial(w.expand(tokens, E).contiguous(), topk, replacement=False,
                              generator=gen)
    expert = picks.reshape(-1)
    token = torch.arange(tokens).repeat_interleave(topk)
    order = torch.sort(expert, stable=True).indices
    counts = torch.bincount(expert, minlength=E)
    offsets = [0] + torch.cumsum(counts, 0).tolist()
    return offsets, token[order], expert[order]


def moe_inputs(device="cpu", tokens=MOE_TOKENS, topk=MOE_TOPK, E=MOE_E, K=MOE_K, N=MOE_N,
               seed=6000):
    """X ~N(0,1) [T,K], W ~N(0,0.02) [E,K,N], G = dO[token of the row] with
    dO ~N(0,1e-3) [tokens,N]."""
    offsets, token, _ = moe_routing(tokens, topk, E, seed)
    T = offsets[-1]
    x = randn_bf16((T, K), 1.0, seed + 1, device)
    w = randn_bf16((E, K, N), 0.02, seed + 2, device)
    dO = randn_bf16((tokens, N), 1e-3, seed + 3, device)
    g = dO[token.to(dO.device)].contiguous()
    return MoEInputs(x, w, g, offsets, token)
