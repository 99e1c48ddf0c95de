"""Seeded synthetic inputs for the MoE layer.

This module only draws random tensors; it holds none of the layer's
arithmetic (no router scores, no top-k, no experts).  Both the HIP path and
the CPU oracle are fed the very same tensors it returns: the oracle receives
host copies of them.

Recipe (every draw is fp32, then scaled, then rounded to the layer's dtype;
torch's fp32->bf16 conversion rounds to nearest-even):
  x  ~ N(0, 1)                 [T][d]
  Wg ~ N(0, 1/d), kept in fp32 [E][d]
  W1, W3 ~ N(0, 1/d)           [E][d_ff][d]
  W2 ~ N(0, 1/d_ff)            [E][d][d_ff]

The skewed workload replaces x by an AR(1) sequence over the token index,
x_t = rho x_{t-1} + sqrt(1 - rho^2) z_t with x_0 = z_0, and adds one fixed
offset mu to every row.  mu is the minimum-norm vector with Wg mu = b, where
b_e = beta * ln p_e and p_e is proportional to (e + 1)^(-s) (a Zipf law,
expert 0 the most popular).  The router has no bias term, so a per-expert
score bias is realised through the input; beta is fixed so that experts 0 and
1 receive about half of all assignments.

Streams: each tensor has its own torch.Generator seeded from
(seed, workload id, tensor id, block).  Draws on a CUDA device and on the CPU
give different numbers for the same seed; every check feeds the oracle copies
of the tensors the device actually used.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import torch

# tensor ids inside a workload's stream space
_X, _WG, _W1, _W3, _W2 = 0, 1, 2, 3, 4

# Fitted by oracle/calibrate_skew.py on CPU draws of the skewed workload
# (T = 16384, seed 0): beta at which experts {0, 1} receive 50% of the
# assignments.
SKEW_BETA = 0.617


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    T: int
    d: int
    d_ff: int
    E: int = 8
    k: int = 2
    dtype: str = "bf16"          # activation and expert-weight dtype
    blocks: int = 1              # >1: stack of h + moe(rmsnorm(h)) blocks
    eps: float = 1e-5            # RMSNorm epsilon (stack only)
    rho: float = 0.0             # AR(1) correlation over tokens (0: i.i.d.)
    zipf_s: float = 0.0          # Zipf exponent of the per-expert bias (0: none)
    beta: float = 0.0            # scale of that bias
    extra: dict = field(default_factory=dict, compare=False)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 0, T=64, d=128, d_ff=448, dtype="f32"),
    "decode": Workload("decode", 1, T=32, d=4096, d_ff=14336),
    "prefill": Workload("prefill", 2, T=4096, d=4096, d_ff=14336),
    "skewed": Workload("skewed", 3, T=16384, d=4096, d_ff=14336, rho=0.9, zipf_s=1.2,
                       beta=SKEW_BETA),
    "stack": Workload("stack", 4, T=2048, d=4096, d_ff=14336, blocks=32, eps=1e-5),
}


def stream_seed(seed: int, wid: int, tensor: int, block: int = 0) -> int:
    """Mix the four stream coordinates into one 63-bit seed."""
    s = 0x9E3779B97F4A7C15
    for v in (seed, wid, tensor, block):
        s = (s ^ (v & 0xFFFFFFFFFFFFFFFF)) * 0xBF58476D1CE4E5B9 & 0xFFFFFFFFFFFFFFFF
        s ^= s >> 31
    return s & 0x7FFFFFFFFFFFFFFF


def _gen(device, seed, wid, tensor, block):
    g = torch.Generator(device=device)
    g.manual_seed(stream_seed(seed, wid, tensor, block))
    return g


def _normal(shape, scale, dtype, device, g, chunk_dim0=False):
    """N(0, scale^2) drawn in fp32 and rounded to dtype (chunked over dim 0 to
    bound the fp32 temporary for large weight stacks)."""
    if not chunk_dim0:
        return (torch.randn(shape, generator=g, device=device, dtype=torch.float32)
                .mul_(scale).to(dtype))
    out = torch.empty(shape, device=device, dtype=dtype)
    for i in range(shape[0]):
        out[i].copy_(torch.randn(shape[1:], generator=g, device=device, dtype=torch.float32)
                     .mul_(scale))
    return out


def zipf_bias(E: int, s: float, beta: float) -> torch.Tensor:
    """b_e = beta * ln p_e with p_e proportional to (e + 1)^(-s), fp64."""
    w = torch.tensor([(e + 1.0) ** (-s) for e in range(E)], dtype=torch.float64)
    p = w / w.sum()
    return beta * torch.log(p)


def min_norm_shift(Wg: torch.Tensor, b: torch.Tensor) -> torch.Tensor:
    """mu = Wg^T (Wg Wg^T)^{-1} b in fp64: the shortest vector with Wg mu = b."""
    W = Wg.double()
    G = W @ W.T
    return W.T @ torch.linalg.solve(G, b.to(W.device, torch.float64))


def make_tokens(w: Workload, device="cpu", seed: int = 0, Wg: torch.Tensor | None = None):
    """Token rows x [T][d] in the workload's dtype."""
    g = _gen(device, seed, w.wid, _X, 0)
    if w.rho == 0.0 and w.zipf_s == 0.0:
        return _normal((w.T, w.d), 1.0, w.torch_dtype, device, g)
    z = torch.randn((w.T, w.d), generator=g, device=device, dtype=torch.float32)
    if w.rho != 0.0:
        c = math.sqrt(1.0 - w.rho * w.rho)
        for t in range(1, w.T):
            z[t].mul_(c).add_(z[t - 1], alpha=w.rho)
    if w.zipf_s != 0.0:
        assert Wg is not None, "the skewed workload needs the gate matrix for its offset"
        mu = min_norm_shift(Wg.to(device), zipf_bias(w.E, w.zipf_s, w.beta))
        z.add_(mu.to(torch.float32))
    return z.to(w.torch_dtype)


def make_weights(w: Workload, device="cpu", seed: int = 0, block: int = 0):
    """Gate (fp32) and stacked expert weights of one block."""
    dt = w.torch_dtype
    Wg = _normal((w.E, w.d), 1.0 / math.sqrt(w.d), torch.float32, device,
                 _gen(device, seed, w.wid, _WG, block))
    big = w.E * w.d * w.d_ff > (1 << 24)
    W1 = _normal((w.E, w.d_ff, w.d), 1.0 / math.sqrt(w.d), dt, device,
                 _gen(device, seed, w.wid, _W1, block), big)
    W3 = _normal((w.E, w.d_ff, w.d), 1.0 / math.sqrt(w.d), dt, device,
                 _gen(device, seed, w.wid, _W3, block), big)
    W2 = _normal((w.E, w.d, w.d_ff), 1.0 / math.sqrt(w.d_ff), dt, device,
                 _gen(device, seed, w.wid, _W2, block), big)
    return dict(Wg=Wg, W1=W1, W3=W3, W2=W2)


def make_layer(w: Workload, device="cpu", seed: int = 0):
    """x plus block-0 weights: everything one layer call needs."""
    wt = make_weights(w, device, seed, 0)
    x = make_tokens(w, device, seed, wt["Wg"])
    return dict(x=x, **wt)


def make_stack(w: Workload, device="cpu", seed: int = 0):
    """h0 and the per-block weights of a stack workload."""
    blocks = [make_weights(w, device, seed, b) for b in range(w.blocks)]
    h0 = make_tokens(w, device, seed, blocks[0]["Wg"])
    return h0, blocks
