"""Seeded synthetic inputs for the NHA operator.

This module draws random tensors and nothing else: it holds none of the
operator's arithmetic, so the GPU path and the fp64 oracle can both be fed
from it without sharing any computation.

Workloads (shapes and distributions) -- q, k, v ~ N(0,1)/sqrt(d); alpha =
sigmoid(N(mu, 1)) per token / KV head / slot; dO ~ N(0,1):

  tiny        B=1  H=2  Hkv=2  T=256   d=32  m=8  w=16   C=16  fp32, mu=3
  340m        B=8  H=16 Hkv=16 T=2048  d=64  m=64 w=64   C=64  bf16, mu=4, RoPE 1e4
  1p3b        B=4  H=16 Hkv=16 T=2048  d=128 m=64 w in {0,64,512,2048} C=64 bf16
  long        B=1  H=16 Hkv=16 T in {8192,16384,32768} d=128 m=64 w=512 C=64 bf16
              (+256 decode tokens)
  gqa         B=1  H=32 Hkv=8  T=8192  d=128 m=32 w=2048 C=64 bf16, RoPE 5e5
  headline    B=4  H=16 Hkv=16 T=8192  d=128 m=64 w=512  C=64 bf16 (1.3B layer
              shape at 8K tokens)

Draw order per workload: q, k, v, alpha-logits, dO, each N(0,1) in fp32 from a
CPU torch.Generator with the workload's seed; then q,k,v /= sqrt(d); alpha =
sigmoid(logit + mu); everything is cast to the workload dtype on the CPU with
round-to-nearest-even.  The cast tensors are what both sides consume (the
oracle gets their exact fp64 upcast).
"""
from dataclasses import dataclass, replace

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Hkv: int
    T: int
    d: int
    m: int
    w: int
    C: int
    dtype: torch.dtype
    rope_base: float
    mu: float
    seed: int

    def with_(self, **kw):
        return replace(self, **kw)


WORKLOADS = {
    "tiny": Workload("tiny", 1, 2, 2, 256, 32, 8, 16, 16, torch.float32, 10000.0, 3.0, 0),
    "340m": Workload("340m", 8, 16, 16, 2048, 64, 64, 64, 64, torch.bfloat16, 10000.0, 4.0, 1),
    "1p3b": Workload("1p3b", 4, 16, 16, 2048, 128, 64, 512, 64, torch.bfloat16, 10000.0, 4.0, 2),
    "long": Workload("long", 1, 16, 16, 8192, 128, 64, 512, 64, torch.bfloat16, 10000.0, 4.0, 3),
    "gqa": Workload("gqa", 1, 32, 8, 8192, 128, 32, 2048, 64, torch.bfloat16, 500000.0, 4.0, 4),
    "headline": Workload("headline", 4, 16, 16, 8192, 128, 64, 512, 64, torch.bfloat16, 10000.0, 4.0, 2),
}


def make_inputs(wl: Workload, T_total=None, with_grad=False, alpha_mu=None, qk_scale=None):
    """Draw (q, k, v, alpha[, dO]) on the CPU in the workload dtype.

    T_total overrides the drawn length (e.g. T + decode tokens; every prefix of
    a longer draw is the shorter workload's input only if drawn in one go, so
    callers that need prefixes draw once at the longest length).
    alpha_mu overrides the gate-logit mean (stress tests use -2).
    qk_scale overrides the 1/sqrt(d) scaling of q and k (stress tests use 1).
    """
    T = wl.T if T_total is None else T_total
    g = torch.Generator(device="cpu").manual_seed(wl.seed)
    shp_q = (wl.B, T, wl.H, wl.d)
    shp_k = (wl.B, T, wl.Hkv, wl.d)
    shp_a = (wl.B, T, wl.Hkv, wl.m)
    q = torch.randn(shp_q, generator=g, dtype=torch.float32)
    k = torch.randn(shp_k, generator=g, dtype=torch.float32)
    v = torch.randn(shp_k, generator=g, dtype=torch.float32)
    a = torch.randn(shp_a, generator=g, dtype=torch.float32)
    dO = torch.randn(shp_q, generator=g, dtype=torch.float32) if with_grad else None
    sq = (1.0 / wl.d ** 0.5) if qk_scale is None else qk_scale
    q = q * sq
    k = k * sq
    v = v / wl.d ** 0.5
    mu = wl.mu if alpha_mu is None else alpha_mu
    a = torch.sigmoid(a + mu)
    out = [x.to(wl.dtype).contiguous() for x in (q, k, v, a)]
    if with_grad:
        out.append(dO.to(wl.dtype).contiguous())
    return tuple(out)


def make_initial_state(wl: Workload, seed_offset=1000):
    """Initial slot states (S0K, S0V), each float32 [B, Hkv, m, d] ~ N(0,1)/sqrt(d)
    (the scale of the keys and values), from their own seeded generator."""
    g = torch.Generator(device="cpu").manual_seed(wl.seed + seed_offset)
    shp = (wl.B, wl.Hkv, wl.m, wl.d)
    s0k = torch.randn(shp, generator=g, dtype=torch.float32) / wl.d ** 0.5
    s0v = torch.randn(shp, generator=g, dtype=torch.float32) / wl.d ** 0.5
    return s0k.contiguous(), s0v.contiguous()


def make_lam(wl: Workload, T_total=None, seed_offset=2000):
    """Fusion coefficients for the weighted-fusion ablation: float32 [B, T, H],
    sigmoid(N(0, 1)) per (token, head), from their own seeded generator."""
    T = wl.T if T_total is None else T_total
    g = torch.Generator(device="cpu").manual_seed(wl.seed + seed_offset)
    return torch.sigmoid(torch.randn((wl.B, T, wl.H), generator=g, dtype=torch.float32)).contiguous()
