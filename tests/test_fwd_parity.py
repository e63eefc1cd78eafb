"""GPU forward parity: the HIP path (through the C ABI) against the fp64 oracle.

Inputs come from softmax_attention_nha_amd.inputs (seeded, synthetic, the
workloads' shapes and distributions); the oracle receives their exact fp64
upcast.  Small cases compare every element; full-size workloads compare one
(batch, KV head) unit -- its query heads -- over a causal prefix the oracle
finishes in seconds (rows t < T' depend only on tokens <= t)."""
import numpy as np
import pytest
import torch

from parity_util import TOL, compare, f64, gpu_fwd, log, oracle_fwd, unit_slice
import softmax_attention_nha_amd as nha
from softmax_attention_nha_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def check_full(wl, w=None, base=None, C=None, **draw):
    w = wl.w if w is None else w
    base = wl.rope_base if base is None else base
    C = wl.C if C is None else C
    log("case %s B=%d T=%d H=%d/%d d=%d m=%d w=%d C=%d base=%g %s %s" % (
        wl.name, wl.B, wl.T, wl.H, wl.Hkv, wl.d, wl.m, w, C, base, wl.dtype, draw))
    q, k, v, a = make_inputs(wl, **draw)
    o, lse = gpu_fwd(q, k, v, a, w, C, base)
    o_ref, l_ref = oracle_fwd(q, k, v, a, w, base)
    tol = TOL[wl.dtype]
    compare("o", f64(o), o_ref, tol["o"], tol["rel"])
    compare("lse", f64(lse), l_ref, tol["lse"], tol["rel"])
    return o, lse


# ---------------------------------------------------------------- fp32 (max-abs 1e-4)
@pytest.mark.parametrize("base", [10000.0, 0.0])
def test_tiny_workload(base):
    check_full(WORKLOADS["tiny"], base=base)


@pytest.mark.parametrize("w", [0, 1, 15, 16, 17, 100, 200, 205])
def test_fp32_window_sweep_ragged_gqa(w):
    wl = WORKLOADS["tiny"].with_(T=200, H=4, Hkv=2, seed=11)
    check_full(wl, w=w)


@pytest.mark.parametrize("C,T,w", [(32, 150, 40), (64, 150, 40), (64, 300, 64), (16, 97, 31)])
def test_fp32_chunk_sizes(C, T, w):
    wl = WORKLOADS["tiny"].with_(T=T, seed=12)
    check_full(wl, w=w, C=C)


@pytest.mark.parametrize("m,d", [(1, 32), (33, 64), (64, 64), (32, 64)])
def test_fp32_slots_and_head_dims(m, d):
    wl = WORKLOADS["tiny"].with_(T=160, m=m, d=d, seed=13)
    check_full(wl, w=24, C=32)


# ---------------------------------------------------------------- bf16, every element at reduced T
@pytest.mark.parametrize("C", [16, 32])
def test_bf16_chunk_sizes_gqa(C):
    # one- and two-wave slot workgroups (C = 16, 32) at d = 128, m = 64 with
    # two query heads per KV head and a ragged last chunk
    wl = WORKLOADS["1p3b"].with_(B=1, T=261, H=4, Hkv=2, seed=14)
    check_full(wl, w=40, C=C)


@pytest.mark.parametrize("name,w", [("340m", None), ("1p3b", 0), ("1p3b", 64), ("1p3b", 512), ("1p3b", 2048),
                                    ("long", None), ("gqa", None)])
def test_bf16_workloads_reduced(name, w):
    wl = WORKLOADS[name]
    wl = wl.with_(B=1, T=576 + 37 if (w is None or w < 600) else 700)
    check_full(wl, w=w)


@pytest.mark.parametrize("d,w,T", [(32, 1, 300), (32, 97, 300), (64, 31, 333), (64, 150, 333), (128, 200, 461),
                                   (128, 17, 140)])
def test_bf16_head_dims_ragged_windows(d, w, T):
    """bf16 at every head dimension with windows that are not a multiple of
    the 64-key tile, so that waves of one query tile need different key tiles
    (and skip the rest) and the band edges fall inside tiles."""
    wl = WORKLOADS["340m"].with_(B=1, T=T, H=4, Hkv=2, d=d, seed=23)
    check_full(wl, w=w)


@pytest.mark.parametrize("B,H,Hkv,d,T,w,fused", [
    (4, 8, 8, 128, 261, 40, True),     # last 128-query tile holds one chunk
    (4, 16, 8, 128, 333, 150, True),   # two query heads per KV head
    (8, 8, 8, 64, 300, 97, True),
    (2, 16, 16, 128, 700, 512, True),  # the window spans several tiles
    (1, 32, 32, 128, 200, 64, True),   # exactly 256 scan waves
    (1, 31, 31, 128, 333, 150, False),  # 248 scan waves: window and slot kernels
    (2, 4, 2, 128, 640, 128, False),
])
def test_bf16_forward_paths(B, H, Hkv, d, T, w, fused):
    """The forward runs both branches in one chunk kernel when the state scan
    has at least 256 waves (B * Hkv * d / 16), else a window kernel beside
    the scan and a slot kernel that merges it: ragged shapes on both sides."""
    wl = WORKLOADS["1p3b"].with_(B=B, T=T, H=H, Hkv=Hkv, d=d, seed=41)
    desc = nha.make_desc(B, T, H, Hkv, d, wl.m, w, wl.C, wl.rope_base, 0.0, wl.dtype)
    names = nha.stage_names(desc)
    assert ("chunk_fwd" in names) == fused and ("slot_fwd" in names) == (not fused), names
    check_full(wl, w=w)


def test_bf16_stress_logits_and_hard_gates():
    wl = WORKLOADS["1p3b"].with_(B=1, T=448, H=2, Hkv=2, seed=21)
    check_full(wl, w=96, qk_scale=1.0, alpha_mu=-2.0)


def test_bf16_gates_that_round_to_one_and_zero():
    wl = WORKLOADS["340m"].with_(B=1, T=320, H=2, Hkv=2, seed=22)
    q, k, v, a = make_inputs(wl)
    a = a.clone()
    a[:, ::7] = 1.0
    a[:, 3::11] = 0.0
    log("case alpha with exact 0/1 entries")
    o, lse = gpu_fwd(q, k, v, a, 64, 64, 10000.0)
    o_ref, l_ref = oracle_fwd(q, k, v, a, 64, 10000.0)
    compare("o", f64(o), o_ref, 2e-2, 1e-2)
    compare("lse", f64(lse), l_ref, 2e-2, 1e-2)


# ---------------------------------------------------------------- full-size workloads, sampled
def check_unit_prefix(wl, w, Tp, b, g):
    G = wl.H // wl.Hkv
    log("case %s full-size B=%d T=%d w=%d: unit b=%d g=%d prefix %d" % (wl.name, wl.B, wl.T, w, b, g, Tp))
    q, k, v, a = make_inputs(wl)
    o, lse = gpu_fwd(q, k, v, a, w, wl.C, wl.rope_base)
    hq = list(range(g * G, (g + 1) * G))
    sl = lambda x, heads: unit_slice(x, b, heads)[:, :Tp]
    o_ref, l_ref = oracle_fwd(sl(q, hq), sl(k, [g]), sl(v, [g]), sl(a, [g]), w, wl.rope_base)
    got_o = f64(o[b:b + 1, :Tp, hq[0]:hq[-1] + 1])
    got_l = f64(lse[b:b + 1, hq[0]:hq[-1] + 1, :Tp])
    tol = TOL[wl.dtype]
    compare("o", got_o, o_ref, tol["o"], tol["rel"])
    compare("lse", got_l, l_ref, tol["lse"], tol["rel"])
    assert torch.isfinite(o.float()).all()


@pytest.mark.parametrize("name,w,Tp", [("340m", None, 2048), ("1p3b", 0, 2048), ("1p3b", 64, 2048),
                                       ("1p3b", 512, 2048), ("1p3b", 2048, 2048), ("long", None, 8192),
                                       ("gqa", None, 2304)])
def test_full_size_workloads_sampled(name, w, Tp):
    wl = WORKLOADS[name]
    check_unit_prefix(wl, wl.w if w is None else w, Tp, wl.B - 1, wl.Hkv - 1)


@pytest.mark.parametrize("T", [16384, 32768])
def test_long_context_lengths_sampled(T):
    wl = WORKLOADS["long"].with_(T=T)
    check_unit_prefix(wl, wl.w, 2048, 0, wl.Hkv // 2)


# ---------------------------------------------------------------- invariants on the GPU path
def test_chunk_size_does_not_change_results():
    wl = WORKLOADS["1p3b"].with_(B=1, T=512, H=2, Hkv=2, seed=31)
    q, k, v, a = make_inputs(wl)
    outs = [gpu_fwd(q, k, v, a, 100, C, 10000.0)[0].float() for C in (16, 32, 64)]
    for x in outs[1:]:
        assert (x - outs[0]).abs().max().item() < 1e-2


@pytest.mark.parametrize("B,H,Hkv", [(1, 8, 2), (4, 32, 8)])
def test_gqa_equals_mha_with_repeated_kv(B, H, Hkv):
    """Bitwise, when both calls take the same forward kernels: the kernel
    choice depends on B * Hkv (window + slot kernels at B = 1 on both sides;
    the one-kernel forward at B = 4 on both), and the two forms round their
    bf16 partials at different points."""
    wl = WORKLOADS["gqa"].with_(B=B, H=H, Hkv=Hkv, T=384, seed=32)
    q, k, v, a = make_inputs(wl)
    G = wl.H // wl.Hkv
    rep = lambda x: x.repeat_interleave(G, dim=2).contiguous()
    names = [nha.stage_names(nha.make_desc(B, wl.T, H, hk, wl.d, wl.m, 128, 64, wl.rope_base, 0.0, wl.dtype))
             for hk in (Hkv, H)]
    assert names[0] == names[1], names
    o1, l1 = gpu_fwd(q, k, v, a, 128, 64, wl.rope_base)
    o2, l2 = gpu_fwd(q, rep(k), rep(v), rep(a), 128, 64, wl.rope_base)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_bitwise_deterministic():
    wl = WORKLOADS["340m"].with_(B=2, T=512, seed=33)
    q, k, v, a = make_inputs(wl)
    r = [gpu_fwd(q, k, v, a, 64, 64, 10000.0) for _ in range(3)]
    for o, l in r[1:]:
        assert torch.equal(o, r[0][0]) and torch.equal(l, r[0][1])
