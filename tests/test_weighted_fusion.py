"""GPU parity of the weighted-fusion ablation (nha_fwd_weighted /
nha_bwd_weighted: separate slot and window softmaxes, o = lam o_slot +
(1 - lam) o_window) against the fp64 oracle's switch for it, including the
coefficient's gradient dlam."""
import numpy as np
import pytest
import torch

import oracle
import softmax_attention_nha_amd as nha
from parity_util import TOL, compare, f64, log, oracle_units
from softmax_attention_nha_amd.inputs import WORKLOADS, make_inputs, make_lam

pytestmark = pytest.mark.gpu


def gpu_weighted(q, k, v, a, lam, dO, w, C, base, want_dlam=True):
    d = torch.device("cuda:0")
    qd, kd, vd, ad, ld = (x.to(d) for x in (q, k, v, a, lam))
    o, lse2 = nha.fwd_weighted(qd, kd, vd, ad, ld, w, C=C, rope_base=base)
    g = nha.bwd_weighted(qd, kd, vd, ad, ld, dO.to(d), w, C=C, rope_base=base, want_dlam=want_dlam)
    torch.cuda.synchronize()
    return o, lse2, g


def check_all(wl, w, lam=None, want_dlam=True):
    log("case weighted %s B=%d T=%d H=%d/%d d=%d m=%d w=%d C=%d %s" % (
        wl.name, wl.B, wl.T, wl.H, wl.Hkv, wl.d, wl.m, w, wl.C, wl.dtype))
    q, k, v, a, dO = make_inputs(wl, with_grad=True)
    lam = make_lam(wl) if lam is None else lam
    o, lse2, g = gpu_weighted(q, k, v, a, lam, dO, w, wl.C, wl.rope_base, want_dlam)
    tol = TOL[wl.dtype]
    o_ref, l_ref = oracle.fwd(f64(q), f64(k), f64(v), f64(a), w, rope_base=wl.rope_base, lam=f64(lam))
    compare("o", f64(o), o_ref, tol["o"], tol["rel"])
    compare("lse2", f64(lse2), l_ref, tol["lse"], tol["rel"])
    ref = oracle.bwd(f64(q), f64(k), f64(v), f64(a), f64(dO), w, rope_base=wl.rope_base, lam=f64(lam))
    names = ("dq", "dk", "dv", "dalpha", "dlam")
    for name, x, r in zip(names, g, ref):
        if x is None:
            assert name == "dlam" and not want_dlam
            continue
        compare(name, f64(x), r, tol["grad"], tol["rel"])


@pytest.mark.parametrize("w", [1, 16, 100, 205])
def test_fp32_window_sweep_gqa(w):
    check_all(WORKLOADS["tiny"].with_(T=200, H=4, Hkv=2, seed=91), w)


@pytest.mark.parametrize("name,w", [("340m", 64), ("1p3b", 512), ("gqa", 300)])
def test_bf16_workloads_reduced(name, w):
    check_all(WORKLOADS[name].with_(B=1, T=661, seed=92), w)


def test_bf16_fixed_coefficient_without_its_gradient():
    wl = WORKLOADS["1p3b"].with_(B=1, T=333, H=4, Hkv=2, seed=93)
    check_all(wl, 96, lam=torch.full((wl.B, wl.T, wl.H), 0.5), want_dlam=False)


def test_headline_shape_sampled_units():
    """B = 4, T = 8192, w = 512: two whole units, every row, fwd + bwd."""
    wl = WORKLOADS["headline"]
    units, G, w = [(0, 2), (wl.B - 1, wl.Hkv - 1)], 1, wl.w
    log("case weighted headline units=%s" % units)
    q, k, v, a, dO = make_inputs(wl, with_grad=True)
    lam = make_lam(wl)
    o, lse2, g = gpu_weighted(q, k, v, a, lam, dO, w, wl.C, wl.rope_base)
    tol = TOL[wl.dtype]
    rf = oracle_units(q, k, v, a, None, w, wl.rope_base, units, G, lam=lam)
    rb = oracle_units(q, k, v, a, dO, w, wl.rope_base, units, G, lam=lam)
    cat = lambda xs: np.concatenate(xs)
    compare("o", cat([f64(o[b:b + 1, :, hg:hg + 1]) for b, hg in units]), cat([r[0] for r in rf]), tol["o"],
            tol["rel"])
    compare("lse2", cat([f64(lse2[:, b:b + 1, hg:hg + 1]) for b, hg in units]), cat([r[1] for r in rf]),
            tol["lse"], tol["rel"])
    sl = [lambda x, b, hg: x[b:b + 1, :, hg:hg + 1]] * 4 + [lambda x, b, hg: x[b:b + 1, :, hg:hg + 1]]
    for i, name in enumerate(("dq", "dk", "dv", "dalpha", "dlam")):
        got = cat([f64(sl[i](g[i], b, hg)) for b, hg in units])
        compare(name, got, cat([r[i] for r in rb]), tol["grad"], tol["rel"])


def test_weighted_equals_unified_parts():
    """Internal consistency on the GPU: lam = 0 gives the window read alone,
    which is the no-slot (m = 0) forward of the same q, k, v."""
    wl = WORKLOADS["340m"].with_(B=1, T=300, H=4, Hkv=2, seed=94)
    w = 64
    q, k, v, a = (x.to("cuda:0") for x in make_inputs(wl))
    o0, lse2 = nha.fwd_weighted(q, k, v, a, torch.zeros(wl.B, wl.T, wl.H, device="cuda:0"), w, rope_base=wl.rope_base)
    a0 = torch.empty(wl.B, wl.T, wl.Hkv, 0, dtype=a.dtype, device="cuda:0")
    ow, lw = nha.fwd(q, k, v, a0, w, rope_base=wl.rope_base)
    torch.cuda.synchronize()
    assert torch.equal(o0, ow)
    assert torch.equal(lse2[1], lw)
