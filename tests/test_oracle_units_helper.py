"""CPU check of the test helper that runs the fp64 oracle one query head at a
time (parity_util.oracle_units): on a small grouped-query case its outputs and
gradients equal the oracle's own grouped call."""
import numpy as np
import torch

import oracle
from parity_util import f64, oracle_units
from softmax_attention_nha_amd.inputs import WORKLOADS, make_inputs


def test_per_head_oracle_equals_grouped_oracle():
    wl = WORKLOADS["gqa"].with_(B=2, T=70, H=8, Hkv=2, d=32, m=5, C=16, dtype=torch.float32, seed=3)
    q, k, v, a, dO = make_inputs(wl, with_grad=True)
    w, G, base = 9, 4, wl.rope_base
    units = [(0, 1), (1, 0)]
    o, lse = oracle.fwd(f64(q), f64(k), f64(v), f64(a), w, rope_base=base)
    dq, dk, dv, da = oracle.bwd(f64(q), f64(k), f64(v), f64(a), f64(dO), w, rope_base=base)
    rf = oracle_units(q, k, v, a, None, w, base, units, G)
    rb = oracle_units(q, k, v, a, dO, w, base, units, G)
    rp = oracle_units(q, k, v, a, None, w, base, units, G, Tp=33)
    for (b, g), (oo, ll), (gq, gk, gv, ga), (po, pl) in zip(units, rf, rb, rp):
        hs = slice(g * G, (g + 1) * G)
        np.testing.assert_allclose(oo, o[b:b + 1, :, hs], rtol=0, atol=1e-12)
        np.testing.assert_allclose(ll, lse[b:b + 1, hs], rtol=0, atol=1e-12)
        np.testing.assert_allclose(po, o[b:b + 1, :33, hs], rtol=0, atol=1e-12)
        np.testing.assert_allclose(pl, lse[b:b + 1, hs, :33], rtol=0, atol=1e-12)
        np.testing.assert_allclose(gq, dq[b:b + 1, :, hs], rtol=0, atol=1e-12)
        np.testing.assert_allclose(gk, dk[b:b + 1, :, g:g + 1], rtol=0, atol=1e-12)
        np.testing.assert_allclose(gv, dv[b:b + 1, :, g:g + 1], rtol=0, atol=1e-12)
        np.testing.assert_allclose(ga, da[b:b + 1, :, g:g + 1], rtol=0, atol=1e-12)


def test_per_head_oracle_equals_grouped_oracle_weighted_fusion():
    from softmax_attention_nha_amd.inputs import make_lam

    wl = WORKLOADS["gqa"].with_(B=2, T=40, H=4, Hkv=2, d=32, m=5, C=16, dtype=torch.float32, seed=5)
    q, k, v, a, dO = make_inputs(wl, with_grad=True)
    lam = make_lam(wl)
    w, G, base = 7, 2, wl.rope_base
    units = [(1, 1), (0, 0)]
    o, lse = oracle.fwd(f64(q), f64(k), f64(v), f64(a), w, rope_base=base, lam=f64(lam))
    g = oracle.bwd(f64(q), f64(k), f64(v), f64(a), f64(dO), w, rope_base=base, lam=f64(lam))
    rf = oracle_units(q, k, v, a, None, w, base, units, G, lam=lam)
    rb = oracle_units(q, k, v, a, dO, w, base, units, G, lam=lam)
    for (b, gg), (oo, ll), grads in zip(units, rf, rb):
        hs = slice(gg * G, (gg + 1) * G)
        np.testing.assert_allclose(oo, o[b:b + 1, :, hs], rtol=0, atol=1e-12)
        np.testing.assert_allclose(ll, lse[:, b:b + 1, hs], rtol=0, atol=1e-12)
        np.testing.assert_allclose(grads[0], g[0][b:b + 1, :, hs], rtol=0, atol=1e-12)
        np.testing.assert_allclose(grads[1], g[1][b:b + 1, :, gg:gg + 1], rtol=0, atol=1e-12)
        np.testing.assert_allclose(grads[3], g[3][b:b + 1, :, gg:gg + 1], rtol=0, atol=1e-12)
        np.testing.assert_allclose(grads[4], g[4][b:b + 1, :, hs], rtol=0, atol=1e-12)
