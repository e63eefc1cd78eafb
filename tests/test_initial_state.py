"""GPU parity of the initial-slot-state entry points (nha_fwd_s0, nha_bwd_s0)
against the fp64 oracle on the same inputs: outputs, the exported final state,
and dq, dk, dv, dalpha plus the gradients of the initial states.  Learnable
initial memory-slot states are item 1 of the ai.info page's Future
Directions; S0 is only decayed by absorbing steps (unchanged until t = w)."""
import numpy as np
import pytest
import torch

import oracle
import softmax_attention_nha_amd as nha
from parity_util import TOL, compare, f64, log
from softmax_attention_nha_amd.inputs import WORKLOADS, make_initial_state, make_inputs

pytestmark = pytest.mark.gpu


def run(wl, w, C, base, rel_override=None):
    log("case s0 %s B=%d T=%d H=%d/%d d=%d m=%d w=%d C=%d %s" % (wl.name, wl.B, wl.T, wl.H, wl.Hkv, wl.d, wl.m, w,
                                                               C, wl.dtype))
    d = torch.device("cuda:0")
    q, k, v, a, dO = make_inputs(wl, with_grad=True)
    s0 = make_initial_state(wl)
    qd, kd, vd, ad, dOd = (x.to(d) for x in (q, k, v, a, dO))
    s0d = tuple(x.to(d) for x in s0)
    state = nha.decode_state(wl.B, wl.H, wl.Hkv, wl.d, wl.m, w, base, dtype=wl.dtype, device=d)
    o, lse = nha.fwd(qd, kd, vd, ad, w, C=C, rope_base=base, s0=s0d, state_out=state)
    dq, dk, dv, da, ds0k, ds0v = nha.bwd(qd, kd, vd, ad, o, lse, dOd, w, C=C, rope_base=base, s0=s0d)
    torch.cuda.synchronize()
    s0n = (s0[0].double().numpy(), s0[1].double().numpy())
    o_ref, l_ref, sk_ref, sv_ref = oracle.fwd(f64(q), f64(k), f64(v), f64(a), w, rope_base=base, s0=s0n,
                                              want_state=True)
    g_ref = oracle.bwd(f64(q), f64(k), f64(v), f64(a), f64(dO), w, rope_base=base, s0=s0n, want_ds0=True)
    tol = TOL[wl.dtype]
    compare("o", f64(o), o_ref, tol["o"], tol["rel"])
    compare("lse", f64(lse), l_ref, tol["lse"], tol["rel"])
    n = wl.B * wl.Hkv * wl.m * wl.d
    st = state.cpu()
    off = (n * 4 + 255) // 256 * 256
    compare("SK_T", st[: n * 4].view(torch.float32).double().numpy().reshape(sk_ref.shape), sk_ref, tol["o"],
            tol["rel"])
    compare("SV_T", st[off: off + n * 4].view(torch.float32).double().numpy().reshape(sv_ref.shape), sv_ref,
            tol["o"], tol["rel"])
    for name, x, r in zip(("dq", "dk", "dv", "dalpha", "dS0K", "dS0V"), (dq, dk, dv, da, ds0k, ds0v), g_ref):
        compare(name, f64(x), r, tol["grad"], (rel_override or {}).get(name, tol["rel"]))


@pytest.mark.parametrize("w,C,T", [(0, 16, 150), (17, 32, 150), (40, 64, 300), (200, 16, 150)])
def test_fp32_initial_state(w, C, T):
    wl = WORKLOADS["tiny"].with_(B=2, T=T, H=4, Hkv=2, seed=51)
    run(wl, w, C, wl.rope_base)


@pytest.mark.parametrize("m", [1, 33])
def test_fp32_initial_state_slot_counts(m):
    wl = WORKLOADS["tiny"].with_(B=1, T=130, H=2, Hkv=2, m=m, d=64, seed=52)
    run(wl, 20, 32, wl.rope_base)


@pytest.mark.parametrize("name,w,T", [("340m", 64, 320), ("1p3b", 512, 700), ("1p3b", 0, 300), ("gqa", 256, 400)])
def test_bf16_initial_state(name, w, T):
    wl = WORKLOADS[name].with_(B=1, T=T, H=4 if name != "gqa" else 8, Hkv=2, seed=53)
    run(wl, w, wl.C, wl.rope_base)


def test_bf16_initial_state_segmented_scan():
    """A walk of 385 chunks with 16 state-scan waves: the bf16 scan runs in
    segments (end states from zero, the segments' start states from the
    initial state, then the walk), forward and standalone backward; the
    exported final state comes from the start-state pass."""
    wl = WORKLOADS["1p3b"].with_(B=1, T=24576 + 37, H=2, Hkv=2, seed=58)
    desc = nha.make_desc(wl.B, wl.T, wl.H, wl.Hkv, wl.d, wl.m, 64, wl.C, wl.rope_base, 0.0, wl.dtype)
    assert "scan_combine" in nha.stage_names(desc) and "scan_combine" in nha.stage_names(desc, backward=1)
    run(wl, 64, wl.C, wl.rope_base)


def test_zero_initial_state_equals_plain_forward_and_backward():
    wl = WORKLOADS["1p3b"].with_(B=1, T=333, H=4, Hkv=2, seed=54)
    w = 64
    log("case s0 zero bf16")
    d = torch.device("cuda:0")
    q, k, v, a, dO = (x.to(d) for x in make_inputs(wl, with_grad=True))
    z = (torch.zeros((wl.B, wl.Hkv, wl.m, wl.d), device=d), torch.zeros((wl.B, wl.Hkv, wl.m, wl.d), device=d))
    o1, l1 = nha.fwd(q, k, v, a, w, C=wl.C, rope_base=wl.rope_base)
    o2, l2 = nha.fwd(q, k, v, a, w, C=wl.C, rope_base=wl.rope_base, s0=z)
    g1 = nha.bwd(q, k, v, a, o1, l1, dO, w, C=wl.C, rope_base=wl.rope_base)
    g2 = nha.bwd(q, k, v, a, o2, l2, dO, w, C=wl.C, rope_base=wl.rope_base, s0=z)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for x, y in zip(g1, g2[:4]):
        assert torch.equal(x, y)
