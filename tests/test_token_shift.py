"""GPU parity of the token-shift ablation (no_token_shift = 1: every token
enters the slots at its own step while the window still holds it; the ai.info
page's findings list the token shift among the parts NHA needs) against the
fp64 oracle run with the same switch: forward, lse, dq/dk/dv/dalpha and the
recurrent decode step."""
import pytest
import torch

import oracle
import softmax_attention_nha_amd as nha
from parity_util import TOL, compare, f64, log
from softmax_attention_nha_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def run(wl, w, C):
    log("case no-token-shift %s B=%d T=%d H=%d/%d d=%d m=%d w=%d C=%d %s" % (
        wl.name, wl.B, wl.T, wl.H, wl.Hkv, wl.d, wl.m, w, C, wl.dtype))
    d = torch.device("cuda:0")
    q, k, v, a, dO = make_inputs(wl, with_grad=True)
    qd, kd, vd, ad, dOd = (x.to(d) for x in (q, k, v, a, dO))
    o, lse = nha.fwd(qd, kd, vd, ad, w, C=C, rope_base=wl.rope_base, token_shift=False)
    g = nha.bwd(qd, kd, vd, ad, o, lse, dOd, w, C=C, rope_base=wl.rope_base, token_shift=False)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.fwd(f64(q), f64(k), f64(v), f64(a), w, rope_base=wl.rope_base, token_shift=False)
    g_ref = oracle.bwd(f64(q), f64(k), f64(v), f64(a), f64(dO), w, rope_base=wl.rope_base, token_shift=False)
    tol = TOL[wl.dtype]
    compare("o", f64(o), o_ref, tol["o"], tol["rel"])
    compare("lse", f64(lse), l_ref, tol["lse"], tol["rel"])
    for name, x, r in zip(("dq", "dk", "dv", "dalpha"), g, g_ref):
        compare(name, f64(x), r, tol["grad"], tol["rel"])


@pytest.mark.parametrize("w,C", [(1, 16), (16, 16), (17, 32), (40, 64), (200, 16)])
def test_fp32_no_token_shift(w, C):
    run(WORKLOADS["tiny"].with_(B=2, T=150, H=4, Hkv=2, seed=81), w, C)


@pytest.mark.parametrize("name,w,T", [("340m", 64, 320), ("1p3b", 512, 700), ("gqa", 256, 400)])
def test_bf16_no_token_shift(name, w, T):
    run(WORKLOADS[name].with_(B=1, T=T, H=4 if name != "gqa" else 8, Hkv=2, seed=82), w, WORKLOADS[name].C)


def test_no_token_shift_decode():
    wl = WORKLOADS["tiny"].with_(H=4, Hkv=2, seed=83)
    T0, steps, w = 64, 24, 16
    log("case no-token-shift decode fp32 T0=%d w=%d" % (T0, w))
    d = torch.device("cuda:0")
    q, k, v, a = make_inputs(wl, T_total=T0 + steps)
    state = nha.decode_state(wl.B, wl.H, wl.Hkv, wl.d, wl.m, w, wl.rope_base, dtype=wl.dtype, device=d)
    nha.fwd(*(x[:, :T0].contiguous().to(d) for x in (q, k, v, a)), w, C=wl.C, rope_base=wl.rope_base,
            state_out=state, token_shift=False)
    qd, kd, vd, ad = (x.to(d) for x in (q, k, v, a))
    outs = [nha.decode_step(qd[:, t].contiguous(), kd[:, t].contiguous(), vd[:, t].contiguous(), ad[:, t].contiguous(),
                            state, w, rope_base=wl.rope_base, token_shift=False) for t in range(T0, T0 + steps)]
    torch.cuda.synchronize()
    o_ref, _ = oracle.fwd(f64(q), f64(k), f64(v), f64(a), w, rope_base=wl.rope_base, token_shift=False)
    compare("o_dec", f64(torch.stack(outs, 1)), o_ref[:, T0:], TOL[torch.float32]["o"], TOL[torch.float32]["rel"])


def test_without_window_the_switch_changes_nothing():
    wl = WORKLOADS["1p3b"].with_(B=1, T=200, H=2, Hkv=2, seed=84)
    d = torch.device("cuda:0")
    q, k, v, a = (x.to(d) for x in make_inputs(wl))
    o1, l1 = nha.fwd(q, k, v, a, 0, C=wl.C, rope_base=wl.rope_base)
    o2, l2 = nha.fwd(q, k, v, a, 0, C=wl.C, rope_base=wl.rope_base, token_shift=False)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
