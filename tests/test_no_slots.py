"""GPU parity of the no-slot ablation (m = 0: the layer reduces to sliding-
window causal softmax attention with RoPE, the pure-window end of its range on
the gist.science page's flexibility section) against the fp64 oracle, whose
m = 0 case is pinned to torch's scaled_dot_product_attention: forward, lse,
dq/dk/dv, and the recurrent decode step."""
import pytest
import torch

import softmax_attention_nha_amd as nha
from parity_util import TOL, compare, f64, gpu_fwd, log, oracle_fwd
from softmax_attention_nha_amd.inputs import WORKLOADS, make_inputs

import oracle

pytestmark = pytest.mark.gpu


def run(wl, w, C):
    log("case no-slots %s B=%d T=%d H=%d/%d d=%d w=%d C=%d %s" % (wl.name, wl.B, wl.T, wl.H, wl.Hkv, wl.d, w, C,
                                                                wl.dtype))
    d = torch.device("cuda:0")
    q, k, v, a, dO = make_inputs(wl.with_(m=0), with_grad=True)
    assert a.shape[-1] == 0
    qd, kd, vd, ad, dOd = (x.to(d) for x in (q, k, v, a, dO))
    o, lse = nha.fwd(qd, kd, vd, ad, w, C=C, rope_base=wl.rope_base)
    dq, dk, dv, da = nha.bwd(qd, kd, vd, ad, o, lse, dOd, w, C=C, rope_base=wl.rope_base)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.fwd(f64(q), f64(k), f64(v), f64(a), w, rope_base=wl.rope_base)
    g_ref = oracle.bwd(f64(q), f64(k), f64(v), f64(a), f64(dO), w, rope_base=wl.rope_base)
    tol = TOL[wl.dtype]
    compare("o", f64(o), o_ref, tol["o"], tol["rel"])
    compare("lse", f64(lse), l_ref, tol["lse"], tol["rel"])
    for name, x, r in zip(("dq", "dk", "dv"), (dq, dk, dv), g_ref):
        compare(name, f64(x), r, tol["grad"], tol["rel"])
    assert da.numel() == 0


@pytest.mark.parametrize("w,C", [(1, 16), (17, 32), (64, 64), (200, 16)])
def test_fp32_no_slots(w, C):
    run(WORKLOADS["tiny"].with_(B=2, T=150, H=4, Hkv=2, seed=71), w, C)


@pytest.mark.parametrize("name,w,T", [("340m", 64, 320), ("1p3b", 512, 700), ("gqa", 256, 400)])
def test_bf16_no_slots(name, w, T):
    run(WORKLOADS[name].with_(B=1, T=T, H=4 if name != "gqa" else 8, Hkv=2, seed=72), w, WORKLOADS[name].C)


def test_no_slots_decode():
    wl = WORKLOADS["tiny"].with_(H=4, Hkv=2, m=0, seed=73)
    T0, steps, w = 64, 24, 16
    log("case no-slots decode fp32 T0=%d w=%d" % (T0, w))
    d = torch.device("cuda:0")
    q, k, v, a = make_inputs(wl, T_total=T0 + steps)
    state = nha.decode_state(wl.B, wl.H, wl.Hkv, wl.d, 0, w, wl.rope_base, dtype=wl.dtype, device=d)
    gpu_fwd(q[:, :T0].contiguous(), k[:, :T0].contiguous(), v[:, :T0].contiguous(), a[:, :T0].contiguous(), w, wl.C,
            wl.rope_base, state_out=state)
    qd, kd, vd, ad = (x.to(d) for x in (q, k, v, a))
    outs = [nha.decode_step(qd[:, t].contiguous(), kd[:, t].contiguous(), vd[:, t].contiguous(), ad[:, t].contiguous(),
                            state, w, rope_base=wl.rope_base) for t in range(T0, T0 + steps)]
    torch.cuda.synchronize()
    o_ref, _ = oracle_fwd(q, k, v, a, w, wl.rope_base)
    compare("o_dec", f64(torch.stack(outs, 1)), o_ref[:, T0:], TOL[torch.float32]["o"], TOL[torch.float32]["rel"])
