"""GPU parity of chunked prefill (nha_fwd_continue / nha_bwd_continue): a
sequence cut into segments, each continuing the decode state the previous
one left, against the fp64 oracle over the whole sequence."""
import numpy as np
import pytest
import torch

import oracle
import softmax_attention_nha_amd as nha
from parity_util import TOL, compare, f64, log
from softmax_attention_nha_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def state_slots(state, wl):
    """(SK, SV) float64 [B,Hkv,m,d] of a decode state (its first two regions)."""
    n = wl.B * wl.Hkv * wl.m * wl.d
    st = state.cpu()
    off = (n * 4 + 255) // 256 * 256
    sk = st[: n * 4].view(torch.float32).double().numpy().reshape(wl.B, wl.Hkv, wl.m, wl.d)
    sv = st[off: off + n * 4].view(torch.float32).double().numpy().reshape(wl.B, wl.Hkv, wl.m, wl.d)
    return sk, sv


def run_segments(wl, w, cuts, q, k, v, a):
    """fwd over the first segment (exporting the state), then fwd_continue for
    every later one (state updated in place).  Returns (o, lse) over the
    whole sequence and the final state."""
    qd, kd, vd, ad = (x.to(DEV) for x in (q, k, v, a))
    state = nha.decode_state(wl.B, wl.H, wl.Hkv, wl.d, wl.m, w, wl.rope_base, dtype=wl.dtype, device=DEV)
    bounds = [0] + list(cuts) + [q.shape[1]]
    os, ls = [], []
    for i in range(len(bounds) - 1):
        t0, t1 = bounds[i], bounds[i + 1]
        if t1 == t0:  # an empty first segment: the next one continues the zero state at position 0
            continue
        seg = [x[:, t0:t1].contiguous() for x in (qd, kd, vd, ad)]
        if i == 0:
            o, lse = nha.fwd(*seg, w, C=wl.C, rope_base=wl.rope_base, state_out=state)
        else:
            o, lse = nha.fwd_continue(*seg, w, state, t0, C=wl.C, rope_base=wl.rope_base, state_out=state)
        os.append(o)
        ls.append(lse)
    torch.cuda.synchronize()
    return torch.cat(os, 1), torch.cat(ls, 2), state


@pytest.mark.parametrize("w,cuts", [(16, [5]), (16, [64]), (16, [0, 100]), (40, [17, 18, 150]), (0, [33]),
                                    (300, [120])])
def test_fp32_segments_equal_whole_sequence(w, cuts):
    wl = WORKLOADS["tiny"].with_(T=200, H=4, Hkv=2, seed=101)
    log("case continue fp32 w=%d cuts=%s" % (w, cuts))
    q, k, v, a = make_inputs(wl)
    o, lse, state = run_segments(wl, w, cuts, q, k, v, a)
    o_ref, l_ref, sk, sv = oracle.fwd(f64(q), f64(k), f64(v), f64(a), w, rope_base=wl.rope_base, want_state=True)
    tol = TOL[torch.float32]
    compare("o", f64(o), o_ref, tol["o"], tol["rel"])
    compare("lse", f64(lse), l_ref, tol["lse"], tol["rel"])
    gk, gv = state_slots(state, wl)
    compare("SK", gk, sk, 1e-5, 1e-5)
    compare("SV", gv, sv, 1e-5, 1e-5)


def test_bf16_segments_then_decode():
    """1.3B head shape, three segments (cuts inside and beyond the window),
    then 24 decode steps from the last segment's state."""
    wl = WORKLOADS["long"].with_(T=1500, H=4, Hkv=2, seed=102)
    w, steps = 512, 24
    log("case continue bf16 + decode")
    q, k, v, a = make_inputs(wl, T_total=wl.T + steps)
    o, lse, state = run_segments(wl, w, [300, 1100], *(x[:, :wl.T] for x in (q, k, v, a)))
    outs = [nha.decode_step(*(x[:, t].contiguous().to(DEV) for x in (q, k, v, a)), state, w, rope_base=wl.rope_base)
            for t in range(wl.T, wl.T + steps)]
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.fwd(f64(q), f64(k), f64(v), f64(a), w, rope_base=wl.rope_base)
    tol = TOL[torch.bfloat16]
    compare("o", f64(o), o_ref[:, :wl.T], tol["o"], tol["rel"])
    compare("lse", f64(lse), l_ref[:, :, :wl.T], tol["lse"], tol["rel"])
    compare("o_dec", f64(torch.stack(outs, 1)), o_ref[:, wl.T:], tol["o"], tol["rel"])


@pytest.mark.parametrize("dtype,T1,w", [(torch.float32, 70, 16), (torch.float32, 9, 16), (torch.bfloat16, 700, 256)])
def test_segment_backward(dtype, T1, w):
    """Gradients of the second segment's loss: w.r.t. its inputs they equal
    the whole-sequence gradients (rows >= T1) of the same loss (zero incoming
    gradient before T1); w.r.t. the ring keys / values the whole sequence's
    dk / dv rows T1 - P .. T1 - 1; w.r.t. the slot states the oracle's dS0 of
    the extended segment started from the state at T1."""
    if dtype == torch.float32:
        wl = WORKLOADS["tiny"].with_(T=150, H=4, Hkv=2, seed=103)
    else:
        wl = WORKLOADS["gqa"].with_(T=1400, H=8, Hkv=2, seed=104)
    log("case continue bwd %s T1=%d w=%d" % (dtype, T1, w))
    q, k, v, a, dO = make_inputs(wl, with_grad=True)
    dO[:, :T1] = 0
    qd, kd, vd, ad, dOd = (x.to(DEV) for x in (q, k, v, a, dO))
    state = nha.decode_state(wl.B, wl.H, wl.Hkv, wl.d, wl.m, w, wl.rope_base, dtype=wl.dtype, device=DEV)
    first = [x[:, :T1].contiguous() for x in (qd, kd, vd, ad)]
    nha.fwd(*first, w, C=wl.C, rope_base=wl.rope_base, state_out=state)
    seg = [x[:, T1:].contiguous() for x in (qd, kd, vd, ad)]
    o2, l2 = nha.fwd_continue(*seg, w, state, T1, C=wl.C, rope_base=wl.rope_base)
    g = nha.bwd_continue(*seg, o2, l2, dOd[:, T1:].contiguous(), w, state, T1, C=wl.C, rope_base=wl.rope_base)
    torch.cuda.synchronize()
    tol = TOL[dtype]
    full = oracle.bwd(f64(q), f64(k), f64(v), f64(a), f64(dO), w, rope_base=wl.rope_base)
    for name, x, r in zip(("dq", "dk", "dv", "dalpha"), g[:4], full):
        compare(name, f64(x), r[:, T1:], tol["grad"], tol["rel"])
    P = min(T1, w)
    ring_rows = [(T1 - P + e) % w for e in range(P)]
    for name, x, r in (("dRK", g[6], full[1]), ("dRV", g[7], full[2])):
        got = f64(x)  # [B,Hkv,w,d]
        ref = np.zeros_like(got)
        ref[:, :, ring_rows] = r[:, T1 - P:T1].transpose(0, 2, 1, 3)
        compare(name, got, ref, tol["grad"], tol["rel"])
    # dS0 of the slots at T1: the oracle over the extended segment
    _, _, s1k, s1v = oracle.fwd(f64(q[:, :T1]), f64(k[:, :T1]), f64(v[:, :T1]), f64(a[:, :T1]), w,
                                rope_base=wl.rope_base, want_state=True)
    ext = lambda x, fill: np.concatenate([np.full_like(x[:, :P], fill) if fill is not None else x[:, T1 - P:T1],
                                          x[:, T1:]], axis=1)
    qe, ke, ve, ae, de = ext(f64(q), 0.0), ext(f64(k), None), ext(f64(v), None), ext(f64(a), 1.0), ext(f64(dO), 0.0)
    r = oracle.bwd(qe, ke, ve, ae, de, w, rope_base=wl.rope_base, s0=(s1k, s1v), want_ds0=True)
    compare("dS0K", f64(g[4]), r[4], tol["grad"], tol["rel"])
    compare("dS0V", f64(g[5]), r[5], tol["grad"], tol["rel"])
