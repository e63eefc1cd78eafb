"""GPU recurrent-inference parity: nha_decode_step continuing from nha_fwd's
exported state (or from the zero state) equals the forward over the
concatenated sequence -- against the fp64 oracle and against the GPU forward."""
import numpy as np
import pytest
import torch

import oracle
import softmax_attention_nha_amd as nha
from parity_util import TOL, compare, f64, gpu_fwd, log, oracle_fwd, unit_slice
from softmax_attention_nha_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def run_decode(wl, T0, steps, w, base):
    """fwd over the first T0 tokens (exporting the state), then `steps` decode
    steps.  Returns (decode outputs [B,steps,H,d], inputs)."""
    d = torch.device("cuda:0")
    q, k, v, a = make_inputs(wl, T_total=T0 + steps)
    state = nha.decode_state(wl.B, wl.H, wl.Hkv, wl.d, wl.m, w, base, dtype=wl.dtype, device=d)
    if T0 > 0:
        gpu_fwd(q[:, :T0].contiguous(), k[:, :T0].contiguous(), v[:, :T0].contiguous(), a[:, :T0].contiguous(),
                w, wl.C, base, state_out=state)
    qd, kd, vd, ad = (x.to(d) for x in (q, k, v, a))
    outs = []
    for t in range(T0, T0 + steps):
        outs.append(nha.decode_step(qd[:, t].contiguous(), kd[:, t].contiguous(), vd[:, t].contiguous(),
                                    ad[:, t].contiguous(), state, w, rope_base=base))
    torch.cuda.synchronize()
    return torch.stack(outs, 1), (q, k, v, a), state


@pytest.mark.parametrize("T0,w", [(0, 16), (64, 16), (64, 0), (40, 200), (100, 1), (21, 7)])
def test_decode_fp32_against_oracle(T0, w):
    wl = WORKLOADS["tiny"].with_(H=4, Hkv=2, seed=41)
    steps = 40
    log("case decode fp32 T0=%d w=%d steps=%d" % (T0, w, steps))
    od, (q, k, v, a), _ = run_decode(wl, T0, steps, w, wl.rope_base)
    o_ref, _ = oracle_fwd(q, k, v, a, w, wl.rope_base)
    compare("o_dec", f64(od), o_ref[:, T0:], TOL[torch.float32]["o"], TOL[torch.float32]["rel"])


def test_exported_state_matches_oracle_final_state():
    wl = WORKLOADS["tiny"].with_(T=100, H=2, Hkv=2, seed=42)
    w = 16
    log("case state export fp32")
    q, k, v, a = make_inputs(wl)
    state = nha.decode_state(wl.B, wl.H, wl.Hkv, wl.d, wl.m, w, wl.rope_base, dtype=wl.dtype,
                             device=torch.device("cuda:0"))
    gpu_fwd(q, k, v, a, w, wl.C, wl.rope_base, state_out=state)
    _, _, sk, sv = oracle.fwd(f64(q), f64(k), f64(v), f64(a), w, rope_base=wl.rope_base, want_state=True)
    n = wl.B * wl.Hkv * wl.m * wl.d
    st = state.cpu()
    sk_gpu = st[: n * 4].view(torch.float32).double().numpy().reshape(sk.shape)
    off = (n * 4 + 255) // 256 * 256
    sv_gpu = st[off: off + n * 4].view(torch.float32).double().numpy().reshape(sv.shape)
    compare("SK", sk_gpu, sk, 1e-5, 1e-5)
    compare("SV", sv_gpu, sv, 1e-5, 1e-5)


def test_long_workload_decode_256_steps():
    wl = WORKLOADS["long"]  # B=1 H=16 d=128 m=64 w=512, T=8192 prefix + 256 recurrent steps
    T0, steps = wl.T, 256
    log("case decode long bf16 T0=%d steps=%d" % (T0, steps))
    od, (q, k, v, a), _ = run_decode(wl, T0, steps, wl.w, wl.rope_base)
    # against the GPU forward over the concatenated sequence (all heads)
    o_full, _ = gpu_fwd(q, k, v, a, wl.w, wl.C, wl.rope_base)
    compare("vs fwd", f64(od), f64(o_full[:, T0:]), 2e-2, 1e-2)
    # against the oracle on two heads
    for g in (0, wl.Hkv - 1):
        sl = lambda x: unit_slice(x, 0, [g])
        o_ref, _ = oracle_fwd(sl(q), sl(k), sl(v), sl(a), wl.w, wl.rope_base)
        compare("vs oracle", f64(od[:, :, g:g + 1]), o_ref[:, T0:], 2e-2, 1e-2)


def test_gqa_decode_bf16():
    wl = WORKLOADS["gqa"].with_(seed=43)
    T0, steps, w = 300, 24, 256
    log("case decode gqa bf16 T0=%d w=%d" % (T0, w))
    od, (q, k, v, a), _ = run_decode(wl, T0, steps, w, wl.rope_base)
    o_ref, _ = oracle_fwd(q, k, v, a, w, wl.rope_base)
    compare("o_dec", f64(od), o_ref[:, T0:], 2e-2, 1e-2)


def test_decode_many_sequences_bf16():
    # B >> 1: every (sequence, KV head) unit steps independently (one split each)
    wl = WORKLOADS["340m"].with_(B=24, T=96, H=8, Hkv=4, m=16, seed=44)
    T0, steps, w = 96, 12, 64
    log("case decode batched bf16 B=%d T0=%d w=%d" % (wl.B, T0, w))
    od, (q, k, v, a), _ = run_decode(wl, T0, steps, w, wl.rope_base)
    o_ref, _ = oracle_fwd(q, k, v, a, w, wl.rope_base)
    compare("o_dec", f64(od), o_ref[:, T0:], 2e-2, 1e-2)


def test_decode_most_keys_per_step():
    # m + w = 4096, the largest key list a step takes: 32 workgroups of 128 keys
    wl = WORKLOADS["1p3b"].with_(B=1, T=4100, H=2, Hkv=2, seed=45)
    T0, steps, w = 4100, 3, 4096 - wl.m
    log("case decode max keys bf16 m=%d w=%d" % (wl.m, w))
    od, (q, k, v, a), _ = run_decode(wl, T0, steps, w, wl.rope_base)
    o_ref, _ = oracle_fwd(q, k, v, a, w, wl.rope_base)
    compare("o_dec", f64(od), o_ref[:, T0:], 2e-2, 1e-2)


def test_decode_bitwise_reproducible():
    # the partial softmax results of the key splits are merged in split order
    wl = WORKLOADS["long"].with_(T=700)
    T0, steps = 600, 6
    log("case decode determinism bf16")
    d = torch.device("cuda:0")
    q, k, v, a = make_inputs(wl, T_total=T0 + steps)
    state = nha.decode_state(wl.B, wl.H, wl.Hkv, wl.d, wl.m, wl.w, wl.rope_base, dtype=wl.dtype, device=d)
    gpu_fwd(q[:, :T0].contiguous(), k[:, :T0].contiguous(), v[:, :T0].contiguous(), a[:, :T0].contiguous(),
            wl.w, wl.C, wl.rope_base, state_out=state)
    runs = []
    for _ in range(2):
        st = state.clone()
        outs = [nha.decode_step(*(x[:, t].contiguous().to(d) for x in (q, k, v, a)), st, wl.w,
                                rope_base=wl.rope_base) for t in range(T0, T0 + steps)]
        torch.cuda.synchronize()
        runs.append((torch.stack(outs, 1).cpu(), st.cpu()))
    assert torch.equal(runs[0][0], runs[1][0])
    assert torch.equal(runs[0][1], runs[1][1])


@pytest.mark.parametrize("B,H,Hkv,d,m,w,T0", [(64, 16, 4, 64, 16, 64, 96), (32, 64, 8, 128, 32, 48, 60),
                                               (256, 2, 1, 32, 8, 0, 20), (128, 4, 2, 128, 64, 200, 230)])
def test_decode_single_launch_many_units(B, H, Hkv, d, m, w, T0):
    """B * Hkv >= the compute-unit count: one workgroup per (sequence, KV
    head) walks all its keys in passes (single launch) -- incl. two passes of
    query heads (G = 8) and no window (w = 0)."""
    wl = WORKLOADS["340m"].with_(B=B, T=T0, H=H, Hkv=Hkv, d=d, m=m, seed=46)
    steps = 6
    log("case decode single launch B=%d H=%d/%d d=%d m=%d w=%d T0=%d" % (B, H, Hkv, d, m, w, T0))
    od, (q, k, v, a), st = run_decode(wl, T0, steps, w, wl.rope_base)
    o_ref, _ = oracle_fwd(q, k, v, a, w, wl.rope_base)
    compare("o_dec", f64(od), o_ref[:, T0:], 2e-2, 1e-2)
    # and bitwise reproducible
    od2, _, st2 = run_decode(wl, T0, steps, w, wl.rope_base)
    assert torch.equal(od, od2) and torch.equal(st, st2)
