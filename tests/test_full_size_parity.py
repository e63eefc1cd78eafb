"""GPU parity at the workloads' full sizes (the shapes bench.py times), against
the fp64 oracle on whole (batch, KV head) units: every row of the unit, over
the full sequence length.

The oracle runs each query head of a unit as its own sequence (see
parity_util.oracle_units), so its threads cover every (unit, head) pair and
each case finishes in seconds to tens of seconds on the host."""
import numpy as np
import pytest
import torch

import softmax_attention_nha_amd as nha
from parity_util import TOL, compare, f64, log, oracle_units
from softmax_attention_nha_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def gpu_run(q, k, v, a, dO, w, C, base):
    d = torch.device("cuda:0")
    qd, kd, vd, ad = (x.to(d) for x in (q, k, v, a))
    o, lse = nha.fwd(qd, kd, vd, ad, w, C=C, rope_base=base)
    grads = None
    if dO is not None:
        grads = nha.bwd(qd, kd, vd, ad, o, lse, dO.to(d), w, C=C, rope_base=base)
    torch.cuda.synchronize()
    return o, lse, grads


def check_units(wl, w, units, with_bwd, Tp=None, rel_override=None, **draw):
    G = wl.H // wl.Hkv
    log("case %s B=%d T=%d H=%d/%d d=%d m=%d w=%d C=%d base=%g units=%s bwd=%s %s" % (
        wl.name, wl.B, wl.T, wl.H, wl.Hkv, wl.d, wl.m, w, wl.C, wl.rope_base, units, with_bwd, draw))
    q, k, v, a, dO = make_inputs(wl, with_grad=True, **draw)
    o, lse, grads = gpu_run(q, k, v, a, dO if with_bwd else None, w, wl.C, wl.rope_base)
    tol = TOL[wl.dtype]
    ref_f = oracle_units(q, k, v, a, None, w, wl.rope_base, units, G, Tp)
    T = Tp or wl.T
    got_o = np.concatenate([f64(o[b:b + 1, :T, g * G:(g + 1) * G]) for b, g in units])
    got_l = np.concatenate([f64(lse[b:b + 1, g * G:(g + 1) * G, :T]) for b, g in units])
    compare("o", got_o, np.concatenate([r[0] for r in ref_f]), tol["o"], tol["rel"])
    compare("lse", got_l, np.concatenate([r[1] for r in ref_f]), tol["lse"], tol["rel"])
    if not with_bwd:
        return
    ref_b = oracle_units(q, k, v, a, dO, w, wl.rope_base, units, G)
    dq, dk, dv, da = grads
    sl = {"dq": lambda x, b, g: x[b:b + 1, :, g * G:(g + 1) * G],
          "dk": lambda x, b, g: x[b:b + 1, :, g:g + 1], "dv": lambda x, b, g: x[b:b + 1, :, g:g + 1],
          "dalpha": lambda x, b, g: x[b:b + 1, :, g:g + 1]}
    for i, (name, x) in enumerate((("dq", dq), ("dk", dk), ("dv", dv), ("dalpha", da))):
        got = np.concatenate([f64(sl[name](x, b, g)) for b, g in units])
        ref = np.concatenate([r[i] for r in ref_b])
        compare(name, got, ref, tol["grad"], (rel_override or {}).get(name, tol["rel"]))


# ---------------------------------------------------------------- backward at full length
def test_gqa_workload_backward_full_length():
    """Llama-shaped GQA: T = 8192, w = 2048, m = 32, four query heads per KV
    head -- tokens 2048 .. 8191 are absorbed, so the slot gradients and dalpha
    are live; two units, every row."""
    wl = WORKLOADS["gqa"]
    check_units(wl, wl.w, [(0, 0), (0, wl.Hkv - 1)], with_bwd=True)


def test_headline_backward_full_length():
    """The benchmarked shape: B = 4, T = 8192 (128 chunks of adjoint scan),
    w = 512; two units of different batch rows, every row."""
    wl = WORKLOADS["headline"]
    check_units(wl, wl.w, [(0, 0), (wl.B - 1, wl.Hkv - 1)], with_bwd=True)


def test_1p3b_no_window_backward():
    """w = 0: the pure gated-slot RNN read by a softmax over the slots, at the
    1.3B shape (T = 2048)."""
    wl = WORKLOADS["1p3b"]
    check_units(wl, 0, [(0, 3), (wl.B - 1, wl.Hkv - 1)], with_bwd=True)


@pytest.mark.parametrize("T", [2048, 8192])
def test_pages_operator_shape_m32_w32(T):
    """The operator-benchmark configuration the pages describe: NHA with m = 32
    slots and w = 32 (d = 128 bf16, 16 heads), forward and backward."""
    wl = WORKLOADS["long"].with_(T=T, m=32)
    check_units(wl, 32, [(0, 0), (0, wl.Hkv - 1)], with_bwd=True)


@pytest.mark.parametrize("name,T,w,unit", [("long", 32768, None, (0, 5)), ("gqa", 24576 + 37, 256, (0, 3))])
def test_long_context_backward_segmented_scan(name, T, w, unit):
    """Forward and backward of one unit over the full length where the state
    scan runs in segments (fewer than 256 scan waves, 384 chunks or more) and
    dalpha's cross-chunk carry uses its exact checkpoints: every row and every
    gradient of the unit against the oracle (GQA: the unit's 4 query heads)."""
    wl = WORKLOADS[name].with_(T=T)
    w = wl.w if w is None else w
    desc = nha.make_desc(wl.B, wl.T, wl.H, wl.Hkv, wl.d, wl.m, w, wl.C, wl.rope_base, 0.0, wl.dtype)
    assert "scan_combine" in nha.stage_names(desc) and "carry_ckpt" in nha.stage_names(desc, backward=1)
    check_units(wl, w, [unit], with_bwd=True)


# ---------------------------------------------------------------- forward at full length
@pytest.mark.parametrize("T", [16384, 32768])
def test_long_context_forward_every_row(T):
    wl = WORKLOADS["long"].with_(T=T)
    check_units(wl, wl.w, [(0, wl.Hkv // 2)], with_bwd=False)


def test_gqa_forward_every_row():
    wl = WORKLOADS["gqa"]
    check_units(wl, wl.w, [(0, 1)], with_bwd=False)


# ---------------------------------------------------------------- backward corners (every element)
def test_bf16_head_dim_32_backward():
    wl = WORKLOADS["340m"].with_(B=1, T=333, H=4, Hkv=2, d=32, seed=71)
    check_units(wl, 40, [(0, 0), (0, 1)], with_bwd=True)


@pytest.mark.parametrize("C", [16, 32])
def test_bf16_32_slots_small_chunks_backward(C):
    """m <= 32 (slot tiles padded to 32) with one- and two-wave slot workgroups."""
    wl = WORKLOADS["gqa"].with_(T=389, C=C, seed=72)
    check_units(wl, 70, [(0, 0), (0, 5)], with_bwd=True)


# ---------------------------------------------------------------- decode after the long prefixes
@pytest.mark.parametrize("T0", [16384, 32768])
def test_long_context_decode_256_steps(T0):
    """nha_fwd over T0 tokens exporting the state, then 256 nha_decode_step
    calls; the steps' outputs against the oracle over T0 + 256 tokens (two KV
    heads, every step)."""
    wl = WORKLOADS["long"].with_(T=T0)
    steps, w, base = 256, wl.w, wl.rope_base
    log("case decode long bf16 T0=%d steps=%d" % (T0, steps))
    d = torch.device("cuda:0")
    q, k, v, a = make_inputs(wl, T_total=T0 + steps)
    state = nha.decode_state(wl.B, wl.H, wl.Hkv, wl.d, wl.m, w, base, dtype=wl.dtype, device=d)
    qd, kd, vd, ad = (x.to(d) for x in (q, k, v, a))
    nha.fwd(qd[:, :T0].contiguous(), kd[:, :T0].contiguous(), vd[:, :T0].contiguous(), ad[:, :T0].contiguous(), w,
            C=wl.C, rope_base=base, state_out=state)
    outs = [nha.decode_step(qd[:, t].contiguous(), kd[:, t].contiguous(), vd[:, t].contiguous(),
                            ad[:, t].contiguous(), state, w, rope_base=base) for t in range(T0, T0 + steps)]
    torch.cuda.synchronize()
    od = torch.stack(outs, 1)  # [B, steps, H, d]
    assert torch.isfinite(od.float()).all()
    units = [(0, 0), (0, wl.Hkv - 1)]
    ref = oracle_units(q, k, v, a, None, w, base, units, 1)
    got = np.concatenate([f64(od[:, :, g:g + 1]) for _, g in units])
    compare("o_dec", got, np.concatenate([r[0][:, T0:] for r in ref]), 2e-2, 1e-2)
