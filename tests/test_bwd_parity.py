"""GPU backward parity: dq, dk, dv, dalpha of the HIP path (through the C ABI)
against the fp64 oracle's adjoint on the same (exactly upcast) inputs.

The backward depends on the whole sequence, so full-size workloads are checked
on one (batch, KV head) unit over the full length where the oracle finishes in
seconds; the Llama-shaped GQA workload runs at a reduced length."""
import numpy as np
import pytest
import torch

import oracle
import softmax_attention_nha_amd as nha
from parity_util import TOL, compare, f64, log, unit_slice
from softmax_attention_nha_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def gpu_fwd_bwd(q, k, v, a, dO, w, C, base):
    d = torch.device("cuda:0")
    qd, kd, vd, ad, dOd = (x.to(d) for x in (q, k, v, a, dO))
    o, lse = nha.fwd(qd, kd, vd, ad, w, C=C, rope_base=base)
    grads = nha.bwd(qd, kd, vd, ad, o, lse, dOd, w, C=C, rope_base=base)
    torch.cuda.synchronize()
    return grads


def check(wl, w=None, C=None, base=None, units=None, rel_override=None, **draw):
    """units: None = every (b, g); else list of (b, g) to compare.
    rel_override: {tensor name: relative-L2 gate} replacing the default."""
    w = wl.w if w is None else w
    C = wl.C if C is None else C
    base = wl.rope_base if base is None else base
    log("case bwd %s B=%d T=%d H=%d/%d d=%d m=%d w=%d C=%d base=%g %s %s" % (
        wl.name, wl.B, wl.T, wl.H, wl.Hkv, wl.d, wl.m, w, C, base, wl.dtype, draw))
    q, k, v, a, dO = make_inputs(wl, with_grad=True, **draw)
    dq, dk, dv, da = gpu_fwd_bwd(q, k, v, a, dO, w, C, base)
    tol = TOL[wl.dtype]
    if units is None:
        ref = oracle.bwd(f64(q), f64(k), f64(v), f64(a), f64(dO), w, rope_base=base)
        got = (f64(dq), f64(dk), f64(dv), f64(da))
    else:
        G = wl.H // wl.Hkv
        got, ref = [[], [], [], []], [[], [], [], []]
        for (b, g) in units:
            hq = list(range(g * G, (g + 1) * G))
            r = oracle.bwd(f64(unit_slice(q, b, hq)), f64(unit_slice(k, b, [g])), f64(unit_slice(v, b, [g])),
                           f64(unit_slice(a, b, [g])), f64(unit_slice(dO, b, hq)), w, rope_base=base)
            gg = (unit_slice(dq, b, hq), unit_slice(dk, b, [g]), unit_slice(dv, b, [g]), unit_slice(da, b, [g]))
            for i in range(4):
                got[i].append(f64(gg[i]))
                ref[i].append(r[i])
        got = [np.concatenate(x) for x in got]
        ref = [np.concatenate(x) for x in ref]
    for name, x, r in zip(("dq", "dk", "dv", "dalpha"), got, ref):
        compare(name, x, r, tol["grad"], (rel_override or {}).get(name, tol["rel"]))


# ---------------------------------------------------------------- fp32 (max-abs 1e-4)
@pytest.mark.parametrize("w", [0, 1, 16, 17, 100, 200, 205])
def test_fp32_window_sweep_ragged_gqa(w):
    check(WORKLOADS["tiny"].with_(T=200, H=4, Hkv=2, seed=51), w=w)


@pytest.mark.parametrize("C,T,w", [(32, 150, 40), (64, 150, 40), (16, 97, 31)])
def test_fp32_chunk_sizes(C, T, w):
    check(WORKLOADS["tiny"].with_(T=T, seed=52), w=w, C=C)


@pytest.mark.parametrize("m", [1, 33])
def test_fp32_slot_counts(m):
    check(WORKLOADS["tiny"].with_(T=130, m=m, seed=53), w=24, C=32)


@pytest.mark.parametrize("base", [10000.0, 0.0])
def test_tiny_workload(base):
    check(WORKLOADS["tiny"], base=base)


# ---------------------------------------------------------------- bf16, every element at reduced T
@pytest.mark.parametrize("C", [16, 32])
def test_bf16_chunk_sizes_gqa(C):
    # one- and two-wave slot workgroups (C = 16, 32: the two load orders of
    # slot pass B) at d = 128, m = 64, two query heads per KV head, ragged T
    check(WORKLOADS["1p3b"].with_(B=1, T=261, H=4, Hkv=2, seed=57), w=40, C=C)


@pytest.mark.parametrize("name,w", [("340m", None), ("1p3b", 0), ("1p3b", 64), ("1p3b", 512), ("1p3b", 2048),
                                    ("gqa", None)])
def test_bf16_workloads_reduced(name, w):
    wl = WORKLOADS[name].with_(B=1, T=640 + 21)
    check(wl, w=w)


def test_bf16_stress_logits_and_hard_gates():
    """Unscaled q, k ~ N(0,1) and alpha = sigmoid(N(-2,1)) (median 0.12).  The
    max-abs gates are the workloads' (5e-2).  dalpha is formed as
    RevCumSum(A - b F)_t / alpha_t - F_t, so the bf16-level rounding of the
    summed terms is divided by alpha_t: with these gates its relative L2 error
    is about 1/alpha times that of the other gradients, and its extra gate is
    5e-2 instead of 1e-2."""
    check(WORKLOADS["1p3b"].with_(B=1, T=400, H=2, Hkv=2, seed=54), w=96, qk_scale=1.0, alpha_mu=-2.0,
          rel_override={"dalpha": 5e-2})


def test_bf16_blocks_around_the_exact_path_threshold():
    """Pass B takes its exact same-block path (fp32 weights from the
    workspace) for 16-row blocks whose decay 2^{sum log2 alpha} falls below
    2^-16 in some slot; pass A writes the fp32 rows of those blocks, testing
    at -15.75.  Slot 0's gates cycle over the blocks through alpha = 0.498046875
    (a block sum of -16.09: exact path in both passes), 0.50390625 (-15.82:
    pass B factorizes, pass A still writes the fp32 rows) and the workload's
    mild gates; both values are exact in bf16."""
    wl = WORKLOADS["1p3b"].with_(B=1, T=320, H=2, Hkv=2, seed=57)
    w = 16
    q, k, v, a, dO = make_inputs(wl, with_grad=True)
    a = a.clone()
    for blk in range(w // 16, wl.T // 16):
        val = (0.498046875, 0.50390625, None)[blk % 3]
        if val is not None:
            a[:, 16 * blk:16 * blk + 16, :, 0] = val
    log("case bwd blocks around the exact-path threshold")
    dq, dk, dv, da = gpu_fwd_bwd(q, k, v, a, dO, w, 64, wl.rope_base)
    ref = oracle.bwd(f64(q), f64(k), f64(v), f64(a), f64(dO), w, rope_base=wl.rope_base)
    tol = TOL[wl.dtype]
    for name, x, r in zip(("dq", "dk", "dv", "dalpha"), (dq, dk, dv, da), ref):
        compare(name, f64(x), r, tol["grad"], tol["rel"])


# ---------------------------------------------------------------- full-size workloads, sampled units
@pytest.mark.parametrize("name,w,T", [("340m", None, None), ("1p3b", 64, None), ("1p3b", 512, None),
                                      ("1p3b", 2048, None), ("gqa", None, 2048)])
def test_full_size_sampled_units(name, w, T):
    wl = WORKLOADS[name]
    if T:
        wl = wl.with_(T=T)
    check(wl, w=w, units=[(wl.B - 1, wl.Hkv - 1), (0, 0)])


# ---------------------------------------------------------------- invariants
def test_bwd_bitwise_deterministic():
    wl = WORKLOADS["340m"].with_(B=1, T=300, H=4, Hkv=4, seed=55)
    q, k, v, a, dO = make_inputs(wl, with_grad=True)
    r = [gpu_fwd_bwd(q, k, v, a, dO, 64, 64, 10000.0) for _ in range(3)]
    for x in r[1:]:
        for g0, g1 in zip(r[0], x):
            assert torch.equal(g0, g1)


@pytest.mark.parametrize("name,B,T,C", [("1p3b", 1, 300, 64), ("1p3b", 4, 300, 64), ("gqa", 1, 260, 32),
                                        ("340m", 1, 200, 16)])
def test_bwd_after_fwd_matches_bwd(name, B, T, C):
    """nha_bwd_after_fwd reads the forward's first stages from its workspace:
    bitwise the same gradients as the standalone backward (1p3b at B = 4:
    after the one-kernel forward; at B = 1: after window + slot kernels)."""
    wl = WORKLOADS[name].with_(B=B, T=T, seed=56)
    q, k, v, a, dO = (x.to("cuda:0") for x in make_inputs(wl, with_grad=True))
    desc = nha.make_desc(wl.B, wl.T, wl.H, wl.Hkv, wl.d, wl.m, wl.w, C, wl.rope_base, 0.0, wl.dtype)
    ws = torch.empty(max(nha.workspace_size(desc), nha.workspace_size(desc, backward=True)), dtype=torch.uint8,
                     device="cuda:0")
    o, lse = nha.fwd(q, k, v, a, wl.w, C=C, rope_base=wl.rope_base, workspace=ws)
    g1 = nha.bwd(q, k, v, a, o, lse, dO, wl.w, C=C, rope_base=wl.rope_base, workspace=ws, after_fwd=True)
    g2 = nha.bwd(q, k, v, a, o, lse, dO, wl.w, C=C, rope_base=wl.rope_base)
    torch.cuda.synchronize()
    for x, y in zip(g1, g2):
        assert torch.equal(x, y)


@pytest.mark.parametrize("B,H,Hkv", [(2, 4, 2), (4, 8, 8)])
def test_side_stream_results_equal_one_stream_results(B, H, Hkv):
    # the production calls run independent launches on the library's side
    # stream; the timed calls run every launch in order on the caller's
    # stream: both must give bitwise the same results (B * Hkv = 4: the
    # window kernel beside the scan; 32: the one-kernel forward)
    wl = WORKLOADS["1p3b"].with_(B=B, T=640, H=H, Hkv=Hkv, seed=61)
    w = 128
    log("case side stream vs one stream bf16")
    d = torch.device("cuda:0")
    q, k, v, a, dO = (x.to(d) for x in make_inputs(wl, with_grad=True))
    desc = nha.make_desc(wl.B, wl.T, wl.H, wl.Hkv, wl.d, wl.m, w, wl.C, wl.rope_base, 0.0, wl.dtype)

    def events(n):
        # the Event objects own the HIP events: keep them alive until the
        # stream has passed every record
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record()
        return evs

    res, keep = [], []
    for timed in (False, True):
        fe = events(len(nha.stage_names(desc)) + 1) if timed else None
        be = events(len(nha.stage_names(desc, backward=1)) + 1) if timed else None
        keep.append((fe, be))
        o, lse = nha.fwd(q, k, v, a, w, C=wl.C, rope_base=wl.rope_base,
                         events=[e.cuda_event for e in fe] if timed else None)
        g = nha.bwd(q, k, v, a, o, lse, dO, w, C=wl.C, rope_base=wl.rope_base,
                    events=[e.cuda_event for e in be] if timed else None)
        torch.cuda.synchronize()
        res.append((o, lse) + tuple(g))
    for x, y in zip(*res):
        assert torch.equal(x, y)


def test_release_side_streams_then_call_again():
    # the production calls create the thread's side stream on first use;
    # releasing it and calling again recreates it, with the same results
    wl = WORKLOADS["340m"].with_(B=1, T=200, H=4, Hkv=2, seed=62)
    q, k, v, a, dO = make_inputs(wl, with_grad=True)
    log("case release side streams")
    r1 = gpu_fwd_bwd(q, k, v, a, dO, 64, 64, 10000.0)
    nha.release_side_streams()
    nha.release_side_streams()  # nothing left: a no-op
    r2 = gpu_fwd_bwd(q, k, v, a, dO, 64, 64, 10000.0)
    for x, y in zip(r1, r2):
        assert torch.equal(x, y)
