"""GPU parity over seeded random shapes: forward (o, lse) and backward (dq,
dk, dv, dalpha) of the HIP path against the fp64 oracle, each case a random
mix of the parameters the other tests sweep one or two at a time -- dtype,
head dimension, slot count, window, chunk size, query heads per KV head,
ragged length, RoPE on or off, and (bf16) enough (batch, KV head) units for
the one-kernel forward in some cases -- so that interactions between them
are exercised too.  The shapes are drawn once from a fixed seed, at sizes the
oracle finishes in well under a second."""
import random

import pytest
import torch

import oracle
import softmax_attention_nha_amd as nha
from parity_util import TOL, compare, f64, log
from softmax_attention_nha_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


def draw_cases(n, seed=20261203):
    rng = random.Random(seed)
    cases = []
    while len(cases) < n:
        dtype = rng.choice([torch.bfloat16, torch.bfloat16, torch.float32])
        d = rng.choice([32, 64, 128])
        m = rng.choice([0, 1, 7, 16, 32, 33, 64])
        w = rng.choice([0, 1, 16, 33, 64, 200])
        if m == 0 and w == 0:
            continue  # no keys at all: rejected by the library
        if dtype == torch.float32 and (d == 128 or (d == 64 and m > 32)):
            continue  # the fp32 backward's tiles exceed a workgroup's LDS there
        C = rng.choice([16, 32, 64])
        G = rng.choice([1, 2, 4])
        # a third of the bf16 cases with B * Hkv * d / 16 >= 256 and C = 64
        # (the one-kernel forward), long enough to absorb tokens
        big = dtype == torch.bfloat16 and rng.random() < 0.35
        if big:
            d, C = 128, 64
        Hkv = 16 if big else rng.choice([1, 2, 3])
        B = 2 if big else rng.choice([1, 2])
        T = rng.randint(w + 1, w + 160) if big else rng.randint(1, 300)
        base = rng.choice([10000.0, 500.0, 0.0])
        cases.append((dtype, B, G * Hkv, Hkv, T, d, m, w, C, base, rng.randrange(1 << 16)))
    return cases


CASES = draw_cases(24)


@pytest.mark.parametrize("case", CASES, ids=["%s-B%dH%dKV%dT%dd%dm%dw%dC%d-b%g" % (
    "bf16" if c[0] == torch.bfloat16 else "f32", *c[1:10]) for c in CASES])
def test_random_shape_fwd_bwd(case):
    dtype, B, H, Hkv, T, d, m, w, C, base, seed = case
    log("case random %s" % (case,))
    wl = WORKLOADS["tiny"].with_(B=B, H=H, Hkv=Hkv, T=T, d=d, m=m, w=w, C=C, dtype=dtype, rope_base=base,
                                 seed=seed)
    q, k, v, a, dO = make_inputs(wl, with_grad=True)
    dev = torch.device("cuda:0")
    qd, kd, vd, ad, dOd = (x.to(dev) for x in (q, k, v, a, dO))
    o, lse = nha.fwd(qd, kd, vd, ad, w, C=C, rope_base=base)
    grads = nha.bwd(qd, kd, vd, ad, o, lse, dOd, w, C=C, rope_base=base)
    torch.cuda.synchronize()
    o_ref, lse_ref = oracle.fwd(f64(q), f64(k), f64(v), f64(a), w, rope_base=base)
    g_ref = oracle.bwd(f64(q), f64(k), f64(v), f64(a), f64(dO), w, rope_base=base)
    tol = TOL[dtype]
    compare("o", f64(o), o_ref, tol["o"], tol["rel"])
    compare("lse", f64(lse), lse_ref, tol["lse"], tol["rel"])
    for name, x, r in zip(("dq", "dk", "dv", "dalpha"), grads, g_ref):
        if m == 0 and name == "dalpha":
            continue  # no gates without slots
        compare(name, f64(x), r, tol["grad"], tol["rel"])


def draw_decode_cases(n, seed=20261204):
    rng = random.Random(seed)
    cases = []
    while len(cases) < n:
        dtype = rng.choice([torch.bfloat16, torch.bfloat16, torch.float32])
        d = rng.choice([32, 64, 128])
        m = rng.choice([0, 1, 7, 32, 33, 64])
        w = rng.choice([0, 1, 5, 16, 40, 100])
        if m == 0 and w == 0:
            continue
        if dtype == torch.float32 and d == 128 and m > 32:
            continue  # the fp32 prefill's tiles exceed the LDS there
        C = rng.choice([16, 32, 64])
        G = rng.choice([1, 2, 4])
        # every third case with B * Hkv >= 256 units (one workgroup per unit
        # fills the chip: the single-launch step)
        many = len(cases) % 3 == 2
        Hkv = 16 if many else rng.choice([1, 2, 3])
        B = 16 if many else rng.choice([1, 2, 3])
        T0 = rng.randint(0, 150)
        steps = rng.randint(1, 24)
        base = rng.choice([10000.0, 500.0, 0.0])
        cases.append((dtype, B, G * Hkv, Hkv, T0, steps, d, m, w, C, base, rng.randrange(1 << 16)))
    return cases


DECODE_CASES = draw_decode_cases(12)


@pytest.mark.parametrize("case", DECODE_CASES, ids=["%s-B%dH%dKV%dT0_%d+%d-d%dm%dw%dC%d-b%g" % (
    "bf16" if c[0] == torch.bfloat16 else "f32", *c[1:11]) for c in DECODE_CASES])
def test_random_shape_prefill_then_decode(case):
    """nha_fwd over the first T0 tokens exporting the state (T0 = 0: the zero
    state), then one nha_decode_step per token: the outputs equal the oracle's
    forward over the whole sequence at those rows."""
    dtype, B, H, Hkv, T0, steps, d, m, w, C, base, seed = case
    log("case random decode %s" % (case,))
    wl = WORKLOADS["tiny"].with_(B=B, H=H, Hkv=Hkv, T=T0 + steps, d=d, m=m, w=w, C=C, dtype=dtype, rope_base=base,
                                 seed=seed)
    q, k, v, a = make_inputs(wl)
    dev = torch.device("cuda:0")
    state = nha.decode_state(B, H, Hkv, d, m, w, base, dtype=dtype, device=dev)
    if T0 > 0:
        nha.fwd(*(x[:, :T0].contiguous().to(dev) for x in (q, k, v, a)), w, C=C, rope_base=base, state_out=state)
    outs = [nha.decode_step(*(x[:, t].contiguous().to(dev) for x in (q, k, v, a)), state, w, rope_base=base)
            for t in range(T0, T0 + steps)]
    torch.cuda.synchronize()
    o_ref, _ = oracle.fwd(f64(q), f64(k), f64(v), f64(a), w, rope_base=base)
    tol = TOL[dtype]
    compare("o_dec", f64(torch.stack(outs, 1)), o_ref[:, T0:], tol["o"], tol["rel"])


def draw_continue_cases(n, seed=20261205):
    rng = random.Random(seed)
    cases = []
    while len(cases) < n:
        dtype = rng.choice([torch.bfloat16, torch.bfloat16, torch.float32])
        d = rng.choice([32, 64, 128])
        m = rng.choice([0, 1, 7, 32, 33, 64])
        w = rng.choice([1, 5, 16, 40, 100])  # a window to continue (the ring)
        if dtype == torch.float32 and (d == 128 or (d == 64 and m > 32)):
            continue  # one workspace serves the continued backward too: its fp32 LDS limit
        C = rng.choice([16, 32, 64])
        G = rng.choice([1, 2, 4])
        Hkv = rng.choice([1, 2, 3])
        B = rng.choice([1, 2])
        T1 = rng.randint(1, 200)
        T2 = rng.randint(1, 200)
        base = rng.choice([10000.0, 500.0, 0.0])
        cases.append((dtype, B, G * Hkv, Hkv, T1, T2, d, m, w, C, base, rng.randrange(1 << 16)))
    return cases


CONTINUE_CASES = draw_continue_cases(10)


@pytest.mark.parametrize("case", CONTINUE_CASES, ids=["%s-B%dH%dKV%dT%d+%d-d%dm%dw%dC%d-b%g" % (
    "bf16" if c[0] == torch.bfloat16 else "f32", *c[1:11]) for c in CONTINUE_CASES])
def test_random_shape_chunked_prefill(case):
    """nha_fwd over T1 tokens exporting the decode state, then
    nha_fwd_continue over the next T2 from that state: the second segment's
    o and lse equal the oracle's forward over all T1 + T2 tokens at its rows."""
    dtype, B, H, Hkv, T1, T2, d, m, w, C, base, seed = case
    log("case random continue %s" % (case,))
    wl = WORKLOADS["tiny"].with_(B=B, H=H, Hkv=Hkv, T=T1 + T2, d=d, m=m, w=w, C=C, dtype=dtype, rope_base=base,
                                 seed=seed)
    q, k, v, a = make_inputs(wl)
    dev = torch.device("cuda:0")
    state = nha.decode_state(B, H, Hkv, d, m, w, base, dtype=dtype, device=dev)
    nha.fwd(*(x[:, :T1].contiguous().to(dev) for x in (q, k, v, a)), w, C=C, rope_base=base, state_out=state)
    o2, l2 = nha.fwd_continue(*(x[:, T1:].contiguous().to(dev) for x in (q, k, v, a)), w, state, T1, C=C,
                              rope_base=base)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.fwd(f64(q), f64(k), f64(v), f64(a), w, rope_base=base)
    tol = TOL[dtype]
    compare("o", f64(o2), o_ref[:, T1:], tol["o"], tol["rel"])
    compare("lse", f64(l2), l_ref[:, :, T1:], tol["lse"], tol["rel"])
