"""Pins of the fp64 oracle against things other than itself (CPU only).

Each test fixes part of the oracle through a closed form, a library routine,
an independent formulation (tests/brute.py: closed-form sums, complex-number
RoPE, torch.softmax) or the mathematics of the gradient (finite differences,
torch.autograd).  Passages followed: the Paper-Notes page 'Native Hybrid
Attention for Efficient Sequence Modeling' -- 整体框架 (two memories, w = 0 is a
pure linear RNN, w = N is full attention), 关键设计 > 层内混合 (K^long_t
recurrence, one softmax scaled by 1/sqrt(d), token shift, RoPE on the window
only) -- and the gist.science page's Flexibilidade Arquitetural (w = 0 / w = N).
"""
import json
import math
import os

import numpy as np
import pytest
import scipy.signal
import scipy.special
import torch
import torch.nn.functional as F

import oracle
from brute import nha_brute, rope_complex

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def rand_case(B, T, H, Hkv, d, m, seed, amu=0.0, qs=0.7):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, T, H, d)) * qs
    k = rng.standard_normal((B, T, Hkv, d)) * qs
    v = rng.standard_normal((B, T, Hkv, d))
    a = 1.0 / (1.0 + np.exp(-(rng.standard_normal((B, T, Hkv, m)) + amu)))
    return q, k, v, a


def t64(x):
    return torch.from_numpy(np.ascontiguousarray(x))


# ---------------------------------------------------------------- worked examples
def test_hand_examples():
    ex = json.load(open(os.path.join(GOLDEN, "hand_examples.json")))
    for c in ex["cases"]:
        B, T, H, Hkv, d, m = c["B"], c["T"], c["H"], c["Hkv"], c["d"], c["m"]
        q = np.array(c["q"], float).reshape(B, T, H, d)
        k = np.array(c["k"], float).reshape(B, T, Hkv, d)
        v = np.array(c["v"], float).reshape(B, T, Hkv, d)
        a = np.array(c["alpha"], float).reshape(B, T, Hkv, m)
        o, lse = oracle.fwd(q, k, v, a, c["w"], rope_base=c["rope_base"], scale=c["scale"])
        np.testing.assert_allclose(o.reshape(T, d), np.array(c["o"]), rtol=0, atol=1e-13, err_msg=c["name"])
        np.testing.assert_allclose(lse.reshape(T), np.array(c["lse"]), rtol=0, atol=1e-13, err_msg=c["name"])


# ---------------------------------------------------------------- RoPE
def test_rope_complex_is_rotation_with_relative_logits():
    """The complex-number RoPE used by the pins: orthogonal, and <R_t q, R_j k>
    depends on j - t only (shift invariance)."""
    rng = np.random.default_rng(5)
    x = t64(rng.standard_normal((1, 9, 1, 8)))
    y = rope_complex(x, 100.0)
    np.testing.assert_allclose(y.norm(dim=-1), x.norm(dim=-1), rtol=1e-13)
    q = t64(rng.standard_normal(8))
    kk = t64(rng.standard_normal(8))
    seq_q = q.expand(1, 9, 1, 8).clone()
    seq_k = kk.expand(1, 9, 1, 8).clone()
    rq, rk = rope_complex(seq_q, 100.0)[0, :, 0], rope_complex(seq_k, 100.0)[0, :, 0]
    a = float(rq[5] @ rk[3])
    b = float(rq[7] @ rk[5])
    assert abs(a - b) < 1e-12


# ---------------------------------------------------------------- w >= T: causal RoPE attention + m null keys
def sdpa_with_slots(q, kslots, vslots, kwin, vwin, allow_win, s):
    """softmax attention of q [T,d] over per-row slot keys [T,m,d] + shared
    window keys [T,d] masked by allow_win [T,T] (torch SDPA, fp64)."""
    T, d = q.shape
    m = kslots.shape[1]
    outs, lses = [], []
    for t in range(T):
        keys = torch.cat([kslots[t], kwin], 0)
        vals = torch.cat([vslots[t], vwin], 0)
        mask = torch.cat([torch.ones(m, dtype=torch.bool), allow_win[t]])
        o = F.scaled_dot_product_attention(q[t][None, None, None], keys[None, None], vals[None, None],
                                           attn_mask=mask[None, None, None], scale=s)
        lg = (keys @ q[t]) * s
        lses.append(torch.logsumexp(lg[mask], 0))
        outs.append(o[0, 0, 0])
    return torch.stack(outs), torch.stack(lses)


@pytest.mark.parametrize("w_extra", [0, 5])
@pytest.mark.parametrize("base", [0.0, 10000.0])
def test_full_window_is_causal_rope_attention_plus_null_slots(w_extra, base):
    B, T, H, Hkv, d, m = 1, 13, 2, 1, 8, 3
    q, k, v, a = rand_case(B, T, H, Hkv, d, m, seed=1)
    w = T + w_extra
    o, lse = oracle.fwd(q, k, v, a, w, rope_base=base)
    s = 1.0 / math.sqrt(d)
    qr = rope_complex(t64(q), base)
    kr = rope_complex(t64(k), base)
    causal = torch.tril(torch.ones(T, T, dtype=torch.bool))
    zeros = torch.zeros(T, m, d, dtype=torch.float64)
    for h in range(H):
        o_ref, l_ref = sdpa_with_slots(qr[0, :, h], zeros, zeros, kr[0, :, 0], t64(v)[0, :, 0], causal, s)
        np.testing.assert_allclose(o[0, :, h], o_ref.numpy(), atol=1e-12)
        np.testing.assert_allclose(lse[0, h], l_ref.numpy(), atol=1e-12)


@pytest.mark.parametrize("w", [1, 3, 7])
def test_alpha_one_freezes_slots_sliding_window(w):
    B, T, H, Hkv, d, m = 1, 15, 1, 1, 8, 4
    q, k, v, _ = rand_case(B, T, H, Hkv, d, m, seed=2)
    a = np.ones((B, T, Hkv, m))
    o, lse = oracle.fwd(q, k, v, a, w, rope_base=500.0)
    s = 1.0 / math.sqrt(d)
    qr, kr = rope_complex(t64(q), 500.0), rope_complex(t64(k), 500.0)
    tt = torch.arange(T)
    band = (tt[None, :] <= tt[:, None]) & (tt[None, :] >= tt[:, None] - w + 1)
    zeros = torch.zeros(T, m, d, dtype=torch.float64)
    o_ref, l_ref = sdpa_with_slots(qr[0, :, 0], zeros, zeros, kr[0, :, 0], t64(v)[0, :, 0], band, s)
    np.testing.assert_allclose(o[0, :, 0], o_ref.numpy(), atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], l_ref.numpy(), atol=1e-12)


@pytest.mark.parametrize("w", [0, 1, 4])
def test_alpha_zero_slots_hold_the_shifted_token(w):
    """alpha == 0: every slot equals the raw (unrotated) k_{t-w}, v_{t-w}; zero before t = w."""
    B, T, H, Hkv, d, m = 1, 12, 1, 1, 6, 3
    q, k, v, _ = rand_case(B, T, H, Hkv, d, m, seed=3)
    a = np.zeros((B, T, Hkv, m))
    o, lse = oracle.fwd(q, k, v, a, w, rope_base=100.0)
    s = 1.0 / math.sqrt(d)
    qr, kr = rope_complex(t64(q), 100.0), rope_complex(t64(k), 100.0)
    kslots = torch.zeros(T, m, d, dtype=torch.float64)
    vslots = torch.zeros(T, m, d, dtype=torch.float64)
    for t in range(w, T):
        kslots[t] = t64(k)[0, t - w, 0]
        vslots[t] = t64(v)[0, t - w, 0]
    tt = torch.arange(T)
    band = (tt[None, :] <= tt[:, None]) & (tt[None, :] >= tt[:, None] - w + 1)
    # window logits use the rotated query, slots the raw query: assemble per row
    outs, lses = [], []
    for t in range(T):
        lg_s = s * (kslots[t] @ t64(q)[0, t, 0])
        lg_w = s * (kr[0, :, 0] @ qr[0, t, 0])
        lg = torch.cat([lg_s, lg_w.masked_fill(~band[t], float("-inf"))])
        p = torch.from_numpy(scipy.special.softmax(lg.numpy()))
        outs.append(p[:m] @ vslots[t] + p[m:] @ t64(v)[0, :, 0])
        lses.append(float(scipy.special.logsumexp(lg.numpy())))
    np.testing.assert_allclose(o[0, :, 0], torch.stack(outs).numpy(), atol=1e-12)
    np.testing.assert_allclose(lse[0, 0], np.array(lses), atol=1e-12)


# ---------------------------------------------------------------- decay arithmetic: EMA via lfilter
@pytest.mark.parametrize("w", [0, 2, 5])
def test_constant_gates_are_an_ema(w):
    """alpha_t[i] == c_i: S_t[i] = (1-c_i) sum_{u<=t-w} c_i^{t-w-u} x_u, i.e. a
    first-order IIR filter of the shifted sequence (scipy.signal.lfilter)."""
    B, T, H, Hkv, d, m = 1, 17, 1, 1, 5, 3
    q, k, v, _ = rand_case(B, T, H, Hkv, d, m, seed=4)
    c = np.array([0.3, 0.75, 0.95])
    a = np.broadcast_to(c, (B, T, Hkv, m)).copy()
    o, lse = oracle.fwd(q, k, v, a, w, rope_base=0.0)
    xs_k = np.zeros((T, d))
    xs_v = np.zeros((T, d))
    xs_k[w:] = k[0, : T - w, 0]
    xs_v[w:] = v[0, : T - w, 0]
    SK = np.stack([scipy.signal.lfilter([1 - ci], [1, -ci], xs_k, axis=0) for ci in c], 1)  # [T,m,d]
    SV = np.stack([scipy.signal.lfilter([1 - ci], [1, -ci], xs_v, axis=0) for ci in c], 1)
    s = 1.0 / math.sqrt(d)
    for t in range(T):
        lg_s = s * SK[t] @ q[0, t, 0]
        j0 = max(0, t - w + 1)
        win = list(range(j0, t + 1)) if w > 0 else []
        lg_w = s * k[0, win, 0] @ q[0, t, 0] if win else np.zeros(0)
        lg = np.concatenate([lg_s, lg_w])
        p = scipy.special.softmax(lg)
        o_ref = p[:m] @ SV[t] + (p[m:] @ v[0, win, 0] if win else 0.0)
        np.testing.assert_allclose(o[0, t, 0], o_ref, atol=1e-12)
        assert abs(lse[0, 0, t] - scipy.special.logsumexp(lg)) < 1e-12


# ---------------------------------------------------------------- time-varying gates: closed-form brute force
@pytest.mark.parametrize("w", [0, 1, 3, 10, 11, 14])
@pytest.mark.parametrize("base", [0.0, 10000.0])
def test_oracle_matches_closed_form(w, base):
    B, T, H, Hkv, d, m = 2, 11, 4, 2, 8, 5
    q, k, v, a = rand_case(B, T, H, Hkv, d, m, seed=10 + w)
    o, lse = oracle.fwd(q, k, v, a, w, rope_base=base)
    o_ref, l_ref = nha_brute(t64(q), t64(k), t64(v), t64(a), w, base)
    np.testing.assert_allclose(o, o_ref.numpy(), atol=1e-12)
    np.testing.assert_allclose(lse, l_ref.numpy(), atol=1e-12)


def test_final_state_export_matches_closed_form():
    B, T, H, Hkv, d, m, w = 1, 9, 2, 2, 4, 3, 2
    q, k, v, a = rand_case(B, T, H, Hkv, d, m, seed=7)
    _, _, sk, sv = oracle.fwd(q, k, v, a, w, want_state=True)
    from brute import slot_states
    SK = slot_states(t64(k), t64(a), w)[:, -1]  # [B,Hkv,m,d]
    SV = slot_states(t64(v), t64(a), w)[:, -1]
    np.testing.assert_allclose(sk, SK.numpy(), atol=1e-13)
    np.testing.assert_allclose(sv, SV.numpy(), atol=1e-13)


# ---------------------------------------------------------------- gradients
@pytest.mark.parametrize("w", [0, 3, 12])
def test_backward_matches_autograd_of_closed_form(w):
    B, T, H, Hkv, d, m = 1, 12, 2, 1, 4, 3
    q, k, v, a = rand_case(B, T, H, Hkv, d, m, seed=20 + w)
    dO = np.random.default_rng(99).standard_normal(q.shape)
    dq, dk, dv, da = oracle.bwd(q, k, v, a, dO, w, rope_base=100.0)
    tq, tk, tv, ta = (t64(x).requires_grad_(True) for x in (q, k, v, a))
    o, _ = nha_brute(tq, tk, tv, ta, w, 100.0)
    (o * t64(dO)).sum().backward()
    np.testing.assert_allclose(dq, tq.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dk, tk.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(dv, tv.grad.numpy(), atol=1e-11)
    np.testing.assert_allclose(da, ta.grad.numpy(), atol=1e-11)


def test_backward_matches_finite_differences():
    B, T, H, Hkv, d, m, w = 1, 10, 2, 1, 4, 3, 3
    q, k, v, a = rand_case(B, T, H, Hkv, d, m, seed=31)
    dO = np.random.default_rng(98).standard_normal(q.shape)
    grads = oracle.bwd(q, k, v, a, dO, w, rope_base=50.0)
    inputs = [q, k, v, a]
    rng = np.random.default_rng(0)
    h = 1e-6
    for which in range(4):
        x = inputs[which]
        for _ in range(12):
            idx = tuple(rng.integers(0, n) for n in x.shape)
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            args_p = list(inputs)
            args_m = list(inputs)
            args_p[which], args_m[which] = xp, xm
            fp = (oracle.fwd(*args_p, w, rope_base=50.0)[0] * dO).sum()
            fm = (oracle.fwd(*args_m, w, rope_base=50.0)[0] * dO).sum()
            fd = (fp - fm) / (2 * h)
            assert abs(fd - grads[which][idx]) < 1e-7 * max(1.0, abs(fd)), (which, idx, fd, grads[which][idx])


def test_dalpha_zero_before_window_fills_and_for_full_window():
    B, T, H, Hkv, d, m = 1, 14, 2, 2, 4, 3
    q, k, v, a = rand_case(B, T, H, Hkv, d, m, seed=41)
    dO = np.random.default_rng(1).standard_normal(q.shape)
    w = 5
    da = oracle.bwd(q, k, v, a, dO, w)[3]
    assert np.all(da[:, :w] == 0.0)
    assert np.abs(da[:, w:]).max() > 0
    da_full = oracle.bwd(q, k, v, a, dO, T)[3]
    assert np.all(da_full == 0.0)


# ---------------------------------------------------------------- invariants
def test_gqa_equals_mha_with_repeated_kv():
    B, T, H, Hkv, d, m, w = 1, 10, 4, 2, 4, 3, 3
    q, k, v, a = rand_case(B, T, H, Hkv, d, m, seed=51)
    dO = np.random.default_rng(2).standard_normal(q.shape)
    G = H // Hkv
    rep = lambda x: np.repeat(x, G, axis=2)
    o1, l1 = oracle.fwd(q, k, v, a, w)
    o2, l2 = oracle.fwd(q, rep(k), rep(v), rep(a), w)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    np.testing.assert_allclose(l1, l2, atol=1e-13)
    g1 = oracle.bwd(q, k, v, a, dO, w)
    g2 = oracle.bwd(q, rep(k), rep(v), rep(a), dO, w)
    np.testing.assert_allclose(g1[0], g2[0], atol=1e-12)
    fold = lambda x: x.reshape(B, T, Hkv, G, -1).sum(3)
    for i in (1, 2, 3):
        np.testing.assert_allclose(g1[i], fold(g2[i]), atol=1e-12)


def test_slot_permutation_equivariance():
    B, T, H, Hkv, d, m, w = 1, 11, 2, 1, 4, 5, 2
    q, k, v, a = rand_case(B, T, H, Hkv, d, m, seed=61)
    dO = np.random.default_rng(3).standard_normal(q.shape)
    perm = np.array([3, 0, 4, 1, 2])
    o1, _ = oracle.fwd(q, k, v, a, w)
    o2, _ = oracle.fwd(q, k, v, a[..., perm], w)
    np.testing.assert_allclose(o1, o2, atol=1e-13)
    da1 = oracle.bwd(q, k, v, a, dO, w)[3]
    da2 = oracle.bwd(q, k, v, a[..., perm], dO, w)[3]
    np.testing.assert_allclose(da1[..., perm], da2, atol=1e-12)


def test_prefix_causality():
    """Outputs at t depend only on tokens <= t: a prefix run equals the prefix of a longer run."""
    B, T, H, Hkv, d, m, w = 1, 16, 2, 1, 4, 3, 4
    q, k, v, a = rand_case(B, T, H, Hkv, d, m, seed=71)
    o1, l1 = oracle.fwd(q, k, v, a, w)
    o2, l2 = oracle.fwd(q[:, :9], k[:, :9], v[:, :9], a[:, :9], w)
    np.testing.assert_allclose(o1[:, :9], o2, atol=1e-14)
    np.testing.assert_allclose(l1[:, :, :9], l2, atol=1e-14)


# ---------------------------------------------------------------- initial slot states
# Learnable initial slot states (ai.info page, "Future Directions", item 1):
# S_{-1} = S0 instead of zero; a state is only decayed by a step that absorbs,
# so S0 is unchanged until t = w and decays by prod alpha afterwards.
def rand_s0(B, Hkv, m, d, seed):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((B, Hkv, m, d)) * 0.8, rng.standard_normal((B, Hkv, m, d))


@pytest.mark.parametrize("w", [0, 3, 12])
def test_initial_state_matches_closed_form(w):
    B, T, H, Hkv, d, m = 2, 11, 4, 2, 8, 5
    q, k, v, a = rand_case(B, T, H, Hkv, d, m, seed=50 + w)
    s0 = rand_s0(B, Hkv, m, d, seed=60 + w)
    o, lse, sk, sv = oracle.fwd(q, k, v, a, w, rope_base=100.0, s0=s0, want_state=True)
    o_ref, l_ref = nha_brute(t64(q), t64(k), t64(v), t64(a), w, 100.0, s0=(t64(s0[0]), t64(s0[1])))
    np.testing.assert_allclose(o, o_ref.numpy(), atol=1e-12)
    np.testing.assert_allclose(lse, l_ref.numpy(), atol=1e-12)
    from brute import slot_states
    np.testing.assert_allclose(sk, slot_states(t64(k), t64(a), w, t64(s0[0]))[:, -1].numpy(), atol=1e-12)
    np.testing.assert_allclose(sv, slot_states(t64(v), t64(a), w, t64(s0[1]))[:, -1].numpy(), atol=1e-12)


def test_initial_state_with_frozen_gates_is_attention_over_fixed_extra_keys():
    # alpha = 1: nothing is absorbed and nothing decays, so every query sees
    # the m fixed keys S0K (raw q, no RoPE) with values S0V beside its window
    B, T, H, Hkv, d, m, w = 1, 9, 2, 2, 4, 3, 4
    q, k, v, _ = rand_case(B, T, H, Hkv, d, m, seed=71)
    a = np.ones((B, T, Hkv, m))
    s0 = rand_s0(B, Hkv, m, d, seed=72)
    o, lse = oracle.fwd(q, k, v, a, w, rope_base=0.0, s0=s0)
    s = 1.0 / math.sqrt(d)
    for t in range(T):
        for h in range(H):
            ls = s * (s0[0][0, h] @ q[0, t, h])  # m slot logits
            j = np.arange(max(0, t - w + 1), t + 1)
            lw = s * (k[0, j, h] @ q[0, t, h])
            lg = np.concatenate([ls, lw])
            p = scipy.special.softmax(lg)
            ref = p[:m] @ s0[1][0, h] + p[m:] @ v[0, j, h]
            np.testing.assert_allclose(o[0, t, h], ref, atol=1e-13)
            assert abs(lse[0, h, t] - scipy.special.logsumexp(lg)) < 1e-13


@pytest.mark.parametrize("w", [0, 3, 12])
def test_initial_state_gradients_match_autograd_of_closed_form(w):
    B, T, H, Hkv, d, m = 1, 12, 4, 2, 4, 3
    q, k, v, a = rand_case(B, T, H, Hkv, d, m, seed=80 + w)
    s0 = rand_s0(B, Hkv, m, d, seed=90 + w)
    dO = np.random.default_rng(97).standard_normal(q.shape)
    dq, dk, dv, da, ds0k, ds0v = oracle.bwd(q, k, v, a, dO, w, rope_base=100.0, s0=s0, want_ds0=True)
    tq, tk, tv, ta, t0k, t0v = (t64(x).requires_grad_(True) for x in (q, k, v, a, s0[0], s0[1]))
    o, _ = nha_brute(tq, tk, tv, ta, w, 100.0, s0=(t0k, t0v))
    (o * t64(dO)).sum().backward()
    for got, ref in ((dq, tq), (dk, tk), (dv, tv), (da, ta), (ds0k, t0k), (ds0v, t0v)):
        np.testing.assert_allclose(got, ref.grad.numpy(), atol=1e-11)


def test_initial_state_gradients_match_finite_differences():
    B, T, H, Hkv, d, m, w = 1, 10, 2, 1, 4, 3, 3
    q, k, v, a = rand_case(B, T, H, Hkv, d, m, seed=33)
    s0 = rand_s0(B, Hkv, m, d, seed=34)
    dO = np.random.default_rng(96).standard_normal(q.shape)
    g = oracle.bwd(q, k, v, a, dO, w, rope_base=50.0, s0=s0, want_ds0=True)
    rng = np.random.default_rng(2)
    h = 1e-6
    for which in (0, 1):
        for _ in range(12):
            idx = tuple(rng.integers(0, n) for n in s0[which].shape)
            sp = [s0[0].copy(), s0[1].copy()]
            sm = [s0[0].copy(), s0[1].copy()]
            sp[which][idx] += h
            sm[which][idx] -= h
            fp = (oracle.fwd(q, k, v, a, w, rope_base=50.0, s0=sp)[0] * dO).sum()
            fm = (oracle.fwd(q, k, v, a, w, rope_base=50.0, s0=sm)[0] * dO).sum()
            fd = (fp - fm) / (2 * h)
            assert abs(fd - g[4 + which][idx]) < 1e-7 * max(1.0, abs(fd)), (which, idx, fd)


def test_zero_initial_state_is_the_default():
    B, T, H, Hkv, d, m, w = 1, 13, 2, 2, 4, 3, 4
    q, k, v, a = rand_case(B, T, H, Hkv, d, m, seed=35)
    z = (np.zeros((B, Hkv, m, d)), np.zeros((B, Hkv, m, d)))
    dO = np.random.default_rng(3).standard_normal(q.shape)
    for x, y in zip(oracle.fwd(q, k, v, a, w), oracle.fwd(q, k, v, a, w, s0=z)):
        assert np.array_equal(x, y)
    for x, y in zip(oracle.bwd(q, k, v, a, dO, w), oracle.bwd(q, k, v, a, dO, w, s0=z)):
        assert np.array_equal(x, y)


# ---------------------------------------------------------------- no slots (m = 0)
# The ablation with no long-term memory (the gist.science page's flexibility
# section: the layer spans a pure window model at one end): m = 0 leaves
# plain (sliding-window) causal softmax attention with RoPE, which torch's
# scaled_dot_product_attention computes directly.
@pytest.mark.parametrize("w", [1, 4, 13, 20])
def test_no_slots_is_sliding_window_rope_attention(w):
    B, T, H, Hkv, d = 1, 13, 4, 2, 8
    q, k, v, a = rand_case(B, T, H, Hkv, d, 0, seed=91)
    o, lse = oracle.fwd(q, k, v, a, w, rope_base=300.0)
    qr, kr = rope_complex(t64(q), 300.0), rope_complex(t64(k), 300.0)
    tt = torch.arange(T)
    band = (tt[None, :] <= tt[:, None]) & (tt[None, :] >= tt[:, None] - w + 1)
    for h in range(H):
        g = h // (H // Hkv)
        ref = F.scaled_dot_product_attention(qr[0, :, h][None], kr[0, :, g][None], t64(v)[0, :, g][None],
                                             attn_mask=band[None])[0]
        np.testing.assert_allclose(o[0, :, h], ref.numpy(), atol=1e-12)
        lg = (qr[0, :, h] @ kr[0, :, g].T) / math.sqrt(d)
        np.testing.assert_allclose(lse[0, h], torch.logsumexp(lg.masked_fill(~band, float("-inf")), -1).numpy(),
                                   atol=1e-12)


@pytest.mark.parametrize("w", [3, 13])
def test_no_slots_gradients_match_autograd_of_attention(w):
    B, T, H, Hkv, d = 1, 13, 2, 1, 8
    q, k, v, a = rand_case(B, T, H, Hkv, d, 0, seed=92)
    dO = np.random.default_rng(5).standard_normal(q.shape)
    dq, dk, dv, da = oracle.bwd(q, k, v, a, dO, w, rope_base=300.0)
    assert da.shape == (B, T, Hkv, 0)
    tq, tk, tv = (t64(x).requires_grad_(True) for x in (q, k, v))
    qr, kr = rope_complex(tq, 300.0), rope_complex(tk, 300.0)
    tt = torch.arange(T)
    band = (tt[None, :] <= tt[:, None]) & (tt[None, :] >= tt[:, None] - w + 1)
    o = torch.stack([F.scaled_dot_product_attention(qr[0, :, h][None], kr[0, :, 0][None], tv[0, :, 0][None],
                                                    attn_mask=band[None])[0] for h in range(H)], 1)[None]
    (o * t64(dO)).sum().backward()
    for got, ref in ((dq, tq), (dk, tk), (dv, tv)):
        np.testing.assert_allclose(got, ref.grad.numpy(), atol=1e-11)


# ---------------------------------------------------------------- no token shift
# The token-shift ablation (ai.info page, findings: both memories and the
# token shift are needed): every token enters the slots at its own step,
# absorption shift 0, while the window still holds it.
@pytest.mark.parametrize("w", [0, 3, 12])
def test_no_token_shift_matches_closed_form(w):
    B, T, H, Hkv, d, m = 2, 11, 4, 2, 8, 5
    q, k, v, a = rand_case(B, T, H, Hkv, d, m, seed=110 + w)
    o, lse = oracle.fwd(q, k, v, a, w, rope_base=100.0, token_shift=False)
    o_ref, l_ref = nha_brute(t64(q), t64(k), t64(v), t64(a), w, 100.0, shift=0)
    np.testing.assert_allclose(o, o_ref.numpy(), atol=1e-12)
    np.testing.assert_allclose(lse, l_ref.numpy(), atol=1e-12)
    if w == 0:  # with no window the shift is 0 either way
        o2, _ = oracle.fwd(q, k, v, a, w, rope_base=100.0)
        assert np.array_equal(o, o2)


def test_no_token_shift_zero_gates_hold_the_current_token():
    # alpha = 0: every slot equals the raw current key / value
    B, T, H, Hkv, d, m, w = 1, 9, 1, 1, 4, 3, 4
    q, k, v, _ = rand_case(B, T, H, Hkv, d, m, seed=120)
    a = np.zeros((B, T, Hkv, m))
    _, _, sk, sv = oracle.fwd(q, k, v, a, w, rope_base=0.0, want_state=True, token_shift=False)
    np.testing.assert_array_equal(sk[0, 0], np.repeat(k[0, -1, 0][None], m, 0))
    np.testing.assert_array_equal(sv[0, 0], np.repeat(v[0, -1, 0][None], m, 0))


@pytest.mark.parametrize("w", [0, 3, 12])
def test_no_token_shift_gradients_match_autograd(w):
    B, T, H, Hkv, d, m = 1, 12, 2, 1, 4, 3
    q, k, v, a = rand_case(B, T, H, Hkv, d, m, seed=130 + w)
    dO = np.random.default_rng(95).standard_normal(q.shape)
    dq, dk, dv, da = oracle.bwd(q, k, v, a, dO, w, rope_base=100.0, token_shift=False)
    tq, tk, tv, ta = (t64(x).requires_grad_(True) for x in (q, k, v, a))
    o, _ = nha_brute(tq, tk, tv, ta, w, 100.0, shift=0)
    (o * t64(dO)).sum().backward()
    for got, ref in ((dq, tq), (dk, tk), (dv, tv), (da, ta)):
        np.testing.assert_allclose(got, ref.grad.numpy(), atol=1e-11)


# ---------------------------------------------------------------- weighted fusion
# The ablation the ai.info page's findings compare the unified softmax with
# ("Unified softmax beats weighted fusion": a fixed-coefficient weighted sum,
# and a learnable sequence-dependent coefficient), i.e. the separate-then-
# summed intra-layer hybrids of the Paper-Notes page's 现有痛点 paragraph: the
# slot and window logits each get their own softmax and o = lam o^L +
# (1 - lam) o^W.
def rand_lam(B, T, H, seed):
    return np.random.default_rng(seed).uniform(0.05, 0.95, (B, T, H))


@pytest.mark.parametrize("w", [1, 3, 12])
def test_weighted_fusion_matches_closed_form(w):
    B, T, H, Hkv, d, m = 2, 11, 4, 2, 8, 5
    q, k, v, a = rand_case(B, T, H, Hkv, d, m, seed=140 + w)
    lam = rand_lam(B, T, H, 141 + w)
    o, lse = oracle.fwd(q, k, v, a, w, rope_base=100.0, lam=lam)
    o_ref, l_ref = nha_brute(t64(q), t64(k), t64(v), t64(a), w, 100.0, lam=t64(lam))
    assert lse.shape == (2, B, H, T)
    np.testing.assert_allclose(o, o_ref.numpy(), atol=1e-12)
    np.testing.assert_allclose(lse, l_ref.numpy(), atol=1e-12)


@pytest.mark.parametrize("w", [2, 13])
def test_weighted_fusion_coefficient_zero_is_sliding_window_attention(w):
    # lam = 0 keeps only the window's own softmax: plain sliding-window RoPE
    # attention (torch scaled_dot_product_attention)
    B, T, H, Hkv, d, m = 1, 13, 4, 2, 8, 3
    q, k, v, a = rand_case(B, T, H, Hkv, d, m, seed=150 + w)
    o, lse = oracle.fwd(q, k, v, a, w, rope_base=300.0, lam=np.zeros((B, T, H)))
    qr, kr = rope_complex(t64(q), 300.0), rope_complex(t64(k), 300.0)
    tt = torch.arange(T)
    band = (tt[None, :] <= tt[:, None]) & (tt[None, :] >= tt[:, None] - w + 1)
    for h in range(H):
        g = h // (H // Hkv)
        ref = F.scaled_dot_product_attention(qr[0, :, h][None], kr[0, :, g][None], t64(v)[0, :, g][None],
                                             attn_mask=band[None])[0]
        np.testing.assert_allclose(o[0, :, h], ref.numpy(), atol=1e-12)


def test_weighted_fusion_zero_gates_read_the_shifted_token():
    # lam = 1 and alpha = 0: every slot holds the raw (k, v)_{t-w}, so the
    # slot softmax reads exactly v_{t-w} (and the m zero slots, i.e. 0, for t < w)
    B, T, H, Hkv, d, m, w = 1, 12, 2, 1, 4, 3, 4
    q, k, v, _ = rand_case(B, T, H, Hkv, d, m, seed=160)
    a = np.zeros((B, T, Hkv, m))
    o, _ = oracle.fwd(q, k, v, a, w, rope_base=100.0, lam=np.ones((B, T, H)))
    ref = np.zeros_like(o)
    ref[0, w:, :, :] = v[0, :T - w, 0][:, None, :]
    np.testing.assert_allclose(o, ref, atol=1e-13)


@pytest.mark.parametrize("w", [1, 5, 12])
def test_weighted_fusion_gradients_match_autograd(w):
    B, T, H, Hkv, d, m = 1, 12, 2, 1, 4, 3
    q, k, v, a = rand_case(B, T, H, Hkv, d, m, seed=170 + w)
    lam = rand_lam(B, T, H, 171 + w)
    dO = np.random.default_rng(172).standard_normal(q.shape)
    dq, dk, dv, da, dlam = oracle.bwd(q, k, v, a, dO, w, rope_base=100.0, lam=lam)
    tq, tk, tv, ta, tl = (t64(x).requires_grad_(True) for x in (q, k, v, a, lam))
    o, _ = nha_brute(tq, tk, tv, ta, w, 100.0, lam=tl)
    (o * t64(dO)).sum().backward()
    for got, ref in ((dq, tq), (dk, tk), (dv, tv), (da, ta), (dlam, tl)):
        np.testing.assert_allclose(got, ref.grad.numpy(), atol=1e-11)


def test_weighted_fusion_coefficient_gradient_matches_finite_differences():
    B, T, H, Hkv, d, m, w = 1, 10, 2, 1, 4, 3, 3
    q, k, v, a = rand_case(B, T, H, Hkv, d, m, seed=180)
    lam = rand_lam(B, T, H, 181)
    dO = np.random.default_rng(182).standard_normal(q.shape)
    dlam = oracle.bwd(q, k, v, a, dO, w, rope_base=50.0, lam=lam)[-1]
    h = 1e-6
    rng = np.random.default_rng(183)
    for _ in range(10):
        idx = tuple(rng.integers(0, n) for n in lam.shape)
        lp, lm = lam.copy(), lam.copy()
        lp[idx] += h
        lm[idx] -= h
        fp = (oracle.fwd(q, k, v, a, w, rope_base=50.0, lam=lp)[0] * dO).sum()
        fm = (oracle.fwd(q, k, v, a, w, rope_base=50.0, lam=lm)[0] * dO).sum()
        fd = (fp - fm) / (2 * h)
        assert abs(fd - dlam[idx]) < 1e-7 * max(1.0, abs(fd))


# ---------------------------------------------------------------- chunked prefill
# A segment that continues the state after pos0 tokens is the whole-sequence
# forward of [the P = min(pos0, w) window tokens; the segment] started from the
# slot states at pos0 (the reduction the continued-segment calls implement):
# its rows P.. equal the whole sequence's rows pos0.., and its final state the
# whole sequence's.  RoPE positions: the oracle rotates row e by e, the whole
# sequence by pos0 - P + e; logits depend on differences only.
@pytest.mark.parametrize("w,pos0", [(4, 0), (4, 2), (4, 9), (6, 6), (0, 5), (30, 11)])
def test_continued_segment_is_the_whole_sequence(w, pos0):
    B, T, H, Hkv, d, m = 1, 20, 2, 1, 8, 3
    q, k, v, a = rand_case(B, T, H, Hkv, d, m, seed=190 + w + pos0)
    o, lse, sk, sv = oracle.fwd(q, k, v, a, w, rope_base=100.0, want_state=True)
    _, _, s1k, s1v = oracle.fwd(q[:, :pos0], k[:, :pos0], v[:, :pos0], a[:, :pos0], w, rope_base=100.0,
                                want_state=True)
    P = min(pos0, w)
    ext = lambda x, fill: np.concatenate([np.full_like(x[:, :P], fill) if fill is not None else x[:, pos0 - P:pos0],
                                          x[:, pos0:]], axis=1)
    qe, ke, ve, ae = ext(q, 0.0), ext(k, None), ext(v, None), ext(a, 1.0)
    oe, le, ek, ev = oracle.fwd(qe, ke, ve, ae, w, rope_base=100.0, s0=(s1k, s1v), want_state=True)
    np.testing.assert_allclose(oe[:, P:], o[:, pos0:], atol=1e-12)
    np.testing.assert_allclose(le[:, :, P:], lse[:, :, pos0:], atol=1e-12)
    np.testing.assert_allclose(ek, sk, atol=1e-13)
    np.testing.assert_allclose(ev, sv, atol=1e-13)
