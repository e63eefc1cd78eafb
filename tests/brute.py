"""Closed-form fp64 torch formulation of the NHA layer, used only to pin the oracle.

It shares nothing with the oracle's code path: instead of running the per-token
recurrence it writes each slot state as the explicit sum the recurrence unrolls
to,

    S_t[i] = sum_{u=w}^{t} ( prod_{j=u+1}^{t} alpha_j[i] ) (1 - alpha_u[i]) x_{u-w},

materialises K^H_t = [S^K_t ; R_j k_j (j in window)] for every t, and applies
torch.softmax over the concatenated logits.  RoPE is computed through complex
multiplication of the (i, i + d/2) pairs by exp(i * t * theta_i), a different
route from the oracle's cos/sin rotation.  It is differentiable, so
torch.autograd provides independent gradients for the oracle's hand-written
adjoint.  Small sizes only (O(T^2 m d) memory).
"""
import math

import torch


def rope_complex(x, base):
    """Rotate-half RoPE via complex numbers. x: [..., T, heads, d] fp64."""
    if base == 0.0:
        return x
    T, d = x.shape[-3], x.shape[-1]
    h = d // 2
    i = torch.arange(h, dtype=torch.float64)
    theta = base ** (-2.0 * i / d)
    ang = torch.arange(T, dtype=torch.float64)[:, None] * theta[None, :]  # [T, h]
    rot = torch.polar(torch.ones_like(ang), ang)[:, None, :]  # [T, 1, h]
    z = torch.complex(x[..., :h], x[..., h:]) * rot
    return torch.cat([z.real, z.imag], dim=-1)


def slot_states(x, alpha, w, s0=None):
    """Closed-form slot states. x: [B,T,Hkv,d], alpha: [B,T,Hkv,m] -> [B,T,Hkv,m,d].
    s0: optional initial state [B,Hkv,m,d], decayed by every absorbing step:
    S_t += (prod_{u<=t, u>=w} alpha_u) S0."""
    B, T, Hkv, d = x.shape
    m = alpha.shape[-1]
    t_idx = torch.arange(T)
    absorbed = (t_idx >= w).to(torch.float64)  # step u absorbs x_{u-w} iff u >= w
    la = torch.log(alpha) * absorbed[None, :, None, None]  # decay applies only when absorbing
    Lc = torch.cumsum(la, dim=1)  # [B,T,Hkv,m]
    # decay[t,u] = exp(Lc[t] - Lc[u]) for u <= t
    dec = torch.exp(Lc[:, :, None] - Lc[:, None, :])  # [B,t,u,Hkv,m]
    mask = (t_idx[:, None] >= t_idx[None, :]).to(torch.float64)  # u <= t
    beta = (1.0 - alpha) * absorbed[None, :, None, None]  # [B,u,Hkv,m]
    xs = torch.zeros_like(x)
    if w < T:
        xs[:, w:] = x[:, : T - w]  # x_{u-w} at step u
    coef = dec * mask[None, :, :, None, None] * beta[:, None]  # [B,t,u,Hkv,m]
    S = torch.einsum("btugm,bugd->btgmd", coef, xs)
    if s0 is not None:
        S = S + torch.exp(Lc)[..., None] * s0[:, None]
    return S


def nha_brute(q, k, v, alpha, w, base=10000.0, scale=0.0, s0=None, shift=None, lam=None):
    """Returns (o [B,T,H,d], lse [B,H,T]); all inputs fp64 torch tensors.
    s0: optional initial slot states (S0K, S0V), each [B,Hkv,m,d].
    shift: the absorption shift of the slots (None: w, the method; 0: every
    token enters the slots at its own step).
    lam: [B,T,H] -- the weighted-fusion ablation: torch.softmax over the slot
    logits and, separately, over the window logits; o = lam o_slot + (1 - lam)
    o_window; lse is then [2,B,H,T] (slot, window)."""
    B, T, H, d = q.shape
    Hkv, m = k.shape[2], alpha.shape[-1]
    G = H // Hkv
    s = scale if scale else 1.0 / math.sqrt(d)
    sh = w if shift is None else shift
    SK = slot_states(k, alpha, sh, None if s0 is None else s0[0])  # [B,T,Hkv,m,d]
    SV = slot_states(v, alpha, sh, None if s0 is None else s0[1])
    qr = rope_complex(q, base)
    kr = rope_complex(k, base)
    rep = lambda x: x.repeat_interleave(G, dim=2)  # KV head -> query heads
    SKh, SVh, krh, vh = rep(SK), rep(SV), rep(kr), rep(v)
    lL = s * torch.einsum("bthd,bthmd->bthm", q, SKh)  # [B,T,H,m]
    lW = s * torch.einsum("bthd,bjhd->bthj", qr, krh)  # [B,T,H,Tj]
    t_idx = torch.arange(T)
    jj = t_idx[None, :]
    tt = t_idx[:, None]
    inwin = (jj <= tt) & (jj >= tt - w + 1) if w > 0 else torch.zeros(T, T, dtype=torch.bool)
    lW = lW.masked_fill(~inwin[None, :, None, :], float("-inf"))
    if lam is not None:
        oL = torch.einsum("bthm,bthmd->bthd", torch.softmax(lL, dim=-1), SVh)
        oW = torch.einsum("bthj,bjhd->bthd", torch.softmax(lW, dim=-1), vh)
        o = lam[..., None] * oL + (1.0 - lam[..., None]) * oW
        lse = torch.stack([torch.logsumexp(lL, dim=-1), torch.logsumexp(lW, dim=-1)])  # [2,B,T,H]
        return o, lse.permute(0, 1, 3, 2).contiguous()
    logits = torch.cat([lL, lW], dim=-1)
    lse = torch.logsumexp(logits, dim=-1)  # [B,T,H]
    p = torch.softmax(logits, dim=-1)
    o = torch.einsum("bthm,bthmd->bthd", p[..., :m], SVh) + torch.einsum(
        "bthj,bjhd->bthd", p[..., m:], vh
    )
    return o, lse.permute(0, 2, 1).contiguous()
