"""fp64 NumPy model of the chunked decomposition the HIP kernels implement.

Test infrastructure: it mirrors, step by step and in float64, the algebra of
the GPU path (chunks of C rows cut into 16-row blocks; every decay factor
referred to a block boundary so that it never exceeds 1; exact running
products inside a block; slot branch merged with the window branch through
their log-sum-exps; reverse adjoint scan over chunks; dalpha from the E - F
identity).  Comparing it with the per-token oracle validates that algebra on
the CPU.  It shares no code with the oracle or with the kernels.

Per (batch, KV head) unit, with a_t = alpha_t, b_t = 1 - alpha_t for t >= w
(a_t = 1, b_t = 0 before), kappa_t = k_{t-w}, nu_t = v_{t-w}:
    S_t = a_t S_{t-1} + b_t (x) kappa_t                      (slot state)
    Lam_t = dS_t + a_{t+1} Lam_{t+1}                         (its adjoint)
"""
import numpy as np

SB = 16


def rope_np(x, base):
    """Rotate-half RoPE of x [T, ..., d] at positions 0..T-1 (cos/sin form)."""
    if base == 0.0:
        return x.copy()
    T, d = x.shape[0], x.shape[-1]
    h = d // 2
    th = base ** (-2.0 * np.arange(h) / d)
    ang = np.arange(T)[:, None] * th[None, :]
    shp = (T,) + (1,) * (x.ndim - 2) + (h,)
    c, s = np.cos(ang).reshape(shp), np.sin(ang).reshape(shp)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], -1)


def rope_np_T(x, base):
    """Inverse rotation R_t^T x."""
    if base == 0.0:
        return x.copy()
    T, d = x.shape[0], x.shape[-1]
    h = d // 2
    th = base ** (-2.0 * np.arange(h) / d)
    ang = np.arange(T)[:, None] * th[None, :]
    shp = (T,) + (1,) * (x.ndim - 2) + (h,)
    c, s = np.cos(ang).reshape(shp), np.sin(ang).reshape(shp)
    x1, x2 = x[..., :h], x[..., h:]
    return np.concatenate([x1 * c + x2 * s, x2 * c - x1 * s], -1)


def gates(alpha, w):
    T = alpha.shape[0]
    ab = (np.arange(T) >= w)[:, None]
    a = np.where(ab, alpha, 1.0)
    b = np.where(ab, 1.0 - alpha, 0.0)
    la = np.log2(np.maximum(a, 2.0 ** -80))
    return a, b, la


def shifted(x, w):
    out = np.zeros_like(x)
    T = x.shape[0]
    if w < T:
        out[w:] = x[: T - w]
    return out


def blocks(n):
    return [(s, min(s + SB, n)) for s in range(0, n, SB)]


def factorizable(G, i0, i1):
    """Same-block pairs use the block-end reference when every slot's total
    decay over the block is >= 2^-16 (the kernels' test)."""
    before = G[i0 - 1] if i0 > 0 else np.zeros_like(G[0])
    return bool(np.all(G[i1 - 1] - before >= -16.0))


# ---------------------------------------------------------------- intra-chunk products
def fwd_read(X, S0, keys, G, a, b, Wts):
    """Forward-in-time read of the chunk's slot states by vectors X [n, d]:
        out[t, i] = <X_t, S_t[i]>,  S_t = 2^{G_t} S0 + sum_{u<=t} 2^{G_t-G_u} b_u (x) keys_u.
    Cross-block pairs via E_J = G at the last row of block J; same-block pairs
    via running products of a.  Wts unused (kept for symmetry)."""
    n = X.shape[0]
    out = (X @ S0.T) * np.exp2(G)
    A = X @ keys.T  # [t, u]
    for (i0, i1) in blocks(n):
        fast = factorizable(G, i0, i1)
        for (j0, j1) in blocks(n):
            if j0 > i0 or (j0 == i0 and not fast):
                break
            E = G[j1 - 1]
            Bj = np.exp2(E - G[j0:j1]) * b[j0:j1]  # <= 1
            Aij = A[i0:i1, j0:j1]
            if j0 == i0:
                Aij = np.tril(Aij)  # u <= t
            out[i0:i1] += np.exp2(G[i0:i1] - E) * (Aij @ Bj)
        if fast:
            continue
        for t in range(i0, i1):
            Dp = np.ones_like(G[0])
            for u in range(t, i0 - 1, -1):
                out[t] += A[t, u] * Dp * b[u]
                Dp = Dp * a[u]
    return out


def fwd_mix(P, S0, keys, G, a, b):
    """Forward-in-time weighted sum of the chunk's slot states:
        out[t] = sum_i P[t, i] S_t[i]   (S_t as in fwd_read, rows of keys)."""
    n = P.shape[0]
    out = (P * np.exp2(G)) @ S0
    for (i0, i1) in blocks(n):
        fast = factorizable(G, i0, i1)
        for (j0, j1) in blocks(n):
            if j0 > i0 or (j0 == i0 and not fast):
                break
            E = G[j1 - 1]
            Bj = np.exp2(E - G[j0:j1]) * b[j0:j1]
            At = (P[i0:i1] * np.exp2(G[i0:i1] - E)) @ Bj.T  # [t, u]
            if j0 == i0:
                At = np.tril(At)
            out[i0:i1] += At @ keys[j0:j1]
        if fast:
            continue
        for t in range(i0, i1):
            Dp = np.ones_like(G[0])
            for u in range(t, i0 - 1, -1):
                out[t] += np.sum(P[t] * Dp * b[u]) * keys[u]
                Dp = Dp * a[u]
    return out


def rev_mix(Wb, L0, W, vecs, G, a):
    """Backward-in-time weighted sum of the chunk's adjoints:
        out[t] = sum_i Wb[t, i] Lam_t[i],
        Lam_t[i] = 2^{G_end - G_t} L0[i] + sum_{u>=t} 2^{G_u - G_t} W[u, i] vecs_u.
    Cross-block pairs via F_I = G at the last row of the query block I."""
    n = Wb.shape[0]
    out = (Wb * np.exp2(G[n - 1] - G)) @ L0
    for (i0, i1) in blocks(n):
        F = G[i1 - 1]
        fast = factorizable(G, i0, i1)
        for (j0, j1) in blocks(n):
            if j0 < i0 or (j0 == i0 and not fast):
                continue
            Y = W[j0:j1] * np.exp2(G[j0:j1] - F)  # <= 1 (>= 1 on the block itself)
            M = (Wb[i0:i1] * np.exp2(F - G[i0:i1])) @ Y.T  # [t, u]
            if j0 == i0:
                M = np.triu(M)  # u >= t
            out[i0:i1] += M @ vecs[j0:j1]
        if fast:
            continue
        for t in range(i0, i1):
            Dp = np.ones_like(G[0])
            for u in range(t, i1):
                out[t] += np.sum(Wb[t] * Dp * W[u]) * vecs[u]
                if u + 1 < i1:
                    Dp = Dp * a[u + 1]
    return out


def rev_read(Y, L0, W, vecs, G, a):
    """Backward-in-time read of the chunk's adjoints by vectors Y [n, d]:
        out[t, i] = <Y_t, Lam_t[i]>   (Lam_t as in rev_mix)."""
    n = Y.shape[0]
    out = (Y @ L0.T) * np.exp2(G[n - 1] - G)
    A = vecs @ Y.T  # [u, t]
    for (i0, i1) in blocks(n):
        F = G[i1 - 1]
        fast = factorizable(G, i0, i1)
        for (j0, j1) in blocks(n):
            if j0 < i0 or (j0 == i0 and not fast):
                continue
            Yw = W[j0:j1] * np.exp2(G[j0:j1] - F)
            Aji = A[j0:j1, i0:i1].T  # [t, u]
            if j0 == i0:
                Aji = np.triu(Aji)  # u >= t
            out[i0:i1] += np.exp2(F - G[i0:i1]) * (Aji @ Yw)
        if fast:
            continue
        for t in range(i0, i1):
            Dp = np.ones_like(G[0])
            for u in range(t, i1):
                out[t] += A[u, t] * Dp * W[u]
                if u + 1 < i1:
                    Dp = Dp * a[u + 1]
    return out


# ---------------------------------------------------------------- window branch (plain band attention)
def window_logits(qr, kr, w, s):
    T = qr.shape[0]
    lg = s * qr @ kr.T
    tt = np.arange(T)
    band = (tt[None, :] <= tt[:, None]) & (tt[None, :] > tt[:, None] - w)
    return np.where(band, lg, -np.inf), band


# ---------------------------------------------------------------- one unit
def unit_fwd(q, k, v, alpha, w, C, base, s):
    """q [T,G,d], k/v [T,d], alpha [T,m] -> o [T,G,d], lse [G,T], chunk-start states."""
    T, G, d = q.shape
    a, b, la = gates(alpha, w)
    kap, nu = shifted(k, w), shifted(v, w)
    qr, kr = rope_np(q, base), rope_np(k, base)
    NC = (T + C - 1) // C
    SK = np.zeros((alpha.shape[1], d))
    SV = np.zeros_like(SK)
    starts = []
    o = np.zeros_like(q)
    lse = np.zeros((G, T))
    for c in range(NC):
        t0, t1 = c * C, min(T, (c + 1) * C)
        starts.append((SK.copy(), SV.copy()))
        Gc = np.cumsum(la[t0:t1], 0)
        for h in range(G):
            lL = s * fwd_read(q[t0:t1, h], SK, kap[t0:t1], Gc, a[t0:t1], b[t0:t1], None)
            muL = lL.max(1, keepdims=True)
            pL = np.exp(lL - muL)
            zL = pL.sum(1, keepdims=True)
            oL = fwd_mix(pL, SV, nu[t0:t1], Gc, a[t0:t1], b[t0:t1]) / zL
            lseL = (muL + np.log(zL))[:, 0]
            # window branch seeded with the slot partial
            lW, _ = window_logits(qr[:, h], kr, w, s) if w > 0 else (np.full((T, T), -np.inf), None)
            lW = lW[t0:t1]
            mu = np.maximum(lseL, lW.max(1))
            pW = np.exp(lW - mu[:, None])
            z = np.exp(lseL - mu) + pW.sum(1)
            o[t0:t1, h] = (np.exp(lseL - mu)[:, None] * oL + pW @ v) / z[:, None]
            lse[h, t0:t1] = mu + np.log(z)
        Wc = np.exp2(Gc[-1] - Gc) * b[t0:t1]
        SK = np.exp2(Gc[-1])[:, None] * SK + Wc.T @ kap[t0:t1]
        SV = np.exp2(Gc[-1])[:, None] * SV + Wc.T @ nu[t0:t1]
    return o, lse, starts


def unit_bwd(q, k, v, alpha, dO, w, C, base, s):
    """Gradients of unit_fwd: (dq [T,G,d], dk [T,d], dv [T,d], dalpha [T,m])."""
    T, G, d = q.shape
    m = alpha.shape[1]
    o, lse, starts = unit_fwd(q, k, v, alpha, w, C, base, s)
    a, b, la = gates(alpha, w)
    kap, nu = shifted(k, w), shifted(v, w)
    qr, kr = rope_np(q, base), rope_np(k, base)
    Dt = np.einsum("tgd,tgd->tg", dO, o)
    NC = (T + C - 1) // C
    dq = np.zeros_like(q)
    dkap = np.zeros_like(k)
    dnu = np.zeros_like(v)
    Acon = np.zeros((T, m))
    pL = np.zeros((T, G, m))
    sdl = np.zeros((T, G, m))
    dLam = []
    for c in range(NC):
        t0, t1 = c * C, min(T, (c + 1) * C)
        SK, SV = starts[c]
        Gc = np.cumsum(la[t0:t1], 0)
        dLK = np.zeros((m, d))
        dLV = np.zeros((m, d))
        for h in range(G):
            lL = s * fwd_read(q[t0:t1, h], SK, kap[t0:t1], Gc, a[t0:t1], b[t0:t1], None)
            p = np.exp(lL - lse[h, t0:t1, None])
            dp = fwd_read(dO[t0:t1, h], SV, nu[t0:t1], Gc, a[t0:t1], b[t0:t1], None)
            dl = p * (dp - Dt[t0:t1, h, None])
            dq[t0:t1, h] += s * fwd_mix(dl, SK, kap[t0:t1], Gc, a[t0:t1], b[t0:t1])
            Acon[t0:t1] += dl * lL + p * dp
            pL[t0:t1, h] = p
            sdl[t0:t1, h] = s * dl
            dLK += (np.exp2(Gc) * s * dl).T @ q[t0:t1, h]
            dLV += (np.exp2(Gc) * p).T @ dO[t0:t1, h]
        dLam.append((dLK, dLV))
    # reverse adjoint scan over chunks
    Lin = [None] * NC
    LK = np.zeros((m, d))
    LV = np.zeros((m, d))
    for c in range(NC - 1, -1, -1):
        t0, t1 = c * C, min(T, (c + 1) * C)
        Lin[c] = (LK.copy(), LV.copy())
        ge = np.exp2(np.cumsum(la[t0:t1], 0)[-1])[:, None]
        LK = ge * LK + dLam[c][0]
        LV = ge * LV + dLam[c][1]
    F = np.zeros((T, m))
    for c in range(NC):
        t0, t1 = c * C, min(T, (c + 1) * C)
        Gc = np.cumsum(la[t0:t1], 0)
        LK0, LV0 = Lin[c]
        dkap[t0:t1] += rev_mix(b[t0:t1], LK0, np.zeros((t1 - t0, m)), np.zeros((t1 - t0, d)), Gc, a[t0:t1])
        dnu[t0:t1] += rev_mix(b[t0:t1], LV0, np.zeros((t1 - t0, m)), np.zeros((t1 - t0, d)), Gc, a[t0:t1])
        F[t0:t1] += rev_read(kap[t0:t1], LK0, np.zeros((t1 - t0, m)), np.zeros((t1 - t0, d)), Gc, a[t0:t1])
        F[t0:t1] += rev_read(nu[t0:t1], LV0, np.zeros((t1 - t0, m)), np.zeros((t1 - t0, d)), Gc, a[t0:t1])
        for h in range(G):
            zL = np.zeros((m, d))
            dkap[t0:t1] += rev_mix(b[t0:t1], zL, sdl[t0:t1, h], q[t0:t1, h], Gc, a[t0:t1])
            dnu[t0:t1] += rev_mix(b[t0:t1], zL, pL[t0:t1, h], dO[t0:t1, h], Gc, a[t0:t1])
            F[t0:t1] += rev_read(kap[t0:t1], zL, sdl[t0:t1, h], q[t0:t1, h], Gc, a[t0:t1])
            F[t0:t1] += rev_read(nu[t0:t1], zL, pL[t0:t1, h], dO[t0:t1, h], Gc, a[t0:t1])
    X = Acon - b * F
    rc = np.cumsum(X[::-1], 0)[::-1]
    dalpha = np.where((np.arange(T) >= w)[:, None], rc / alpha - F, 0.0)
    # window branch
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    if w > 0:
        dkr = np.zeros_like(k)
        for h in range(G):
            lW, band = window_logits(qr[:, h], kr, w, s)
            pW = np.exp(lW - lse[h][:, None])
            dpW = dO[:, h] @ v.T
            dlW = np.where(band, pW * (dpW - Dt[:, h, None]), 0.0)
            dq[:, h] += rope_np_T(s * dlW @ kr, base)
            dkr += s * dlW.T @ qr[:, h]
            dv += pW.T @ dO[:, h]
        dk += rope_np_T(dkr, base)
    # slot-path contributions land on the shifted rows
    if w < T:
        dk[: T - w] += dkap[w:]
        dv[: T - w] += dnu[w:]
    return dq, dk, dv, dalpha


def run(fn, q, k, v, alpha, *extra, w, C, base, scale=0.0):
    """Apply unit function over [B,T,H,d] / [B,T,Hkv,d] / [B,T,Hkv,m] arrays."""
    B, T, H, d = q.shape
    Hkv = k.shape[2]
    G = H // Hkv
    s = scale if scale else 1.0 / np.sqrt(d)
    outs = None
    for bb in range(B):
        for g in range(Hkv):
            hs = slice(g * G, (g + 1) * G)
            ex = [e[bb, :, hs] for e in extra]
            r = fn(q[bb, :, hs], k[bb, :, g], v[bb, :, g], alpha[bb, :, g], *ex, w, C, base, s)
            if outs is None:
                outs = [None] * len(r)
            for i, x in enumerate(r):
                outs[i] = outs[i] if outs[i] is not None else []
                outs[i].append((bb, g, x))
    return outs


def model_fwd(q, k, v, alpha, w, C, base=10000.0, scale=0.0):
    B, T, H, d = q.shape
    Hkv = k.shape[2]
    G = H // Hkv
    o = np.zeros_like(q)
    lse = np.zeros((B, H, T))
    s = scale if scale else 1.0 / np.sqrt(d)
    for bb in range(B):
        for g in range(Hkv):
            hs = slice(g * G, (g + 1) * G)
            oo, ll, _ = unit_fwd(q[bb, :, hs], k[bb, :, g], v[bb, :, g], alpha[bb, :, g], w, C, base, s)
            o[bb, :, hs] = oo
            lse[bb, hs] = ll
    return o, lse


def model_bwd(q, k, v, alpha, dO, w, C, base=10000.0, scale=0.0):
    B, T, H, d = q.shape
    Hkv = k.shape[2]
    G = H // Hkv
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    da = np.zeros_like(alpha)
    s = scale if scale else 1.0 / np.sqrt(d)
    for bb in range(B):
        for g in range(Hkv):
            hs = slice(g * G, (g + 1) * G)
            r = unit_bwd(q[bb, :, hs], k[bb, :, g], v[bb, :, g], alpha[bb, :, g], dO[bb, :, hs], w, C, base, s)
            dq[bb, :, hs], dk[bb, :, g], dv[bb, :, g], da[bb, :, g] = r
    return dq, dk, dv, da
