"""Helpers for the GPU parity tests: run the HIP path through the binding and
the fp64 oracle on the same (exactly upcast) inputs, then compare."""
import sys

import numpy as np
import torch

import oracle
import softmax_attention_nha_amd as nha

# Tolerances.  fp32 inputs: max-abs 1e-4.  bf16 inputs with fp32 accumulation:
# max-abs 2e-2 on outputs and 5e-2 on gradients; in addition (these max-abs
# gates are loose at the workloads' small output magnitudes) a relative L2
# error of 1e-2 per tensor.
TOL = {
    torch.float32: dict(o=1e-4, lse=1e-4, grad=1e-4, rel=1e-5),
    torch.bfloat16: dict(o=2e-2, lse=2e-2, grad=5e-2, rel=1e-2),
}


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def f64(x):
    return x.detach().float().cpu().double().numpy()


def dev():
    return torch.device("cuda:0")


def gpu_fwd(q, k, v, a, w, C, base, state_out=None):
    d = dev()
    o, lse = nha.fwd(q.to(d), k.to(d), v.to(d), a.to(d), w, C=C, rope_base=base, state_out=state_out)
    torch.cuda.synchronize()
    return o, lse


def oracle_fwd(q, k, v, a, w, base, threads=0):
    return oracle.fwd(f64(q), f64(k), f64(v), f64(a), w, rope_base=base, threads=threads)


def unit_slice(x, b, heads):
    """Slice batch b and the given head indices (query or KV heads) of [B,T,heads,*]."""
    return x[b:b + 1, :, heads[0]:heads[-1] + 1].contiguous()


def compare(name, got, ref, atol, rel):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (name, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite values" % name
    err = np.abs(got - ref)
    mx = float(err.max()) if err.size else 0.0
    nrm = float(np.linalg.norm(ref))
    r = float(np.linalg.norm(got - ref) / nrm) if nrm > 0 else float(np.linalg.norm(got - ref))
    log("  %-8s max|err|=%.3e  rel-L2=%.3e  max|ref|=%.3e" % (name, mx, r, float(np.abs(ref).max()) if ref.size else 0))
    assert mx <= atol, "%s: max abs error %.3e > %.1e" % (name, mx, atol)
    assert r <= rel, "%s: relative L2 error %.3e > %.1e" % (name, r, rel)
    return mx, r


def _per_head(x, b, heads):
    """[B,T,*,d] -> one sequence per listed head: [len(heads),T,1,d] (fp64)."""
    return np.ascontiguousarray(f64(x[b, :, heads[0]:heads[-1] + 1]).transpose(1, 0, 2)[:, :, None, :])


def oracle_units(q, k, v, a, dO, w, base, units, G, Tp=None, lam=None):
    """The fp64 oracle on the (b, g) units listed, with every query head of a
    unit run as a sequence of its own over its KV head (the operator is
    grouped-query attention: a query head reads only its KV head, and the
    loss is a sum over query heads, so dk, dv and dalpha of a unit are the sums
    of the per-head gradients -- the GQA invariant the oracle pins check).
    The oracle's threads then cover every (unit, query head).  Tp: first Tp
    tokens only (forward: rows t < Tp depend on tokens <= t only).
    lam: [B,T,H] coefficients of the weighted-fusion ablation (then lse is
    [2,1,G,T] and the gradients end with dlam [1,T,G]).
    Returns per unit: (o [1,T,G,d], lse [1,G,T]) when dO is None, else
    (dq [1,T,G,d], dk, dv [1,T,1,d], dalpha [1,T,1,m])."""
    qs, ks, vs, as_, ds, ls = [], [], [], [], [], []
    for (b, g) in units:
        hq = list(range(g * G, (g + 1) * G))
        qs.append(_per_head(q, b, hq))
        if lam is not None:
            ls.append(np.ascontiguousarray(f64(lam[b, :, g * G:(g + 1) * G]).T[:, :, None]))
        rep = lambda x: np.repeat(_per_head(x, b, [g]), G, axis=0)
        ks.append(rep(k))
        vs.append(rep(v))
        as_.append(rep(a))
        if dO is not None:
            ds.append(_per_head(dO, b, hq))
    cut = lambda xs: np.ascontiguousarray(np.concatenate(xs)[:, :Tp] if Tp else np.concatenate(xs))
    lm = cut(ls)[..., 0] if lam is not None else None  # [units*G, T, 1] -> [units*G, T]
    if lm is not None:
        lm = lm[:, :, None]
    if dO is None:
        o, lse = oracle.fwd(cut(qs), cut(ks), cut(vs), cut(as_), w, rope_base=base, lam=lm)
        out = []
        for i in range(len(units)):
            oo = o[i * G:(i + 1) * G, :, 0].transpose(1, 0, 2)[None]
            if lam is None:
                ll = lse[i * G:(i + 1) * G, 0][None]
            else:
                ll = lse[:, i * G:(i + 1) * G, 0][:, None]
            out.append((oo, ll))
        return out
    r = oracle.bwd(cut(qs), cut(ks), cut(vs), cut(as_), cut(ds), w, rope_base=base, lam=lm)
    dq, dk, dv, da = r[:4]
    out = []
    for i in range(len(units)):
        s = slice(i * G, (i + 1) * G)
        one = (dq[s, :, 0].transpose(1, 0, 2)[None], dk[s].sum(0, keepdims=True),
               dv[s].sum(0, keepdims=True), da[s].sum(0, keepdims=True))
        if lam is not None:
            one += (r[4][s, :, 0].T[None],)
        out.append(one)
    return out
