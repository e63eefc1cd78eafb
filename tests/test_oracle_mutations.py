"""The pins catch plausible mistakes: each case plants one mistake in a copy of
the oracle's C source (on the CPU, in a temporary directory), builds it, and
checks that the independent references the pin tests use -- the hand-derived
examples, the closed-form torch formulation and its autograd -- disagree with
the planted oracle, while they agree with the real one."""
import ctypes
import json
import os
import subprocess

import numpy as np
import pytest
import torch

import oracle
from brute import nha_brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
SRC = open(os.path.join(os.path.dirname(oracle.__file__), "nha_oracle.c")).read()

# (name, text in nha_oracle.c, replacement): one planted mistake each
MUTATIONS = [
    ("absorbed token weighted by alpha, not 1 - alpha", "double ai = a[i], bi = 1.0 - a[i];",
     "double ai = a[i], bi = a[i];"),
    ("token shift one too short", "absorb(m, d, alpha + AIDX(b, t, g), k + KIDX(b, t - Dm.sh, g), SK);",
     "absorb(m, d, alpha + AIDX(b, t, g), k + KIDX(b, t - Dm.sh + (t + 1 < D->T ? 1 : 0), g), SK);"),
    ("RoPE rotation sign", "y[i] = x[i] * c[i] - x[i + h] * s[i];", "y[i] = x[i] * c[i] + x[i + h] * s[i];"),
    ("slot logits unscaled", "for (int i = 0; i < m; ++i) p[i] = s * dot(SK + (size_t)i * d, qv, d);",
     "for (int i = 0; i < m; ++i) p[i] = dot(SK + (size_t)i * d, qv, d);"),
    ("RoPE on the slots", "for (int i = 0; i < m; ++i) p[i] = s * dot(SK + (size_t)i * d, qv, d);",
     "for (int i = 0; i < m; ++i) p[i] = s * dot(SK + (size_t)i * d, qr, d);"),
    # (a window one too wide would read past the sequence in the backward:
    # the narrow one plants the same kind of mistake without leaving the arrays)
    ("window one too narrow", "  int j0 = t - w + 1;\n  if (j0 < 0) j0 = 0;\n  int nw = (w > 0) ? (t - j0 + 1) : 0;",
     "  int j0 = t - w + 2;\n  if (j0 < 0) j0 = 0;\n  int nw = (w > 0) ? (t - j0 + 1) : 0;"),
    ("D_t dropped from the slot gradient", "dl[i] = cL * p[i] * (dp - DL);", "dl[i] = cL * p[i] * dp;"),
    ("dalpha sign", "acc += lk[c] * (sk[c] - kap[c]) + lv[c] * (sv[c] - nu[c]);",
     "acc += lk[c] * (kap[c] - sk[c]) + lv[c] * (sv[c] - nu[c]);"),
    ("value adjoint not decayed", "              lv[c] *= a[i];\n", ""),
    ("window dk not rotated back", "rope_apply_T(D, cs, sn, t, dkr + (size_t)t * d, tmp);",
     "memcpy(tmp, dkr + (size_t)t * d, sizeof(double) * d);"),
    ("weighted fusion: dlam sign", "if (dlam) dlam[((size_t)b * T + t) * H + h] = DL - DW;",
     "if (dlam) dlam[((size_t)b * T + t) * H + h] = DW - DL;"),
    ("weighted fusion: window value source unscaled", "dvr[c] += cW * p[m + j] * dov[c];",
     "dvr[c] += p[m + j] * dov[c];"),
]


def build_variant(src, tmp_path, tag):
    c = os.path.join(tmp_path, "oracle_%s.c" % tag)
    so = os.path.join(tmp_path, "oracle_%s.so" % tag)
    with open(c, "w") as fh:
        fh.write(src)
    subprocess.check_call(["gcc", "-O1", "-fopenmp", "-shared", "-fPIC", "-std=c99", c, "-o", so, "-lm"])
    return oracle.configure(ctypes.CDLL(so))


def disagreements():
    """Which independent references the loaded oracle disagrees with."""
    bad = []
    ex = json.load(open(os.path.join(GOLDEN, "hand_examples.json")))
    for c in ex["cases"]:
        B, T, H, Hkv, d, m = c["B"], c["T"], c["H"], c["Hkv"], c["d"], c["m"]
        o, lse = oracle.fwd(np.array(c["q"], float).reshape(B, T, H, d), np.array(c["k"], float).reshape(B, T, Hkv, d),
                            np.array(c["v"], float).reshape(B, T, Hkv, d),
                            np.array(c["alpha"], float).reshape(B, T, Hkv, m), c["w"], rope_base=c["rope_base"],
                            scale=c["scale"])
        if not (np.allclose(o.reshape(T, d), c["o"], atol=1e-12) and np.allclose(lse.reshape(T), c["lse"], atol=1e-12)):
            bad.append("hand " + c["name"])
    rng = np.random.default_rng(7)
    B, T, H, Hkv, d, m, w = 1, 11, 2, 1, 8, 3, 3
    q, k = rng.standard_normal((B, T, H, d)) * 0.7, rng.standard_normal((B, T, Hkv, d)) * 0.7
    v = rng.standard_normal((B, T, Hkv, d))
    a = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, T, Hkv, m))))
    lam = rng.uniform(0.1, 0.9, (B, T, H))
    dO = rng.standard_normal(q.shape)
    t64 = lambda x: torch.from_numpy(np.ascontiguousarray(x))
    for lm in (None, lam):
        o, _ = oracle.fwd(q, k, v, a, w, rope_base=100.0, lam=lm)
        tq, tk, tv, ta = (t64(x).requires_grad_(True) for x in (q, k, v, a))
        tl = t64(lm).requires_grad_(True) if lm is not None else None
        ob, _ = nha_brute(tq, tk, tv, ta, w, 100.0, lam=tl)
        if not np.allclose(o, ob.detach().numpy(), atol=1e-11):
            bad.append("closed form" + (" weighted" if lm is not None else ""))
        (ob * t64(dO)).sum().backward()
        g = oracle.bwd(q, k, v, a, dO, w, rope_base=100.0, lam=lm)
        refs = [tq, tk, tv, ta] + ([tl] if lm is not None else [])
        for x, r in zip(g, refs):
            if not np.allclose(x, r.grad.numpy(), atol=1e-10):
                bad.append("autograd" + (" weighted" if lm is not None else ""))
                break
    return bad


@pytest.fixture
def swap_lib():
    saved = oracle._lib
    yield
    oracle._lib = saved


def test_unmodified_source_passes(tmp_path, swap_lib):
    oracle._lib = build_variant(SRC, str(tmp_path), "same")
    assert disagreements() == []


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[x[0] for x in MUTATIONS])
def test_planted_mistake_is_caught(name, old, new, tmp_path, swap_lib):
    assert SRC.count(old) >= 1, "mutation site not found: %s" % name
    oracle._lib = build_variant(SRC.replace(old, new), str(tmp_path), "mut")
    assert disagreements(), "planted mistake not caught: %s" % name
