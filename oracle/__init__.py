"""fp64 CPU oracle of the NHA layer operator -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's ``cpu_baseline``
leg may import this package.  The product path (``softmax_attention_nha_amd``)
never imports, links or calls it, and this package imports nothing from there.

The arithmetic lives in ``nha_oracle.c`` (plain C, fp64, OpenMP over
(batch, KV head)); see the header of that file for what is computed and which
passage of the pages each step follows.  This module only builds and calls it.

Parity status of its parts (details in the tests that pin them):
  * forward (slots, window, RoPE, joint softmax): pinned by closed forms,
    library routines and an independent brute force;
  * backward: pinned by central finite differences of the forward and by
    torch.autograd through an independent fp64 torch formulation;
  * initial slot states and their gradients: pinned by the same closed form
    (with the decayed initial state added), its autograd, finite differences
    and the frozen-gate case;
  * weighted-fusion ablation (separate slot and window softmaxes mixed by a
    coefficient): pinned by an independent torch formulation, its autograd
    (incl. the coefficient's gradient), finite differences, and the closed
    forms at coefficient 0 (sliding-window attention) and with zero gates;
  * which gate absorbs a shifted token (alpha_t versus alpha_{t-w}) and the
    rotate-half RoPE pairing: the pages do not fix them -- parity unpinned for
    those two choices (self-consistency only).
"""
import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nha_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force=True):
    """Compile liboracle.so with gcc (fp64, OpenMP)."""
    if not force and os.path.exists(_LIB) and os.path.getmtime(_LIB) >= os.path.getmtime(_SRC):
        return _LIB
    tmp = _LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c99", _SRC, "-o", tmp, "-lm"]
    subprocess.check_call(cmd)
    os.replace(tmp, _LIB)
    return _LIB


def configure(lib):
    """Set the argument types of a loaded oracle library (this one, or a copy
    built from modified sources by the mutation tests)."""
    P = ctypes.POINTER(ctypes.c_double)
    i, dbl = ctypes.c_int, ctypes.c_double
    lib.nha_oracle_fwd.argtypes = [i] * 8 + [dbl, dbl] + [P] * 12 + [i]
    lib.nha_oracle_fwd.restype = i
    lib.nha_oracle_bwd.argtypes = [i] * 8 + [dbl, dbl] + [P] * 15 + [i]
    lib.nha_oracle_bwd.restype = i
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _lib = configure(ctypes.CDLL(_LIB))
    return _lib


def _ptr(a):
    if a is None:
        return ctypes.cast(None, ctypes.POINTER(ctypes.c_double))
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _f64(a):
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _dims(q, k, alpha):
    B, T, H, d = q.shape
    Hkv = k.shape[2]
    m = alpha.shape[3]
    assert k.shape == (B, T, Hkv, d) and alpha.shape == (B, T, Hkv, m)
    return B, T, H, Hkv, d, m


def _s0(s0, B, Hkv, m, d):
    if s0 is None:
        return None, None
    s0k, s0v = _f64(s0[0]), _f64(s0[1])
    assert s0k.shape == (B, Hkv, m, d) and s0v.shape == (B, Hkv, m, d)
    return s0k, s0v


def _lam(lam, B, T, H):
    if lam is None:
        return None
    lam = _f64(lam)
    assert lam.shape == (B, T, H)
    return lam


def fwd(q, k, v, alpha, w, rope_base=10000.0, scale=0.0, threads=0, want_state=False, s0=None, token_shift=True,
        lam=None):
    """Forward. Arrays in the operator's layouts (see nha_oracle.c).

    token_shift=False: the ablation in which every token enters the slots at
    its own step (absorption shift 0 instead of w).

    lam: the weighted-fusion ablation -- [B,T,H] coefficients; the slot and
    window logits get separate softmaxes and o = lam o_slot + (1 - lam) o_win.
    The returned lse is then [2,B,H,T]: the slot softmax's, then the window's.

    s0: optional initial slot states (S0K, S0V), each [B,Hkv,m,d] (zero when
    None).  Returns (o [B,T,H,d], lse [B,H,T]) and, with want_state, also the
    final slot states (SK, SV) each [B,Hkv,m,d]."""
    q, k, v, alpha = _f64(q), _f64(k), _f64(v), _f64(alpha)
    B, T, H, Hkv, d, m = _dims(q, k, alpha)
    s0k, s0v = _s0(s0, B, Hkv, m, d)
    lam = _lam(lam, B, T, H)
    o = np.zeros((B, T, H, d))
    lse = np.zeros((B, H, T))
    lse_w = np.zeros((B, H, T)) if lam is not None else None
    sk = np.zeros((B, Hkv, m, d)) if want_state else None
    sv = np.zeros((B, Hkv, m, d)) if want_state else None
    rc = _load().nha_oracle_fwd(B, T, H, Hkv, d, m, int(w), -1 if token_shift else 0, float(rope_base), float(scale),
                                _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(s0k), _ptr(s0v), _ptr(lam), _ptr(o),
                                _ptr(lse), _ptr(lse_w), _ptr(sk), _ptr(sv), int(threads))
    if rc:
        raise ValueError("oracle: invalid dimensions")
    if lam is not None:
        lse = np.stack([lse, lse_w])
    if want_state:
        return o, lse, sk, sv
    return o, lse


def bwd(q, k, v, alpha, dO, w, rope_base=10000.0, scale=0.0, threads=0, s0=None, want_ds0=False,
        token_shift=True, lam=None):
    """Backward. Returns (dq, dk, dv, dalpha) in the input layouts, and with
    want_ds0 also the gradients (dS0K, dS0V) of the initial slot states.
    lam: the weighted-fusion ablation (see fwd); the gradient of lam [B,T,H]
    is then appended to the result."""
    q, k, v, alpha, dO = _f64(q), _f64(k), _f64(v), _f64(alpha), _f64(dO)
    B, T, H, Hkv, d, m = _dims(q, k, alpha)
    s0k, s0v = _s0(s0, B, Hkv, m, d)
    lam = _lam(lam, B, T, H)
    dlam = np.zeros((B, T, H)) if lam is not None else None
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    da = np.zeros_like(alpha)
    ds0k = np.zeros((B, Hkv, m, d)) if want_ds0 else None
    ds0v = np.zeros((B, Hkv, m, d)) if want_ds0 else None
    rc = _load().nha_oracle_bwd(B, T, H, Hkv, d, m, int(w), -1 if token_shift else 0, float(rope_base), float(scale),
                                _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(s0k), _ptr(s0v), _ptr(lam), _ptr(dO),
                                _ptr(dq), _ptr(dk), _ptr(dv), _ptr(da), _ptr(ds0k), _ptr(ds0v), _ptr(dlam),
                                int(threads))
    if rc:
        raise ValueError("oracle: invalid dimensions")
    out = (dq, dk, dv, da)
    if want_ds0:
        out += (ds0k, ds0v)
    if lam is not None:
        out += (dlam,)
    return out
