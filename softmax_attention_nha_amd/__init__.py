"""Native Hybrid Attention (NHA) layer operator for AMD Instinct MI355X (gfx950).

Thin ctypes binding over ``libnha.so`` (the C ABI in ``include/nha.h``).  This
module only marshals arguments: it checks tensor shapes/dtypes/devices,
allocates outputs and workspaces through PyTorch, and passes raw device
pointers plus the current HIP stream.  Every step of the operator runs in the
library's HIP kernels; there is no fallback path.  If the library is missing,
``load()`` raises.

    from softmax_attention_nha_amd import fwd, bwd, decode_state, decode_step
    o, lse = fwd(q, k, v, alpha, w=512)                # q [B,T,H,d], k/v [B,T,Hkv,d]
    dq, dk, dv, dalpha = bwd(q, k, v, alpha, o, lse, dO, w=512)
"""
import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnha.so")

NHA_OK, NHA_ERR_INVALID_ARG, NHA_ERR_UNSUPPORTED, NHA_ERR_WORKSPACE, NHA_ERR_HIP = range(5)
NHA_DTYPE_F32, NHA_DTYPE_BF16 = 0, 1
_DTYPES = {torch.float32: NHA_DTYPE_F32, torch.bfloat16: NHA_DTYPE_BF16}

EXPORTED = (
    "nha_fwd_workspace_size",
    "nha_bwd_workspace_size",
    "nha_check_desc",
    "nha_decode_state_size",
    "nha_fwd",
    "nha_bwd",
    "nha_decode_step",
    "nha_status_string",
    "nha_stage_names",
    "nha_fwd_timed",
    "nha_bwd_timed",
    "nha_bwd_after_fwd",
    "nha_bwd_after_fwd_timed",
    "nha_fwd_s0",
    "nha_bwd_s0",
    "nha_release_side_streams",
    "nha_fwd_noalloc",
    "nha_weighted_workspace_size",
    "nha_fwd_weighted",
    "nha_bwd_weighted",
    "nha_continue_workspace_size",
    "nha_fwd_continue",
    "nha_bwd_continue",
)


class NhaDesc(ctypes.Structure):
    _fields_ = [
        ("B", ctypes.c_int32),
        ("T", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("Hkv", ctypes.c_int32),
        ("d", ctypes.c_int32),
        ("m", ctypes.c_int32),
        ("w", ctypes.c_int32),
        ("C", ctypes.c_int32),
        ("rope_base", ctypes.c_float),
        ("scale", ctypes.c_float),
        ("dtype", ctypes.c_int32),
        ("no_token_shift", ctypes.c_int32),
    ]


class NhaError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__("%s: %s" % (what, _lib_status(status)))


_lib = None


def load():
    """Load libnha.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            "libnha.so not found at %s: build it with `python -m softmax_attention_nha_amd.build` "
            "(or __graft_entry__.build())" % LIB_PATH
        )
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, st = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    D = ctypes.POINTER(NhaDesc)
    lib.nha_fwd_workspace_size.argtypes = [D]
    lib.nha_fwd_workspace_size.restype = sz
    lib.nha_bwd_workspace_size.argtypes = [D]
    lib.nha_bwd_workspace_size.restype = sz
    lib.nha_decode_state_size.argtypes = [D]
    lib.nha_decode_state_size.restype = sz
    lib.nha_check_desc.argtypes = [D]
    lib.nha_check_desc.restype = st
    lib.nha_fwd.argtypes = [D, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.nha_fwd.restype = st
    lib.nha_bwd.argtypes = [D, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.nha_bwd.restype = st
    lib.nha_decode_step.argtypes = [D, vp, vp, vp, vp, vp, vp, vp]
    lib.nha_decode_step.restype = st
    lib.nha_stage_names.argtypes = [D, st, st, ctypes.POINTER(ctypes.c_char_p), st]
    lib.nha_stage_names.restype = st
    lib.nha_fwd_timed.argtypes = [D, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, ctypes.POINTER(vp)]
    lib.nha_fwd_timed.restype = st
    lib.nha_bwd_timed.argtypes = [D, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, ctypes.POINTER(vp)]
    lib.nha_bwd_timed.restype = st
    lib.nha_bwd_after_fwd.argtypes = [D, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.nha_bwd_after_fwd.restype = st
    lib.nha_bwd_after_fwd_timed.argtypes = [D, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp,
                                            ctypes.POINTER(vp)]
    lib.nha_bwd_after_fwd_timed.restype = st
    lib.nha_fwd_s0.argtypes = [D] + [vp] * 10 + [sz, vp]
    lib.nha_fwd_s0.restype = st
    lib.nha_bwd_s0.argtypes = [D] + [vp] * 16 + [sz, vp]
    lib.nha_bwd_s0.restype = st
    lib.nha_fwd_noalloc.argtypes = [D, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.nha_fwd_noalloc.restype = st
    lib.nha_weighted_workspace_size.argtypes = [D]
    lib.nha_weighted_workspace_size.restype = sz
    lib.nha_fwd_weighted.argtypes = [D] + [vp] * 8 + [sz, vp]
    lib.nha_fwd_weighted.restype = st
    lib.nha_bwd_weighted.argtypes = [D] + [vp] * 12 + [sz, vp]
    lib.nha_bwd_weighted.restype = st
    ll = ctypes.c_longlong
    lib.nha_continue_workspace_size.argtypes = [D]
    lib.nha_continue_workspace_size.restype = sz
    lib.nha_fwd_continue.argtypes = [D, ll] + [vp] * 9 + [sz, vp]
    lib.nha_fwd_continue.restype = st
    lib.nha_bwd_continue.argtypes = [D, ll] + [vp] * 17 + [sz, vp]
    lib.nha_bwd_continue.restype = st
    lib.nha_release_side_streams.argtypes = []
    lib.nha_release_side_streams.restype = st
    lib.nha_status_string.argtypes = [st]
    lib.nha_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _lib_status(s):
    try:
        return load().nha_status_string(int(s)).decode()
    except Exception:  # pragma: no cover - only when the library itself is missing
        return "status %d" % s


def make_desc(B, T, H, Hkv, d, m, w, C=64, rope_base=10000.0, scale=0.0, dtype=torch.bfloat16, token_shift=True):
    """token_shift=False: the ablation in which every token enters the slots
    at its own step (instead of when it leaves the window)."""
    return NhaDesc(int(B), int(T), int(H), int(Hkv), int(d), int(m), int(w), int(C), float(rope_base),
                   float(scale), _DTYPES[dtype], 0 if token_shift else 1)


def stage_names(desc, backward=False, with_state=False):
    """Names of the kernel launches one fwd (backward=0) / bwd (1) /
    bwd(after_fwd=True) (2) call enqueues, in order."""
    lib = load()
    names = (ctypes.c_char_p * 16)()
    n = lib.nha_stage_names(ctypes.byref(desc), int(backward), int(with_state), names, 16)
    if n < 0:
        raise NhaError(lib.nha_check_desc(ctypes.byref(desc)), "stage names")
    return [names[i].decode() for i in range(n)]


def _events_arg(events):
    if events is None:
        return None
    arr = (ctypes.c_void_p * len(events))(*[ctypes.c_void_p(e) for e in events])
    return arr


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check(t, name, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s: expected shape %s, got %s" % (name, tuple(shape), tuple(t.shape)))
    if t.dtype != dtype:
        raise ValueError("%s: expected dtype %s, got %s" % (name, dtype, t.dtype))
    if t.device != device:
        raise ValueError("%s: expected device %s, got %s" % (name, device, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)


def _check_bytes(t, name, nbytes, device):
    """A raw device buffer (workspace, decode state): contiguous uint8 on
    `device` holding at least `nbytes` bytes."""
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.dtype != torch.uint8:
        raise ValueError("%s: expected dtype torch.uint8, got %s" % (name, t.dtype))
    if t.device != device:
        raise ValueError("%s: expected device %s, got %s" % (name, device, t.device))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if t.numel() < nbytes:
        raise ValueError("%s: %d bytes needed for this shape, got %d" % (name, nbytes, t.numel()))


def _desc_from(q, k, alpha, w, C, rope_base, scale, token_shift=True):
    if q.dim() != 4 or k.dim() != 4 or alpha.dim() != 4:
        raise ValueError("q, k, alpha must be 4-D: [B,T,H,d], [B,T,Hkv,d], [B,T,Hkv,m]")
    B, T, H, d = q.shape
    Hkv, m = k.shape[2], alpha.shape[3]
    if q.dtype not in _DTYPES:
        raise ValueError("dtype must be float32 or bfloat16")
    return make_desc(B, T, H, Hkv, d, m, w, C, rope_base, scale, q.dtype, token_shift)


def workspace_size(desc, backward=False):
    lib = load()
    n = (lib.nha_bwd_workspace_size if backward else lib.nha_fwd_workspace_size)(ctypes.byref(desc))
    if n == 0:
        # nha_check_desc applies the forward's rules: a descriptor it accepts
        # with no backward workspace is one the backward does not support
        rc = lib.nha_check_desc(ctypes.byref(desc))
        raise NhaError(rc if rc != NHA_OK else NHA_ERR_UNSUPPORTED,
                       "backward workspace size" if backward else "workspace size")
    return n


def decode_state_size(desc):
    lib = load()
    n = lib.nha_decode_state_size(ctypes.byref(desc))
    if n == 0:
        raise NhaError(lib.nha_check_desc(ctypes.byref(desc)), "decode state size")
    return n


def _workspace(workspace, n, dev):
    """The caller's workspace when it is large enough, else a new one."""
    if workspace is not None:
        _check_bytes(workspace, "workspace", 0, dev)
        if workspace.numel() >= n:
            return workspace
    return torch.empty(n, dtype=torch.uint8, device=dev)


def _check_s0(s0, B, Hkv, m, d, dev):
    if len(s0) != 2:
        raise ValueError("s0 must be (S0K, S0V)")
    for t, nm in zip(s0, ("s0k", "s0v")):
        _check(t, nm, (B, Hkv, m, d), torch.float32, dev)


def fwd(q, k, v, alpha, w, C=64, rope_base=10000.0, scale=0.0, state_out=None, workspace=None, out=None,
        lse_out=None, events=None, s0=None, token_shift=True):
    """Chunkwise-parallel forward. Returns (o [B,T,H,d], lse [B,H,T] float32).

    state_out: optional uint8 decode state tensor (decode_state()) that receives
    the state after the last token.  s0: optional initial slot states
    (S0K, S0V), float32 [B,Hkv,m,d] each (nha_fwd_s0; no timing events).
    token_shift=False: the ablation without token shift."""
    desc = _desc_from(q, k, alpha, w, C, rope_base, scale, token_shift)
    dev, dt = q.device, q.dtype
    B, T, H, d = q.shape
    Hkv, m = k.shape[2], alpha.shape[3]
    _check(q, "q", (B, T, H, d), dt, dev)
    _check(k, "k", (B, T, Hkv, d), dt, dev)
    _check(v, "v", (B, T, Hkv, d), dt, dev)
    _check(alpha, "alpha", (B, T, Hkv, m), dt, dev)
    lib = load()
    if out is not None:
        _check(out, "out", (B, T, H, d), dt, dev)
    if lse_out is not None:
        _check(lse_out, "lse_out", (B, H, T), torch.float32, dev)
    if state_out is not None:
        _check_bytes(state_out, "state_out", decode_state_size(desc), dev)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev) if lse_out is None else lse_out
    n = workspace_size(desc)
    ws = _workspace(workspace, n, dev)
    if s0 is not None:
        _check_s0(s0, B, Hkv, m, d, dev)
        rc = lib.nha_fwd_s0(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(s0[0]), _ptr(s0[1]),
                            _ptr(o), _ptr(lse), _ptr(state_out), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev))
        if rc != NHA_OK:
            raise NhaError(rc, "nha_fwd_s0")
        return o, lse
    rc = lib.nha_fwd_timed(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(o), _ptr(lse),
                           _ptr(state_out), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev),
                           _events_arg(events))
    if rc != NHA_OK:
        raise NhaError(rc, "nha_fwd")
    return o, lse


def fwd_noalloc(q, k, v, alpha, w, C=64, rope_base=10000.0, scale=0.0, out=None, lse_out=None, state_out=None,
                token_shift=True):
    """nha_fwd_noalloc: the forward without a workspace argument (the library's
    scratch array serves as one; shapes whose workspace exceeds it raise
    NhaError with NHA_ERR_WORKSPACE).  Returns (o, lse)."""
    desc = _desc_from(q, k, alpha, w, C, rope_base, scale, token_shift)
    dev, dt = q.device, q.dtype
    B, T, H, d = q.shape
    Hkv, m = k.shape[2], alpha.shape[3]
    _check(q, "q", (B, T, H, d), dt, dev)
    _check(k, "k", (B, T, Hkv, d), dt, dev)
    _check(v, "v", (B, T, Hkv, d), dt, dev)
    _check(alpha, "alpha", (B, T, Hkv, m), dt, dev)
    if out is not None:
        _check(out, "out", (B, T, H, d), dt, dev)
    if lse_out is not None:
        _check(lse_out, "lse_out", (B, H, T), torch.float32, dev)
    if state_out is not None:
        _check_bytes(state_out, "state_out", decode_state_size(desc), dev)
    lib = load()
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev) if lse_out is None else lse_out
    rc = lib.nha_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(o), _ptr(lse),
                             _ptr(state_out), _stream(dev))
    if rc != NHA_OK:
        raise NhaError(rc, "nha_fwd_noalloc")
    return o, lse


def bwd(q, k, v, alpha, o, lse, dO, w, C=64, rope_base=10000.0, scale=0.0, workspace=None, out=None,
        events=None, after_fwd=False, s0=None, token_shift=True):
    """Gradients of fwd. Returns (dq, dk, dv, dalpha); dalpha is float32.

    after_fwd=True calls nha_bwd_after_fwd: `workspace` must then be the one
    the forward of these inputs ran with, untouched since (the forward's RoPE'd
    q/k, gate products and chunk-start states are read from it).  s0: the
    forward's initial slot states (S0K, S0V) (nha_bwd_s0); the result then ends
    with their gradients: (dq, dk, dv, dalpha, dS0K, dS0V).  token_shift as
    for fwd."""
    desc = _desc_from(q, k, alpha, w, C, rope_base, scale, token_shift)
    dev, dt = q.device, q.dtype
    B, T, H, d = q.shape
    Hkv, m = k.shape[2], alpha.shape[3]
    for t, nm, shp in ((q, "q", (B, T, H, d)), (k, "k", (B, T, Hkv, d)), (v, "v", (B, T, Hkv, d)),
                       (alpha, "alpha", (B, T, Hkv, m)), (o, "o", (B, T, H, d)), (dO, "dO", (B, T, H, d))):
        _check(t, nm, shp, dt, dev)
    _check(lse, "lse", (B, H, T), torch.float32, dev)
    lib = load()
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        da = torch.empty((B, T, Hkv, m), dtype=torch.float32, device=dev)
    else:
        if len(out) != 4:
            raise ValueError("out must be (dq, dk, dv, dalpha)")
        dq, dk, dv, da = out
        _check(dq, "dq", (B, T, H, d), dt, dev)
        _check(dk, "dk", (B, T, Hkv, d), dt, dev)
        _check(dv, "dv", (B, T, Hkv, d), dt, dev)
        _check(da, "dalpha", (B, T, Hkv, m), torch.float32, dev)
    n = workspace_size(desc, backward=True)
    if after_fwd:
        if workspace is None:
            raise ValueError("after_fwd needs the forward's workspace, of at least %d bytes" % n)
        _check_bytes(workspace, "workspace", n, dev)
        ws = workspace
    else:
        ws = _workspace(workspace, n, dev)
    if s0 is not None:
        if after_fwd:
            raise ValueError("s0 with after_fwd is not provided (nha_bwd_s0 recomputes the prologue)")
        _check_s0(s0, B, Hkv, m, d, dev)
        ds0k, ds0v = torch.empty_like(s0[0]), torch.empty_like(s0[1])
        rc = lib.nha_bwd_s0(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(s0[0]), _ptr(s0[1]),
                            _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(da), _ptr(ds0k),
                            _ptr(ds0v), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev))
        if rc != NHA_OK:
            raise NhaError(rc, "nha_bwd_s0")
        return dq, dk, dv, da, ds0k, ds0v
    fn = lib.nha_bwd_after_fwd_timed if after_fwd else lib.nha_bwd_timed
    rc = fn(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq),
            _ptr(dk), _ptr(dv), _ptr(da), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev), _events_arg(events))
    if rc != NHA_OK:
        raise NhaError(rc, "nha_bwd")
    return dq, dk, dv, da


def release_side_streams():
    """Destroy the calling thread's library side streams (nha_release_side_streams)."""
    rc = load().nha_release_side_streams()
    if rc != NHA_OK:
        raise NhaError(rc, "nha_release_side_streams")


def weighted_workspace_size(desc):
    lib = load()
    n = lib.nha_weighted_workspace_size(ctypes.byref(desc))
    if n == 0:
        # past nha_check_desc: m < 1 or w < 1 (invalid for this mode), else
        # the backward's LDS limit (unsupported)
        rc = lib.nha_check_desc(ctypes.byref(desc))
        if rc == NHA_OK:
            rc = NHA_ERR_INVALID_ARG if desc.m < 1 or desc.w < 1 else NHA_ERR_UNSUPPORTED
        raise NhaError(rc, "weighted workspace size")
    return n


def _check_lam(lam, B, T, H, dev):
    _check(lam, "lam", (B, T, H), torch.float32, dev)


def fwd_weighted(q, k, v, alpha, lam, w, C=64, rope_base=10000.0, scale=0.0, workspace=None, out=None,
                 lse_out=None, token_shift=True):
    """The weighted-fusion ablation (nha_fwd_weighted): separate slot and
    window softmaxes, o = lam o_slot + (1 - lam) o_window with lam float32
    [B,T,H].  Returns (o, lse2) with lse2 [2,B,H,T] (slot, window)."""
    desc = _desc_from(q, k, alpha, w, C, rope_base, scale, token_shift)
    dev, dt = q.device, q.dtype
    B, T, H, d = q.shape
    Hkv, m = k.shape[2], alpha.shape[3]
    for t, nm, shp in ((q, "q", (B, T, H, d)), (k, "k", (B, T, Hkv, d)), (v, "v", (B, T, Hkv, d)),
                       (alpha, "alpha", (B, T, Hkv, m))):
        _check(t, nm, shp, dt, dev)
    _check_lam(lam, B, T, H, dev)
    if out is not None:
        _check(out, "out", (B, T, H, d), dt, dev)
    if lse_out is not None:
        _check(lse_out, "lse_out", (2, B, H, T), torch.float32, dev)
    lib = load()
    o = torch.empty_like(q) if out is None else out
    lse2 = torch.empty((2, B, H, T), dtype=torch.float32, device=dev) if lse_out is None else lse_out
    ws = _workspace(workspace, weighted_workspace_size(desc), dev)
    rc = lib.nha_fwd_weighted(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(lam), _ptr(o),
                              _ptr(lse2), _ptr(ws), ctypes.c_size_t(ws.numel()), _stream(dev))
    if rc != NHA_OK:
        raise NhaError(rc, "nha_fwd_weighted")
    return o, lse2


def bwd_weighted(q, k, v, alpha, lam, dO, w, C=64, rope_base=10000.0, scale=0.0, workspace=None, out=None,
                 want_dlam=True, token_shift=True):
    """Gradients of fwd_weighted: (dq, dk, dv, dalpha, dlam) -- dlam float32
    [B,T,H], or None with want_dlam=False (a fixed coefficient)."""
    desc = _desc_from(q, k, alpha, w, C, rope_base, scale, token_shift)
    dev, dt = q.device, q.dtype
    B, T, H, d = q.shape
    Hkv, m = k.shape[2], alpha.shape[3]
    for t, nm, shp in ((q, "q", (B, T, H, d)), (k, "k", (B, T, Hkv, d)), (v, "v", (B, T, Hkv, d)),
                       (alpha, "alpha", (B, T, Hkv, m)), (dO, "dO", (B, T, H, d))):
        _check(t, nm, shp, dt, dev)
    _check_lam(lam, B, T, H, dev)
    if out is None:
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        da = torch.empty((B, T, Hkv, m), dtype=torch.float32, device=dev)
        dlam = torch.empty((B, T, H), dtype=torch.float32, device=dev) if want_dlam else None
    else:
        if len(out) != 5:
            raise ValueError("out must be (dq, dk, dv, dalpha, dlam or None)")
        dq, dk, dv, da, dlam = out
        _check(dq, "dq", (B, T, H, d), dt, dev)
        _check(dk, "dk", (B, T, Hkv, d), dt, dev)
        _check(dv, "dv", (B, T, Hkv, d), dt, dev)
        _check(da, "dalpha", (B, T, Hkv, m), torch.float32, dev)
        if dlam is not None:
            _check(dlam, "dlam", (B, T, H), torch.float32, dev)
    lib = load()
    ws = _workspace(workspace, weighted_workspace_size(desc), dev)
    rc = lib.nha_bwd_weighted(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(lam), _ptr(dO),
                              _ptr(dq), _ptr(dk), _ptr(dv), _ptr(da), _ptr(dlam), _ptr(ws),
                              ctypes.c_size_t(ws.numel()), _stream(dev))
    if rc != NHA_OK:
        raise NhaError(rc, "nha_bwd_weighted")
    return dq, dk, dv, da, dlam


def continue_workspace_size(desc):
    lib = load()
    n = lib.nha_continue_workspace_size(ctypes.byref(desc))
    if n == 0:
        rc = lib.nha_check_desc(ctypes.byref(desc))
        raise NhaError(rc if rc != NHA_OK else NHA_ERR_UNSUPPORTED, "continue workspace size")
    return n


def fwd_continue(q, k, v, alpha, w, state_in, pos0, C=64, rope_base=10000.0, scale=0.0, state_out=None,
                 workspace=None, out=None, lse_out=None):
    """Chunked prefill (nha_fwd_continue): the forward over a segment that
    continues `state_in` (a decode state after pos0 tokens).  state_out may be
    state_in itself.  Returns (o, lse) of the segment."""
    desc = _desc_from(q, k, alpha, w, C, rope_base, scale)
    dev, dt = q.device, q.dtype
    B, T, H, d = q.shape
    Hkv, m = k.shape[2], alpha.shape[3]
    for t, nm, shp in ((q, "q", (B, T, H, d)), (k, "k", (B, T, Hkv, d)), (v, "v", (B, T, Hkv, d)),
                       (alpha, "alpha", (B, T, Hkv, m))):
        _check(t, nm, shp, dt, dev)
    n_state = decode_state_size(desc)
    _check_bytes(state_in, "state_in", n_state, dev)
    if state_out is not None:
        _check_bytes(state_out, "state_out", n_state, dev)
    if out is not None:
        _check(out, "out", (B, T, H, d), dt, dev)
    if lse_out is not None:
        _check(lse_out, "lse_out", (B, H, T), torch.float32, dev)
    lib = load()
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty((B, H, T), dtype=torch.float32, device=dev) if lse_out is None else lse_out
    ws = _workspace(workspace, continue_workspace_size(desc), dev)
    rc = lib.nha_fwd_continue(ctypes.byref(desc), ctypes.c_longlong(int(pos0)), _ptr(state_in), _ptr(q), _ptr(k),
                              _ptr(v), _ptr(alpha), _ptr(o), _ptr(lse), _ptr(state_out), _ptr(ws),
                              ctypes.c_size_t(ws.numel()), _stream(dev))
    if rc != NHA_OK:
        raise NhaError(rc, "nha_fwd_continue")
    return o, lse


def bwd_continue(q, k, v, alpha, o, lse, dO, w, state_in, pos0, C=64, rope_base=10000.0, scale=0.0,
                 workspace=None, want_ring=True):
    """Gradients of fwd_continue: (dq, dk, dv, dalpha, dS0K, dS0V, dRK, dRV) --
    the last four w.r.t. the state it continued (slots float32 [B,Hkv,m,d];
    ring keys / values in the state's ring layout [B,Hkv,w,d], None with
    want_ring=False)."""
    desc = _desc_from(q, k, alpha, w, C, rope_base, scale)
    dev, dt = q.device, q.dtype
    B, T, H, d = q.shape
    Hkv, m = k.shape[2], alpha.shape[3]
    for t, nm, shp in ((q, "q", (B, T, H, d)), (k, "k", (B, T, Hkv, d)), (v, "v", (B, T, Hkv, d)),
                       (alpha, "alpha", (B, T, Hkv, m)), (o, "o", (B, T, H, d)), (dO, "dO", (B, T, H, d))):
        _check(t, nm, shp, dt, dev)
    _check(lse, "lse", (B, H, T), torch.float32, dev)
    _check_bytes(state_in, "state_in", decode_state_size(desc), dev)
    lib = load()
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    da = torch.empty((B, T, Hkv, m), dtype=torch.float32, device=dev)
    ds0k = torch.empty((B, Hkv, m, d), dtype=torch.float32, device=dev)
    ds0v = torch.empty_like(ds0k)
    drk = torch.empty((B, Hkv, w, d), dtype=dt, device=dev) if want_ring and w > 0 else None
    drv = torch.empty_like(drk) if drk is not None else None
    ws = _workspace(workspace, continue_workspace_size(desc), dev)
    rc = lib.nha_bwd_continue(ctypes.byref(desc), ctypes.c_longlong(int(pos0)), _ptr(state_in), _ptr(q), _ptr(k),
                              _ptr(v), _ptr(alpha), _ptr(o), _ptr(lse), _ptr(dO), _ptr(dq), _ptr(dk), _ptr(dv),
                              _ptr(da), _ptr(ds0k), _ptr(ds0v), _ptr(drk), _ptr(drv), _ptr(ws),
                              ctypes.c_size_t(ws.numel()), _stream(dev))
    if rc != NHA_OK:
        raise NhaError(rc, "nha_bwd_continue")
    return dq, dk, dv, da, ds0k, ds0v, drk, drv


def decode_state(B, H, Hkv, d, m, w, rope_base=10000.0, scale=0.0, dtype=torch.bfloat16, device="cuda"):
    """A zero decode state (the state before the first token)."""
    desc = make_desc(B, 1, H, Hkv, d, m, w, 64, rope_base, scale, dtype)
    return torch.zeros(decode_state_size(desc), dtype=torch.uint8, device=device)


def decode_step(q_t, k_t, v_t, alpha_t, state, w, rope_base=10000.0, scale=0.0, out=None, token_shift=True):
    """One recurrent step. q_t [B,H,d], k_t/v_t [B,Hkv,d], alpha_t [B,Hkv,m]. Returns o_t [B,H,d]."""
    if q_t.dim() != 3 or k_t.dim() != 3 or alpha_t.dim() != 3:
        raise ValueError("q_t, k_t, alpha_t must be 3-D: [B,H,d], [B,Hkv,d], [B,Hkv,m]")
    B, H, d = q_t.shape
    Hkv, m = k_t.shape[1], alpha_t.shape[2]
    dev, dt = q_t.device, q_t.dtype
    if dt not in _DTYPES:
        raise ValueError("dtype must be float32 or bfloat16")
    _check(q_t, "q_t", (B, H, d), dt, dev)
    _check(k_t, "k_t", (B, Hkv, d), dt, dev)
    _check(v_t, "v_t", (B, Hkv, d), dt, dev)
    _check(alpha_t, "alpha_t", (B, Hkv, m), dt, dev)
    desc = make_desc(B, 1, H, Hkv, d, m, w, 64, rope_base, scale, dt, token_shift)
    _check_bytes(state, "state", decode_state_size(desc), dev)
    if out is not None:
        _check(out, "out", (B, H, d), dt, dev)
    o = torch.empty_like(q_t) if out is None else out
    rc = load().nha_decode_step(ctypes.byref(desc), _ptr(q_t), _ptr(k_t), _ptr(v_t), _ptr(alpha_t), _ptr(state),
                                _ptr(o), _stream(dev))
    if rc != NHA_OK:
        raise NhaError(rc, "nha_decode_step")
    return o
