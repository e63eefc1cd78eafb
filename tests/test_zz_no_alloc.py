"""GPU check of the allocation-free forward (nha_fwd_noalloc, through the C
ABI): two calls in a row -- the second with a smaller input, so the scratch
array still holds the first call's larger contents -- give the outputs and
exported decode state of nha_fwd with a workspace, bitwise (the same kernels);
a shape whose workspace exceeds the scratch array is refused before any work."""
import ctypes

import pytest
import torch

import softmax_attention_nha_amd as nha
from parity_util import log
from softmax_attention_nha_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 64 << 20  # NHA_NOALLOC_SCRATCH_BYTES in include/nha.h


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr() if t is not None else 0)


def _setup(wl, w):
    dev = torch.device("cuda:0")
    q, k, v, a = (x.to(dev) for x in make_inputs(wl))
    desc = nha.make_desc(wl.B, wl.T, wl.H, wl.Hkv, wl.d, wl.m, w, wl.C, wl.rope_base, 0.0, wl.dtype)
    assert nha.workspace_size(desc) <= SCRATCH_BYTES
    o = torch.full_like(q, float("nan"))
    lse = torch.full((wl.B, wl.H, wl.T), float("nan"), dtype=torch.float32, device=dev)
    state = torch.zeros(nha.decode_state_size(desc), dtype=torch.uint8, device=dev)
    # bytes of the state before its per-step scratch region (the last one,
    # [B*H][32][d+4] floats, which has no meaning between calls)
    part = (wl.B * wl.H * 32 * (wl.d + 4) * 4 + 255) // 256 * 256
    return desc, (q, k, v, a), (o, lse, state), state.numel() - part


def test_noalloc_forward_equals_workspace_forward_twice():
    # the 1.3B head shape (d = 128, m = 64) over one sequence of 2048 tokens,
    # then a smaller, ragged GQA case (T = 777, w = 100)
    cases = [(WORKLOADS["long"].with_(T=2048, seed=81), 512),
             (WORKLOADS["gqa"].with_(T=777, H=8, Hkv=2, seed=82), 100)]
    lib = nha.load()
    dev = torch.device("cuda:0")
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    runs = [_setup(wl, w) for wl, w in cases]
    refs = []
    for desc, (q, k, v, a), _, _ in runs:
        o = torch.empty_like(q)
        lse = torch.empty((desc.B, desc.H, desc.T), dtype=torch.float32, device=dev)
        state = torch.zeros(nha.decode_state_size(desc), dtype=torch.uint8, device=dev)
        ws = torch.empty(nha.workspace_size(desc), dtype=torch.uint8, device=dev)
        rc = lib.nha_fwd(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(o), _ptr(lse), _ptr(state),
                         _ptr(ws), ctypes.c_size_t(ws.numel()), stream)
        assert rc == nha.NHA_OK
        refs.append((o, lse, state))
    torch.cuda.synchronize()
    # the two allocation-free calls, back to back
    for (desc, (q, k, v, a), (o, lse, state), _), (wl, w) in zip(runs, cases):
        log("case noalloc B=%d T=%d H=%d/%d d=%d m=%d w=%d" % (wl.B, wl.T, wl.H, wl.Hkv, wl.d, wl.m, w))
        rc = lib.nha_fwd_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(o), _ptr(lse),
                                 _ptr(state), stream)
        assert rc == nha.NHA_OK
    torch.cuda.synchronize()
    for (_, _, (o, lse, state), n), (ro, rl, rs) in zip(runs, refs):
        assert torch.isfinite(ro.float()).all()
        assert torch.equal(o, ro) and torch.equal(lse, rl)
        assert torch.equal(state[:n], rs[:n])


def test_noalloc_refuses_shapes_beyond_the_scratch():
    wl = WORKLOADS["headline"]
    desc = nha.make_desc(wl.B, wl.T, wl.H, wl.Hkv, wl.d, wl.m, wl.w, wl.C, wl.rope_base, 0.0, wl.dtype)
    assert nha.workspace_size(desc) > SCRATCH_BYTES
    A = ctypes.c_void_p(4096)  # never dereferenced: refused on the host
    rc = nha.load().nha_fwd_noalloc(ctypes.byref(desc), A, A, A, A, A, None, None, None)
    assert rc == nha.NHA_ERR_WORKSPACE
