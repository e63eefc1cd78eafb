"""GPU check that the production calls can be captured into a HIP graph: the
forward followed by the backward that re-uses its workspace, captured once
(with the library's side stream joining the capture through its events) and
replayed three times -- each replay after the outputs were cleared, with an
eager step and a synchronisation between replays -- equals the eager results
bitwise every time."""
import pytest
import torch

import softmax_attention_nha_amd as nha
from parity_util import log
from softmax_attention_nha_amd.inputs import WORKLOADS, make_inputs

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("B", [1, 4])
def test_fwd_bwd_graph_replays_equal_eager(B):
    # the 1.3B head shape over B sequences of 2048 tokens, w = 512 (B = 1:
    # the window kernel beside the scan on the side stream; B = 4: the
    # one-kernel forward)
    wl = WORKLOADS["1p3b"].with_(B=B)
    w = 512
    dev = torch.device("cuda:0")
    q, k, v, a, dO = (x.to(dev) for x in make_inputs(wl, with_grad=True))
    desc = nha.make_desc(wl.B, wl.T, wl.H, wl.Hkv, wl.d, wl.m, w, wl.C, wl.rope_base, 0.0, wl.dtype)
    ws = torch.empty(max(nha.workspace_size(desc), nha.workspace_size(desc, backward=True)), dtype=torch.uint8,
                     device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((wl.B, wl.H, wl.T), dtype=torch.float32, device=dev)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
             torch.empty((wl.B, wl.T, wl.Hkv, wl.m), dtype=torch.float32, device=dev))
    outs = (o, lse) + grads

    def step():
        nha.fwd(q, k, v, a, w, C=wl.C, rope_base=wl.rope_base, workspace=ws, out=o, lse_out=lse)
        nha.bwd(q, k, v, a, o, lse, dO, w, C=wl.C, rope_base=wl.rope_base, workspace=ws, out=grads,
                after_fwd=True)

    step()
    torch.cuda.synchronize()
    ref = [x.clone() for x in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    names = ("o", "lse", "dq", "dk", "dv", "dalpha")
    for rep in range(3):
        for x in outs:
            x.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, x, r in zip(names, outs, ref):
            assert torch.equal(x, r), "replay %d: %s differs from the eager result" % (rep, name)
        log("  replay %d: all six outputs bitwise equal to eager" % rep)
        step()  # eager work between replays
        torch.cuda.synchronize()
        for name, x, r in zip(names, outs, ref):
            assert torch.equal(x, r), "eager step after replay %d: %s differs" % (rep, name)
