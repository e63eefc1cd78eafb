"""Host-side checks of bench.py's accounting (no GPU): the algorithmic work
its roofline divides by, counted here independently by enumeration, and the
refusal of more than one GPU.

Window pairs: each query t attends to the keys t - w + 1 .. t that exist, the
band of the sliding window (Paper-Notes page, 关键设计 > 层内混合); slot rows:
row u of a chunk absorbs token u - w when u >= w, and a query reads the rows
of its own chunk up to itself (the chunkwise form of 关键设计 > Chunkwise
并行计算)."""
import os
import subprocess
import sys

import pytest
import torch

import bench
from softmax_attention_nha_amd.inputs import WORKLOADS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def pairs_by_enumeration(T, w):
    # every (query, key) with t - w < j <= t and j >= 0
    return sum(1 for t in range(T) for j in range(max(0, t - w + 1), t + 1))


@pytest.mark.parametrize("T,w", [(37, 5), (37, 0), (20, 20), (20, 64), (64, 1), (100, 33)])
def test_window_flops_count_every_pair_once(T, w):
    B, H, d = 2, 3, 8
    assert bench.flops_window(B, H, T, d, w) == 4.0 * d * B * H * pairs_by_enumeration(T, w)


@pytest.mark.parametrize("T,w,C", [(150, 40, 64), (97, 31, 16), (64, 64, 32), (130, 0, 32), (70, 3, 64)])
def test_slot_flops_count_absorbed_rows_of_the_chunk(T, w, C):
    B, H, d, m = 1, 2, 16, 5
    tot = 0
    for t in range(w, T):
        c0 = C * (t // C)
        rows = [u for u in range(c0, t + 1) if u >= w]  # absorbing rows of t's chunk up to t
        tot += 4 * m * d + (4 * d + 4 * m) * len(rows)
    assert bench.flops_slot(B, H, T, d, m, w, C) == B * H * tot
    assert bench.flops_slot(B, H, T, d, 0, w, C) == 0.0


def test_headline_dkdv_kernel_work_and_bound():
    """The window dk/dv kernel at B=4 H=16 T=8192 d=128 w=512 bf16: 8d flops
    per pair; its own bytes per (batch, token) are q, dO (read), k, v (read),
    dk, dv (written) and lse, D_t: 2 H d 2 + 4 Hkv d 2 + 2 H 4 = 24704."""
    wl = WORKLOADS["headline"]
    e = 2
    flops, nbytes, impl = bench.stage_work("win_bwd_dkdv", wl, wl.w, e)
    pairs = pairs_by_enumeration(wl.T, wl.w)
    assert pairs == 4063488
    assert flops == 8.0 * wl.d * wl.B * wl.H * pairs
    assert nbytes == 24704.0 * wl.B * wl.T
    # 329 flop/B, above the 2500 TFLOP/s / 8 TB/s ridge (312.5 flop/B)
    assert flops / nbytes > 2500.0 / 8.0 > 300.0
    r = bench.roofline("win_bwd_dkdv", 437.0, wl, wl.w, e)
    assert r["bound"] == "mfma" and r["unit"] == "TFLOP/s" and r["peak"] == 2500.0
    assert r["frac"] == pytest.approx(flops / 437e-6 / 1e12 / 2500.0, rel=1e-3)


def test_headline_slot_pass_b_is_hbm_bound():
    wl = WORKLOADS["headline"]
    flops, nbytes, _ = bench.stage_work("slot_bwd_b", wl, wl.w, 2)
    assert 0 < flops / nbytes < 2500.0 / 8.0
    r = bench.roofline("slot_bwd_b", 440.0, wl, wl.w, 2)
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert r["frac"] == pytest.approx(nbytes / 440e-6 / 1e9 / 8000.0, rel=1e-3)


def test_forward_flops_are_the_three_parts():
    wl = WORKLOADS["headline"]
    f = bench.flops_fwd(wl, wl.w)
    assert f == (bench.flops_window(wl.B, wl.H, wl.T, wl.d, wl.w)
                 + bench.flops_slot(wl.B, wl.H, wl.T, wl.d, wl.m, wl.w, wl.C)
                 + 4.0 * wl.m * wl.d * wl.B * wl.Hkv * (wl.T - wl.w))


def test_every_stage_the_library_names_has_its_work_defined():
    import softmax_attention_nha_amd as nha
    wl = WORKLOADS["headline"]
    desc = nha.make_desc(wl.B, wl.T, wl.H, wl.Hkv, wl.d, wl.m, wl.w, wl.C, wl.rope_base, 0.0, wl.dtype)
    for backward in (0, 1):
        for name in nha.stage_names(desc, backward=backward):
            flops, nbytes, impl = bench.stage_work(name, wl, wl.w, 2)
            assert flops is not None, name


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""
