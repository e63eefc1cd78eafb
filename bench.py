#!/usr/bin/env python
"""Benchmark of the NHA layer operator (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload headline]

A step is one pass of the whole training hot path over one batch of synthetic
input already resident in HBM: nha_fwd (RoPE, gate prep, slot-state scan, slot
branch, window branch) followed by its backward, nha_bwd_after_fwd with the
forward's workspace (the backward reads the forward's RoPE'd q/k, gate
products and chunk-start states instead of recomputing them, as a training
step keeps forward intermediates).  K steps are timed with HIP events between
two device synchronisations; each kernel launch is also bracketed by HIP
events recorded by the library on the same stream (nha_fwd_timed /
nha_bwd_after_fwd_timed), which gives the live per-kernel durations used for
the roofline of the dominant kernel.  Prints ONE JSON line.

Workload (default): the 1.3B-scale layer shape at 8K tokens -- B=4, H=Hkv=16,
T=8192, d=128, m=64 slots, w=512, C=64, bf16 inputs with fp32 accumulation,
RoPE base 10000 -- q,k,v ~ N(0,1)/sqrt(d), alpha = sigmoid(N(4,1)), dO ~ N(0,1).

cpu_baseline: the fp64 oracle (test infrastructure, never tuned) timed on the
host cores over a bounded sample of the same workload, reported as tokens/s.
"""
import argparse
import json
import math
import os
import sys
import time

import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import softmax_attention_nha_amd as nha  # noqa: E402
from softmax_attention_nha_amd.inputs import WORKLOADS, make_inputs  # noqa: E402

METRIC = "NHA layer fwd+bwd tokens/s and TFLOP/s (% bf16 MFMA peak), 1 GPU, T=2K-8K"
PEAK_TFLOPS = {torch.bfloat16: 2500.0, torch.float32: 157.3}  # dense MFMA, MI355X
PEAK_HBM_GBS = 8000.0


# ---------------------------------------------------------------- algorithmic work
def n_win(t, w):
    return min(w, t + 1)


def flops_window(B, H, T, d, w):
    """QK^T + PV over the band: 4 d flops per (query, window key) pair."""
    if w <= 0:
        return 0.0
    full = max(0, T - w)
    ramp = min(T, w)
    pairs = ramp * (ramp + 1) / 2 + full * w
    return 4.0 * d * B * H * pairs


def flops_slot(B, H, T, d, m, w, C):
    """Slot read (4 m d per query) plus the intra-chunk terms (4d + 4m per
    (query, earlier absorbed row of the same chunk)); none without slots."""
    if m == 0:
        return 0.0
    tot = 0.0
    for t in range(w, T):
        c = t - max(C * (t // C), w) + 1
        tot += 4.0 * m * d + (4.0 * d + 4.0 * m) * c
    return B * H * tot


def flops_state(B, Hkv, T, d, m, w):
    """Slot-state build: 4 m d per absorbed token (K and V)."""
    return 4.0 * m * d * B * Hkv * max(0, T - w)


def flops_fwd(wl, w, sh=None):
    """sh: the slots' absorption shift (None: w; 0 without token shift)."""
    sh = w if sh is None else sh
    return (flops_window(wl.B, wl.H, wl.T, wl.d, w) + flops_slot(wl.B, wl.H, wl.T, wl.d, wl.m, sh, wl.C)
            + flops_state(wl.B, wl.Hkv, wl.T, wl.d, wl.m, sh))


def bytes_fwd(wl, e):
    """Minimum HBM traffic of the forward: read q,k,v,alpha; write o, lse."""
    return wl.B * (wl.H * wl.T * (2 * wl.d * e + 4) + wl.Hkv * wl.T * (2 * wl.d * e + wl.m * e))


def stage_work(stage, wl, w, e):
    """(flops, algorithmic bytes, implementation bytes) of one launch of `stage`.

    Flops: the algorithmic flops of the part of the method the kernel
    computes -- window kernels 4d per (query, in-window key) pair in the
    forward, 6d (dq pass: QK^T, dO V^T, dS K) and 8d (dk/dv pass: QK^T, dO V^T,
    P^T dO, dS^T Q) in the backward; slot kernels, per query t >= w with c(t)
    earlier absorbed rows of its chunk, one read (2md + (2d+2m)c) and one mix
    (same) in the forward, two reads and one mix in pass A, two reverse reads
    and two reverse mixes in pass B; the state scan 4md per absorbed token per
    KV head; the adjoint's sources 4md per token per query head (bf16: in
    pass A, which hands the scan per-chunk sums; the scan then takes 4 flops
    per slot-state element per chunk and query head: decay, add, both sides;
    fp32: in the scan).

    Algorithmic bytes: the operator's own tensors the kernel reads or writes,
    each once -- q, k, v, alpha, dO (inputs), o, dq, dk, dv, dalpha (outputs),
    and the per-row softmax statistics lse and D_t = <dO_t, o_t> (4 bytes per
    (row, head)).  RoPE'd q/k stand in for q/k.  Implementation bytes: the
    workspace intermediates the kernel moves between launches (gate products,
    chunk-start states, slot partials, adjoints, slot parts of the gradients),
    reported apart and not counted in the roofline.  e = element bytes, mp = m
    padded to 32 or 64, NC chunks of C rows."""
    B, H, Hkv, T, d, m, C = wl.B, wl.H, wl.Hkv, wl.T, wl.d, wl.m, wl.C
    G, NC = H // Hkv, -(-T // C)
    mp = 32 if m <= 32 else 64
    units = B * Hkv
    fw = flops_window(B, H, T, d, w)
    fs = flops_slot(B, H, T, d, m, w, C)
    absorbed = max(0, T - w)
    BT = float(B * T)
    q_b, kv_b, a_b = BT * H * d * e, BT * Hkv * d * e, BT * Hkv * m * e  # one of q (or o, dO, dq); k; alpha
    row = BT * H * 4.0  # lse or D
    # the slot passes' per-(row, slot) exchange: s dl and p (fp16 for bf16
    # inputs, fp32 otherwise) and A (fp32); the fp32 rows of blocks on the
    # exact same-block path (strong decays) are not counted
    xw = 8.0 if e == 2 else 12.0
    # segments of the state scan (the library's rule: bf16, fewer than 256
    # scan waves, at least 384 chunks; up to 768 waves of at least 8 chunks)
    nseg, base = 1, B * Hkv * (d // 16)
    if e == 2 and m > 0 and base < 256 and NC >= 384:
        nseg = min(768 // base, 16, NC // 8)
        if nseg >= 2:
            L = -(-NC // nseg)
            nseg = -(-NC // L)
        else:
            nseg = 1
    table = {
        "rope_cs": (0.0, 0.0, 8.0 * T * (d // 2)),
        "rope": (0.0, q_b + kv_b, q_b + kv_b),
        "chunk_gates": (0.0, a_b, units * NC * mp * (C * e + 4.0)),
        "state_scan": (flops_state(B, Hkv, T, d, m, w), 2.0 * B * Hkv * absorbed * d * e,
                       units * NC * (mp * C * e + 4.0 * mp + 2.0 * mp * d * e)),
        # the window branch runs first (into the workspace); the slot kernel
        # merges it and writes o and lse
        "slot_fwd": (fs, 2 * q_b + 2 * kv_b + a_b + row, B * H * NC * 2.0 * mp * d * e + (q_b + row if w else 0)),
        "win_fwd": (fw, q_b + 2 * kv_b, q_b + row),
        # both branches in one kernel (bf16, C = 64): q, RoPE'd q / k, v, the
        # absorbed k / v rows, alpha read, o and lse written; the chunk-start
        # states read
        "chunk_fwd": (fw + fs, 2 * q_b + 2 * kv_b + a_b + row, B * H * NC * 2.0 * mp * d * e + q_b + kv_b),
        "bwd_prep": (0.0, 2 * q_b + row, 0.0),
        "slot_bwd_a": (1.5 * fs + (4.0 * m * d * B * H * T if e == 2 else 0.0), 3 * q_b + 2 * kv_b + a_b + 2 * row,
                       B * H * NC * (2.0 * mp * d * e + 2.0 * mp * (d if e == 2 else C) * e + xw * C * mp) + q_b),
        "adj_scan": ((4.0 * m * d * units * NC * G, 0.0, units * NC * (G * 2.0 * mp * d * e + 4.0 * mp + 2.0 * mp * d * e))
                     if e == 2 else
                     (4.0 * m * d * B * H * T, 2 * q_b, units * NC * (G * 2.0 * mp * C * e + 4.0 * mp + 2.0 * mp * d * e))),
        "slot_bwd_b": (2.0 * fs, 2 * kv_b + a_b + BT * Hkv * m * 4.0 + 2 * q_b,
                       units * NC * (2.0 * mp * d * e + 4.0 * mp + G * xw * C * mp) + 2 * kv_b),
        "dalpha_tail": (0.0, a_b + 2 * BT * Hkv * m * 4.0, units * NC * mp * 4.0),
        "win_bwd_dq": (1.5 * fw, 3 * q_b + 2 * kv_b + 2 * row, q_b),
        "win_bwd_dkdv": (2.0 * fw, 2 * q_b + 4 * kv_b + 2 * row, 2 * kv_b),
        "export_state": (0.0, 4.0 * B * Hkv * min(w, T) * d * e, 0.0),
        # the segmented scan (long walks at few waves): segment end states
        # and decays, their start states, then the walk ("state_scan")
        "state_scan_seg": (flops_state(B, Hkv, T, d, m, w), 2.0 * B * Hkv * absorbed * d * e,
                           units * NC * (mp * C * e + 4.0 * mp) + nseg * units * (2.0 * m * d * 4 + 4.0 * mp)),
        "scan_combine": (0.0, 0.0, nseg * units * (4.0 * m * d * 4 + 4.0 * mp)),
        # dalpha's exact carries at every 16th chunk: adjoint and state rows
        "carry_ckpt": (0.0, 0.0, units * ((NC - 1) // 16) * (2 * 2.0 * mp * d * e + 4.0 * mp)),
    }
    return table.get(stage, (None, None, None))


def roofline(stage, us, wl, w, e):
    """Roofline of one kernel against its algorithmic work: intensity I =
    flops / algorithmic bytes; bound "mfma" when I is at or above the ridge
    P / BW, else "hbm"; frac = achieved / peak of that bound.  Both fractions
    and the implementation traffic are reported beside it."""
    flops, nbytes, impl = stage_work(stage, wl, w, e)
    if flops is None:
        return None
    dur = us / 1e6
    peak = PEAK_TFLOPS[wl.dtype]
    tf = flops / dur / 1e12
    gbs = nbytes / dur / 1e9
    # (no algorithmic bytes -- a kernel on workspace intermediates only: the
    # intensity is unbounded)
    mfma_bound = flops > 0 and (nbytes == 0 or flops / nbytes >= peak * 1e12 / (PEAK_HBM_GBS * 1e9))
    r = {"kernel": stage}
    if mfma_bound:
        r.update(bound="mfma", achieved=round(tf, 2), peak=peak, unit="TFLOP/s", frac=round(tf / peak, 4))
    else:
        r.update(bound="hbm", achieved=round(gbs, 1), peak=PEAK_HBM_GBS, unit="GB/s",
                 frac=round(gbs / PEAK_HBM_GBS, 4))
    tr = measured_traffic(stage)
    r.update(traffic=tr.get("fetch_write") if tr else None,
             traffic_dram_requests=tr.get("dram_requests") if tr else None,
             avg_us=round(us, 2), flops_per_launch=flops, algorithmic_bytes_per_launch=nbytes,
             implementation_bytes_per_launch=impl,
             intensity_flop_per_byte=round(flops / nbytes, 1) if nbytes else None,
             mfma_tflops=round(tf, 2), mfma_frac=round(tf / peak, 4),
             hbm_GBs=round(gbs, 1), hbm_frac=round(gbs / PEAK_HBM_GBS, 4))
    return r


# ---------------------------------------------------------------- CPU baseline
def cpu_baseline(wl, w, q, k, v, a, dO, with_bwd):
    import oracle  # test infrastructure: only this leg of the benchmark uses it

    cores = int(os.environ.get("OMP_NUM_THREADS", "0")) or os.cpu_count() or 1
    cores = min(cores, os.cpu_count() or cores)
    Tp = int(os.environ.get("NHA_CPU_SAMPLE_T", "8192"))
    Tp = min(Tp, wl.T)
    units = wl.Hkv  # one batch row, every KV head
    threads = min(cores, units)
    f64 = lambda x: x[:1, :Tp].float().double().numpy()
    qs, ks, vs, as_, ds = f64(q), f64(k), f64(v), f64(a), f64(dO)
    t0 = time.perf_counter()
    oracle.fwd(qs, ks, vs, as_, w, rope_base=wl.rope_base, threads=threads)
    if with_bwd:
        oracle.bwd(qs, ks, vs, as_, ds, w, rope_base=wl.rope_base, threads=threads)
    dt = time.perf_counter() - t0
    return {
        "value": round(Tp / dt, 2),
        "unit": "tokens/s",
        "cores": threads,
        "kind": "oracle",
        "sample": "batch row 0, all %d heads, first %d of %d tokens, %s in fp64 (%.1f s)" % (
            wl.H, Tp, wl.T, "fwd+bwd" if with_bwd else "fwd", dt),
        "threads_note": "cores = OpenMP threads the oracle ran with: min(host CPUs, %d KV heads of the batch row)" % (
            units),
        "host_cpu_model": _cpu_model(),
        "host_logical_cpus": os.cpu_count(),
        "host_cpus_available": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
    }


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


# ---------------------------------------------------------------- context figures
def copy_bandwidth(mib=1024, reps=5):
    """Attainable HBM bandwidth: a plain device copy of `mib` MiB (read + write
    bytes over the median event time)."""
    n = mib * (1 << 20)
    src = torch.ones(n // 4, device="cuda:0")
    dst = torch.empty_like(src)
    dst.copy_(src)
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b) / 1e3)
    t = sorted(ts)[reps // 2]
    del src, dst
    return {"bytes": 2 * n, "GBs": round(2 * n / t / 1e9, 1), "note": "torch device copy of %d MiB, median of %d" % (
        mib, reps)}


def device_clock_under_load(run_step, seconds=1.5):
    """The engine clock while the step runs: enqueue about `seconds` of steps,
    then read rocm-smi's current clock levels while they execute."""
    import subprocess

    t0 = time.perf_counter()
    run_step()
    torch.cuda.synchronize()
    per = max(time.perf_counter() - t0, 1e-4)
    for _ in range(max(1, int(seconds / per))):
        run_step()
    out = None
    try:
        r = subprocess.run(["rocm-smi", "--showclocks"], capture_output=True, text=True, timeout=20)
        lines = [x.strip() for x in r.stdout.splitlines() if "sclk" in x.lower() or "mclk" in x.lower()]
        out = {"rocm_smi": lines[:4], "note": "rocm-smi --showclocks while about %.1f s of steps ran" % seconds}
    except (OSError, subprocess.SubprocessError) as ex:
        out = {"rocm_smi": None, "note": "rocm-smi unavailable: %s" % type(ex).__name__}
    torch.cuda.synchronize()
    props = torch.cuda.get_device_properties(0)
    rate = getattr(props, "clock_rate", None)
    if rate:
        out["max_engine_clock_MHz"] = round(rate / 1e3)
    return out


def b1_timings(steps, flush_mib=512):
    """The headline shape at B = 1 (151 MB of algorithmic forward traffic fits
    the 256 MB Infinity Cache): median fwd / bwd times with warm caches, and
    with a flush_mib buffer written before every call."""
    wl = WORKLOADS["headline"].with_(B=1)
    dev = torch.device("cuda:0")
    q, k, v, a, dO = (x.to(dev) for x in make_inputs(wl, with_grad=True))
    desc = nha.make_desc(wl.B, wl.T, wl.H, wl.Hkv, wl.d, wl.m, wl.w, wl.C, wl.rope_base, 0.0, wl.dtype)
    ws = torch.empty(max(nha.workspace_size(desc), nha.workspace_size(desc, backward=True)), dtype=torch.uint8,
                     device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((wl.B, wl.H, wl.T), dtype=torch.float32, device=dev)
    grads = (torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
             torch.empty((wl.B, wl.T, wl.Hkv, wl.m), dtype=torch.float32, device=dev))
    junk = torch.empty(flush_mib * (1 << 20) // 4, dtype=torch.float32, device=dev)
    res = {}
    for flush in (False, True):
        tf, tb = [], []
        for i in range(steps + 2):
            if flush:
                junk.fill_(float(i))
            e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
            e0.record()
            nha.fwd(q, k, v, a, wl.w, C=wl.C, rope_base=wl.rope_base, workspace=ws, out=o, lse_out=lse)
            e1.record()
            if flush:
                junk.fill_(float(-i))
                e1b = torch.cuda.Event(enable_timing=True)
                e1b.record()
            else:
                e1b = e1
            nha.bwd(q, k, v, a, o, lse, dO, wl.w, C=wl.C, rope_base=wl.rope_base, workspace=ws, out=grads,
                    after_fwd=True)
            e2.record()
            e2.synchronize()
            if i >= 2:
                tf.append(e0.elapsed_time(e1))
                tb.append(e1b.elapsed_time(e2))
        res["flushed" if flush else "warm"] = {"fwd_ms": round(sorted(tf)[len(tf) // 2], 4),
                                               "bwd_ms": round(sorted(tb)[len(tb) // 2], 4)}
    res["workload"] = "B=1 H=16 T=8192 d=128 m=64 w=512 C=64 bf16"
    res["flush"] = "a %d MiB buffer written before each fwd and each bwd (flushed)" % flush_mib
    del junk, ws
    return res


# ---------------------------------------------------------------- HBM traffic from counters
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
STAGE_KERNEL = {  # stage name -> kernel symbol fragment in the profiler's output
    "slot_bwd_b": "k_bwd_slot_b", "slot_bwd_a": "k_bwd_slot_a", "slot_fwd": "k_slot_fwd", "win_fwd": "k_win_fwd",
    "win_bwd_dq": "k_win_bwd_dq", "win_bwd_dkdv": "k_win_bwd_dkdv", "adj_scan": "k_adj_scan",
    "state_scan": "k_state_scan", "chunk_fwd": "k_chunk_fwd",
}


# translation unit of each kernel that counters are taken for
KERNEL_SOURCE = {"k_bwd_slot_b": "nha_bwd.hip", "k_bwd_slot_a": "nha_bwd.hip", "k_adj_scan": "nha_bwd.hip",
                 "k_chunk_fwd": "nha_fwd.hip",
                 "k_win_bwd_dq": "nha_bwd.hip", "k_win_bwd_dkdv": "nha_bwd.hip", "k_slot_fwd": "nha_fwd.hip",
                 "k_win_fwd": "nha_fwd.hip", "k_state_scan": "nha_fwd.hip"}


def source_digest(kernel):
    """sha256 over the kernel's translation unit and the shared headers:
    counters taken on other sources are stale."""
    import hashlib

    h = hashlib.sha256()
    src = os.path.join(ROOT, "softmax_attention_nha_amd", "csrc")
    for f in sorted(os.listdir(src)):
        if f.endswith(".h") or f == KERNEL_SOURCE.get(kernel, "nha_bwd.hip"):
            with open(os.path.join(src, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()


def copy_calibrate(mib):
    """Three plain copies of `mib` MiB: the per-dispatch FETCH_SIZE / WRITE_SIZE
    of this kernel against its known byte count gives the counters' scale."""
    n = mib * (1 << 20)
    src = torch.ones(n // 4, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 3}), flush=True)


def _pmc_per_dispatch(folder, counter, name_part):
    """Mean value of `counter` per dispatch of the kernels whose name contains
    name_part, from a rocprofv3 --pmc --output-format csv folder."""
    import csv
    import glob

    vals = {}
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if name_part in r["Kernel_Name"] and r["Counter_Name"] == counter:
                    key = (f, r["Dispatch_Id"])
                    vals[key] = vals.get(key, 0.0) + float(r["Counter_Value"])
    if not vals:
        raise SystemExit("no %s values for %s under %s" % (counter, name_part, folder))
    return sum(vals.values()) / len(vals), len(vals)


def traffic_summary(dirs, kernels, copy_mib, dram_dirs=None):
    """profiles/traffic.json: per-launch HBM bytes of each kernel in `kernels`
    (comma-separated), two ways:
      fetch_write    its FETCH_SIZE / WRITE_SIZE (KiB per dispatch) scaled by
                     what the same counters read for a plain copy of copy_mib
                     MiB (dirs: kernel FETCH, kernel WRITE, copy FETCH, copy
                     WRITE runs);
      dram_requests  32 B x (TCC_EA0_RDREQ_DRAM_32B + TCC_EA0_WRREQ_WRITE_DRAM_32B)
                     -- the L2's requests to memory counted in 32-byte units
                     (64- and 128-byte requests count 2 and 4) -- from one run
                     with both counters (dram_dirs: kernel run, copy run); the
                     copy's reading is reported beside it as the check."""
    cf, _ = _pmc_per_dispatch(dirs[2], "FETCH_SIZE", "copy")
    cw, _ = _pmc_per_dispatch(dirs[3], "WRITE_SIZE", "copy")
    n = copy_mib * (1 << 20)
    ff, fw = cf * 1024.0 / n, cw * 1024.0 / n  # counter bytes per true byte, from the copy
    out = {
        "copy_mib": copy_mib,
        "copy_fetch_kib": round(cf, 1),
        "copy_write_kib": round(cw, 1),
        "fetch_scale": round(ff, 4),
        "write_scale": round(fw, 4),
        "kernels": {},
    }
    if dram_dirs:
        crd, _ = _pmc_per_dispatch(dram_dirs[1], "TCC_EA0_RDREQ_DRAM_32B", "copy")
        cwr, _ = _pmc_per_dispatch(dram_dirs[1], "TCC_EA0_WRREQ_WRITE_DRAM_32B", "copy")
        out["copy_dram_read_bytes"] = round(32.0 * crd)
        out["copy_dram_write_bytes"] = round(32.0 * cwr)
    for kernel in kernels.split(","):
        fetch, nf = _pmc_per_dispatch(dirs[0], "FETCH_SIZE", kernel)
        write, nw = _pmc_per_dispatch(dirs[1], "WRITE_SIZE", kernel)
        ent = {
            "fetch_kib_per_dispatch": round(fetch, 1),
            "write_kib_per_dispatch": round(write, 1),
            "dispatches": [nf, nw],
            "hbm_bytes_per_launch": round(fetch * 1024.0 / ff + write * 1024.0 / fw),
            "source_sha256": source_digest(kernel),
        }
        if dram_dirs:
            rd, nr = _pmc_per_dispatch(dram_dirs[0], "TCC_EA0_RDREQ_DRAM_32B", kernel)
            wr, _ = _pmc_per_dispatch(dram_dirs[0], "TCC_EA0_WRREQ_WRITE_DRAM_32B", kernel)
            ent["dram_read_bytes"] = round(32.0 * rd)
            ent["dram_write_bytes"] = round(32.0 * wr)
            ent["dram_request_bytes_per_launch"] = round(32.0 * (rd + wr))
        out["kernels"][kernel] = ent
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def _kernel_short(name):
    """Short kernel name from a demangled (nha::k_x<...>(...)) or mangled
    (_ZN3nha<len>k_x...) profiler name; None for other kernels."""
    if "nha::" in name:
        return name.split("nha::")[1].split("<")[0].split("(")[0]
    if name.startswith("_ZN3nha"):
        rest = name[len("_ZN3nha"):]
        digits = ""
        while rest and rest[0].isdigit():
            digits, rest = digits + rest[0], rest[1:]
        return rest[: int(digits)] if digits else None
    return None


def counter_summary(folders):
    """Markdown table of per-kernel SQ counters (mean per dispatch) from a
    rocprofv3 --pmc csv folder, with the executed bf16 MFMA work
    (SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 flop) and, given a --kernel-trace
    --stats folder as well, its rate against the kernel's average duration;
    LDS bank-conflict share = SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE; LDS
    wait share = SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES."""
    import csv
    import glob

    folder = folders[0]
    vals = {}
    for f in glob.glob(os.path.join(folder, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            for r in csv.DictReader(fh):
                k = _kernel_short(r["Kernel_Name"])
                if not k:
                    continue
                d = vals.setdefault(k, {}).setdefault((f, r["Dispatch_Id"]), {})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    dur = {}
    if len(folders) > 1:
        for f in glob.glob(os.path.join(folders[1], "**", "*kernel_stats.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    k = _kernel_short(r["Name"])
                    if k:
                        dur[k] = float(r["AverageNs"]) / 1e3
    print("| kernel | dispatches | executed bf16 MFMA GFLOP | avg us (trace) | MFMA TFLOP/s (% of 2500) "
          "| LDS bank-conflict / LDS active | LDS wait / wave cycles |")
    print("|---|---|---|---|---|---|---|")
    for k, disp in sorted(vals.items()):
        n = len(disp)
        mean = lambda c: sum(x.get(c, 0.0) for x in disp.values()) / n
        gf = mean("SQ_INSTS_VALU_MFMA_MOPS_BF16") * 512 / 1e9
        lds_act = mean("SQ_LDS_IDX_ACTIVE")
        bc = mean("SQ_LDS_BANK_CONFLICT") / lds_act if lds_act else 0.0
        wc = mean("SQ_WAVE_CYCLES")
        lw = mean("SQ_WAIT_INST_LDS") / wc if wc else 0.0
        us = dur.get(k)
        rate = ("%.0f (%.1f %%)" % (gf / us * 1e3, gf / us * 1e3 / 25)) if us and gf else "—"
        print("| %s | %d | %.2f | %s | %s | %.3f | %.3f |" % (k, n, gf, "%.1f" % us if us else "—", rate, bc, lw))


def trace_summary(folder):
    """Markdown table (calls, average and total duration per kernel) of a
    rocprofv3 --kernel-trace --stats --output-format csv folder."""
    import csv
    import glob
    import re

    rows = []
    for f in glob.glob(os.path.join(folder, "**", "*kernel_stats.csv"), recursive=True):
        with open(f) as fh:
            rows += list(csv.DictReader(fh))
    tot = sum(float(r["TotalDurationNs"]) for r in rows) or 1.0
    print("| kernel | calls | avg us | % of GPU time |")
    print("|---|---|---|---|")
    for r in sorted(rows, key=lambda r: -float(r["TotalDurationNs"])):
        m = re.search(r"(k_[a-z0-9_]+)", r["Name"])
        name = m.group(1) if m else r["Name"][:40]
        print("| %s | %s | %.1f | %.1f |" % (name, r["Calls"], float(r["AverageNs"]) / 1e3,
                                           100.0 * float(r["TotalDurationNs"]) / tot))


def measured_traffic(stage):
    """HBM bytes per launch of `stage` from profiles/traffic.json --
    {"fetch_write": .., "dram_requests": ..} -- or None when absent, for
    another kernel, or taken on other kernel sources."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    kernel = STAGE_KERNEL.get(stage)
    e = t.get("kernels", {}).get(kernel)
    if e is None or e.get("source_sha256") != source_digest(kernel):
        return None
    return {"fetch_write": e.get("hbm_bytes_per_launch"), "dram_requests": e.get("dram_request_bytes_per_launch")}


# ---------------------------------------------------------------- sweeps
# (label, workload, overrides, window, with backward, decode tokens after the forward)
SWEEP = [
    ("w_sweep", "1p3b", {}, 0, True, 0),
    ("w_sweep", "1p3b", {}, 64, True, 0),
    ("w_sweep", "1p3b", {}, 512, True, 0),
    ("w_sweep", "1p3b", {}, 2048, True, 0),  # w = T: causal attention plus the m slot keys
    ("T_sweep", "long", {"T": 8192}, 512, False, 256),
    ("T_sweep", "long", {"T": 16384}, 512, False, 256),
    ("T_sweep", "long", {"T": 32768}, 512, False, 256),
    ("config", "340m", {}, 64, True, 0),
    ("config", "gqa", {}, 2048, True, 0),
    ("config", "headline", {}, 512, True, 0),
    # many sequences decoding together (B = 32 at 2K tokens of prefix each)
    ("decode_batched", "long", {"B": 32, "T": 2048}, 512, False, 64),
    # ablation: no slots (m = 0, sliding-window attention alone) at the headline shape
    ("ablation_no_slots", "headline", {"m": 0}, 512, True, 0),
    # ablation: no token shift (every token enters the slots at its own step)
    ("ablation_no_token_shift", "headline", {}, 512, True, 0),
    # ablation: weighted fusion (separate slot and window softmaxes mixed by a
    # per-token coefficient, with its gradient)
    ("ablation_weighted_fusion", "headline", {}, 512, True, 0),
]
# The operator benchmark shape the pages describe (NHA with m = 32 slots and
# w = 32 against a 64-slot gated-slot model and full attention, over the
# sequence length); the pages print no B, H, d or T list, so these are one
# sequence of 16 heads of dimension 128 at T = 2K .. 32K.  NHA w = 0, m = 64
# is the gated-slot point; w = T the full causal attention curve (plus m null
# slots).
for _T in (2048, 4096, 8192, 16384, 32768):
    SWEEP.append(("operator_nha_m32_w32", "long", {"T": _T, "m": 32}, 32, True, 0))
    SWEEP.append(("operator_slots_m64_w0", "long", {"T": _T, "m": 64}, 0, True, 0))
    SWEEP.append(("operator_full_attention_w_eq_T", "long", {"T": _T, "m": 32}, _T, True, 0))


def sweep_point(label, wl, w, with_bwd, ndec, steps, warmup):
    """Whole-call times (HIP events around each call) of one configuration."""
    dev = torch.device("cuda:0")
    e = 2 if wl.dtype == torch.bfloat16 else 4
    q, k, v, a, dO = make_inputs(wl, T_total=wl.T + ndec, with_grad=True)
    T = wl.T
    qd, kd, vd, ad, dOd = (x[:, :T].contiguous().to(dev) for x in (q, k, v, a, dO))
    shift = label != "ablation_no_token_shift"
    desc = nha.make_desc(wl.B, T, wl.H, wl.Hkv, wl.d, wl.m, w, wl.C, wl.rope_base, 0.0, wl.dtype, shift)
    ws = torch.empty(max(nha.workspace_size(desc), nha.workspace_size(desc, backward=with_bwd)), dtype=torch.uint8,
                     device=dev)
    o = torch.empty_like(qd)
    lse = torch.empty((wl.B, wl.H, T), dtype=torch.float32, device=dev)
    grads = (torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd),
             torch.empty((wl.B, T, wl.Hkv, wl.m), dtype=torch.float32, device=dev))
    state = nha.decode_state(wl.B, wl.H, wl.Hkv, wl.d, wl.m, w, wl.rope_base, 0.0, wl.dtype, dev) if ndec else None

    def fwd():
        nha.fwd(qd, kd, vd, ad, w, C=wl.C, rope_base=wl.rope_base, workspace=ws, out=o, lse_out=lse,
                state_out=state, token_shift=shift)

    def bwd():
        nha.bwd(qd, kd, vd, ad, o, lse, dOd, w, C=wl.C, rope_base=wl.rope_base, workspace=ws, out=grads,
                after_fwd=True, token_shift=shift)

    if label == "ablation_weighted_fusion":
        from softmax_attention_nha_amd.inputs import make_lam

        lam = make_lam(wl).to(dev)
        ws = torch.empty(nha.weighted_workspace_size(desc), dtype=torch.uint8, device=dev)
        lse2 = torch.empty((2, wl.B, wl.H, T), dtype=torch.float32, device=dev)
        wgrads = grads + (torch.empty((wl.B, T, wl.H), dtype=torch.float32, device=dev),)

        def fwd():  # noqa: F811 -- the ablation's own calls
            nha.fwd_weighted(qd, kd, vd, ad, lam, w, C=wl.C, rope_base=wl.rope_base, workspace=ws, out=o,
                             lse_out=lse2)

        def bwd():  # noqa: F811 -- recomputes both reads, then the gradients incl. dlam
            nha.bwd_weighted(qd, kd, vd, ad, lam, dOd, w, C=wl.C, rope_base=wl.rope_base, workspace=ws,
                             out=wgrads)

    ev = [torch.cuda.Event(enable_timing=True) for _ in range(3 * steps)]
    for _ in range(warmup):
        fwd()
        if with_bwd:
            bwd()
    torch.cuda.synchronize()
    for i in range(steps):
        ev[3 * i].record()
        fwd()
        ev[3 * i + 1].record()
        if with_bwd:
            bwd()
        ev[3 * i + 2].record()
    torch.cuda.synchronize()
    fwd_ms = sorted(ev[3 * i].elapsed_time(ev[3 * i + 1]) for i in range(steps))[steps // 2]
    bwd_ms = sorted(ev[3 * i + 1].elapsed_time(ev[3 * i + 2]) for i in range(steps))[steps // 2]
    F = flops_fwd(wl, w, None if shift else 0)
    peak = PEAK_TFLOPS[wl.dtype]
    line = {
        "sweep": label,
        "workload": "B=%d H=%d Hkv=%d T=%d d=%d m=%d w=%d C=%d %s" % (
            wl.B, wl.H, wl.Hkv, T, wl.d, wl.m, w, wl.C, "bf16" if e == 2 else "f32"),
        "fwd_ms": round(fwd_ms, 4),
        "fwd_tokens_per_s": round(wl.B * T / (fwd_ms / 1e3), 1),
        "fwd_gflop": round(F / 1e9, 2),
        "fwd_tflops": round(F / (fwd_ms / 1e3) / 1e12, 2),
        "fwd_mfma_frac": round(F / (fwd_ms / 1e3) / 1e12 / peak, 4),
        "fwd_hbm_frac": round(bytes_fwd(wl.with_(T=T), e) / (fwd_ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
        "full_causal_attention_gflop": round(4.0 * wl.d * wl.B * wl.H * T * (T + 1) / 2 / 1e9, 2),
    }
    if with_bwd:
        line.update(bwd_ms=round(bwd_ms, 4),
                    fwdbwd_tokens_per_s=round(wl.B * T / ((fwd_ms + bwd_ms) / 1e3), 1),
                    step_tflops=round(3.5 * F / ((fwd_ms + bwd_ms) / 1e3) / 1e12, 2),
                    step_mfma_frac=round(3.5 * F / ((fwd_ms + bwd_ms) / 1e3) / 1e12 / peak, 4))
    if ndec:
        # the state left by the forward, then ndec recurrent steps on the next tokens
        fwd()
        toks = [[x[:, T + i].contiguous().to(dev) for x in (q, k, v, a)] for i in range(ndec)]
        outs = torch.empty((wl.B, wl.H, wl.d), dtype=wl.dtype, device=dev)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(ndec):
            nha.decode_step(toks[i][0], toks[i][1], toks[i][2], toks[i][3], state, w, rope_base=wl.rope_base,
                            out=outs)
        e1.record()
        torch.cuda.synchronize()
        line["decode_us_per_step"] = round(e0.elapsed_time(e1) * 1e3 / ndec, 2)
        line["decode_note"] = ("one step = one token of each of the B sequences; eager: one Python call per step "
                               "(host-bound); graph: the same calls captured in a HIP graph")
        # the same ndec steps captured once in a HIP graph (the state keeps
        # advancing between replays; only the timing is of interest here)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(ndec):
                nha.decode_step(toks[i][0], toks[i][1], toks[i][2], toks[i][3], state, w, rope_base=wl.rope_base,
                                out=outs)
        g.replay()
        torch.cuda.synchronize()
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        line["decode_graph_us_per_step"] = round(e0.elapsed_time(e1) * 1e3 / ndec, 2)
        line["decode_graph_tokens_per_s"] = round(wl.B * ndec / (e0.elapsed_time(e1) / 1e3), 1)
    print(json.dumps(line), flush=True)


# ---------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="headline", choices=sorted(WORKLOADS))
    ap.add_argument("--w", type=int, default=None, help="override the window size")
    ap.add_argument("--T", type=int, default=None, help="override the sequence length")
    ap.add_argument("--B", type=int, default=None, help="override the batch")
    ap.add_argument("--fwd-only", action="store_true", help="diagnostic: time the forward alone")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-context", action="store_true",
                    help="skip the context figures (device clock, copy bandwidth, B = 1 warm / flushed timings)")
    ap.add_argument("--one-stream", action="store_true",
                    help="skip the production-call region: time only the one-stream pass with an event around "
                         "every launch (for kernel traces whose averages match the per-kernel events)")
    ap.add_argument("--copy-calibrate", type=int, default=0, metavar="MIB",
                    help="run 3 plain device copies of MIB MiB (a known-size kernel for the HBM counters) and exit")
    ap.add_argument("--traffic-summary", nargs=4, metavar=("FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR",
                                                           "COPY_WRITE_DIR"),
                    help="turn four rocprofv3 --pmc output folders into profiles/traffic.json and exit")
    ap.add_argument("--traffic-kernel", default="k_bwd_slot_b,k_win_bwd_dkdv",
                    help="kernel names (comma-separated) for --traffic-summary")
    ap.add_argument("--traffic-copy-mib", type=int, default=1024)
    ap.add_argument("--traffic-dram", nargs=2, metavar=("KERNEL_DIR", "COPY_DIR"),
                    help="with --traffic-summary: rocprofv3 --pmc folders of one run each with "
                         "TCC_EA0_RDREQ_DRAM_32B and TCC_EA0_WRREQ_WRITE_DRAM_32B (kernel run, copy run)")
    ap.add_argument("--sweep", action="store_true",
                    help="time the w sweep, the T sweep (with decode), the other configurations; one JSON line each")
    ap.add_argument("--only", metavar="LABEL", help="with --sweep: only the points of this sweep label")
    ap.add_argument("--counter-summary", nargs="+", metavar="DIR",
                    help="print a markdown table of per-kernel SQ counters from a rocprofv3 --pmc csv folder "
                         "(and, optionally, a --kernel-trace --stats folder for the durations) and exit")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="print a markdown table of a rocprofv3 --kernel-trace --stats csv folder and exit")
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(args.trace_summary)
        return
    if args.counter_summary:
        counter_summary(args.counter_summary)
        return
    if args.copy_calibrate:
        copy_calibrate(args.copy_calibrate)
        return
    if args.traffic_summary:
        traffic_summary(args.traffic_summary, args.traffic_kernel, args.traffic_copy_mib, args.traffic_dram)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this operator build has no multi-GPU path "
              "(every (batch, KV head) unit is independent; see DESIGN.md for how it would shard). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if args.sweep:
        for label, name, over, w, with_bwd, ndec in SWEEP:
            if args.only and label != args.only:
                continue
            sweep_point(label, WORKLOADS[name].with_(**over), w, with_bwd, ndec, max(args.steps // 2, 5),
                        max(args.warmup // 2, 2))
        return

    wl = WORKLOADS[args.workload]
    if args.T:
        wl = wl.with_(T=args.T)
    if args.B:
        wl = wl.with_(B=args.B)
    w = wl.w if args.w is None else args.w
    dev = torch.device("cuda:0")
    e = 2 if wl.dtype == torch.bfloat16 else 4

    q, k, v, a, dO = make_inputs(wl, with_grad=True)
    qd, kd, vd, ad, dOd = (x.to(dev) for x in (q, k, v, a, dO))
    desc = nha.make_desc(wl.B, wl.T, wl.H, wl.Hkv, wl.d, wl.m, w, wl.C, wl.rope_base, 0.0, wl.dtype)
    ws = torch.empty(max(nha.workspace_size(desc), nha.workspace_size(desc, backward=True)), dtype=torch.uint8,
                     device=dev)
    o = torch.empty_like(qd)
    lse = torch.empty((wl.B, wl.H, wl.T), dtype=torch.float32, device=dev)
    grads = (torch.empty_like(qd), torch.empty_like(kd), torch.empty_like(vd),
             torch.empty((wl.B, wl.T, wl.Hkv, wl.m), dtype=torch.float32, device=dev))
    fstages = nha.stage_names(desc)
    do_bwd = not args.fwd_only
    bstages = nha.stage_names(desc, backward=2) if do_bwd else []

    def new_events(n):
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for ev in evs:
            ev.record()  # materialise the underlying hipEvent_t
        return evs

    def step(fev=None, bev=None):
        nha.fwd(qd, kd, vd, ad, w, C=wl.C, rope_base=wl.rope_base, workspace=ws, out=o, lse_out=lse,
                events=[x.cuda_event for x in fev] if fev else None)
        if do_bwd:
            nha.bwd(qd, kd, vd, ad, o, lse, dOd, w, C=wl.C, rope_base=wl.rope_base, workspace=ws, out=grads,
                    events=[x.cuda_event for x in bev] if bev else None, after_fwd=True)

    for _ in range(args.warmup):
        if args.one_stream:  # warm up the same one-stream launch order that is timed
            step(new_events(len(fstages) + 1), new_events(len(bstages) + 1) if do_bwd else None)
        else:
            step()
    torch.cuda.synchronize()
    K = args.steps
    # the timed region: K steps of the production calls (independent launches
    # of a call overlap on the library's side stream)
    ms = None
    if not args.one_stream:
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record()
        for i in range(K):
            step()
        end.record()
        end.synchronize()
        torch.cuda.synchronize()
        ms = start.elapsed_time(end) / K
    # per-kernel durations: K more steps of the timed calls, which run every
    # launch in order on this stream with a HIP event before and after each
    fevs = [new_events(len(fstages) + 1) for _ in range(K)]
    bevs = [new_events(len(bstages) + 1) for _ in range(K)] if do_bwd else [None] * K
    torch.cuda.synchronize()
    s0, s1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s0.record()
    for i in range(K):
        step(fevs[i], bevs[i])
    s1.record()
    s1.synchronize()
    torch.cuda.synchronize()
    ms_serial = s0.elapsed_time(s1) / K
    if ms is None:
        ms = ms_serial

    # per-kernel durations from the live events
    per = {}
    for evs, names in ((fevs, fstages), (bevs, bstages)):
        if not names:
            continue
        for j, nm in enumerate(names):
            per[nm] = sum(evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(K)) / K
    fwd_ms = sum(per[n] for n in fstages)
    bwd_ms = sum(per[n] for n in bstages) if do_bwd else 0.0

    F_fwd = flops_fwd(wl, w)
    F_step = F_fwd * (3.5 if do_bwd else 1.0)  # backward counted as 2.5 x forward (FlashAttention convention)
    tokens = wl.B * wl.T
    value = tokens / (ms / 1e3)
    tflops = F_step / (ms / 1e3) / 1e12
    peak = PEAK_TFLOPS[wl.dtype]

    dom = max(per, key=per.get)
    roof = roofline(dom, per[dom] * 1e3, wl, w, e)
    # the next-longest kernel too: where two kernels take about the same time
    # the dominant one can differ from box to box
    rest = [n for n in per if n != dom]
    nxt = max(rest, key=per.get) if rest else None

    ok = bool(torch.isfinite(o.float()).all().item())
    if do_bwd:
        ok = ok and all(bool(torch.isfinite(g.float()).all().item()) for g in grads)

    line = {
        "metric": METRIC if do_bwd else METRIC + " [diagnostic: forward only]",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "ms_per_step_one_stream": round(ms_serial, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {
            "workload": "NHA layer %s: B=%d H=%d Hkv=%d T=%d d=%d m=%d w=%d C=%d rope_base=%g" % (
                "fwd+bwd" if do_bwd else "fwd", wl.B, wl.H, wl.Hkv, wl.T, wl.d, wl.m, w, wl.C, wl.rope_base),
            "global_batch": wl.B,
            "seq_len": wl.T,
            "parallelism": "single GPU",
        },
        "tflops": round(tflops, 2),
        "mfma_peak_frac": round(tflops / peak, 4),
        "fwd_ms": round(fwd_ms, 4),
        "bwd_ms": round(bwd_ms, 4),
        "timing_note": ("value and ms_per_step: the production calls (independent launches overlap on the "
                        "library's side stream); kernels_us, fwd_ms, bwd_ms and the roofline: K more steps of the "
                        "timed calls, one stream, a HIP event around every launch (ms_per_step_one_stream)"
                        if not args.one_stream else
                        "--one-stream: every figure from the timed calls (one stream, an event around every launch)"),
        "fwd_tflops": round(F_fwd / (fwd_ms / 1e3) / 1e12, 2),
        "fwd_mfma_peak_frac": round(F_fwd / (fwd_ms / 1e3) / 1e12 / peak, 4),
        "fwd_hbm_GBs_min_traffic": round(bytes_fwd(wl, e) / (fwd_ms / 1e3) / 1e9, 1),
        "fwd_hbm_frac": round(bytes_fwd(wl, e) / (fwd_ms / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
        "kernels_us": {kname: round(x * 1e3, 2) for kname, x in per.items()},
        "outputs_finite": ok,
        "roofline": roof,
        "roofline_next_kernel": roofline(nxt, per[nxt] * 1e3, wl, w, e) if nxt else None,
    }
    if not args.no_context and args.workload == "headline" and do_bwd:
        line["device_clock"] = device_clock_under_load(step)
        line["copy_bandwidth"] = copy_bandwidth()
        line["b1"] = b1_timings(max(5, K // 2))
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(wl, w, q, k, v, a, dO, do_bwd)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
