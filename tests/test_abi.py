"""C-ABI checks that need no GPU: the library loads, exports every function
declared in include/nha.h, and rejects bad arguments with the documented status
before any HIP call."""
import ctypes
import os
import re

import pytest
import torch

import softmax_attention_nha_amd as nha

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    src = open(os.path.join(ROOT, "include", "nha.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(nha_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_exported_set():
    assert declared_functions() == sorted(nha.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = nha.load()
    for name in declared_functions():
        assert hasattr(lib, name), name


def desc(**kw):
    base = dict(B=1, T=256, H=2, Hkv=2, d=32, m=8, w=16, C=16, rope_base=10000.0, scale=0.0, dtype=torch.float32)
    base.update(kw)
    return nha.make_desc(**base)


def status(d):
    return nha.load().nha_check_desc(ctypes.byref(d))


@pytest.mark.parametrize("kw,expected", [
    ({}, nha.NHA_OK),
    ({"dtype": torch.bfloat16, "d": 128, "m": 64, "w": 512, "C": 64}, nha.NHA_OK),
    ({"H": 3}, nha.NHA_ERR_INVALID_ARG),          # H % Hkv != 0
    ({"B": 0}, nha.NHA_ERR_INVALID_ARG),
    ({"T": 0}, nha.NHA_ERR_INVALID_ARG),
    ({"w": -1}, nha.NHA_ERR_INVALID_ARG),
    ({"m": 0, "w": 0}, nha.NHA_ERR_INVALID_ARG),  # no slots and no window: no keys
    ({"m": 0, "w": 8}, nha.NHA_OK),                # no slots: sliding-window attention
    ({"m": -1}, nha.NHA_ERR_INVALID_ARG),
    ({"rope_base": -1.0}, nha.NHA_ERR_INVALID_ARG),
    ({"scale": -0.5}, nha.NHA_ERR_INVALID_ARG),
    ({"d": 96}, nha.NHA_ERR_UNSUPPORTED),
    ({"m": 65}, nha.NHA_ERR_UNSUPPORTED),
    ({"C": 48}, nha.NHA_ERR_UNSUPPORTED),
    ({"d": 128, "m": 64, "C": 64}, nha.NHA_ERR_UNSUPPORTED),  # fp32 tiles exceed the LDS budget
])
def test_descriptor_validation(kw, expected):
    assert status(desc(**kw)) == expected


def test_sizes_zero_for_invalid_and_positive_for_valid():
    lib = nha.load()
    good, bad = desc(), desc(H=3)
    assert lib.nha_fwd_workspace_size(ctypes.byref(good)) > 0
    assert lib.nha_bwd_workspace_size(ctypes.byref(good)) > 0
    assert lib.nha_decode_state_size(ctypes.byref(good)) > 0
    for f in (lib.nha_fwd_workspace_size, lib.nha_bwd_workspace_size, lib.nha_decode_state_size):
        assert f(ctypes.byref(bad)) == 0


@pytest.mark.parametrize("rope_base", [10000.0, 0.0])
def test_decode_state_size_matches_documented_layout(rope_base):
    """SK, SV, RK, RV, RKR (RoPE only), pos, then the 32-split scratch."""
    d = desc(B=2, H=4, Hkv=2, d=64, m=8, w=16, dtype=torch.bfloat16, rope_base=rope_base)
    a256 = lambda x: (x + 255) // 256 * 256
    units = 2 * 2
    rings = 3 if rope_base > 0 else 2
    expect = (2 * a256(units * 8 * 64 * 4) + rings * a256(units * 16 * 64 * 2) + a256(units * 8)
              + a256(2 * 4 * 32 * (64 + 4) * 4))
    assert nha.decode_state_size(d) == expect


A = ctypes.c_void_p(4096)   # 16-byte aligned, never dereferenced on these paths
MIS = ctypes.c_void_p(4098)  # misaligned


def fwd_rc(d, q=A, ws=A, ws_bytes=1 << 40, lse=None):
    return nha.load().nha_fwd(ctypes.byref(d), q, A, A, A, A, lse, None, ws, ctypes.c_size_t(ws_bytes), None)


def test_fwd_argument_errors():
    d = desc()
    assert fwd_rc(d, q=ctypes.c_void_p(0)) == nha.NHA_ERR_INVALID_ARG
    assert fwd_rc(d, q=MIS) == nha.NHA_ERR_INVALID_ARG
    assert fwd_rc(d, lse=MIS) == nha.NHA_ERR_INVALID_ARG
    assert fwd_rc(d, ws=ctypes.c_void_p(0)) == nha.NHA_ERR_INVALID_ARG
    assert fwd_rc(d, ws_bytes=nha.workspace_size(d) - 1) == nha.NHA_ERR_WORKSPACE
    assert fwd_rc(desc(H=3)) == nha.NHA_ERR_INVALID_ARG
    assert fwd_rc(desc(d=96)) == nha.NHA_ERR_UNSUPPORTED


def test_bwd_argument_errors():
    lib = nha.load()
    d = desc()
    args = [A] * 11
    rc = lib.nha_bwd(ctypes.byref(d), *args[:5], None, *args[5:10], A, ctypes.c_size_t(1 << 40), None)
    assert rc == nha.NHA_ERR_INVALID_ARG  # lse is required
    n = nha.workspace_size(d, backward=True)
    rc = lib.nha_bwd(ctypes.byref(d), *args[:5], A, *args[5:10], A, ctypes.c_size_t(n - 1), None)
    assert rc == nha.NHA_ERR_WORKSPACE
    # the variant that reuses the forward's workspace checks the same things
    rc = lib.nha_bwd_after_fwd(ctypes.byref(d), *args[:5], None, *args[5:10], A, ctypes.c_size_t(1 << 40), None)
    assert rc == nha.NHA_ERR_INVALID_ARG
    rc = lib.nha_bwd_after_fwd(ctypes.byref(d), *args[:5], A, *args[5:10], A, ctypes.c_size_t(n - 1), None)
    assert rc == nha.NHA_ERR_WORKSPACE


def test_initial_state_argument_errors():
    lib = nha.load()
    d = desc()
    big = ctypes.c_size_t(1 << 40)
    # nha_fwd_s0(desc, q, k, v, alpha, s0k, s0v, o, lse, state_out, ws, ws_bytes, stream)
    assert lib.nha_fwd_s0(ctypes.byref(d), A, A, A, A, None, A, A, None, None, A, big, None) == nha.NHA_ERR_INVALID_ARG
    assert lib.nha_fwd_s0(ctypes.byref(d), A, A, A, A, A, MIS, A, None, None, A, big, None) == nha.NHA_ERR_INVALID_ARG
    n = nha.workspace_size(d)
    rc = lib.nha_fwd_s0(ctypes.byref(d), A, A, A, A, A, A, A, None, None, A, ctypes.c_size_t(n - 1), None)
    assert rc == nha.NHA_ERR_WORKSPACE
    # nha_bwd_s0(desc, q, k, v, alpha, s0k, s0v, o, lse, dO, dq, dk, dv, dalpha, ds0k, ds0v, ws, ws_bytes, stream)
    args = [A] * 15
    rc = lib.nha_bwd_s0(ctypes.byref(d), *args[:13], None, A, A, big, None)
    assert rc == nha.NHA_ERR_INVALID_ARG  # ds0k is required
    rc = lib.nha_bwd_s0(ctypes.byref(d), *args[:7], None, *args[8:15], A, big, None)
    assert rc == nha.NHA_ERR_INVALID_ARG  # lse is required
    nb = nha.workspace_size(d, backward=True)
    rc = lib.nha_bwd_s0(ctypes.byref(d), *args, A, ctypes.c_size_t(nb - 1), None)
    assert rc == nha.NHA_ERR_WORKSPACE


def test_stage_lists():
    """The backward after a forward skips the forward's first stages."""
    d = desc()
    full, after = nha.stage_names(d, backward=1), nha.stage_names(d, backward=2)
    fwd = nha.stage_names(d)
    assert after == [x for x in full if x not in ("rope_cs", "rope", "chunk_gates", "state_scan_seg", "scan_combine",
                                                  "state_scan")]
    assert full[:len(full) - len(after)] == fwd[:len(full) - len(after)]


@pytest.mark.parametrize("B,H,Hkv,d,C,dtype,fused", [
    (4, 16, 16, 128, 64, torch.bfloat16, True),   # 512 scan waves
    (2, 16, 16, 128, 64, torch.bfloat16, True),   # 256
    (8, 8, 8, 64, 64, torch.bfloat16, True),      # 256 at d = 64
    (1, 16, 16, 128, 64, torch.bfloat16, False),  # 128
    (1, 32, 8, 128, 64, torch.bfloat16, False),   # 64
    (4, 8, 4, 64, 64, torch.bfloat16, False),     # 64
    (4, 16, 16, 128, 32, torch.bfloat16, False),  # chunk of 32: not two per 128-query tile
    (8, 8, 8, 64, 64, torch.float32, False),      # fp32 path
])
def test_forward_kernel_choice(B, H, Hkv, d, C, dtype, fused):
    """The one-kernel forward (both branches per 128-query tile) is taken for
    bf16 with C = 64 when the state scan has at least 256 waves (one per batch
    row, KV head and 16 state columns); otherwise window + slot kernels."""
    dd = nha.make_desc(B, 2048, H, Hkv, d, 64, 512, C, 10000.0, 0.0, dtype)
    names = nha.stage_names(dd)
    if fused:
        assert "chunk_fwd" in names and "win_fwd" not in names and "slot_fwd" not in names, names
    else:
        assert "chunk_fwd" not in names and names[-2:] == ["win_fwd", "slot_fwd"], names
    # no window or no slots: never the chunk kernel
    for w, m in ((0, 64), (512, 0)):
        assert "chunk_fwd" not in nha.stage_names(nha.make_desc(B, 2048, H, Hkv, d, m, w, C, 10000.0, 0.0, dtype))


@pytest.mark.parametrize("B,H,Hkv,d,T,dtype,segmented", [
    (1, 16, 16, 128, 32768, torch.bfloat16, True),   # 128 scan waves, 512 chunks
    (1, 32, 8, 128, 24576, torch.bfloat16, True),    # 64 waves, 384 chunks
    (1, 16, 16, 128, 24512, torch.bfloat16, False),  # 383 chunks: one walk
    (1, 16, 16, 128, 8192, torch.bfloat16, False),
    (2, 16, 16, 128, 32768, torch.bfloat16, False),  # 256 waves: one walk
    (1, 16, 16, 64, 32768, torch.float32, False),    # fp32 scan: one walk
])
def test_state_scan_segments(B, H, Hkv, d, T, dtype, segmented):
    """Below 256 state-scan waves (B * Hkv * d / 16) and from 384 chunks on,
    the bf16 scan runs in segments of at least 8 chunks: segment end states,
    the segments' start states, then the walk (three launches, forward and
    standalone backward)."""
    dd = nha.make_desc(B, T, H, Hkv, d, 64, 512, 64, 10000.0, 0.0, dtype)
    for names in (nha.stage_names(dd), nha.stage_names(dd, backward=1)):
        i = names.index("state_scan")
        if segmented:
            assert names[i - 2:i] == ["state_scan_seg", "scan_combine"], names
        else:
            assert "state_scan_seg" not in names and "scan_combine" not in names, names
    assert "state_scan" not in nha.stage_names(dd, backward=2)


def test_decode_argument_errors():
    lib = nha.load()
    d = desc()
    assert lib.nha_decode_step(ctypes.byref(d), A, A, A, A, ctypes.c_void_p(0), A, None) == nha.NHA_ERR_INVALID_ARG
    assert lib.nha_decode_step(ctypes.byref(d), A, A, MIS, A, A, A, None) == nha.NHA_ERR_INVALID_ARG
    big = desc(w=1 << 20)
    assert lib.nha_decode_step(ctypes.byref(big), A, A, A, A, A, A, None) == nha.NHA_ERR_UNSUPPORTED


@pytest.mark.skipif(torch.cuda.is_available(), reason="checks the no-device path")
def test_launch_without_device_reports_hip_error():
    assert fwd_rc(desc()) == nha.NHA_ERR_HIP


def test_status_strings():
    lib = nha.load()
    for s in range(5):
        assert lib.nha_status_string(s).startswith(b"NHA_")


def test_token_shift_switch_validation():
    d = desc()
    d.no_token_shift = 1
    assert status(d) == nha.NHA_OK
    d.no_token_shift = 2
    assert status(d) == nha.NHA_ERR_INVALID_ARG


def test_release_side_streams_without_any_is_a_no_op():
    # nothing was created by this thread: no HIP call, NHA_OK
    assert nha.load().nha_release_side_streams() == nha.NHA_OK
    nha.release_side_streams()


# ---------------------------------------------------------------- binding checks (raise before any library call)
def _cpu_inputs(B=1, T=64, H=2, Hkv=2, d=32, m=8, dtype=torch.float32):
    q = torch.zeros(B, T, H, d, dtype=dtype)
    k = torch.zeros(B, T, Hkv, d, dtype=dtype)
    return q, k, k.clone(), torch.zeros(B, T, Hkv, m, dtype=dtype)


def test_binding_rejects_a_too_small_or_mistyped_decode_state():
    q, k, v, a = _cpu_inputs()
    d = nha.make_desc(1, 64, 2, 2, 32, 8, 16, 16, 10000.0, 0.0, torch.float32)
    n = nha.decode_state_size(d)
    with pytest.raises(ValueError, match="state_out"):
        nha.fwd(q, k, v, a, 16, C=16, state_out=torch.zeros(n - 1, dtype=torch.uint8))
    with pytest.raises(ValueError, match="state_out"):
        nha.fwd(q, k, v, a, 16, C=16, state_out=torch.zeros(n, dtype=torch.float32))
    # a state sized for bf16 rings is too small for fp32 ones
    nb = nha.decode_state_size(nha.make_desc(1, 64, 2, 2, 32, 8, 16, 16, 10000.0, 0.0, torch.bfloat16))
    assert nb < n
    with pytest.raises(ValueError, match="state_out"):
        nha.fwd(q, k, v, a, 16, C=16, state_out=torch.zeros(nb, dtype=torch.uint8))
    # a state sized without RoPE (no RoPE'd ring) is too small with RoPE
    nr = nha.decode_state_size(nha.make_desc(1, 64, 2, 2, 32, 8, 16, 16, 0.0, 0.0, torch.float32))
    assert nr < n
    with pytest.raises(ValueError, match="state_out"):
        nha.fwd(q, k, v, a, 16, C=16, state_out=torch.zeros(nr, dtype=torch.uint8))


def test_binding_rejects_mismatched_outputs():
    q, k, v, a = _cpu_inputs()
    with pytest.raises(ValueError, match="out"):
        nha.fwd(q, k, v, a, 16, C=16, out=torch.zeros(1, 64, 2, 16))
    with pytest.raises(ValueError, match="lse_out"):
        nha.fwd(q, k, v, a, 16, C=16, lse_out=torch.zeros(1, 2, 64, dtype=torch.float64))
    with pytest.raises(ValueError, match="workspace"):
        nha.fwd(q, k, v, a, 16, C=16, workspace=torch.zeros(16, dtype=torch.float32))
    o, lse = torch.zeros_like(q), torch.zeros(1, 2, 64)
    good = (torch.zeros_like(q), torch.zeros_like(k), torch.zeros_like(v), torch.zeros(1, 64, 2, 8))
    for i, name in enumerate(("dq", "dk", "dv", "dalpha")):
        bad = list(good)
        bad[i] = bad[i][:, :32].contiguous()
        with pytest.raises(ValueError, match=name):
            nha.bwd(q, k, v, a, o, lse, q, 16, C=16, out=tuple(bad))
    with pytest.raises(ValueError, match="workspace"):
        nha.bwd(q, k, v, a, o, lse, q, 16, C=16, out=good, after_fwd=True,
                workspace=torch.zeros(8, dtype=torch.uint8))


def test_binding_decode_step_checks_every_tensor():
    B, H, Hkv, d, m, w = 1, 2, 2, 32, 8, 16
    q = torch.zeros(B, H, d)
    k = torch.zeros(B, Hkv, d)
    a = torch.zeros(B, Hkv, m)
    n = nha.decode_state_size(nha.make_desc(B, 1, H, Hkv, d, m, w, 64, 10000.0, 0.0, torch.float32))
    state = torch.zeros(n, dtype=torch.uint8)
    with pytest.raises(ValueError, match="q_t"):
        nha.decode_step(torch.zeros(B, H, 2 * d)[:, :, ::2], k, k, a, state, w)  # non-contiguous
    with pytest.raises(ValueError, match="out"):
        nha.decode_step(q, k, k, a, state, w, out=torch.zeros(B, H, d + 1))
    with pytest.raises(ValueError, match="state"):
        nha.decode_step(q, k, k, a, state[: n - 8], w)
    with pytest.raises(ValueError, match="state"):
        nha.decode_step(q, k, k, a, torch.zeros(n, dtype=torch.int8), w)


def test_weighted_fusion_argument_errors():
    lib = nha.load()
    big = ctypes.c_size_t(1 << 40)
    d = desc()
    n = lib.nha_weighted_workspace_size(ctypes.byref(d))
    assert n >= max(nha.workspace_size(d), nha.workspace_size(d, backward=True))
    for bad in (desc(m=0, w=8), desc(w=0), desc(H=3)):  # both softmaxes need keys; invalid shape
        assert lib.nha_weighted_workspace_size(ctypes.byref(bad)) == 0
        assert lib.nha_fwd_weighted(ctypes.byref(bad), A, A, A, A, A, A, None, A, big, None) == nha.NHA_ERR_INVALID_ARG
    # nha_fwd_weighted(desc, q, k, v, alpha, lam, o, lse2, ws, ws_bytes, stream)
    assert lib.nha_fwd_weighted(ctypes.byref(d), A, A, A, A, None, A, None, A, big, None) == nha.NHA_ERR_INVALID_ARG
    assert lib.nha_fwd_weighted(ctypes.byref(d), A, A, A, A, MIS, A, None, A, big, None) == nha.NHA_ERR_INVALID_ARG
    assert lib.nha_fwd_weighted(ctypes.byref(d), A, A, A, A, A, A, None, A, ctypes.c_size_t(n - 1),
                                None) == nha.NHA_ERR_WORKSPACE
    # nha_bwd_weighted(desc, q, k, v, alpha, lam, dO, dq, dk, dv, dalpha, dlam, ws, ws_bytes, stream)
    args = [A] * 10
    assert lib.nha_bwd_weighted(ctypes.byref(d), *args[:4], None, *args[5:10], None, A, big,
                                None) == nha.NHA_ERR_INVALID_ARG
    assert lib.nha_bwd_weighted(ctypes.byref(d), *args, MIS, A, big, None) == nha.NHA_ERR_INVALID_ARG
    assert lib.nha_bwd_weighted(ctypes.byref(d), *args, None, A, ctypes.c_size_t(n - 1),
                                None) == nha.NHA_ERR_WORKSPACE


def test_backward_lds_limit_is_reported_as_unsupported():
    # the fp32 backward's tiles exceed a workgroup's LDS at d = 128 (any m)
    # and at d = 64 with m > 32: no backward workspace, and the binding names
    # the reason although nha_check_desc (the forward's rules) accepts them
    lib = nha.load()
    for d, m, fwd_ok, bwd_ok in [(32, 64, True, True), (64, 32, True, True), (64, 33, True, False),
                                 (128, 0, True, False), (128, 32, True, False), (128, 33, False, False)]:
        desc = nha.make_desc(1, 100, 2, 2, d, m, 16, 64, 10000.0, 0.0, torch.float32)
        assert (lib.nha_fwd_workspace_size(ctypes.byref(desc)) > 0) == fwd_ok, (d, m)
        assert (lib.nha_bwd_workspace_size(ctypes.byref(desc)) > 0) == bwd_ok, (d, m)
        if not bwd_ok:
            with pytest.raises(nha.NhaError) as ei:
                nha.workspace_size(desc, backward=True)
            assert ei.value.status == nha.NHA_ERR_UNSUPPORTED
        if fwd_ok:
            assert lib.nha_check_desc(ctypes.byref(desc)) == nha.NHA_OK
        # bf16 has no such limit
        desc = nha.make_desc(1, 100, 2, 2, d, m, 16, 64, 10000.0, 0.0, torch.bfloat16)
        assert nha.workspace_size(desc, backward=True) > 0 and nha.workspace_size(desc) > 0
    # chunked prefill: one workspace serves the continued forward and
    # backward, so its size applies the backward's limit to both
    with pytest.raises(nha.NhaError) as ei:
        nha.continue_workspace_size(nha.make_desc(1, 100, 2, 2, 128, 7, 16, 64, 10000.0, 0.0, torch.float32))
    assert ei.value.status == nha.NHA_ERR_UNSUPPORTED
    assert nha.continue_workspace_size(nha.make_desc(1, 100, 2, 2, 128, 64, 16, 64, 10000.0, 0.0, torch.bfloat16)) > 0
    # the weighted-fusion mode: m = 0 is invalid there, the LDS limit unsupported
    with pytest.raises(nha.NhaError) as ei:
        nha.weighted_workspace_size(nha.make_desc(1, 100, 2, 2, 64, 0, 16, 64, 10000.0, 0.0, torch.float32))
    assert ei.value.status == nha.NHA_ERR_INVALID_ARG
    with pytest.raises(nha.NhaError) as ei:
        nha.weighted_workspace_size(nha.make_desc(1, 100, 2, 2, 128, 16, 16, 64, 10000.0, 0.0, torch.float32))
    assert ei.value.status == nha.NHA_ERR_UNSUPPORTED
