"""C-ABI checks that run without a GPU.

The library must load, export every function include/libretention.h declares,
and reject invalid arguments before making any HIP call (so these calls are
safe on a machine without a device: nothing is launched).
"""
import ctypes
import os
import re

import pytest

from retnet_retention_chunkwise_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "libretention.h")

INVALID, UNSUPPORTED = _lib.RET_ERR_INVALID_ARG, _lib.RET_ERR_UNSUPPORTED
FAKE = ctypes.c_void_p(0x10000)        # aligned, never dereferenced: every call below fails validation first
FAKE_MIS = ctypes.c_void_p(0x10004)    # not 16-byte aligned


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(retention_\w+)\s*\(", text, flags=re.M)))


def gam(*vals):
    return (ctypes.c_float * len(vals))(*vals)


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert set(names) == set(_lib.SIGNATURES), names
    for n in names:
        assert hasattr(lib, n), n
    assert lib.retention_version() == 100


def chunk(lib, q=FAKE, k=FAKE, v=FAKE, g=None, sin=None, sout=None, y=ctypes.c_void_p(0x20000), B=1, H=2, T=8,
          dk=16, dv=16, C=4, dt=0, ws=None, wsb=0):
    g = gam(0.5, 0.9) if g is None else g
    return lib.retention_chunkwise_fwd(q, k, v, g, sin, sout, y, B, H, T, dk, dv, C, dt, ws, wsb, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(B=0), INVALID, "B=0"),
    (dict(H=0), INVALID, "H=0"),
    (dict(T=-1), INVALID, "T=-1"),
    (dict(dk=0), INVALID, "dk=0"),
    (dict(C=0), INVALID, "chunk length"),
    (dict(C=129), UNSUPPORTED, "exceeds"),
    (dict(dk=257), UNSUPPORTED, "exceed"),
    (dict(dv=513), UNSUPPORTED, "exceed"),
    (dict(dt=7), UNSUPPORTED, "dtype"),
    (dict(q=None), INVALID, "required"),
    (dict(y=None), INVALID, "required"),
    (dict(q=FAKE_MIS), UNSUPPORTED, "aligned"),
    (dict(g=(ctypes.c_float * 2)(0.5, 1.5)), INVALID, "gamma[1]"),
    (dict(g=(ctypes.c_float * 2)(-0.1, 0.5)), INVALID, "gamma[0]"),
    (dict(g=(ctypes.c_float * 2)(float("nan"), 0.5)), INVALID, "gamma[0]"),
    (dict(g=(ctypes.c_float * 2)(0.5, float("inf"))), INVALID, "gamma[1]"),
    (dict(y=FAKE), INVALID, "overlaps"),
    (dict(sin=ctypes.c_void_p(0x40000), sout=ctypes.c_void_p(0x40010)), INVALID, "overlap"),
    (dict(B=1 << 16, H=1 << 10, T=1 << 10, g=(ctypes.c_float * 1024)(*([0.5] * 1024))), UNSUPPORTED, "2^31"),
])
def test_chunkwise_rejects(lib, kw, status, needle):
    assert chunk(lib, **kw) == status
    assert needle in _lib.last_error(), _lib.last_error()


def test_null_gamma_rejected(lib):
    st = lib.retention_chunkwise_fwd(FAKE, FAKE, FAKE, None, None, None, FAKE, 1, 1, 4, 4, 4, 4, 0, None, 0, None)
    assert st == INVALID and "gamma" in _lib.last_error()


def test_recurrent_step_rejects(lib):
    g = gam(0.5)
    st = lib.retention_recurrent_step(FAKE, FAKE, FAKE, g, None, ctypes.c_void_p(0x90000), 1, 1, 4, 4, 0, None)
    assert st == INVALID and "required" in _lib.last_error()
    st = lib.retention_recurrent_step(FAKE, FAKE, FAKE, gam(2.0), ctypes.c_void_p(0x50000),
                                      ctypes.c_void_p(0x90000), 1, 1, 4, 4, 0, None)
    assert st == INVALID and "gamma[0]" in _lib.last_error()
    st = lib.retention_recurrent_step(FAKE, FAKE, FAKE, g, ctypes.c_void_p(0x50000), ctypes.c_void_p(0x50000),
                                      1, 1, 4, 4, 0, None)
    assert st == INVALID and "overlaps" in _lib.last_error()


def test_parallel_rejects(lib):
    st = lib.retention_parallel_fwd(FAKE, FAKE, FAKE, gam(0.5), None, None, 1, 1, 4, 4, 4, 0, None)
    assert st == INVALID
    st = lib.retention_parallel_fwd(FAKE, FAKE, FAKE, gam(0.5), None, ctypes.c_void_p(0x90000), 1, 1, 4, 300, 4, 0,
                                    None)
    assert st == UNSUPPORTED


def test_workspace_query(lib):
    assert lib.retention_chunkwise_workspace_bytes(1, 2, 64, 16, 16, 16, 0) == 0
    bad = ctypes.c_size_t(-1).value
    assert lib.retention_chunkwise_workspace_bytes(0, 2, 64, 16, 16, 16, 0) == bad
    assert lib.retention_chunkwise_workspace_bytes(1, 2, 64, 16, 16, 0, 0) == bad
    assert lib.retention_chunkwise_workspace_bytes(1, 2, 64, 16, 16, 16, 5) == bad


def test_workspace_for_segmented_long_sequences(lib):
    """bf16 calls with few (batch, head, 64-column) walkers over a long sequence
    are split into sequence segments: one fp32 state slot per segment, plus one
    per sub-segment of the state-only launch (nsub per segment but the last,
    about 768 work items in all, each at least 4 chunks of 64 tokens)."""
    # B1 H8 T65536 dk256 dv512 C128: 64 walkers -> 4 segments of 16384 tokens;
    # 64 x 3 items per sub-segment -> 4 sub-segments: 4 + 4 * 3 = 16 slots
    assert lib.retention_chunkwise_workspace_bytes(1, 8, 65536, 256, 512, 128, 1) == 16 * 8 * 256 * 512 * 4
    # 256 walkers (B4 H8 dv512) fill the device: no segments
    assert lib.retention_chunkwise_workspace_bytes(4, 8, 2048, 256, 512, 64, 1) == 0
    # short sequences (fewer than 16 chunks) and fp32 calls never segment
    assert lib.retention_chunkwise_workspace_bytes(1, 1, 15 * 64, 64, 64, 64, 1) == 0
    assert lib.retention_chunkwise_workspace_bytes(1, 1, 65536, 64, 64, 64, 0) == 0
    # 1 walker, 32 chunks: at most T/(8 chunks) = 4 segments of 512 tokens,
    # split in 2 sub-segments of 256 (the 4-chunk minimum): 4 + 2 * 3 = 10 slots
    assert lib.retention_chunkwise_workspace_bytes(1, 1, 2048, 64, 64, 64, 1) == 10 * 64 * 64 * 4


def test_segmented_call_requires_workspace(lib):
    q, k, v, y = (ctypes.c_void_p(a << 36) for a in (1, 2, 3, 4))
    args = dict(q=q, k=k, v=v, y=y, B=1, H=1, T=2048, dk=64, dv=64, C=64, dt=1)
    need = lib.retention_chunkwise_workspace_bytes(1, 1, 2048, 64, 64, 64, 1)
    assert chunk(lib, **args) == INVALID and "workspace" in _lib.last_error()
    assert chunk(lib, ws=ctypes.c_void_p(5 << 36), wsb=need - 16, **args) == INVALID
    assert "workspace" in _lib.last_error()
    assert chunk(lib, ws=ctypes.c_void_p((4 << 36) + 4096), wsb=need, **args) == INVALID
    assert "workspace overlaps" in _lib.last_error()


def test_error_text_is_cleared_by_success_path_query(lib):
    chunk(lib, B=0)
    assert _lib.last_error() != ""


def test_python_wrapper_refuses_cpu_tensors():
    import torch

    q = torch.zeros(1, 1, 4, 4)
    with pytest.raises(ValueError):
        _lib.chunkwise_fwd(q, q, q, [0.5], 4)
    with pytest.raises(ValueError):
        _lib.recurrent_step(q[0], q[0], q[0], [0.5], torch.zeros(1, 1, 4, 4))


def test_host_dispatch_of_every_parity_shape_without_a_device(lib):
    """With no GPU present, every chunkwise parity shape passes validation and
    segment planning on the host and fails only at the launch (RET_ERR_HIP).
    Skipped where a GPU is visible: the pointers here are placeholders."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("placeholder pointers must never reach a real device")
    import test_parity_gpu as parity
    for (B, H, T, dk, dv, C, dt, _, _) in parity.CHUNK_CASES:
        d = 1 if dt == "bf16" else 0
        need = lib.retention_chunkwise_workspace_bytes(B, H, T, dk, dv, C, d)
        q, k, v, y, w = (ctypes.c_void_p(a << 36) for a in (1, 2, 3, 4, 5))
        st = lib.retention_chunkwise_fwd(q, k, v, gam(*([0.5] * H)), None, None, y, B, H, T, dk, dv, C, d,
                                         w if need else None, need, None)
        assert st == 3, (B, H, T, dk, dv, C, dt, _lib.last_error())
    for (B, H, T, dk, dv, dt, _, _, _) in parity.SHORT_CASES:
        d = 1 if dt == "bf16" else 0
        assert lib.retention_chunkwise_workspace_bytes(B, H, T, dk, dv, 64, d) == 0
        q, k, v, y = (ctypes.c_void_p(a << 36) for a in (1, 2, 3, 4))
        st = lib.retention_chunkwise_fwd(q, k, v, gam(*([0.5] * H)), None, None, y, B, H, T, dk, dv, 64, d, None, 0,
                                         None)
        assert st == 3, (B, H, T, dk, dv, dt, _lib.last_error())


def bwd(lib, q=FAKE, k=ctypes.c_void_p(0x100000), v=ctypes.c_void_p(0x200000), sin=None,
        dy=ctypes.c_void_p(0x300000), dso=None, gq=ctypes.c_void_p(0x400000), gk=ctypes.c_void_p(0x500000),
        gv=ctypes.c_void_p(0x600000), gsi=None, B=1, H=2, T=8, dk=16, dv=16, C=4, dt=0):
    return lib.retention_chunkwise_bwd(q, k, v, gam(0.5, 0.9), sin, dy, dso, gq, gk, gv, gsi, B, H, T, dk, dv, C, dt,
                                       None, 0, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(B=0), INVALID, "B=0"),
    (dict(C=0), INVALID, "chunk length"),
    (dict(C=129), UNSUPPORTED, "exceeds"),
    (dict(dk=257), UNSUPPORTED, "exceed"),
    (dict(dt=3), UNSUPPORTED, "dtype"),
    (dict(dy=None), INVALID, "required"),
    (dict(gk=None), INVALID, "required"),
    (dict(gv=FAKE_MIS), UNSUPPORTED, "aligned"),
    (dict(gq=FAKE), INVALID, "overlaps an input"),
    (dict(gk=ctypes.c_void_p(0x400100)), INVALID, "outputs overlap"),
    (dict(dso=ctypes.c_void_p(0x700000), gsi=ctypes.c_void_p(0x700010)), INVALID, "overlaps an input"),
])
def test_chunkwise_bwd_rejects(lib, kw, status, needle):
    assert bwd(lib, **kw) == status
    assert needle in _lib.last_error(), _lib.last_error()


def test_chunkwise_bwd_in_place_state_gradient_passes_validation(lib):
    """grad_state_in == grad_state_out is accepted; with no device the call then
    fails only at the launch.  Skipped where a GPU is visible."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("placeholder pointers must never reach a real device")
    st = bwd(lib, dso=ctypes.c_void_p(0x700000), gsi=ctypes.c_void_p(0x700000))
    assert st == 3, _lib.last_error()


def test_host_dispatch_of_every_backward_parity_shape_without_a_device(lib):
    """Every backward parity shape passes validation on the host and fails only
    at the launch when no GPU is present.  Skipped where a GPU is visible."""
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("placeholder pointers must never reach a real device")
    import test_parity_gpu as parity
    for (B, H, T, dk, dv, C, dt, _, _, _) in parity.BWD_CASES:
        d = 1 if dt == "bf16" else 0
        ptrs = [ctypes.c_void_p(a << 36) for a in range(1, 9)]
        need = lib.retention_chunkwise_bwd_workspace_bytes(B, H, T, dk, dv, C, d)
        st = lib.retention_chunkwise_bwd(ptrs[0], ptrs[1], ptrs[2], gam(*([0.5] * H)), None, ptrs[3], None,
                                         ptrs[4], ptrs[5], ptrs[6], None, B, H, T, dk, dv, C, d,
                                         ptrs[7] if need else None, need, None)
        assert st == 3, (B, H, T, dk, dv, C, dt, _lib.last_error())


def gn(lib, y=ctypes.c_void_p(0x100000), w=None, b=None, eps=1e-5, out=ctypes.c_void_p(0x200000), B=1, H=2, T=8,
       dv=16, dt=0):
    return lib.retention_group_norm(y, w, b, eps, out, B, H, T, dv, dt, None)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(B=0), INVALID, "B=0"),
    (dict(T=-1), INVALID, "T=-1"),
    (dict(dv=0), INVALID, "dv=0"),
    (dict(dv=513), UNSUPPORTED, "exceeds"),
    (dict(dt=2), UNSUPPORTED, "dtype"),
    (dict(eps=-1.0), INVALID, "eps"),
    (dict(eps=float("nan")), INVALID, "eps"),
    (dict(y=None), INVALID, "required"),
    (dict(out=FAKE_MIS), UNSUPPORTED, "aligned"),
    (dict(out=ctypes.c_void_p(0x100010)), INVALID, "overlaps y"),
    (dict(w=ctypes.c_void_p(0x200000)), INVALID, "weight or bias"),
])
def test_group_norm_rejects(lib, kw, status, needle):
    assert gn(lib, **kw) == status
    assert needle in _lib.last_error(), _lib.last_error()


def test_group_norm_empty_and_in_place_pass_validation(lib):
    """T = 0 is a no-op; out == y is accepted (with no device the call then
    fails only at the launch; skipped where a GPU is visible)."""
    assert gn(lib, T=0) == _lib.RET_OK
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("placeholder pointers must never reach a real device")
    assert gn(lib, out=ctypes.c_void_p(0x100000)) == 3


def test_host_dispatch_of_every_group_norm_parity_shape_without_a_device(lib):
    import torch
    if torch.cuda.device_count() > 0:
        pytest.skip("placeholder pointers must never reach a real device")
    import test_parity_gpu as parity
    for (B, H, T, dv, dt, affine, eps, in_place) in parity.GN_CASES:
        d = 1 if dt == "bf16" else 0
        y = ctypes.c_void_p(1 << 36)
        out = y if in_place else ctypes.c_void_p(2 << 36)
        w = ctypes.c_void_p(3 << 36) if affine else None
        b = ctypes.c_void_p(4 << 36) if affine else None
        assert lib.retention_group_norm(y, w, b, eps, out, B, H, T, dv, d, None) == 3, _lib.last_error()


def test_backward_workspace_for_segmented_long_sequences(lib):
    """bf16 backward calls with few (batch, head, column) walkers over a long
    sequence are split into sequence segments of 64-token chunks: per pass (dV,
    dK, dQ) one fp32 state slot per segment and per sub-segment of the
    state-only launch."""
    # B1 H8 T65536 dk256 dv512: 64 walkers -> 4 segments, 4 sub-segments each: 16 slots
    assert lib.retention_chunkwise_bwd_workspace_bytes(1, 8, 65536, 256, 512, 128, 1) == 3 * 16 * 8 * 256 * 512 * 4
    # the 1.3B layer (B4 H8 T2048): 256 walkers, no segments
    assert lib.retention_chunkwise_bwd_workspace_bytes(4, 8, 2048, 256, 512, 64, 1) == 0
    # fp32 inputs (generic passes) and short sequences never segment
    assert lib.retention_chunkwise_bwd_workspace_bytes(1, 1, 65536, 64, 64, 64, 0) == 0
    assert lib.retention_chunkwise_bwd_workspace_bytes(1, 1, 15 * 64, 64, 64, 64, 1) == 0
    bad = ctypes.c_size_t(-1).value
    assert lib.retention_chunkwise_bwd_workspace_bytes(1, 1, 64, 64, 64, 0, 1) == bad


def test_segmented_backward_requires_workspace(lib):
    q, k, v, dy, gq, gk, gv = (ctypes.c_void_p(a << 36) for a in range(1, 8))
    need = lib.retention_chunkwise_bwd_workspace_bytes(1, 2, 4096, 64, 64, 64, 1)
    assert need > 0
    args = dict(q=q, k=k, v=v, dy=dy, gq=gq, gk=gk, gv=gv, B=1, H=2, T=4096, dk=64, dv=64, C=64, dt=1)
    assert bwd(lib, **args) == INVALID and "workspace" in _lib.last_error()
    st = lib.retention_chunkwise_bwd(q, k, v, gam(0.5, 0.9), None, dy, None, gq, gk, gv, None, 1, 2, 4096, 64, 64, 64,
                                     1, ctypes.c_void_p((1 << 36) + 4096), need, None)
    assert st == INVALID and "workspace overlaps" in _lib.last_error()


@pytest.mark.parametrize("bad", ["shape", "dtype"])
def test_python_wrapper_checks_caller_outputs_before_any_launch(bad):
    """A caller-supplied y of the wrong shape or dtype is refused with
    ValueError before any device work: the kernels write exactly B*H*(T)*dv
    elements of the input dtype into it."""
    import torch

    B, H, T, dk, dv = 1, 2, 5, 4, 6
    q = torch.zeros(B, H, T, dk)
    v = torch.zeros(B, H, T, dv)
    st = torch.zeros(B, H, dk, dv)
    wrong_y = (torch.zeros(B, H, T, dv - 1) if bad == "shape" else torch.zeros(B, H, T, dv, dtype=torch.bfloat16))
    for call in (lambda: _lib.parallel_fwd(q, q, v, [0.5, 0.5], y=wrong_y),
                 lambda: _lib.chunkwise_fwd(q, q, v, [0.5, 0.5], 4, y=wrong_y)):
        with pytest.raises(ValueError, match="y must be"):
            call()
    wrong_step_y = (torch.zeros(B, H, dv + 1) if bad == "shape" else torch.zeros(B, H, dv, dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="y must be"):
        _lib.recurrent_step(q[:, :, 0], q[:, :, 0], v[:, :, 0], [0.5, 0.5], st, y=wrong_step_y)


def test_recurrent_step_rejects_state_overlapping_inputs(lib):
    """The decode step rewrites the state in place while other workgroups read
    q, k and v: a state overlapping any of them is refused."""
    B, H, dk, dv = 1, 1, 4, 4
    base = 0x100000
    q, k, v = (ctypes.c_void_p(base + i * 0x1000) for i in range(3))
    y = ctypes.c_void_p(0x900000)
    for overlapped in (0, 1, 2):
        st_ptr = ctypes.c_void_p(base + overlapped * 0x1000)
        st = lib.retention_recurrent_step(q, k, v, gam(0.5), st_ptr, y, B, H, dk, dv, 0, None)
        assert st == INVALID and "the state overlaps" in _lib.last_error(), _lib.last_error()


def test_noalloc_rejects_calls_beyond_its_static_scratch(lib):
    """retention_chunkwise_fwd_noalloc refuses, before any HIP call, a call whose
    workspace would exceed the static scratch, and names both sizes; the
    long-context workload (B1 H8 T65536 dk256 dv512 C128) fits exactly."""
    limit = 64 << 20
    assert lib.retention_chunkwise_workspace_bytes(1, 8, 65536, 256, 512, 128, 1) == limit
    # 31 heads x 8 column tiles = 248 walkers: 2 segments, 4 sub-segments -> 6 slots of 15.5 MiB
    need = lib.retention_chunkwise_workspace_bytes(1, 31, 65536, 256, 512, 128, 1)
    assert need > limit
    q, k, v, y = (ctypes.c_void_p(a << 36) for a in (1, 2, 3, 4))
    st = lib.retention_chunkwise_fwd_noalloc(q, k, v, gam(*([0.9] * 31)), None, None, y, 1, 31, 65536, 256, 512,
                                             128, 1, None)
    assert st == UNSUPPORTED
    msg = _lib.last_error()
    assert "static scratch" in msg and str(need) in msg and str(limit) in msg, msg
    # argument errors are reported as by retention_chunkwise_fwd
    st = lib.retention_chunkwise_fwd_noalloc(None, k, v, gam(0.5), None, None, y, 1, 1, 8, 16, 16, 4, 0, None)
    assert st == INVALID and "required" in _lib.last_error()


def fgn(lib, q=FAKE, k=ctypes.c_void_p(0x20000000), v=ctypes.c_void_p(0x40000000), state_in=None, state_out=None,
        w=None, b=None, eps=1e-5, y=ctypes.c_void_p(0x80000000), B=1, H=2, T=300, dk=64, dv=128, C=64, dt=1,
        ws=None, wsb=0, g=None):
    g = gam(0.9, 0.5) if g is None else g
    return lib.retention_chunkwise_fwd_group_norm(q, k, v, g, state_in, state_out, w, b, ctypes.c_float(eps), y, B,
                                                  H, T, dk, dv, C, dt, ws, wsb, None)


def test_fused_group_norm_workspace_query(lib):
    """The fused GroupNorm's workspace: 256 bytes, the forward's segment slots
    (rounded up to 256 bytes) and 8 bytes per row and column tile; calls that
    do not take the fused kernel need the forward's workspace only."""
    q = lib.retention_chunkwise_fwd_group_norm_workspace_bytes
    fwd = lib.retention_chunkwise_workspace_bytes
    # layer1p3b: one segment, 8 column tiles
    assert q(4, 8, 2048, 256, 512, 64, 1) == 256 + 4 * 8 * 8 * 2048 * 8
    # long64k: 4 segments of 16384 positions, 16 state slots
    assert q(1, 8, 65536, 256, 512, 128, 1) == 256 + fwd(1, 8, 65536, 256, 512, 128, 1) + 4 * 8 * 8 * 16384 * 8
    # not fused: blocks of up to 64 tokens, fp32, dv above 512 or not a multiple of 64
    assert q(1, 2, 64, 64, 128, 16, 1) == fwd(1, 2, 64, 64, 128, 16, 1) == 0
    assert q(1, 2, 300, 64, 128, 64, 0) == fwd(1, 2, 300, 64, 128, 64, 0)
    assert q(1, 2, 300, 64, 100, 64, 1) == fwd(1, 2, 300, 64, 100, 64, 1)
    bad = ctypes.c_size_t(-1).value
    assert q(0, 2, 300, 64, 128, 64, 1) == bad and q(1, 2, 300, 64, 128, 0, 1) == bad


@pytest.mark.parametrize("kw,status,needle", [
    (dict(B=0), INVALID, "retention_chunkwise_fwd_group_norm"),
    (dict(eps=-1.0), INVALID, "eps"),
    (dict(eps=float("inf")), INVALID, "eps"),
    (dict(w=FAKE_MIS), UNSUPPORTED, "aligned"),
    (dict(w=ctypes.c_void_p(0x80000000 + 4096)), INVALID, "weight or bias"),
    (dict(), INVALID, "workspace"),                                 # the fused call needs its records
    (dict(ws=ctypes.c_void_p(0xC0000000), wsb=64), INVALID, "workspace"),
    (dict(ws=ctypes.c_void_p(0x80000000 + 8192), wsb=1 << 20), INVALID, "workspace overlaps"),
])
def test_fused_group_norm_rejects(lib, kw, status, needle):
    assert fgn(lib, **kw) == status
    assert needle in _lib.last_error(), _lib.last_error()


def test_fused_group_norm_testing_hook_validates_and_restores(lib):
    """retention_testing_gn_wait (host-side settings only, no HIP call)."""
    assert lib.retention_testing_gn_wait(0, -1) == INVALID
    assert "spin_limit" in _lib.last_error()
    assert lib.retention_testing_gn_wait(8, -2) == INVALID
    assert "silent_tile" in _lib.last_error()
    assert lib.retention_testing_gn_wait(8, 1) == _lib.RET_OK
    assert lib.retention_testing_gn_wait(1 << 16, -1) == _lib.RET_OK
