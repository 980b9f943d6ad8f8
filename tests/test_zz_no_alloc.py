"""The allocation-free chunkwise forward (retention_chunkwise_fwd_noalloc),
called through the C ABI, against retention_chunkwise_fwd with a caller
workspace on the same inputs: bit-identical y and final state (both run the
same kernels in the same order; only the workspace address differs), and both
within the bf16 tolerance of the oracle.  Two calls in a row, the second with a
smaller input, so that the second reads the static scratch the first left
behind."""
import ctypes

import pytest
import torch

import oracle
import retnet_retention_chunkwise_amd as ret
from retnet_retention_chunkwise_amd import _lib
from retnet_retention_chunkwise_amd.workloads import make_inputs
from helpers import rel_l2, say

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _noalloc(q, k, v, gs, C, state_in, state_out, y):
    B, H, T, dk = q.shape
    dv = v.shape[-1]
    lib = _lib.load()
    g = (ctypes.c_float * H)(*gs)
    p = lambda t: None if t is None else ctypes.c_void_p(t.data_ptr())
    st = lib.retention_chunkwise_fwd_noalloc(p(q), p(k), p(v), g, p(state_in), p(state_out), p(y), B, H, T, dk, dv,
                                             C, _lib.RET_BF16, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, _lib.last_error()


@pytest.mark.parametrize("first,second", [
    # (B, H, T, dk, dv, C, gammas): both segmented (few walkers, long sequence)
    ((1, 2, 4096, 128, 128, 64, [0.999, 0.9]), (1, 1, 2048, 64, 128, 128, [0.99])),
])
def test_noalloc_matches_workspace_entry_point(first, second):
    for i, (B, H, T, dk, dv, C, gs) in enumerate((first, second)):
        say(f"noalloc call {i}: B{B} H{H} T{T} dk{dk} dv{dv} C{C}")
        need = ret.chunkwise_workspace_bytes(B, H, T, dk, dv, C, torch.bfloat16)
        assert 0 < need <= _lib.load().retention_chunkwise_workspace_bytes(B, H, T, dk, dv, C, 1)
        q, k, v, s0 = make_inputs(B, H, T, dk, dv, "bf16", seed=70 + i, with_state=True)
        qd, kd, vd, sd = (t.to(DEV) for t in (q, k, v, s0))
        ws = torch.full((need // 4 + 64,), float("nan"), device=DEV).view(torch.uint8)
        y_ws, s_ws = ret.chunkwise_fwd(qd, kd, vd, gs, C, state_in=sd, workspace=ws)
        y_na = torch.full_like(y_ws, float("nan"))
        s_na = torch.full_like(s_ws, float("nan"))
        _noalloc(qd, kd, vd, gs, C, sd, s_na, y_na)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ws), i
        assert torch.equal(s_na, s_ws), i
        y_ref, s_ref = oracle.recurrent(q, k, v, torch.tensor(gs), s0)
        ry, rs = rel_l2(y_na, y_ref), rel_l2(s_na, s_ref)
        say(f"noalloc call {i}: identical to the workspace entry point; rel-L2 y {ry:.2e}, state {rs:.2e}")
        assert ry <= 2e-2 and rs <= 2e-2


def test_noalloc_in_place_state_and_unsegmented_call():
    """state_out aliasing state_in, and a call that needs no workspace (enough
    walkers to fill the device) through the same entry point."""
    for (B, H, T, dk, dv, C) in ((1, 2, 3000, 128, 128, 64), (4, 8, 300, 256, 512, 64)):
        say(f"noalloc in place: B{B} H{H} T{T} dk{dk} dv{dv} C{C}")
        gs = [0.99 - 0.05 * h for h in range(H)]
        q, k, v, s0 = make_inputs(B, H, T, dk, dv, "bf16", seed=72, with_state=True)
        qd, kd, vd, sd = (t.to(DEV) for t in (q, k, v, s0))
        y_ws, s_ws = ret.chunkwise_fwd(qd, kd, vd, gs, C, state_in=sd)
        st = sd.clone()
        y_na = torch.empty_like(y_ws)
        _noalloc(qd, kd, vd, gs, C, st, st, y_na)
        torch.cuda.synchronize()
        assert torch.equal(y_na, y_ws) and torch.equal(st, s_ws)
