"""GPU parity of the chunkwise forward with the per-head GroupNorm fused into it
(retention_chunkwise_fwd_group_norm) against the fp64 oracle: the oracle's
chunkwise output, normalised by the oracle's group_norm.  The fused kernel
normalises the outputs rounded to the input dtype, as the two separate calls
do; both sides see the same input values."""
import ctypes

import pytest
import torch

import oracle
import retnet_retention_chunkwise_amd as ret
from retnet_retention_chunkwise_amd import _lib
from retnet_retention_chunkwise_amd.workloads import WORKLOADS, make_inputs
from helpers import rel_l2, say, tol

pytestmark = pytest.mark.gpu

DEV = "cuda"


def affine(H, dv, seed):
    gen = torch.Generator().manual_seed(seed)
    return torch.randn(H, dv, generator=gen), torch.randn(H, dv, generator=gen)


def err_word(ws):
    return int(ws[:4].view(torch.int32).item()) if ws is not None and ws.numel() else 0


FUSED_CASES = [
    # B, H, T, dk, dv, C, dtype, state_in, affine, gammas
    (2, 3, 300, 256, 512, 64, "bf16", True, True, [0.99, 0.9, 0.97]),        # 64-token tiles, ragged tail
    (1, 2, 333, 128, 256, 128, "bf16", True, True, [0.999, 0.95]),           # 128-token tiles, 4 column tiles
    (1, 2, 250, 64, 192, 100, "bf16", False, False, [0.98, 0.5]),            # C below the tile, 3 column tiles
    (1, 2, 300, 256, 512, 128, "bf16", True, True, [0.3, 0.5]),              # small gamma: V kept unscaled
    (1, 1, 4097, 256, 512, 128, "bf16", True, True, [0.999]),                # sequence segments
    (1, 2, 3000, 128, 128, 64, "bf16", False, True, [0.995, 0.9]),           # segments, 2 column tiles
    (2, 40, 200, 64, 512, 64, "bf16", True, True, None),                     # 640 workgroups (> 256 compute units)
    (1, 2, 65, 256, 512, 64, "bf16", True, True, [0.97, 0.9]),               # shortest fused call: 2 chunks
    (1, 130, 96, 64, 64, 32, "bf16", True, True, None),                     # 2 head groups, one column tile
    (3, 2, 777, 128, 320, 100, "bf16", False, True, [0.95, 0.999]),         # 5 column tiles, ragged, C < tile
    (1, 1, 9000, 64, 128, 128, "bf16", True, False, [0.9999]),              # segments, gamma near 1
    (1, 3, 129, 128, 512, 128, "bf16", False, True, [0.9, 0.99, 0.6]),       # 128-token tiles, 1-row tail
    (1, 2, 100, 64, 128, 32, "f32", True, True, [0.9, 0.99]),                # fp32: forward, then GroupNorm
    (1, 2, 64, 64, 128, 16, "bf16", True, True, [0.9, 0.99]),                # short block: forward, then GroupNorm
    (1, 2, 20, 64, 128, 16, "bf16", True, True, [0.9, 0.99]),                # short block: forward, then GroupNorm
]


@pytest.mark.parametrize("B,H,T,dk,dv,C,dt,with_state,aff,gs", FUSED_CASES)
def test_fused_group_norm_vs_oracle(B, H, T, dk, dv, C, dt, with_state, aff, gs):
    say(f"fused group norm B{B} H{H} T{T} dk{dk} dv{dv} C{C} {dt} state={with_state} affine={aff}")
    gs = gs if gs is not None else [0.9 + 0.099 * h / max(1, H - 1) for h in range(H)]
    q, k, v, s0 = make_inputs(B, H, T, dk, dv, dt, seed=80, with_state=True)
    s0 = s0 if with_state else None
    w, b = affine(H, dv, 81) if aff else (None, None)
    y_ref, s_ref = oracle.chunkwise(q, k, v, torch.tensor(gs), C, state_in=s0)
    ref = oracle.group_norm(y_ref, w, b, 1e-5)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    sd = None if s0 is None else s0.to(DEV)
    wd = None if w is None else w.to(DEV)
    bd = None if b is None else b.to(DEV)
    need = int(_lib.load().retention_chunkwise_fwd_group_norm_workspace_bytes(B, H, T, dk, dv, C,
                                                                              1 if dt == "bf16" else 0))
    ws = torch.full((need + 16,), 0x55, dtype=torch.uint8, device=DEV) if need else None
    y, s = ret.chunkwise_fwd_group_norm(qd, kd, vd, gs, C, wd, bd, 1e-5, state_in=sd, workspace=ws)
    torch.cuda.synchronize()
    r, rs = rel_l2(y, ref), rel_l2(s, s_ref)
    say(f"fused group norm: rel-L2 {r:.3e}, state {rs:.3e}, error word {err_word(ws)}")
    assert torch.isfinite(y.float()).all()
    assert r <= tol(q.dtype) and rs <= tol(q.dtype)
    assert err_word(ws) == 0
    # the two separate calls on the GPU give the same normalised output up to
    # the statistics' rounding order
    y2, _ = ret.chunkwise_fwd(qd, kd, vd, gs, C, state_in=sd, state_out=False)
    n2 = ret.group_norm(y2, wd, bd, 1e-5)
    torch.cuda.synchronize()
    say(f"fused vs separate calls: rel-L2 {rel_l2(y, n2):.3e}")
    assert rel_l2(y, n2) <= 1e-2


def test_fused_group_norm_wait_gives_up_and_reports():
    """Failure path, forced from the host: column tile 1 publishes no
    statistics and a wait polls at most 8 times, so every workgroup of the
    call gives up and still finishes; the error word reports it and
    check=True raises.  With the defaults restored the same call is correct."""
    B, H, T, dk, dv, C = 1, 2, 640, 128, 256, 64
    gs = [0.97, 0.9]
    say(f"fused group norm, forced give-up: B{B} H{H} T{T} dk{dk} dv{dv} C{C}")
    q, k, v = make_inputs(B, H, T, dk, dv, "bf16", seed=83)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    need = int(_lib.load().retention_chunkwise_fwd_group_norm_workspace_bytes(B, H, T, dk, dv, C, 1))
    assert need > ret.chunkwise_workspace_bytes(B, H, T, dk, dv, C, torch.bfloat16)  # the fused kernel runs
    ws = torch.zeros(need, dtype=torch.uint8, device=DEV)
    try:
        ret.testing_gn_wait(8, 1)
        ret.chunkwise_fwd_group_norm(qd, kd, vd, gs, C, state_out=False, workspace=ws)
        torch.cuda.synchronize()
        say(f"error word after the forced give-up: {err_word(ws)}")
        assert err_word(ws) == 1
        assert ret.fused_group_norm_failed(ws, B, H, T, dk, dv, C, torch.bfloat16)
        with pytest.raises(RuntimeError, match="gave up"):
            ret.chunkwise_fwd_group_norm(qd, kd, vd, gs, C, state_out=False, workspace=ws, check=True)
    finally:
        ret.testing_gn_wait()
    y, _ = ret.chunkwise_fwd_group_norm(qd, kd, vd, gs, C, state_out=False, workspace=ws, check=True)
    torch.cuda.synchronize()
    assert err_word(ws) == 0
    y_ref, _ = oracle.chunkwise(q, k, v, torch.tensor(gs), C)
    r = rel_l2(y, oracle.group_norm(y_ref, None, None, 1e-5))
    say(f"after restoring the defaults: rel-L2 {r:.3e}")
    assert r <= tol(q.dtype)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("key", ["layer1p3b", "layer6p7b", "long64k"])
def test_fused_group_norm_full_size_whole_tensor(key):
    """The fused call at full workload size, every head against the oracle."""
    wl = WORKLOADS[key]
    say(f"fused group norm, full workload {key}")
    q, k, v = make_inputs(wl.B, wl.H, wl.T, wl.dk, wl.dv, wl.dtype, seed=0)
    w, b = affine(wl.H, wl.dv, 82)
    need = int(_lib.load().retention_chunkwise_fwd_group_norm_workspace_bytes(wl.B, wl.H, wl.T, wl.dk, wl.dv, wl.C,
                                                                              1))
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    y, _ = ret.chunkwise_fwd_group_norm(q.to(DEV), k.to(DEV), v.to(DEV), list(wl.gammas), wl.C, w.to(DEV), b.to(DEV),
                                        1e-5, state_out=False, workspace=ws)
    torch.cuda.synchronize()
    assert err_word(ws) == 0
    num = den = 0.0
    hs = max(1, min(wl.H, (1 << 22) // wl.T))
    for bb in range(wl.B):
        for h0 in range(0, wl.H, hs):
            sl = (slice(bb, bb + 1), slice(h0, h0 + hs))
            y_ref, _ = oracle.chunkwise(q[sl], k[sl], v[sl], torch.tensor(wl.gammas[h0:h0 + hs]), wl.C)
            ref = oracle.group_norm(y_ref, w[h0:h0 + hs], b[h0:h0 + hs], 1e-5)
            d = y[sl].cpu().double() - ref
            num += float(d.pow(2).sum())
            den += float(ref.pow(2).sum())
    r = (num / den) ** 0.5
    say(f"fused group norm {key}: whole-tensor rel-L2 {r:.3e}")
    assert r <= 2e-2


def test_fused_group_norm_in_a_captured_graph():
    """Captured in a HIP graph (the record fill is a kernel, not a memset) and
    replayed three times with eager work in between: every replay equals the
    eager call bit for bit."""
    B, H, T, dk, dv, C = 1, 2, 2048, 128, 256, 64  # segmented
    gs = [0.99, 0.9]
    say("fused group norm in a graph")
    q, k, v = (t.to(DEV) for t in make_inputs(B, H, T, dk, dv, "bf16", seed=83))
    w, b = (t.to(DEV) for t in affine(H, dv, 84))
    need = int(_lib.load().retention_chunkwise_fwd_group_norm_workspace_bytes(B, H, T, dk, dv, C, 1))
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    y_e, s_e = ret.chunkwise_fwd_group_norm(q, k, v, gs, C, w, b, workspace=ws)
    y = torch.empty_like(y_e)
    s = torch.empty_like(s_e)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ret.chunkwise_fwd_group_norm(q, k, v, gs, C, w, b, state_out=s, y=y, workspace=ws)
    for rep in range(3):
        y.zero_()
        graph.replay()
        ret.chunkwise_fwd(q, k, v, gs, C, state_out=False)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y, y_e) and torch.equal(s, s_e), rep
        assert err_word(ws) == 0
