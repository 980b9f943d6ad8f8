"""GPU parity of libretention against the fp64 CPU oracle (MI355X).

Every test calls the HIP kernels through the C ABI (via the ctypes binding)
on seeded synthetic inputs and compares element by element with the oracle on
the same input values: rel-L2 <= 1e-4 for fp32 inputs and <= 2e-2 for bf16
inputs, on y and on the carried state.  Full-size forward workloads are
checked over the whole tensor (every head, and the worst single row); the
full-size backward on sampled heads and windows.
"""
import pytest
import torch

import oracle
import retnet_retention_chunkwise_amd as ret
from retnet_retention_chunkwise_amd.workloads import WORKLOADS, make_decode_inputs, make_inputs
from helpers import rel_l2, say, tol

pytestmark = pytest.mark.gpu

DEV = "cuda"


def to_dev(*ts):
    return [None if t is None else t.to(DEV) for t in ts]


def check(name, got, want, bound):
    r = rel_l2(got, want)
    say(f"{name}: rel-L2 {r:.3e} (bound {bound:.0e})")
    assert torch.isfinite(got.float()).all(), name
    assert r <= bound, (name, r)


def gammas_for(H, lo=0.3):
    return [lo + (1.0 - lo) * h / max(1, H - 1) for h in range(H)]


# ------------------------------------------------------------------ tiny
def test_tiny_all_three_forms():
    wl = WORKLOADS["tiny"]
    say("tiny workload: parallel, chunkwise C=16, 64 recurrent steps (fp32)")
    q, k, v = make_inputs(wl.B, wl.H, wl.T, wl.dk, wl.dv, wl.dtype, seed=0)
    g = list(wl.gammas)
    y_ref, s_ref = oracle.recurrent(q, k, v, torch.tensor(g, dtype=torch.float64))
    qd, kd, vd = to_dev(q, k, v)
    check("tiny parallel", ret.parallel_fwd(qd, kd, vd, g), y_ref, 1e-4)
    y, s = ret.chunkwise_fwd(qd, kd, vd, g, wl.C)
    check("tiny chunkwise y", y, y_ref, 1e-4)
    check("tiny chunkwise state", s, s_ref, 1e-4)
    state = torch.zeros(wl.B, wl.H, wl.dk, wl.dv, device=DEV)
    ys = []
    for n in range(wl.T):
        ys.append(ret.recurrent_step(qd[:, :, n].contiguous(), kd[:, :, n].contiguous(), vd[:, :, n].contiguous(), g,
                                     state))
    check("tiny recurrent y", torch.stack(ys, dim=2), y_ref, 1e-4)
    check("tiny recurrent state", state, s_ref, 1e-4)


# ------------------------------------------------------- chunkwise edge cases
CHUNK_CASES = [
    # B, H, T, dk, dv, C, dtype, with_state, gammas
    (1, 3, 100, 16, 16, 16, "f32", True, [0.0, 0.5, 1.0]),
    (2, 2, 257, 64, 96, 32, "f32", True, [0.9, 0.99]),
    (1, 1, 1, 8, 8, 16, "f32", False, [0.7]),
    (1, 2, 50, 7, 5, 8, "f32", True, [0.6, 0.95]),
    (1, 2, 300, 16, 16, 1, "f32", False, [0.8, 0.3]),
    (1, 2, 300, 32, 48, 128, "f32", True, [0.999, 0.5]),
    (1, 130, 20, 4, 4, 4, "f32", True, None),
    # fp32 inputs on fp32 MFMA (dk, dv in {64..512}): every d_a instance, ragged tails
    (2, 2, 257, 64, 64, 32, "f32", True, [0.9, 0.99]),
    (1, 3, 100, 64, 128, 16, "f32", True, [0.0, 0.5, 1.0]),
    (1, 2, 300, 128, 256, 64, "f32", False, [0.995, 0.8]),
    (1, 2, 201, 256, 512, 128, "f32", True, [0.97, 0.999]),
    (1, 2, 300, 64, 128, 64, "bf16", True, [0.97, 0.6]),
    (2, 2, 200, 48, 80, 32, "bf16", False, [0.0, 1.0]),
    (1, 2, 129, 256, 512, 128, "bf16", True, [0.99, 0.9]),
    (2, 3, 385, 128, 192, 64, "bf16", True, [0.999, 0.95, 0.5]),
    (1, 2, 70, 256, 64, 16, "bf16", True, [0.9, 0.97]),
    (1, 1, 33, 32, 64, 32, "bf16", False, [1.0]),
    # every MFMA tile layout: 128-token tiles with two LDS copies (dk 64/128) and
    # one copy (dk 256), chunk lengths equal to and below the tile
    (1, 2, 300, 128, 128, 128, "bf16", True, [0.99, 0.7]),
    (1, 2, 250, 128, 128, 100, "bf16", True, [0.98, 0.5]),
    (1, 1, 200, 64, 64, 96, "bf16", True, [0.9]),
    (1, 2, 250, 256, 128, 100, "bf16", True, [0.995, 0.8]),
    (2, 2, 130, 64, 192, 40, "bf16", True, [0.97, 0.3]),
    # zeta-staged V near its limit gamma^(tile-1) = 2^-99 (64- and 128-token tiles)
    (1, 2, 200, 64, 64, 64, "bf16", True, [0.3367, 0.5]),
    (1, 2, 300, 128, 64, 128, "bf16", True, [0.5823, 0.9]),
    # few (batch, head, column tile) walkers over a long sequence: split into
    # sequence segments (state-only pass, scan over segments, full pass)
    (1, 1, 2048, 64, 64, 64, "bf16", True, [0.99]),
    (1, 2, 3000, 128, 192, 40, "bf16", True, [0.995, 0.9]),
    (1, 1, 4097, 256, 64, 128, "bf16", True, [0.999]),
    (1, 1, 1024, 64, 64, 1, "bf16", False, [0.97]),
    (1, 2, 2500, 256, 128, 100, "bf16", False, [1.0, 0.0]),
    # segments together with more than 128 heads (two head-group launches
    # sharing one workspace indexed by global head)
    (1, 130, 1024, 64, 64, 64, "bf16", True, None),
]


@pytest.mark.parametrize("B,H,T,dk,dv,C,dt,with_state,gs", CHUNK_CASES)
def test_chunkwise_vs_oracle(B, H, T, dk, dv, C, dt, with_state, gs):
    say(f"chunkwise B{B} H{H} T{T} dk{dk} dv{dv} C{C} {dt} state={with_state}")
    gs = gs if gs is not None else gammas_for(H)
    q, k, v, s0 = make_inputs(B, H, T, dk, dv, dt, seed=1, with_state=True)
    if not with_state:
        s0 = None
    y_ref, s_ref = oracle.recurrent(q, k, v, torch.tensor(gs, dtype=torch.float32), s0)
    qd, kd, vd, sd = to_dev(q, k, v, s0)
    y, s = ret.chunkwise_fwd(qd, kd, vd, gs, C, state_in=sd)
    torch.cuda.synchronize()
    bound = tol(q.dtype)
    check("y", y, y_ref, bound)
    check("state_out", s, s_ref, bound)


# ----------------------- short blocks (T <= 64): streaming kernels (bf16 MFMA / fp32 MFMA / VALU)
SHORT_CASES = [
    # B, H, T, dk, dv, dtype, state_in, state_out ("new" / "inplace" / None), gammas
    (2, 3, 1, 64, 128, "f32", True, "new", [0.0, 0.9, 1.0]),
    (1, 2, 2, 7, 5, "f32", True, "inplace", [0.5, 0.99]),
    (2, 2, 3, 33, 300, "f32", False, "new", [0.8, 1.0]),
    (1, 3, 4, 256, 512, "f32", True, None, [0.3, 0.7, 0.999]),
    (2, 2, 5, 48, 260, "f32", True, "inplace", [0.0, 0.6]),
    (1, 2, 8, 128, 37, "f32", True, "new", [0.95, 0.5]),
    (2, 2, 9, 16, 64, "f32", False, None, [0.9, 0.1]),
    (1, 2, 16, 256, 512, "f32", True, "inplace", [0.97, 1.0]),
    (1, 130, 11, 4, 4, "f32", True, "new", None),
    (2, 4, 1, 256, 512, "bf16", True, "inplace", [0.9, 0.95, 0.99, 0.999]),
    (2, 2, 6, 64, 192, "bf16", True, "new", [0.0, 0.8]),
    (1, 2, 16, 128, 256, "bf16", False, "new", [0.99, 0.5]),
    (1, 2, 13, 100, 301, "bf16", True, "inplace", [0.7, 1.0]),
    # 17..32 tokens (two 16-token blocks on the fp32 MFMA streaming kernel)
    (1, 2, 17, 64, 64, "f32", True, "new", [0.0, 0.9]),
    (2, 2, 32, 256, 512, "bf16", True, "inplace", [0.99, 1.0]),
    (1, 3, 25, 128, 128, "f32", False, "new", [0.5, 0.8, 0.999]),
    (1, 2, 29, 48, 192, "bf16", True, None, [0.95, 0.6]),
    # bf16 blocks of up to 64 tokens with dk % 32 == 0 (bf16 MFMA streaming kernel)
    (1, 2, 33, 256, 512, "bf16", True, "new", [0.99, 0.9]),
    (2, 3, 48, 128, 192, "bf16", False, "new", [0.0, 0.8, 1.0]),
    (1, 2, 64, 256, 512, "bf16", True, "inplace", [0.97, 0.999]),
    (1, 2, 40, 64, 64, "bf16", True, None, [0.5, 0.95]),
    (2, 2, 5, 32, 128, "bf16", True, "new", [0.9, 1.0]),
    (1, 130, 21, 32, 64, "bf16", True, "inplace", None),
    (1, 2, 57, 96, 320, "bf16", True, "new", [0.3, 0.99]),
]


@pytest.mark.parametrize("B,H,T,dk,dv,dt,with_in,out,gs", SHORT_CASES)
def test_short_block_vs_oracle(B, H, T, dk, dv, dt, with_in, out, gs):
    """Blocks of at most 64 tokens (bf16) or 32 tokens take a one-pass
    streaming kernel (any C):
    y and the carried state against the oracle, with state_in absent or given,
    state_out absent, separate or the same buffer as state_in."""
    say(f"short block B{B} H{H} T{T} dk{dk} dv{dv} {dt} state_in={with_in} state_out={out}")
    gs = gs if gs is not None else gammas_for(H)
    q, k, v, s0 = make_inputs(B, H, T, dk, dv, dt, seed=11, with_state=True)
    if not with_in:
        s0 = None
    y_ref, s_ref = oracle.recurrent(q, k, v, torch.tensor(gs, dtype=torch.float32), s0)
    qd, kd, vd, sd = to_dev(q, k, v, s0)
    if out == "inplace":
        so = sd
    else:
        so = out == "new"
    y, s = ret.chunkwise_fwd(qd, kd, vd, gs, 64, state_in=sd, state_out=so)
    torch.cuda.synchronize()
    bound = tol(q.dtype)
    check("y", y, y_ref, bound)
    if out is not None:
        check("state_out", s, s_ref, bound)
    else:
        assert s is None


# ------------------------------------------------------------------ backward
BWD_CASES = [
    # B, H, T, dk, dv, C, dtype, state_in, grad_state_out, gammas
    (1, 2, 37, 16, 24, 16, "f32", True, True, [0.9, 0.5]),
    (2, 3, 100, 64, 64, 64, "f32", False, True, [0.0, 0.8, 1.0]),
    (1, 2, 5, 7, 5, 4, "f32", True, False, [0.6, 0.99]),
    (1, 1, 1, 8, 8, 1, "f32", True, True, [0.7]),
    (1, 130, 20, 4, 4, 4, "f32", True, True, None),
    (2, 2, 70, 256, 512, 64, "f32", True, True, [0.97, 0.999]),
    (1, 3, 100, 64, 64, 16, "f32", True, False, [0.0, 0.6, 1.0]),
    (2, 2, 129, 128, 256, 64, "f32", False, True, [0.99, 0.9]),
    (1, 130, 33, 64, 64, 32, "f32", True, True, None),
    (1, 2, 129, 128, 256, 64, "bf16", True, True, [0.99, 0.9]),
    (1, 2, 200, 256, 512, 64, "bf16", True, True, [0.97, 0.999]),
    (2, 2, 77, 48, 80, 32, "bf16", False, False, [0.0, 1.0]),
    # bf16 MFMA passes: every d_a instance (64..512), ragged last chunks, gamma 0 and 1
    (2, 2, 100, 64, 64, 16, "bf16", True, True, [0.0, 1.0]),
    (1, 3, 65, 128, 128, 64, "bf16", False, True, [0.5, 0.9, 0.999]),
    (1, 2, 31, 64, 512, 32, "bf16", True, False, [0.95, 0.7]),
    (2, 2, 257, 256, 512, 128, "bf16", False, False, [0.999, 0.8]),
    (1, 2, 1, 256, 256, 1, "bf16", True, True, [0.9, 0.6]),
    (1, 130, 40, 64, 64, 32, "bf16", True, True, None),
    # a small gamma (gamma^64 < 2^-100): V kept unscaled, zeta applied in
    # registers, in both directions and at d_a = 512
    (1, 2, 150, 256, 512, 64, "bf16", True, True, [0.2, 0.9]),
    # few walkers over long sequences: sequence segments (state-only launch,
    # scan over segments in each pass's direction, full launch), incl. a short
    # last segment and gamma = 1
    (1, 1, 4096, 64, 64, 64, "bf16", True, True, [0.999]),
    (1, 2, 3001, 128, 256, 64, "bf16", True, True, [0.995, 0.9]),
    (1, 1, 2500, 256, 512, 128, "bf16", False, False, [1.0]),
    (1, 130, 1024, 64, 64, 64, "bf16", True, True, None),
    (1, 1, 2048, 128, 128, 64, "bf16", True, True, [0.3]),
]


def bwd_inputs(B, H, T, dk, dv, dt, seed):
    q, k, v, s0 = make_inputs(B, H, T, dk, dv, dt, seed=seed, with_state=True)
    _, _, dy, ds = make_inputs(B, H, T, dk, dv, dt, seed=seed + 1000, with_state=True)
    return q, k, v, s0, dy, ds


@pytest.mark.parametrize("B,H,T,dk,dv,C,dt,with_in,with_dout,gs", BWD_CASES)
def test_chunkwise_bwd_vs_oracle(B, H, T, dk, dv, C, dt, with_in, with_dout, gs):
    """Gradients of the chunkwise forward (dQ, dK, dV, dS_in) against the
    oracle's chain-rule gradients of the recurrent form."""
    say(f"backward B{B} H{H} T{T} dk{dk} dv{dv} C{C} {dt} state_in={with_in} grad_state_out={with_dout}")
    gs = gs if gs is not None else gammas_for(H)
    q, k, v, s0, dy, ds = bwd_inputs(B, H, T, dk, dv, dt, seed=40)
    s0 = s0 if with_in else None
    ds = ds if with_dout else None
    ref = oracle.recurrent_backward(q, k, v, torch.tensor(gs, dtype=torch.float32), dy, s0, ds)
    qd, kd, vd, sd, dyd, dsd = to_dev(q, k, v, s0, dy, ds)
    got = ret.chunkwise_bwd(qd, kd, vd, gs, C, dyd, state_in=sd, grad_state_out=dsd)
    torch.cuda.synchronize()
    bound = tol(q.dtype)
    for name, g, r in zip(("grad_q", "grad_k", "grad_v", "grad_state_in"), got, ref):
        check(name, g, r, bound)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_chunkwise_bwd_sampled_heads_at_layer_size(dt):
    """The backward at the 1.3B-scale layer shape (B4 H8 T2048 dk256 dv512):
    two sampled heads against the oracle (their gradients depend only on their
    own inputs)."""
    wl = WORKLOADS["layer1p3b"]
    say(f"backward at layer size, {dt}")
    q, k, v, s0, dy, ds = bwd_inputs(wl.B, wl.H, wl.T, wl.dk, wl.dv, dt, seed=42)
    gs = list(wl.gammas)
    qd, kd, vd, sd, dyd, dsd = to_dev(q, k, v, s0, dy, ds)
    got = ret.chunkwise_bwd(qd, kd, vd, gs, wl.C, dyd, state_in=sd, grad_state_out=dsd)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (3, 7)):
        sl = lambda t: t[b:b + 1, h:h + 1]
        ref = oracle.recurrent_backward(sl(q), sl(k), sl(v), torch.tensor([gs[h]]), sl(dy), sl(s0), sl(ds))
        for name, gg, r in zip(("grad_q", "grad_k", "grad_v", "grad_state_in"), got, ref):
            check(f"{name} (b{b} h{h})", sl(gg), r, tol(q.dtype))


def test_segmented_bwd_in_place_and_explicit_workspace():
    """A segmented bf16 backward with grad_state_in = grad_state_out (in place)
    and a caller-provided workspace."""
    B, H, T, dk, dv = 1, 2, 2048, 64, 128
    gs = [0.99, 0.7]
    say("segmented backward, in place, explicit workspace")
    q, k, v, s0, dy, ds = bwd_inputs(B, H, T, dk, dv, "bf16", seed=43)
    ref = oracle.recurrent_backward(q, k, v, torch.tensor(gs), dy, s0, ds)
    qd, kd, vd, sd, dyd, dsd = to_dev(q, k, v, s0, dy, ds)
    need = int(ret.load().retention_chunkwise_bwd_workspace_bytes(B, H, T, dk, dv, 64, 1))
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    got = ret.chunkwise_bwd(qd, kd, vd, gs, 64, dyd, state_in=sd, grad_state_out=dsd, grad_state_in=dsd, workspace=ws)
    torch.cuda.synchronize()
    for name, g, r in zip(("grad_q", "grad_k", "grad_v", "grad_state_in"), got, ref):
        check(name, g, r, 2e-2)


def test_segmented_calls_with_negligible_sub_segments():
    """Segmented forward and backward whose state-only pass leaves out the
    sub-segments that reach the next segment only through gamma^d <= 2^-40.
    B1 H5 T8192 dk64 dv64 C64: 5 walkers -> 16 segments of 512 positions, 2
    sub-segments of 256 each in the state-only pass; the first sub-segment of a
    segment (d = 256) is left out for gamma = 0 and 0.5 and walked for
    1 - 2^-5, 0.999 and 1.  Both directions against the oracle."""
    B, H, T, dk, dv, C = 1, 5, 8192, 64, 64, 64
    gs = [0.0, 0.5, 1 - 2 ** -5, 0.999, 1.0]
    say(f"segmented forward and backward with negligible sub-segments, gammas {gs}")
    q, k, v, s0, dy, ds = bwd_inputs(B, H, T, dk, dv, "bf16", seed=47)
    y_ref, s_ref = oracle.recurrent(q, k, v, torch.tensor(gs, dtype=torch.float64), s0)
    qd, kd, vd, sd, dyd, dsd = to_dev(q, k, v, s0, dy, ds)
    assert ret.chunkwise_workspace_bytes(B, H, T, dk, dv, C, torch.bfloat16) > 0  # segmented
    y, s_out = ret.chunkwise_fwd(qd, kd, vd, gs, C, state_in=sd)
    torch.cuda.synchronize()
    for h in range(H):
        check(f"y (gamma {gs[h]})", y[:, h], y_ref[:, h], 2e-2)
        check(f"state (gamma {gs[h]})", s_out[:, h], s_ref[:, h], 2e-2)
    ref = oracle.recurrent_backward(q, k, v, torch.tensor(gs, dtype=torch.float32), dy, s0, ds)
    got = ret.chunkwise_bwd(qd, kd, vd, gs, C, dyd, state_in=sd, grad_state_out=dsd)
    torch.cuda.synchronize()
    for name, g, r in zip(("grad_q", "grad_k", "grad_v", "grad_state_in"), got, ref):
        check(name, g, r, 2e-2)


def test_chunkwise_bwd_in_place_state_gradient_and_empty_sequence():
    """grad_state_in may be the grad_state_out buffer; T = 0 copies it through."""
    B, H, T, dk, dv = 1, 2, 50, 32, 64
    gs = [0.9, 0.6]
    say("backward in place / T = 0")
    q, k, v, s0, dy, ds = bwd_inputs(B, H, T, dk, dv, "f32", seed=41)
    ref = oracle.recurrent_backward(q, k, v, torch.tensor(gs), dy, s0, ds)
    qd, kd, vd, sd, dyd, dsd = to_dev(q, k, v, s0, dy, ds)
    got = ret.chunkwise_bwd(qd, kd, vd, gs, 16, dyd, state_in=sd, grad_state_out=dsd, grad_state_in=dsd)
    torch.cuda.synchronize()
    for name, g, r in zip(("grad_q", "grad_k", "grad_v", "grad_state_in"), got, ref):
        check(name, g, r, 1e-4)
    e = lambda t: t[:, :, :0].contiguous()
    ds2 = ds.to(DEV)
    _, _, _, gsi = ret.chunkwise_bwd(e(qd), e(kd), e(vd), gs, 16, e(dyd), grad_state_out=ds2)
    torch.cuda.synchronize()
    assert torch.equal(gsi.cpu(), ds)


# --------------------------------------------------------------- group norm
GN_CASES = [
    # B, H, T, dv, dtype, affine, eps, in_place
    (2, 3, 100, 512, "bf16", True, 1e-5, False),
    (1, 2, 77, 64, "f32", True, 1e-5, True),
    (1, 4, 33, 300, "bf16", False, 1e-3, False),
    (1, 1, 5, 7, "f32", True, 0.0, False),
    (2, 130, 3, 16, "f32", False, 1e-5, True),
    (1, 2, 40, 256, "f32", True, 1e-6, False),
    (1, 2, 9, 100, "f32", True, 1e-5, False),
]


@pytest.mark.parametrize("B,H,T,dv,dt,affine,eps,in_place", GN_CASES)
def test_group_norm_vs_oracle(B, H, T, dv, dt, affine, eps, in_place):
    say(f"group norm B{B} H{H} T{T} dv{dv} {dt} affine={affine} eps={eps} in_place={in_place}")
    gen = torch.Generator().manual_seed(60)
    y = (torch.randn(B, H, T, dv, generator=gen) * 2.0 + 0.5).to(torch.bfloat16 if dt == "bf16" else torch.float32)
    w = torch.randn(H, dv, generator=gen) if affine else None
    b = torch.randn(H, dv, generator=gen) if affine else None
    ref = oracle.group_norm(y, w, b, eps)
    yd, wd, bd = to_dev(y, w, b)
    out = ret.group_norm(yd, wd, bd, eps, out=yd if in_place else None)
    torch.cuda.synchronize()
    check("group norm", out, ref, tol(y.dtype))


def test_group_norm_of_chunkwise_output_at_layer_size():
    """The chunkwise forward followed by the per-head GroupNorm at the 1.3B-scale
    layer shape, sampled heads against the oracle."""
    wl = WORKLOADS["layer1p3b"]
    say("chunkwise + group norm at layer size")
    q, k, v = make_inputs(wl.B, wl.H, wl.T, wl.dk, wl.dv, wl.dtype, seed=61)
    gen = torch.Generator().manual_seed(62)
    w = torch.randn(wl.H, wl.dv, generator=gen)
    b = torch.randn(wl.H, wl.dv, generator=gen)
    qd, kd, vd, wd, bd = to_dev(q, k, v, w, b)
    y, _ = ret.chunkwise_fwd(qd, kd, vd, list(wl.gammas), wl.C, state_out=False)
    out = ret.group_norm(y, wd, bd, 1e-5)
    torch.cuda.synchronize()
    for bb, h in ((0, 0), (2, 5)):
        sl = lambda t: t[bb:bb + 1, h:h + 1]
        y_ref, _ = oracle.recurrent(sl(q), sl(k), sl(v), torch.tensor([wl.gammas[h]]))
        ref = oracle.group_norm(y_ref, w[h:h + 1], b[h:h + 1], 1e-5)
        check(f"group norm of y (b{bb} h{h})", sl(out), ref, tol(q.dtype))


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_parallel_vs_oracle(dt):
    B, H, T, dk, dv = 2, 3, 150, 32, 64
    say(f"parallel B{B} H{H} T{T} dk{dk} dv{dv} {dt}")
    gs = [0.0, 0.8, 1.0]
    q, k, v, s0 = make_inputs(B, H, T, dk, dv, dt, seed=2, with_state=True)
    y_ref = oracle.parallel(q, k, v, torch.tensor(gs, dtype=torch.float32), s0)
    qd, kd, vd, sd = to_dev(q, k, v, s0)
    check("parallel y", ret.parallel_fwd(qd, kd, vd, gs, state_in=sd), y_ref, tol(q.dtype))


@pytest.mark.parametrize("dt,dv", [("f32", 64), ("bf16", 512), ("f32", 30), ("bf16", 6)])
def test_recurrent_steps_vs_oracle(dt, dv):
    B, H, dk, steps = 3, 4, 64, 12
    say(f"recurrent steps B{B} H{H} dk{dk} dv{dv} {dt}")
    gs = [0.0, 0.5, 0.9, 1.0]
    q, k, v, s0 = make_decode_inputs(B, H, dk, dv, steps, dt, seed=3)
    state = s0.to(DEV)
    S = s0
    ys, yr = [], []
    for n in range(steps):
        ys.append(ret.recurrent_step(q[n].to(DEV), k[n].to(DEV), v[n].to(DEV), gs, state).cpu())
        y_n, S = oracle.recurrent_step(q[n], k[n], v[n], torch.tensor(gs, dtype=torch.float32), S)
        yr.append(y_n)
    check("decode y", torch.stack(ys), torch.stack(yr), tol(q.dtype))
    check("decode state", state, S, tol(q.dtype))


# ------------------------------------------------------- state semantics
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_split_sequence_with_state_handoff(dt):
    B, H, T, dk, dv, C = 1, 2, 260, 64, 128, 32
    say(f"state handoff {dt}")
    gs = [0.95, 0.7]
    q, k, v, s0 = make_inputs(B, H, T, dk, dv, dt, seed=4, with_state=True)
    qd, kd, vd, sd = to_dev(q, k, v, s0)
    y_all, s_all = ret.chunkwise_fwd(qd, kd, vd, gs, C, state_in=sd)
    t = 100  # not a multiple of C
    st = sd.clone()
    y1, _ = ret.chunkwise_fwd(qd[:, :, :t].contiguous(), kd[:, :, :t].contiguous(), vd[:, :, :t].contiguous(), gs, C,
                              state_in=st, state_out=st)       # in place: state_out aliases state_in
    y2, _ = ret.chunkwise_fwd(qd[:, :, t:].contiguous(), kd[:, :, t:].contiguous(), vd[:, :, t:].contiguous(), gs, C,
                              state_in=st, state_out=st)
    y_ref, s_ref = oracle.recurrent(q, k, v, torch.tensor(gs, dtype=torch.float32), s0)
    check("split y", torch.cat([y1, y2], dim=2), y_ref, tol(q.dtype))
    check("split state", st, s_ref, tol(q.dtype))
    check("split vs one call", torch.cat([y1, y2], dim=2), y_all, tol(q.dtype))


def test_segmented_handoff_in_place_and_explicit_workspace():
    """Segmented calls (few heads, long sequence) with state_out aliasing
    state_in, and a caller-provided workspace that starts out as NaN."""
    B, H, T, dk, dv, C = 1, 2, 3000, 128, 128, 64
    say("segmented handoff, in-place state, NaN-filled workspace")
    gs = [0.999, 0.9]
    q, k, v, s0 = make_inputs(B, H, T, dk, dv, "bf16", seed=7, with_state=True)
    qd, kd, vd, sd = to_dev(q, k, v, s0)
    t = 1100
    parts = [(0, t), (t, T)]
    for a, b in parts:
        assert ret.chunkwise_workspace_bytes(B, H, b - a, dk, dv, C, qd.dtype) > 0
    st = sd.clone()
    ys = []
    for a, b in parts:
        need = ret.chunkwise_workspace_bytes(B, H, b - a, dk, dv, C, qd.dtype)
        ws = torch.full((need // 4 + 64,), float("nan"), device=DEV)
        y, _ = ret.chunkwise_fwd(qd[:, :, a:b].contiguous(), kd[:, :, a:b].contiguous(), vd[:, :, a:b].contiguous(),
                                 gs, C, state_in=st, state_out=st, workspace=ws.view(torch.uint8))
        ys.append(y)
    y_ref, s_ref = oracle.recurrent(q, k, v, torch.tensor(gs, dtype=torch.float32), s0)
    check("segmented split y", torch.cat(ys, dim=2), y_ref, 2e-2)
    check("segmented split state", st, s_ref, 2e-2)


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_prefill_decode_continuation(dt):
    """Inference use of the three forms on one sequence: a chunkwise prefill of
    300 tokens, 5 recurrent decode steps, then chunkwise continuations of 16
    and 1 new tokens from the carried state (C = 16 and 1), against the oracle
    on the concatenated 322 tokens."""
    B, H, dk, dv = 2, 4, 64, 128
    T0, nd, T1, T2 = 300, 5, 16, 1
    T = T0 + nd + T1 + T2
    say(f"prefill -> decode -> continuation, {dt}")
    gs = [0.999, 0.99, 0.95, 0.8]
    q, k, v, s0 = make_inputs(B, H, T, dk, dv, dt, seed=8, with_state=True)
    y_ref, s_ref = oracle.recurrent(q, k, v, torch.tensor(gs, dtype=torch.float32), s0)
    qd, kd, vd, sd = to_dev(q, k, v, s0)
    st = sd.clone()
    parts = []
    y, _ = ret.chunkwise_fwd(qd[:, :, :T0].contiguous(), kd[:, :, :T0].contiguous(), vd[:, :, :T0].contiguous(), gs, 64,
                             state_in=st, state_out=st)
    parts.append(y)
    for n in range(T0, T0 + nd):
        parts.append(ret.recurrent_step(qd[:, :, n].contiguous(), kd[:, :, n].contiguous(), vd[:, :, n].contiguous(),
                                        gs, st).unsqueeze(2))
    a = T0 + nd
    for Tn, C in ((T1, 16), (T2, 1)):
        y, _ = ret.chunkwise_fwd(qd[:, :, a:a + Tn].contiguous(), kd[:, :, a:a + Tn].contiguous(),
                                 vd[:, :, a:a + Tn].contiguous(), gs, C, state_in=st, state_out=st)
        parts.append(y)
        a += Tn
    torch.cuda.synchronize()
    check("continued y", torch.cat(parts, dim=2), y_ref, tol(q.dtype))
    check("continued state", st, s_ref, tol(q.dtype))


@pytest.mark.parametrize("Tn,C", [(1, 1), (7, 4), (16, 16), (64, 64), (100, 32)])
def test_multi_token_decode_from_state(Tn, C):
    """Chunkwise continuation of a batch of decode streams: Tn new tokens per
    stream from a carried fp32 state (the decode workload's head shapes)."""
    B, H, dk, dv = 8, 4, 256, 512
    say(f"multi-token decode Tn={Tn} C={C}")
    gs = gammas_for(H, 0.9)
    q, k, v, s0 = make_inputs(B, H, Tn, dk, dv, "bf16", seed=9, with_state=True)
    y_ref, s_ref = oracle.recurrent(q, k, v, torch.tensor(gs, dtype=torch.float32), s0)
    qd, kd, vd, sd = to_dev(q, k, v, s0)
    y, s = ret.chunkwise_fwd(qd, kd, vd, gs, C, state_in=sd)
    torch.cuda.synchronize()
    check("y", y, y_ref, 2e-2)
    check("state", s, s_ref, 2e-2)


def test_empty_sequence_copies_state():
    say("T = 0")
    B, H, dk, dv = 1, 2, 16, 32
    e = torch.empty(B, H, 0, dk, device=DEV)
    ev = torch.empty(B, H, 0, dv, device=DEV)
    s_in = torch.randn(B, H, dk, dv, device=DEV)
    y, s = ret.chunkwise_fwd(e, e, ev, [0.5, 0.5], 16, state_in=s_in)
    assert y.shape == (B, H, 0, dv)
    assert torch.equal(s, s_in)
    _, s0 = ret.chunkwise_fwd(e, e, ev, [0.5, 0.5], 16)
    assert torch.count_nonzero(s0) == 0


def test_chunk_length_independence_on_gpu():
    B, H, T, dk, dv = 1, 2, 257, 128, 128
    say("chunk length independence, bf16")
    gs = [0.98, 0.8]
    q, k, v = to_dev(*make_inputs(B, H, T, dk, dv, "bf16", seed=5))
    y_ref, s_ref = oracle.recurrent(q.cpu(), k.cpu(), v.cpu(), torch.tensor(gs, dtype=torch.float32))
    for C in (8, 16, 32, 64, 100, 128):
        y, s = ret.chunkwise_fwd(q, k, v, gs, C)
        check(f"C={C} y", y, y_ref, 2e-2)
        check(f"C={C} state", s, s_ref, 2e-2)


def test_deterministic_reruns():
    say("bitwise determinism of reruns")
    B, H, T, dk, dv, C = 2, 4, 512, 256, 512, 64
    q, k, v = to_dev(*make_inputs(B, H, T, dk, dv, "bf16", seed=6))
    gs = gammas_for(H, 0.9)
    y1, s1 = ret.chunkwise_fwd(q, k, v, gs, C)
    y2, s2 = ret.chunkwise_fwd(q, k, v, gs, C)
    assert torch.equal(y1, y2) and torch.equal(s1, s2)


def test_side_stream_matches_default_stream():
    """Every entry point enqueued on a non-default stream (the binding passes
    torch's current stream through the C ABI) gives the default-stream results
    bit for bit, including a segmented call with its workspace."""
    say("side stream")
    B, H, T, dk, dv, C = 1, 2, 2048, 128, 256, 64  # few walkers: segmented forward and backward
    gs = [0.99, 0.8]
    q, k, v, s0, dy, ds = to_dev(*bwd_inputs(B, H, T, dk, dv, "bf16", seed=46))
    q1, k1 = q[:, :, 0].contiguous(), k[:, :, 0].contiguous()
    v1 = v[:, :, 0].contiguous()

    def run():
        y, s = ret.chunkwise_fwd(q, k, v, gs, C, state_in=s0)
        g = ret.chunkwise_bwd(q, k, v, gs, C, dy, state_in=s0, grad_state_out=ds)
        st = s0.clone()
        yd = ret.recurrent_step(q1, k1, v1, gs, st)
        n = ret.group_norm(y)
        return (y, s, *g, st, yd, n)

    ref = run()
    torch.cuda.synchronize()
    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        got = run()
    side.synchronize()
    for i, (a, b) in enumerate(zip(got, ref)):
        assert torch.equal(a, b), i


def test_chunkwise_in_a_captured_graph_matches_eager():
    """Launches captured in a HIP graph (as the benchmark issues them) give the
    eager result bit for bit on every replay, with eager work and
    synchronisations between the replays."""
    say("chunkwise forward and backward captured in a graph, replayed 3 times")
    B, H, T, dk, dv, C = 2, 4, 300, 256, 512, 64
    q, k, v, s0 = to_dev(*make_inputs(B, H, T, dk, dv, "bf16", seed=12, with_state=True))
    dy = torch.randn(B, H, T, dv, device=DEV).div_(16).to(torch.bfloat16)
    gs = gammas_for(H, 0.9)
    y_eager, s_eager = ret.chunkwise_fwd(q, k, v, gs, C, state_in=s0)
    g_eager = ret.chunkwise_bwd(q, k, v, gs, C, dy, state_in=s0)
    y = torch.empty_like(y_eager)
    s = torch.empty_like(s_eager)
    gq, gk, gv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    gsi = torch.empty_like(s0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ret.chunkwise_fwd(q, k, v, gs, C, state_in=s0, state_out=s, y=y)
        out = ret.chunkwise_bwd(q, k, v, gs, C, dy, state_in=s0, grad_state_in=gsi)
    for rep in range(3):
        y.zero_()
        s.zero_()
        gsi.zero_()
        graph.replay()
        other, _ = ret.chunkwise_fwd(v[:, :, :, :dk].contiguous(), k, v, gs, C)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager) and torch.equal(s, s_eager), rep
        for a, b in zip(out, g_eager):
            assert torch.equal(a, b), rep


def test_segmented_calls_in_a_captured_graph_match_eager():
    """Segmented forward and backward (state-only launch with negligible
    sub-segments and positions left out, segment scan on 16-byte and on
    single-element accesses, full launch) captured in a HIP graph give the eager
    result bit for bit on every replay."""
    B, H, T, dk, dv, C = 1, 5, 8192, 64, 64, 64
    gs = [0.0, 0.5, 1 - 2 ** -5, 0.999, 1.0]
    say("segmented forward and backward captured in a graph, replayed 3 times")
    q, k, v, s0 = to_dev(*make_inputs(B, H, T, dk, dv, "bf16", seed=13, with_state=True))
    dy = torch.randn(B, H, T, dv, device=DEV).div_(16).to(torch.bfloat16)
    nf = ret.chunkwise_workspace_bytes(B, H, T, dk, dv, C, torch.bfloat16)
    nb = int(ret.load().retention_chunkwise_bwd_workspace_bytes(B, H, T, dk, dv, C, 1))
    assert nf > 0 and nb > 0
    wf = torch.empty(nf, dtype=torch.uint8, device=DEV)
    wb = torch.empty(nb, dtype=torch.uint8, device=DEV)
    y_eager, s_eager = ret.chunkwise_fwd(q, k, v, gs, C, state_in=s0, workspace=wf)
    g_eager = ret.chunkwise_bwd(q, k, v, gs, C, dy, state_in=s0, workspace=wb)
    y = torch.empty_like(y_eager)
    s = torch.empty_like(s_eager)
    gsi = torch.empty_like(s0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ret.chunkwise_fwd(q, k, v, gs, C, state_in=s0, state_out=s, y=y, workspace=wf)
        out = ret.chunkwise_bwd(q, k, v, gs, C, dy, state_in=s0, grad_state_in=gsi, workspace=wb)
    for rep in range(3):
        y.zero_()
        s.zero_()
        gsi.zero_()
        wf.zero_()
        graph.replay()
        other, _ = ret.chunkwise_fwd(k, q, v, gs, C)  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager) and torch.equal(s, s_eager), rep
        for a, b in zip(out, g_eager):
            assert torch.equal(a, b), rep


# ------------------------------------------------------- full-size workloads
def sampled_heads(B, H):
    return sorted({(0, 0), (B // 2, H // 2), (B - 1, H - 1)})


def test_f32_forward_at_layer_size_sampled_heads():
    """fp32 inputs at the 1.3B-scale layer shape (fp32 MFMA path): sampled
    heads against the oracle at the fp32 bound."""
    wl = WORKLOADS["layer1p3b"]
    say("fp32 forward at layer size")
    q, k, v, s0 = make_inputs(wl.B, wl.H, wl.T, wl.dk, wl.dv, "f32", seed=44, with_state=True)
    qd, kd, vd, sd = to_dev(q, k, v, s0)
    y, s = ret.chunkwise_fwd(qd, kd, vd, list(wl.gammas), wl.C, state_in=sd)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (3, 7)):
        sl = lambda t: t[b:b + 1, h:h + 1]
        y_ref, s_ref = oracle.recurrent(sl(q), sl(k), sl(v), torch.tensor([wl.gammas[h]]), sl(s0))
        check(f"y (b{b} h{h})", sl(y), y_ref, 1e-4)
        check(f"state (b{b} h{h})", sl(s), s_ref, 1e-4)


class WholeTensor:
    """rel-L2 over a whole tensor accumulated slice by slice (sum of squared
    differences over sum of squared oracle values, in float64), plus the
    worst single row (one token of one head): its error over its own norm and
    over the root-mean-square row norm of its head."""

    def __init__(self, name):
        self.name, self.num, self.den = name, 0.0, 0.0
        self.row_own = self.row_rms = 0.0
        self.where = None

    def add(self, got, want, rows=True):
        g = got.detach().to("cpu", torch.float64)
        w = want.detach().to("cpu", torch.float64)
        assert torch.isfinite(g).all(), self.name
        d = g - w
        self.num += float(d.pow(2).sum())
        self.den += float(w.pow(2).sum())
        if rows:
            dn = d.pow(2).sum(-1).sqrt()                       # [..., T]
            wn = w.pow(2).sum(-1).sqrt()
            rms = w.pow(2).sum(-1).mean(-1, keepdim=True).sqrt()
            own = dn / wn.clamp_min(1e-300)
            rel = dn / rms.clamp_min(1e-300)
            if float(own.max()) > self.row_own:
                self.row_own = float(own.max())
            if float(rel.max()) > self.row_rms:
                self.row_rms = float(rel.max())
                self.where = tuple(int(i) for i in torch.nonzero(rel == rel.max())[0])

    def check(self, bound, row_own_bound=None, row_rms_bound=None):
        r = (self.num / self.den) ** 0.5
        rows = "" if self.where is None else (f"; worst row: {self.row_own:.3e} of its own norm, {self.row_rms:.3e} "
                                              f"of its head's rms row norm (at {self.where})")
        say(f"{self.name}: whole-tensor rel-L2 {r:.3e} (bound {bound:.0e}){rows}")
        assert r <= bound, (self.name, r)
        if row_own_bound is not None:
            assert self.row_own <= row_own_bound, (self.name, self.row_own)
        if row_rms_bound is not None:
            assert self.row_rms <= row_rms_bound, (self.name, self.row_rms)


# Per-row bounds of the full-size checks: no single token row of any head may
# be off by more than 10% of its own norm or 5% of its head's typical (rms)
# row norm.  A row computed from a wrong state, tile or segment is off by
# about 100%, while rounding (bf16 inputs, bf16 operands of the products, bf16
# output) leaves a few 1e-3 per row.
ROW_OWN_BOUND = 0.1
ROW_RMS_BOUND = 0.05


@pytest.mark.timeout(600)
@pytest.mark.parametrize("key", ["layer1p3b", "layer6p7b", "long64k"])
def test_full_size_workload_whole_tensor(key):
    """The chunkwise forward of a full workload (bf16), every head against the
    fp64 oracle: rel-L2 over the whole y and the whole final state, and the
    worst single row, computed head slice by head slice on the host."""
    wl = WORKLOADS[key]
    say(f"full workload {key}: {wl.description}")
    q, k, v = make_inputs(wl.B, wl.H, wl.T, wl.dk, wl.dv, wl.dtype, seed=0)
    qd, kd, vd = to_dev(q, k, v)
    y, s = ret.chunkwise_fwd(qd, kd, vd, list(wl.gammas), wl.C)
    torch.cuda.synchronize()
    del qd, kd, vd
    say(f"{key}: kernel done, checking every head against the oracle")
    ty, ts = WholeTensor(f"{key} y"), WholeTensor(f"{key} state")
    hs = max(1, min(wl.H, (1 << 22) // wl.T))  # heads per oracle slice (bounded host memory)
    for b in range(wl.B):
        for h0 in range(0, wl.H, hs):
            sl = (slice(b, b + 1), slice(h0, h0 + hs))
            g = torch.tensor(wl.gammas[h0:h0 + hs], dtype=torch.float32)
            y_ref, s_ref = oracle.chunkwise(q[sl], k[sl], v[sl], g, wl.C)
            ty.add(y[sl], y_ref)
            ts.add(s[sl], s_ref, rows=False)
    ty.check(2e-2, ROW_OWN_BOUND, ROW_RMS_BOUND)
    ts.check(2e-2)


@pytest.mark.timeout(600)
def test_full_size_long_backward():
    """The backward of the long-context workload (B1 H8 T65536 dk256 dv512 bf16,
    C=128), which runs in sequence segments with sub-segmented state-only
    launches.  Against the oracle on sampled heads: dQ of the first W tokens
    (it depends only on state_in and earlier tokens), dK, dV of the last W
    (only on later tokens and grad_state_out), and all three in a window in
    the middle of the sequence.
    All four gradients at full size through a split of the sequence: the
    backward of the second part (state_in = the forward's state at the split)
    hands its grad_state_in to the backward of the first part as its
    grad_state_out, and the pieces must match the one-call gradients."""
    wl = WORKLOADS["long64k"]
    say(f"full-size backward: {wl.description}")
    q, k, v, s0, dy, ds = bwd_inputs(wl.B, wl.H, wl.T, wl.dk, wl.dv, wl.dtype, seed=45)
    gs = list(wl.gammas)
    T, W = wl.T, 512
    qd, kd, vd, sd, dyd, dsd = to_dev(q, k, v, s0, dy, ds)
    got = ret.chunkwise_bwd(qd, kd, vd, gs, wl.C, dyd, state_in=sd, grad_state_out=dsd)
    torch.cuda.synchronize()
    say("long backward done, checking sampled heads against the oracle")
    for b, h in sampled_heads(wl.B, wl.H):
        g = torch.tensor([gs[h]], dtype=torch.float32)
        first = lambda t: t[b:b + 1, h:h + 1, :W]
        last = lambda t: t[b:b + 1, h:h + 1, T - W:]
        head = oracle.recurrent_backward(first(q), first(k), first(v), g, first(dy), s0[b:b + 1, h:h + 1], None)
        check(f"grad_q first {W} (b{b} h{h})", first(got[0]), head[0], 2e-2)
        tail = oracle.recurrent_backward(last(q), last(k), last(v), g, last(dy), None, ds[b:b + 1, h:h + 1])
        check(f"grad_k last {W} (b{b} h{h})", last(got[1]), tail[1], 2e-2)
        check(f"grad_v last {W} (b{b} h{h})", last(got[2]), tail[2], 2e-2)
    # A window in the middle, inside a segment of the GPU's split and not on a
    # chunk boundary, against the oracle alone: the oracle's forward over the
    # prefix gives the state entering the window (dQ there depends on it), and
    # the oracle's backward over the suffix gives the gradient that reaches the
    # window's last state from every later token and grad_state_out (its
    # grad_state_in); the window's own backward from those two is then exact.
    t0 = T // 2 + 3 * wl.C + 37
    t1 = t0 + W
    hl = [h for _, h in sampled_heads(wl.B, wl.H)]
    gh = torch.tensor([gs[h] for h in hl], dtype=torch.float32)
    sel = lambda t, lo, hi: t[:, hl, lo:hi].contiguous()
    say(f"long backward: oracle forward over the prefix [0, {t0}) and backward over the suffix [{t1}, {T})")
    _, s_t0 = oracle.chunkwise(sel(q, 0, t0), sel(k, 0, t0), sel(v, 0, t0), gh, wl.C, state_in=s0[:, hl])
    carry = oracle.recurrent_backward(sel(q, t1, T), sel(k, t1, T), sel(v, t1, T), gh, sel(dy, t1, T), None,
                                      ds[:, hl])[3]
    win = oracle.recurrent_backward(sel(q, t0, t1), sel(k, t0, t1), sel(v, t0, t1), gh, sel(dy, t0, t1), s_t0, carry)
    for i, name in enumerate(("grad_q", "grad_k", "grad_v")):
        check(f"{name} window [{t0}, {t1}) (heads {hl})", got[i][:, hl, t0:t1], win[i], 2e-2)
    t = T // 2 + 1000  # not a segment boundary of either part
    part = lambda x, lo, hi: x[:, :, lo:hi].contiguous()
    _, s_mid = ret.chunkwise_fwd(part(qd, 0, t), part(kd, 0, t), part(vd, 0, t), gs, wl.C, state_in=sd)
    g2 = ret.chunkwise_bwd(part(qd, t, T), part(kd, t, T), part(vd, t, T), gs, wl.C, part(dyd, t, T),
                           state_in=s_mid, grad_state_out=dsd)
    g1 = ret.chunkwise_bwd(part(qd, 0, t), part(kd, 0, t), part(vd, 0, t), gs, wl.C, part(dyd, 0, t),
                           state_in=sd, grad_state_out=g2[3])
    torch.cuda.synchronize()
    for i, name in enumerate(("grad_q", "grad_k", "grad_v")):
        check(f"split {name}", torch.cat([g1[i], g2[i]], dim=2), got[i], 2e-2)
    check("split grad_state_in", g1[3], got[3], 2e-2)


def test_largest_supported_tensors():
    """The largest tensors the ABI accepts at dk 256, dv 512: B1 H63 T65536, so v,
    y and the value gradient hold 2.11e9 elements (over 4 GB of bf16; byte
    offsets pass 2^32).  Forward, backward and GroupNorm on the GPU; the last
    head (largest offsets) against the oracle: y and the state in full, dQ of
    the first W tokens and dK, dV of the last W, GroupNorm on its last rows.
    Inputs come from a seeded generator on the GPU; the checked head is copied
    to the host for the oracle."""
    B, H, T, dk, dv, C, W = 1, 63, 65536, 256, 512, 64, 256
    assert B * H * T * dv < 2 ** 31
    say(f"largest tensors: B{B} H{H} T{T} dk{dk} dv{dv}")
    gen = torch.Generator(device=DEV).manual_seed(47)
    rnd = lambda d, scale: (torch.randn(B, H, T, d, device=DEV, generator=gen) * scale).to(torch.bfloat16)
    q, k = rnd(dk, dk ** -0.5), rnd(dk, dk ** -0.5)
    v = rnd(dv, dk ** -0.5)
    gs = [1 - 2 ** (-5 - 8 * h / H) for h in range(H)]
    y, s = ret.chunkwise_fwd(q, k, v, gs, C)
    torch.cuda.synchronize()
    h = H - 1
    g = torch.tensor([gs[h]], dtype=torch.float32)
    head = lambda t: t[:, h:h + 1].cpu()
    qh, kh, vh = head(q), head(k), head(v)
    say("largest tensors: forward done, oracle on the last head")
    y_ref, s_ref = oracle.chunkwise(qh, kh, vh, g, C)
    check("y (last head)", head(y), y_ref, 2e-2)
    check("state (last head)", head(s), s_ref, 2e-2)
    out = ret.group_norm(y)
    torch.cuda.synchronize()
    check("group norm (last head, last rows)", head(out)[:, :, -W:], oracle.group_norm(head(y)[:, :, -W:], None, None,
                                                                                      1e-5), 2e-2)
    del out, s
    dy = rnd(dv, 1.0)
    got = ret.chunkwise_bwd(q, k, v, gs, C, dy, grad_state_in=False)
    torch.cuda.synchronize()
    say("largest tensors: backward done")
    dyh = head(dy)
    first = oracle.recurrent_backward(qh[:, :, :W], kh[:, :, :W], vh[:, :, :W], g, dyh[:, :, :W])
    check("grad_q first tokens (last head)", head(got[0])[:, :, :W], first[0], 2e-2)
    last = oracle.recurrent_backward(qh[:, :, -W:], kh[:, :, -W:], vh[:, :, -W:], g, dyh[:, :, -W:])
    check("grad_k last tokens (last head)", head(got[1])[:, :, -W:], last[1], 2e-2)
    check("grad_v last tokens (last head)", head(got[2])[:, :, -W:], last[2], 2e-2)


@pytest.mark.timeout(600)
def test_full_size_decode_1000_steps_every_head():
    """The decode workload (batch 128, H 16, fp32 256x512 state, 1000 chained
    steps) on the GPU; every head against the oracle.  The oracle side uses the
    identity of the recurrent and chunkwise forms: 1000 decode steps from S0
    equal one chunkwise pass over the 1000 stacked tokens with state_in = S0
    (the oracle's own tests pin that identity), run in batch slices."""
    wl = WORKLOADS["decode"]
    say(f"full decode: {wl.description}")
    q, k, v, s0 = make_decode_inputs(wl.B, wl.H, wl.dk, wl.dv, wl.steps, wl.dtype, seed=0)
    qd, kd, vd = to_dev(q, k, v)
    state = s0.to(DEV)
    ys = torch.empty(wl.steps, wl.B, wl.H, wl.dv, dtype=qd.dtype, device=DEV)
    g = list(wl.gammas)
    for n in range(wl.steps):
        ret.recurrent_step(qd[n], kd[n], vd[n], g, state, y=ys[n])
    torch.cuda.synchronize()
    del qd, kd, vd
    say("decode: 1000 steps done, checking every head against the oracle")
    ty, ts = WholeTensor("decode y (1000 steps, every head)"), WholeTensor("decode final state (every head)")
    gt = torch.tensor(wl.gammas, dtype=torch.float32)
    bs = 8
    for b0 in range(0, wl.B, bs):
        stack = lambda t: t[:, b0:b0 + bs].permute(1, 2, 0, 3).contiguous()   # [b, H, steps, d]
        y_ref, s_ref = oracle.chunkwise(stack(q), stack(k), stack(v), gt, 100, state_in=s0[b0:b0 + bs])
        ty.add(ys[:, b0:b0 + bs].permute(1, 2, 0, 3), y_ref)
        ts.add(state[b0:b0 + bs], s_ref, rows=False)
    ty.check(2e-2, ROW_OWN_BOUND, ROW_RMS_BOUND)
    ts.check(2e-2)
