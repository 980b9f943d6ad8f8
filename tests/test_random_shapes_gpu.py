"""Seeded sweep of random shapes through every entry point on the GPU.

Each case draws a shape from the sets the kernels dispatch on (MFMA-sized
d_k/d_v and odd ones, T around the 16/32-token and chunk boundaries, one or
two heads past the 128-head launch groups), a dtype, decays including 0 and 1,
and which states are present, then compares the library with the fp64 oracle
at the dtype's bound.  The case list is a pure function of the seed.
"""
import random

import pytest
import torch

import oracle
import retnet_retention_chunkwise_amd as ret
from retnet_retention_chunkwise_amd.workloads import make_inputs
from helpers import rel_l2, say, tol

pytestmark = pytest.mark.gpu

DEV = "cuda"
DKS = [16, 48, 64, 128, 256]
DVS = [16, 40, 64, 128, 192, 256, 512]
TS = [1, 2, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100, 129, 200]
CS = [1, 8, 16, 32, 64, 100, 128]


def cases(n, seed):
    rnd = random.Random(seed)
    out = []
    for _ in range(n):
        dk, dv = rnd.choice(DKS), rnd.choice(DVS)
        H = rnd.choice([1, 2, 3, 129]) if dk * dv <= 64 * 64 else rnd.choice([1, 2, 3])
        B = rnd.choice([1, 2])
        T = rnd.choice(TS)
        C = rnd.choice(CS)
        dt = rnd.choice(["f32", "bf16"])
        gs = [rnd.choice([0.0, 1.0, rnd.uniform(0.3, 0.999)]) for _ in range(H)]
        out.append((B, H, T, dk, dv, C, dt, rnd.random() < 0.6, rnd.random() < 0.6, gs))
    return out


def check(name, got, want, bound):
    r = rel_l2(got, want)
    assert torch.isfinite(got.float()).all(), name
    assert r <= bound, (name, r)


@pytest.mark.parametrize("case", cases(24, 2026), ids=lambda c: "B{}H{}T{}dk{}dv{}C{}{}".format(*c[:7]))
def test_forward_random_shape(case):
    B, H, T, dk, dv, C, dt, with_in, with_out, gs = case
    say(f"forward {case[:9]}")
    q, k, v, s0 = make_inputs(B, H, T, dk, dv, dt, seed=70, with_state=True)
    s0 = s0 if with_in else None
    y_ref, s_ref = oracle.recurrent(q, k, v, torch.tensor(gs, dtype=torch.float64), s0)
    qd, kd, vd = q.to(DEV), k.to(DEV), v.to(DEV)
    sd = s0.to(DEV) if s0 is not None else None
    y, s = ret.chunkwise_fwd(qd, kd, vd, gs, C, state_in=sd, state_out=with_out)
    torch.cuda.synchronize()
    check("y", y, y_ref, tol(q.dtype))
    if with_out:
        check("state_out", s, s_ref, tol(q.dtype))


@pytest.mark.parametrize("case", cases(16, 2027), ids=lambda c: "B{}H{}T{}dk{}dv{}C{}{}".format(*c[:7]))
def test_backward_random_shape(case):
    B, H, T, dk, dv, C, dt, with_in, with_dout, gs = case
    say(f"backward {case[:9]}")
    q, k, v, s0 = make_inputs(B, H, T, dk, dv, dt, seed=71, with_state=True)
    _, _, dy, ds = make_inputs(B, H, T, dk, dv, dt, seed=72, with_state=True)
    s0 = s0 if with_in else None
    ds = ds if with_dout else None
    ref = oracle.recurrent_backward(q, k, v, torch.tensor(gs, dtype=torch.float64), dy, s0, ds)
    dev = lambda t: None if t is None else t.to(DEV)
    got = ret.chunkwise_bwd(dev(q), dev(k), dev(v), gs, C, dev(dy), state_in=dev(s0), grad_state_out=dev(ds))
    torch.cuda.synchronize()
    for name, g, r in zip(("grad_q", "grad_k", "grad_v", "grad_state_in"), got, ref):
        check(name, g, r, tol(q.dtype))


def long_cases(n, seed):
    """bf16 MFMA shapes with few (batch, head, column-tile) walkers over long
    sequences, so that calls run in sequence segments (state-only launch over
    sub-segments, scan, full launch) with random segment and sub-segment
    counts, chunk lengths and decays."""
    rnd = random.Random(seed)
    out = []
    for _ in range(n):
        dk, dv = rnd.choice([64, 128, 256]), rnd.choice([64, 128, 256, 512])
        H, B = rnd.choice([1, 2, 3]), rnd.choice([1, 2])
        T = rnd.randint(900, 4200)
        C = rnd.choice([16, 32, 48, 64, 100, 128])
        gs = [rnd.choice([0.0, 0.2, 1.0, rnd.uniform(0.5, 0.999)]) for _ in range(H)]
        out.append((B, H, T, dk, dv, C, "bf16", rnd.random() < 0.7, rnd.random() < 0.7, gs))
    return out


@pytest.mark.parametrize("case", long_cases(8, 2029), ids=lambda c: "B{}H{}T{}dk{}dv{}C{}".format(*c[:6]))
def test_segmented_random_shape(case):
    B, H, T, dk, dv, C, dt, with_in, with_dout, gs = case
    say(f"segmented forward + backward {case[:9]}")
    q, k, v, s0 = make_inputs(B, H, T, dk, dv, dt, seed=74, with_state=True)
    _, _, dy, ds = make_inputs(B, H, T, dk, dv, dt, seed=75, with_state=True)
    s0 = s0 if with_in else None
    ds = ds if with_dout else None
    g64 = torch.tensor(gs, dtype=torch.float64)
    y_ref, s_ref = oracle.recurrent(q, k, v, g64, s0)
    ref = oracle.recurrent_backward(q, k, v, g64, dy, s0, ds)
    dev = lambda t: None if t is None else t.to(DEV)
    y, s = ret.chunkwise_fwd(dev(q), dev(k), dev(v), gs, C, state_in=dev(s0))
    got = ret.chunkwise_bwd(dev(q), dev(k), dev(v), gs, C, dev(dy), state_in=dev(s0), grad_state_out=dev(ds))
    torch.cuda.synchronize()
    check("y", y, y_ref, tol(q.dtype))
    check("state_out", s, s_ref, tol(q.dtype))
    for name, g, r in zip(("grad_q", "grad_k", "grad_v", "grad_state_in"), got, ref):
        check(name, g, r, tol(q.dtype))


@pytest.mark.parametrize("case", cases(12, 2028), ids=lambda c: "B{}H{}T{}dv{}{}".format(c[0], c[1], c[2], c[4], c[6]))
def test_group_norm_random_shape(case):
    B, H, T, _, dv, _, dt, affine, in_place, _ = case
    say(f"group norm B{B} H{H} T{T} dv{dv} {dt}")
    gen = torch.Generator().manual_seed(73)
    y = (torch.randn(B, H, T, dv, generator=gen) * 3 - 1).to(torch.bfloat16 if dt == "bf16" else torch.float32)
    w = torch.randn(H, dv, generator=gen) if affine else None
    b = torch.randn(H, dv, generator=gen) if affine else None
    ref = oracle.group_norm(y, w, b, 1e-5)
    yd = y.to(DEV)
    out = ret.group_norm(yd, None if w is None else w.to(DEV), None if b is None else b.to(DEV), 1e-5,
                         out=yd if in_place else None)
    torch.cuda.synchronize()
    check("group norm", out, ref, tol(y.dtype))


@pytest.mark.parametrize("case", cases(16, 2028), ids=lambda c: "B{}H{}T{}dk{}dv{}C{}{}".format(*c[:7]))
def test_fused_group_norm_random_shape(case):
    """The forward with the per-head GroupNorm fused in (or, for shapes the
    fused kernel does not take, the forward followed by the standalone pass)
    against the oracle's GroupNorm of the oracle's output."""
    B, H, T, dk, dv, C, dt, with_in, affine, gs = case
    say(f"fused group norm {case[:9]}")
    q, k, v, s0 = make_inputs(B, H, T, dk, dv, dt, seed=73, with_state=True)
    s0 = s0 if with_in else None
    gen = torch.Generator().manual_seed(74)
    w, b = (torch.randn(H, dv, generator=gen), torch.randn(H, dv, generator=gen)) if affine else (None, None)
    y_ref, _ = oracle.recurrent(q, k, v, torch.tensor(gs, dtype=torch.float64), s0)
    ref = oracle.group_norm(y_ref, w, b, 1e-5)
    dev = lambda t: None if t is None else t.to(DEV)
    y, _ = ret.chunkwise_fwd_group_norm(dev(q), dev(k), dev(v), gs, C, dev(w), dev(b), 1e-5, state_in=dev(s0),
                                        state_out=False)
    torch.cuda.synchronize()
    check("y", y, ref, tol(q.dtype))
