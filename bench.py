"""Benchmark of the retention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline] [--only a,b,...]

A step is one chunkwise retention forward (retention_chunkwise_fwd: intra-chunk
(Q K^T .* D) V, cross-chunk Q R gamma^(j+1), state update, fp32 state carried
across every chunk and written out at the end) over one batch of the
long-context workload: B=1, H=8, T=65536, d_k=256, d_v=512, bf16, C=128
(512 chunks), gamma_h = 1 - 2^(-5-h), seeded synthetic inputs.  It is the
largest single-GPU configuration; with only 64 (head, 64-column) walkers it
runs in sequence segments (a state-only pass over the earlier segments, a scan
of their end states, and the full pass), and the timed call is that whole
sequence of launches.  Inputs are resident in HBM before timing; one input set
(1.61 GB, six times the 256 MB last-level cache) is read cold by every step.

Measured in the same run, each in an object of its own with its roofline:
  layer6p7b    chunkwise B2 H16 T8192 C=128 (805 MB, one input set)
  layer1p3b    chunkwise B4 H8 T2048 C=64 (201 MB, four rotating input sets)
  decode       1000 chained recurrent steps, batch 128, H16, fp32 state
  continuation 16 (and 32, 64) new tokens per decode stream from the carried state
  backward     dQ, dK, dV, dS_in of the layer1p3b workload
  group_norm   per-head GroupNorm of a layer1p3b output

Prints ONE JSON line.  "value" is whole-job throughput over the K timed steps,
issued as one captured HIP graph and replayed (the launches back to back);
the eager loop's time, host work included, is "ms_per_step_eager".  The
roofline of a chunkwise call uses algorithmic HBM bytes (bf16 Q, K, V in and
Y out: 3072 bytes per head-token, plus the fp32 final state) over the call's
duration in that replay, timed with HIP events on the launch stream.
"""
import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "retnet_retention_chunkwise_amd", "csrc")
SECTIONS = ("long64k", "layer6p7b", "layer1p3b", "decode", "continuation", "backward", "group_norm")


def head_token_flops(dk, dv, C):
    # two d_k x d_v contractions (cross term, state update) + causal intra-chunk
    # Q K^T and P V: 4 dk dv + (C+1)(dk+dv) flops per head-token
    return 4 * dk * dv + (C + 1) * (dk + dv)


def source_digest(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(name, kernel_src):
    """HBM bytes per launch (or call) from committed rocprofv3 counter runs
    (FETCH_SIZE + WRITE_SIZE, copy-calibrated), if they were taken on the
    current kernel source; else None."""
    from retnet_retention_chunkwise_amd.rocprof_summary import read_traffic_file

    p = os.path.join(PROFILES, name)
    if not os.path.exists(p):
        return None
    rec = read_traffic_file(p)
    if rec.get("kernel_source_sha256_16") != source_digest(kernel_src):
        return None
    try:
        return float(rec["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def load_mfma_counters(name, kernel_src):
    """Executed bf16 MFMA share and MFMA-busy share of a kernel from a committed
    rocprofv3 counter summary (SQ_INSTS_VALU_MFMA_MOPS_BF16,
    SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE), if it was taken on the current
    kernel source; else None."""
    from retnet_retention_chunkwise_amd.rocprof_summary import read_traffic_file

    p = os.path.join(PROFILES, name)
    if not os.path.exists(p):
        return None
    rec = read_traffic_file(p)
    if rec.get("kernel_source_sha256_16") != source_digest(kernel_src):
        return None
    try:
        frac_key = next(k for k in rec if k.startswith("executed_mfma_frac"))
        return {"profile": name, "kernel": rec["kernel"],
                "executed_mfma_frac": float(rec[frac_key]),
                "executed_bf16_mfma_tflops": float(rec["executed_bf16_mfma_tflops"].split()[0]),
                "mfma_busy_frac": float(rec["mfma_busy_frac"].split()[0])}
    except (KeyError, ValueError, StopIteration):
        return None


def host_cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown CPU"


def cpu_baseline_chunkwise(wl, sample_B, sample_T):
    """The fp64 oracle (recurrent form) on a bounded sample: the first sample_B
    batch elements, all heads, the first sample_T tokens.  Returns tokens/s in
    the GPU metric's unit (a token counts once across all heads)."""
    import torch

    import oracle
    from retnet_retention_chunkwise_amd.workloads import make_inputs

    q, k, v = make_inputs(sample_B, wl.H, sample_T, wl.dk, wl.dv, wl.dtype, seed=0)
    g = torch.tensor(wl.gammas, dtype=torch.float32)
    t0 = time.perf_counter()
    oracle.recurrent(q, k, v, g)
    dt = time.perf_counter() - t0
    cores = torch.get_num_threads()
    return {
        "value": sample_B * sample_T / dt, "unit": "tokens/s", "cores": cores, "kind": "oracle",
        "sample": f"fp64 recurrent-form oracle on {sample_B} of {wl.B} batch elements x all {wl.H} heads x "
                  f"{sample_T} of {wl.T} tokens of the {wl.key} workload: {dt:.1f} s on {cores} threads "
                  f"of {host_cpu_model()}",
    }


def cpu_baseline_decode(wl, n_steps, n_batch):
    import torch

    import oracle
    from retnet_retention_chunkwise_amd.workloads import make_decode_inputs

    q, k, v, s0 = make_decode_inputs(n_batch, wl.H, wl.dk, wl.dv, n_steps, wl.dtype, seed=0)
    g = torch.tensor(wl.gammas, dtype=torch.float32)
    S = s0
    t0 = time.perf_counter()
    for n in range(n_steps):
        _, S = oracle.recurrent_step(q[n], k[n], v[n], g, S)
    dt = time.perf_counter() - t0
    cores = torch.get_num_threads()
    # steps/s of the full batch: the sample covers n_batch of wl.B sequences
    return {
        "value": n_steps / dt * n_batch / wl.B, "unit": "steps/s", "cores": cores, "kind": "oracle",
        "sample": f"fp64 oracle decode steps, {n_batch} of {wl.B} sequences x {wl.H} heads, {n_steps} steps "
                  f"({dt:.1f} s on {cores} threads of {host_cpu_model()}), scaled to the full batch",
    }


def graph_time_ms(fn, n, stream):
    """fn(i) for i in 0..n-1 captured in one HIP graph, replayed once untimed and
    once timed; returns ms per call of the timed replay."""
    import torch

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(n):
            fn(i)
    graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    del graph
    return e0.elapsed_time(e1) / n


def eager_time_ms(fn, n, stream):
    """fn(i) issued eagerly n times: (ms per call over the whole loop, median ms
    of the per-call event pairs, which also hold each call's dispatch)."""
    import torch

    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    e0.record(stream)
    for i in range(n):
        ev[i][0].record(stream)
        fn(i)
        ev[i][1].record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n, statistics.median(a.elapsed_time(b) for a, b in ev)


CHUNKWISE_TRAFFIC = {
    "long64k": "chunkwise_mfma_long64k_traffic.txt",
    "layer6p7b": "chunkwise_mfma_layer6p7b_traffic.txt",
    "layer1p3b": "chunkwise_mfma_layer1p3b_traffic.txt",
}


def bench_chunkwise(key, dev, steps, warmup, n_rot):
    """One chunkwise workload: every call writes y and the fp32 final state
    (state_out), with the workspace preallocated; returns its bench object."""
    import torch

    import retnet_retention_chunkwise_amd as ret
    from retnet_retention_chunkwise_amd.workloads import WORKLOADS, make_inputs

    wl = WORKLOADS[key]
    sets = []
    for r in range(n_rot):
        q, k, v = make_inputs(wl.B, wl.H, wl.T, wl.dk, wl.dv, wl.dtype, seed=r)
        sets.append((q.to(dev), k.to(dev), v.to(dev)))
        del q, k, v
    y = torch.empty(wl.B, wl.H, wl.T, wl.dv, dtype=sets[0][0].dtype, device=dev)
    st = torch.empty(wl.B, wl.H, wl.dk, wl.dv, dtype=torch.float32, device=dev)
    need = ret.chunkwise_workspace_bytes(wl.B, wl.H, wl.T, wl.dk, wl.dv, wl.C, y.dtype)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev) if need else None
    g = list(wl.gammas)

    def call(i):
        qd, kd, vd = sets[i % n_rot]
        ret.chunkwise_fwd(qd, kd, vd, g, wl.C, y=y, state_out=st, workspace=ws)

    stream = torch.cuda.current_stream(dev)  # the stream the library launches on
    for i in range(warmup):
        call(i)
    torch.cuda.synchronize()
    ms_eager, ms_pairs = eager_time_ms(call, steps, stream)
    ms = graph_time_ms(call, steps, stream)
    head_tokens = wl.B * wl.H * wl.T
    state_bytes = wl.B * wl.H * wl.dk * wl.dv * 4
    alg_bytes = head_tokens * (2 * wl.dk + 2 * wl.dk + 2 * wl.dv + 2 * wl.dv) + state_bytes
    alg_flops = head_tokens * head_token_flops(wl.dk, wl.dv, wl.C)
    gbs = alg_bytes / (ms * 1e-3) / 1e9
    tflops = alg_flops / (ms * 1e-3) / 1e12
    traffic = load_traffic(CHUNKWISE_TRAFFIC[key], os.path.join(CSRC, "chunkwise_mfma.hip"))
    counters = load_mfma_counters(f"chunkwise_fwd_{key}_mfma_counters.txt", os.path.join(CSRC, "chunkwise_mfma.hip"))
    segs = "one launch" if not need else "state-only pass + segment scan + full pass (one call)"
    gn = bench_fused_group_norm(wl, sets, y, st, ws, steps, warmup, stream, ms, alg_bytes)
    del sets, y, st, ws
    torch.cuda.empty_cache()
    return {
        "workload": f"{key}: chunkwise fwd B={wl.B} H={wl.H} T={wl.T} dk={wl.dk} dv={wl.dv} bf16 C={wl.C}, "
                    f"gamma per head as the workload states, fp32 state carried across {wl.T // wl.C} chunks "
                    f"and written out",
        "tokens_per_s": wl.B * wl.T / (ms * 1e-3),
        "ms_per_step": ms,
        "ms_per_step_eager": ms_eager,
        "input_sets": n_rot,
        "roofline": {
            "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
            "traffic": traffic, "kernel": f"retention_chunkwise_fwd call: {segs}",
            "kernel_us": ms * 1e3, "kernel_us_event_pairs": ms_pairs * 1e3,
            "algorithmic_bytes_per_launch": alg_bytes, "algorithmic_flops_per_launch": alg_flops,
            "mfma_tflops": tflops, "mfma_frac": tflops / BF16_PEAK_TFLOPS,
            "mfma_counters": counters,
        },
        "group_norm_fused": gn,
    }


def bench_fused_group_norm(wl, sets, y, st, ws, steps, warmup, stream, ms_fwd, fwd_bytes):
    """The same workload with the per-head GroupNorm (affine) of its output:
    the fused call (retention_chunkwise_fwd_group_norm) against the forward
    followed by retention_group_norm in place, both as graph replays over the
    same rotating input sets."""
    import torch

    import retnet_retention_chunkwise_amd as ret

    gen = torch.Generator().manual_seed(7)
    w = torch.randn(wl.H, wl.dv, generator=gen).to(y.device)
    b = torch.randn(wl.H, wl.dv, generator=gen).to(y.device)
    lib = ret.load()
    need = int(lib.retention_chunkwise_fwd_group_norm_workspace_bytes(wl.B, wl.H, wl.T, wl.dk, wl.dv, wl.C, 1))
    wsf = torch.empty(max(need, 16), dtype=torch.uint8, device=y.device)
    g = list(wl.gammas)
    n_rot = len(sets)

    def fused(i):
        qd, kd, vd = sets[i % n_rot]
        ret.chunkwise_fwd_group_norm(qd, kd, vd, g, wl.C, w, b, 1e-5, y=y, state_out=st, workspace=wsf)

    def separate(i):
        qd, kd, vd = sets[i % n_rot]
        ret.chunkwise_fwd(qd, kd, vd, g, wl.C, y=y, state_out=st, workspace=ws)
        ret.group_norm(y, w, b, 1e-5, out=y)

    for i in range(warmup):
        fused(i)
    torch.cuda.synchronize()
    ms_fused = graph_time_ms(fused, steps, stream)
    err = int(wsf[:4].view(torch.int32).item())
    for i in range(warmup // 4):
        separate(i)
    torch.cuda.synchronize()
    ms_sep = graph_time_ms(separate, steps, stream)
    alg = fwd_bytes + 2 * wl.H * wl.dv * 4
    gbs = alg / (ms_fused * 1e-3) / 1e9
    traffic = load_traffic(f"chunkwise_fused_group_norm_{wl.key}_traffic.txt", os.path.join(CSRC, "chunkwise_mfma.hip"))
    return {
        "workload": "the same call with the per-head GroupNorm (affine weight and bias, eps 1e-5) of its output",
        "fused_us": ms_fused * 1e3, "forward_then_group_norm_us": ms_sep * 1e3, "forward_alone_us": ms_fwd * 1e3,
        "fused_extra_us": (ms_fused - ms_fwd) * 1e3, "separate_extra_us": (ms_sep - ms_fwd) * 1e3,
        "wait_gave_up": err,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": traffic, "algorithmic_bytes_per_launch": alg},
    }


def bench_decode(dev, decode_steps):
    import torch

    import retnet_retention_chunkwise_amd as ret
    from retnet_retention_chunkwise_amd.workloads import WORKLOADS, make_decode_inputs

    dw = WORKLOADS["decode"]
    dq, dk_, dv_, s0 = make_decode_inputs(dw.B, dw.H, dw.dk, dw.dv, decode_steps, dw.dtype, seed=0)
    dq, dk_, dv_ = dq.to(dev), dk_.to(dev), dv_.to(dev)
    state = s0.to(dev)
    ydec = torch.empty(dw.B, dw.H, dw.dv, dtype=dq.dtype, device=dev)
    gd = list(dw.gammas)
    stream = torch.cuda.current_stream(dev)
    for n in range(10):  # warm-up steps (the state keeps evolving; the timed steps continue from it)
        ret.recurrent_step(dq[n % decode_steps], dk_[n % decode_steps], dv_[n % decode_steps], gd, state, y=ydec)
    torch.cuda.synchronize()
    ms_loop, ms_pairs = eager_time_ms(lambda n: ret.recurrent_step(dq[n], dk_[n], dv_[n], gd, state, y=ydec),
                                      decode_steps, stream)
    kernel_us = ms_pairs * 1e3
    state_bytes = dw.B * dw.H * dw.dk * dw.dv * 4
    dec_bytes = 2 * state_bytes + dw.B * dw.H * (2 * dw.dk + 2 * dw.dk + 2 * dw.dv + 2 * dw.dv)
    gbs = dec_bytes / (kernel_us * 1e-6) / 1e9
    traffic = load_traffic("recurrent_step_decode_traffic.txt", os.path.join(CSRC, "recurrent_step.hip"))
    del dq, dk_, dv_, state
    torch.cuda.empty_cache()
    return {
        "workload": f"recurrent step: batch 128, H=16, fp32 state 256x512 per head, bf16 q/k/v, "
                    f"{decode_steps} chained steps",
        "steps_per_s": 1e3 / ms_loop,
        "us_per_step": ms_loop * 1e3,
        "kernel_us": kernel_us,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": traffic, "algorithmic_bytes_per_launch": dec_bytes},
    }


def bench_continuation(dev, tokens=(16, 32, 64)):
    """chunkwise on T new tokens per stream from the decode state, in place,
    for each T in tokens (the bf16 MFMA streaming kernel); the first T is the
    object's own figure, every T is listed in "by_tokens"."""
    import torch

    import retnet_retention_chunkwise_amd as ret
    from retnet_retention_chunkwise_amd.workloads import WORKLOADS, make_decode_inputs, make_inputs

    dw = WORKLOADS["decode"]
    *_, s0 = make_decode_inputs(dw.B, dw.H, dw.dk, dw.dv, 1, dw.dtype, seed=0)
    cstate = s0.to(dev)
    gd = list(dw.gammas)
    stream = torch.cuda.current_stream(dev)
    state_bytes = dw.B * dw.H * dw.dk * dw.dv * 4
    rows = []
    for ct in tokens:
        cq, ck, cv = (t.to(dev) for t in make_inputs(dw.B, dw.H, ct, dw.dk, dw.dv, dw.dtype, seed=1))
        cy = torch.empty(dw.B, dw.H, ct, dw.dv, dtype=cq.dtype, device=dev)
        call = lambda i: ret.chunkwise_fwd(cq, ck, cv, gd, ct, state_in=cstate, state_out=cstate, y=cy)
        for i in range(3):
            call(i)
        torch.cuda.synchronize()
        _, ms_pairs = eager_time_ms(call, 20, stream)
        us = ms_pairs * 1e3
        nbytes = 2 * state_bytes + dw.B * dw.H * ct * (2 * dw.dk + 2 * dw.dk + 2 * dw.dv + 2 * dw.dv)
        rows.append({"tokens": ct, "kernel_us": us, "tokens_per_s": dw.B * ct / (us * 1e-6),
                     "achieved_gbs": nbytes / (us * 1e-6) / 1e9, "algorithmic_bytes_per_launch": nbytes})
        del cq, ck, cv, cy
    del cstate
    torch.cuda.empty_cache()
    h = rows[0]
    traffic = load_traffic(f"short_bf16_continuation{h['tokens']}_traffic.txt", os.path.join(CSRC, "short_bf16.hip"))
    return {
        "workload": f"chunkwise fwd on {h['tokens']} new tokens per stream from a carried state, in place: batch 128, "
                    "H=16, fp32 state 256x512 per head, bf16 q/k/v (also 32 and 64 tokens in by_tokens)",
        "tokens_per_s": h["tokens_per_s"],
        "kernel_us": h["kernel_us"],
        "roofline": {"bound": "hbm", "achieved": h["achieved_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": h["achieved_gbs"] / HBM_PEAK_GBS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": h["algorithmic_bytes_per_launch"]},
        "by_tokens": rows,
    }


def bench_backward(dev):
    """gradients of the layer1p3b forward: dQ, dK, dV and dS_in from dY and dS_out;
    3 rotating input sets (about 270 MB each, together larger than the GPU's
    256 MB last-level cache)"""
    import torch

    import retnet_retention_chunkwise_amd as ret
    from retnet_retention_chunkwise_amd.workloads import WORKLOADS, make_inputs

    wl = WORKLOADS["layer1p3b"]
    bsets = []
    for r in range(3):
        bq, bk, bv, bs0 = make_inputs(wl.B, wl.H, wl.T, wl.dk, wl.dv, wl.dtype, seed=7 + 2 * r, with_state=True)
        _, _, bdy, bds = make_inputs(wl.B, wl.H, wl.T, wl.dk, wl.dv, wl.dtype, seed=8 + 2 * r, with_state=True)
        bsets.append(tuple(t.to(dev) for t in (bq, bk, bv, bs0, bdy, bds)))
    g = list(wl.gammas)

    def call(i):
        bq, bk, bv, bs0, bdy, bds = bsets[i % len(bsets)]
        ret.chunkwise_bwd(bq, bk, bv, g, wl.C, bdy, state_in=bs0, grad_state_out=bds)

    stream = torch.cuda.current_stream(dev)
    for i in range(12):
        call(i)
    torch.cuda.synchronize()
    _, ms_pairs = eager_time_ms(call, 21, stream)
    us = graph_time_ms(call, 21, stream) * 1e3
    head_tokens = wl.B * wl.H * wl.T
    tokens = wl.B * wl.T
    nbytes = head_tokens * (2 * wl.dk * 2 + 2 * wl.dv * 2 + 2 * wl.dk * 2 + wl.dv * 2)  # q,k,v,dy in; dq,dk,dv out
    flops = 3 * head_tokens * head_token_flops(wl.dk, wl.dv, wl.C)  # three chunkwise passes
    traffic = load_traffic("chunkwise_mfma_bwd_passes_layer1p3b_traffic.txt", os.path.join(CSRC, "chunkwise_mfma.hip"))
    del bsets
    torch.cuda.empty_cache()
    gbs = nbytes / (us * 1e-6) / 1e9
    tf = flops / (us * 1e-6) / 1e12
    return {
        "workload": "chunkwise backward (dQ, dK, dV, dS_in) of the layer1p3b workload: B=4 H=8 T=2048 dk=256 "
                    "dv=512 bf16 C=64, with state_in and grad_state_out, 3 rotating input sets",
        "tokens_per_s": tokens / (us * 1e-6),
        "kernel_us": us,
        "kernel_us_event_pairs": ms_pairs * 1e3,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": traffic, "algorithmic_bytes_per_launch": nbytes,
                     "algorithmic_flops_per_launch": flops, "mfma_tflops": tf, "mfma_frac": tf / BF16_PEAK_TFLOPS},
    }


def bench_group_norm(dev):
    import torch

    import retnet_retention_chunkwise_amd as ret
    from retnet_retention_chunkwise_amd.workloads import WORKLOADS

    wl = WORKLOADS["layer1p3b"]
    gy = [torch.randn(wl.B, wl.H, wl.T, wl.dv, device=dev).to(torch.bfloat16) for _ in range(4)]
    gw = torch.randn(wl.H, wl.dv, device=dev)
    gb = torch.randn(wl.H, wl.dv, device=dev)
    gout = torch.empty_like(gy[0])
    stream = torch.cuda.current_stream(dev)
    call = lambda i: ret.group_norm(gy[i % 4], gw, gb, 1e-5, out=gout)
    for i in range(200):  # steady clocks
        call(i)
    torch.cuda.synchronize()
    _, ms_pairs = eager_time_ms(call, 20, stream)
    us = graph_time_ms(call, 100, stream) * 1e3
    head_tokens = wl.B * wl.H * wl.T
    nbytes = 2 * head_tokens * wl.dv * 2 + 2 * wl.H * wl.dv * 4  # y in, out out (bf16); weight, bias
    traffic = load_traffic("group_norm_layer1p3b_traffic.txt", os.path.join(CSRC, "group_norm.hip"))
    del gy, gw, gb, gout
    torch.cuda.empty_cache()
    gbs = nbytes / (us * 1e-6) / 1e9
    return {
        "workload": "per-head GroupNorm of a layer1p3b output: [4,8,2048,512] bf16, affine weight/bias, 4 rotating inputs",
        "kernel_us": us,
        "kernel_us_event_pairs": ms_pairs * 1e3,
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs / HBM_PEAK_GBS, "traffic": traffic, "algorithmic_bytes_per_launch": nbytes},
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU needs ~30 ms of work to reach its steady clocks: the warm-up steps
    # come first (400 x ~0.6 ms for the headline workload)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", default="", help=f"comma-separated subset of {','.join(SECTIONS)} (profiling runs)")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (counter calibration under rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)
    only = [s for s in args.only.split(",") if s]
    for s in only:
        if s not in SECTIONS:
            print(f"unknown section {s!r}; choose from {', '.join(SECTIONS)}", file=sys.stderr)
            sys.exit(2)
    want = lambda s: not only or s in only

    import torch

    import retnet_retention_chunkwise_amd as ret
    from retnet_retention_chunkwise_amd.workloads import WORKLOADS

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    dev = torch.device("cuda:0")
    ret.load()
    if args.calibrate_copy_mib:
        n = args.calibrate_copy_mib * 1024 * 1024 // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = not args.no_cpu_baseline
    res = {}
    # long sequences need fewer steps for the same time: the headline runs
    # args.steps steps, the other chunkwise workloads scale theirs
    plan = {"long64k": (1, 1), "layer6p7b": (1, 2), "layer1p3b": (4, 8)}
    for key, (n_rot, mult) in plan.items():
        if want(key):
            res[key] = bench_chunkwise(key, dev, args.steps * mult, args.warmup * mult, n_rot)
            print(f"[bench] {key}: {res[key]['ms_per_step'] * 1e3:.1f} us per call", file=sys.stderr, flush=True)
    if want("decode"):
        res["decode"] = bench_decode(dev, args.decode_steps)
    if want("continuation"):
        res["continuation"] = bench_continuation(dev)
    if want("backward"):
        res["backward"] = bench_backward(dev)
    if want("group_norm"):
        res["group_norm"] = bench_group_norm(dev)
    if cpu:
        samples = {"long64k": (1, 65536), "layer6p7b": (1, 8192), "layer1p3b": (4, 2048)}
        for key, (sb, stt) in samples.items():
            if key in res:
                res[key]["cpu_baseline"] = cpu_baseline_chunkwise(WORKLOADS[key], sb, stt)
        if "decode" in res:
            res["decode"]["cpu_baseline"] = cpu_baseline_decode(WORKLOADS["decode"], 64, 16)

    head_key = "long64k" if "long64k" in res else next((k for k in plan if k in res), None)
    out = {
        "metric": "retention tokens/sec (chunkwise fwd) + decode steps/sec; % MFMA / HBM peak",
        "value": None, "unit": "tokens/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": None, "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)/sqrt(dk) bf16 q, k, v; the headline's one input set is 1.61 GB, "
                "read cold by every step)",
    }
    if head_key is not None:
        wl = WORKLOADS[head_key]
        h = res.pop(head_key)
        out["value"] = h["tokens_per_s"]
        out["ms_per_step"] = h["ms_per_step"]
        out["ms_per_step_eager"] = h["ms_per_step_eager"]
        out["config"] = {"workload": h["workload"], "global_batch": wl.B, "seq_len": wl.T,
                         "parallelism": "single GPU"}
        out["roofline"] = h["roofline"]
        out["group_norm_fused"] = h["group_norm_fused"]
        if "cpu_baseline" in h:
            out["cpu_baseline"] = h["cpu_baseline"]
    out.update(res)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
