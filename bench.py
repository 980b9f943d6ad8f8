"""Benchmark of the retention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]

A step is one chunkwise retention forward (retention_chunkwise_fwd: intra-chunk
(Q K^T .* D) V, cross-chunk Q R gamma^(j+1), state update, carried fp32 state)
over one batch of the 1.3B-scale layer workload: B=4, H=8, T=2048, d_k=256,
d_v=512, bf16, C=64, gamma_h = 1 - 2^(-5-h), seeded synthetic inputs.  Inputs
are resident in HBM before timing; four input sets rotate so that each step
reads cold data (one set, 201 MB, would fit in the 256 MB last-level cache).

The recurrent decode step (retention_recurrent_step, batch 128, H=16, fp32
256x512 state per head, 1000 chained steps) is measured in the same run and
reported in the "decode" object, and a chunkwise continuation of 16 new tokens
per stream from that state (the fp32-MFMA streaming kernel) in the
"continuation" object, the backward of the chunkwise workload in "backward"
and the per-head GroupNorm of its output in "group_norm".

Prints ONE JSON line.  "value" is whole-job throughput over the K timed steps,
issued as one captured HIP graph (the eager loop's time, host work included,
is "ms_per_step_eager").
The roofline of the chunkwise kernel uses algorithmic HBM bytes (bf16 Q, K, V
in and Y out: 3072 bytes per head-token) over the kernel's duration per launch
in the graph replay, timed with HIP events on the launch stream (the median of
per-launch event pairs around eager launches, which also hold each launch's
dispatch, is reported beside it).
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


def head_token_flops(dk, dv, C):
    # two d_k x d_v contractions (cross term, state update) + causal intra-chunk
    # Q K^T and P V: 4 dk dv + (C+1)(dk+dv) flops per head-token
    return 4 * dk * dv + (C + 1) * (dk + dv)


def source_digest(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(name, kernel_src):
    """HBM bytes per launch from committed rocprofv3 counter runs (FETCH_SIZE +
    WRITE_SIZE, copy-calibrated), if they were taken on the current kernel
    source; else None."""
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
    return sample_B * sample_T / dt, dt, torch.get_num_threads()


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
    # steps/s of the full batch: the sample covers n_batch of wl.B sequences
    return n_steps / dt * n_batch / wl.B, dt, torch.get_num_threads()


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU needs ~30 ms of work to reach its steady clocks: 400 warm-up steps
    # (~35 ms) before 200 timed ones (~17 ms)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB first (counter calibration under rocprofv3)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); the library has no multi-GPU path",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import retnet_retention_chunkwise_amd as ret
    from retnet_retention_chunkwise_amd.workloads import WORKLOADS, make_decode_inputs, make_inputs

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

    # ------------------------------------------------ chunkwise forward
    wl = WORKLOADS["layer1p3b"]
    n_rot = 4
    sets = []
    for r in range(n_rot):
        q, k, v = make_inputs(wl.B, wl.H, wl.T, wl.dk, wl.dv, wl.dtype, seed=r)
        sets.append((q.to(dev), k.to(dev), v.to(dev), torch.empty(wl.B, wl.H, wl.T, wl.dv, dtype=q.dtype, device=dev)))
    g = list(wl.gammas)
    for i in range(args.warmup):
        qd, kd, vd, yd = sets[i % n_rot]
        ret.chunkwise_fwd(qd, kd, vd, g, wl.C, y=yd, state_out=False)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)  # the stream the library launches on
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    # whole-job time over the timed region, and each launch bracketed by its own
    # event pair (the kernel's duration for the roofline)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    e0.record(stream)
    for i in range(args.steps):
        qd, kd, vd, yd = sets[i % n_rot]
        ev[i][0].record(stream)
        ret.chunkwise_fwd(qd, kd, vd, g, wl.C, y=yd, state_out=False)
        ev[i][1].record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step_eager = e0.elapsed_time(e1) / args.steps
    kernel_ms = statistics.median(a.elapsed_time(b) for a, b in ev)  # median launch duration
    # The same K steps captured once in a HIP graph and replayed: the launches
    # run back to back without the host's per-call work in between (the way a
    # serving or training loop would issue them).  One untimed replay first.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(args.steps):
            qd, kd, vd, yd = sets[i % n_rot]
            ret.chunkwise_fwd(qd, kd, vd, g, wl.C, y=yd, state_out=False)
    graph.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    del graph
    # kernel duration for the roofline: the graph replay's time per launch
    # (back-to-back launches; an event pair around one eager launch also holds
    # its dispatch, several us, reported as kernel_us_event_pairs)
    kernel_ms_pairs = kernel_ms
    kernel_ms = ms_per_step
    tokens = wl.B * wl.T
    value = tokens / (ms_per_step * 1e-3)
    head_tokens = wl.B * wl.H * wl.T
    alg_bytes = head_tokens * (2 * wl.dk + 2 * wl.dk + 2 * wl.dv + 2 * wl.dv)  # q, k, v in, y out (bf16)
    alg_flops = head_tokens * head_token_flops(wl.dk, wl.dv, wl.C)
    achieved_gbs = alg_bytes / (kernel_ms * 1e-3) / 1e9
    achieved_tflops = alg_flops / (kernel_ms * 1e-3) / 1e12
    kernel_src = os.path.join(ROOT, "retnet_retention_chunkwise_amd", "csrc", "chunkwise_mfma.hip")
    traffic = load_traffic("chunkwise_mfma_layer1p3b_traffic.txt", kernel_src)
    del sets
    torch.cuda.empty_cache()

    # ------------------------------------------------ recurrent decode
    dw = WORKLOADS["decode"]
    dq, dk_, dv_, s0 = make_decode_inputs(dw.B, dw.H, dw.dk, dw.dv, args.decode_steps, dw.dtype, seed=0)
    dq, dk_, dv_ = dq.to(dev), dk_.to(dev), dv_.to(dev)
    state = s0.to(dev)
    ydec = torch.empty(dw.B, dw.H, dw.dv, dtype=dq.dtype, device=dev)
    gd = list(dw.gammas)
    for n in range(10):  # warm-up steps (the state keeps evolving; the timed steps continue from it)
        m = n % args.decode_steps
        ret.recurrent_step(dq[m], dk_[m], dv_[m], gd, state, y=ydec)
    torch.cuda.synchronize()
    dev_ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(args.decode_steps)]
    e0.record(stream)
    for n in range(args.decode_steps):
        dev_ev[n][0].record(stream)
        ret.recurrent_step(dq[n], dk_[n], dv_[n], gd, state, y=ydec)
        dev_ev[n][1].record(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    dec_ms = e0.elapsed_time(e1)
    dec_kernel_us = statistics.median(a.elapsed_time(b) for a, b in dev_ev) * 1e3
    dec_us_step = dec_ms * 1e3 / args.decode_steps
    state_bytes = dw.B * dw.H * dw.dk * dw.dv * 4
    dec_bytes = 2 * state_bytes + dw.B * dw.H * (2 * dw.dk + 2 * dw.dk + 2 * dw.dv + 2 * dw.dv)
    dec_gbs = dec_bytes / (dec_kernel_us * 1e-6) / 1e9
    dec_src = os.path.join(ROOT, "retnet_retention_chunkwise_amd", "csrc", "recurrent_step.hip")
    dec_traffic = load_traffic("recurrent_step_decode_traffic.txt", dec_src)
    del dq, dk_, dv_, state
    torch.cuda.empty_cache()

    # ------------------------------------- multi-token continuation (16 tokens)
    # chunkwise on 16 new tokens per stream from the decode state, in place
    # (the fp32-MFMA short-block streaming kernel)
    ct = 16
    cq, ck, cv = make_inputs(dw.B, dw.H, ct, dw.dk, dw.dv, dw.dtype, seed=1)
    cq, ck, cv = cq.to(dev), ck.to(dev), cv.to(dev)
    cstate = s0.to(dev)
    cy = torch.empty(dw.B, dw.H, ct, dw.dv, dtype=cq.dtype, device=dev)
    for _ in range(3):
        ret.chunkwise_fwd(cq, ck, cv, gd, ct, state_in=cstate, state_out=cstate, y=cy)
    torch.cuda.synchronize()
    cev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
    for a, b in cev:
        a.record(stream)
        ret.chunkwise_fwd(cq, ck, cv, gd, ct, state_in=cstate, state_out=cstate, y=cy)
        b.record(stream)
    torch.cuda.synchronize()
    cont_us = statistics.median(a.elapsed_time(b) for a, b in cev) * 1e3
    cont_bytes = 2 * state_bytes + dw.B * dw.H * ct * (2 * dw.dk + 2 * dw.dk + 2 * dw.dv + 2 * dw.dv)
    cont_gbs = cont_bytes / (cont_us * 1e-6) / 1e9
    cont_src = os.path.join(ROOT, "retnet_retention_chunkwise_amd", "csrc", "short_mfma.hip")
    cont_traffic = load_traffic("short_mfma_continuation16_traffic.txt", cont_src)
    del cq, ck, cv, cstate, cy, s0
    torch.cuda.empty_cache()

    # ------------------------------------------------ backward (layer1p3b)
    # gradients of the chunkwise forward: dQ, dK, dV and dS_in from dY and dS_out;
    # 3 rotating input sets (about 270 MB each, together larger than the GPU's
    # 256 MB last-level cache), as the forward rotates its inputs
    bsets = []
    for r in range(3):
        bq, bk, bv, bs0 = make_inputs(wl.B, wl.H, wl.T, wl.dk, wl.dv, wl.dtype, seed=7 + 2 * r, with_state=True)
        _, _, bdy, bds = make_inputs(wl.B, wl.H, wl.T, wl.dk, wl.dv, wl.dtype, seed=8 + 2 * r, with_state=True)
        bsets.append(tuple(t.to(dev) for t in (bq, bk, bv, bs0, bdy, bds)))

    def bwd_call(i):
        bq, bk, bv, bs0, bdy, bds = bsets[i % len(bsets)]
        ret.chunkwise_bwd(bq, bk, bv, g, wl.C, bdy, state_in=bs0, grad_state_out=bds)

    for i in range(12):
        bwd_call(i)
    torch.cuda.synchronize()
    bev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(21)]
    for i, (a, b) in enumerate(bev):
        a.record(stream)
        bwd_call(i)
        b.record(stream)
    torch.cuda.synchronize()
    bwd_us_pairs = statistics.median(a.elapsed_time(b) for a, b in bev) * 1e3
    # as for the forward: calls captured in a HIP graph and replayed back to
    # back (one untimed replay first); the event pairs above also hold the
    # host's work between the launches of a call
    nbg = 21
    bgraph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(bgraph):
        for i in range(nbg):
            bwd_call(i)
    bgraph.replay()
    torch.cuda.synchronize()
    e0.record(stream)
    bgraph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    bwd_us = e0.elapsed_time(e1) * 1e3 / nbg
    del bgraph
    bwd_bytes = head_tokens * (2 * wl.dk * 2 + 2 * wl.dv * 2 + 2 * wl.dk * 2 + wl.dv * 2)  # q,k,v,dy in; dq,dk,dv out
    bwd_flops = 3 * alg_flops  # three chunkwise passes of the forward's per-token work
    bwd_traffic = load_traffic("chunkwise_mfma_bwd_passes_layer1p3b_traffic.txt", kernel_src)
    del bsets
    torch.cuda.empty_cache()

    # ------------------------------------------- per-head GroupNorm (layer1p3b y)
    gy = [torch.randn(wl.B, wl.H, wl.T, wl.dv, device=dev).to(torch.bfloat16) for _ in range(4)]
    gw = torch.randn(wl.H, wl.dv, device=dev)
    gb = torch.randn(wl.H, wl.dv, device=dev)
    gout = torch.empty_like(gy[0])
    for i in range(3):
        ret.group_norm(gy[i % 4], gw, gb, 1e-5, out=gout)
    torch.cuda.synchronize()
    gev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
    for i, (a, b) in enumerate(gev):
        a.record(stream)
        ret.group_norm(gy[i % 4], gw, gb, 1e-5, out=gout)
        b.record(stream)
    torch.cuda.synchronize()
    gn_us = statistics.median(a.elapsed_time(b) for a, b in gev) * 1e3
    gn_bytes = 2 * head_tokens * wl.dv * 2 + 2 * wl.H * wl.dv * 4  # y in, out out (bf16); weight, bias
    gn_src = os.path.join(ROOT, "retnet_retention_chunkwise_amd", "csrc", "group_norm.hip")
    gn_traffic = load_traffic("group_norm_layer1p3b_traffic.txt", gn_src)
    del gy, gw, gb, gout
    torch.cuda.empty_cache()

    out = {
        "metric": "retention tokens/sec (chunkwise fwd) + decode steps/sec; % MFMA / HBM peak",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "ms_per_step_eager": ms_per_step_eager,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1)/sqrt(dk) inputs, 4 rotating input sets)",
        "config": {"workload": "layer1p3b: chunkwise fwd B=4 H=8 T=2048 dk=256 dv=512 bf16 C=64, "
                               "gamma_h=1-2^(-5-h), fp32 state",
                   "global_batch": wl.B, "seq_len": wl.T, "parallelism": "single GPU"},
        "roofline": {
            "bound": "hbm",
            "achieved": achieved_gbs,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved_gbs / HBM_PEAK_GBS,
            "traffic": traffic,
            "kernel": "chunkwise_mfma_kernel<64, 256, true, true, 0> (64-token tile, d_k 256, zeta-staged V, forward in time)",
            "kernel_us": kernel_ms * 1e3,
            "kernel_us_event_pairs": kernel_ms_pairs * 1e3,
            "algorithmic_bytes_per_launch": alg_bytes,
            "algorithmic_flops_per_launch": alg_flops,
            "mfma_tflops": achieved_tflops,
            "mfma_frac": achieved_tflops / BF16_PEAK_TFLOPS,
        },
        "decode": {
            "workload": "recurrent step: batch 128, H=16, fp32 state 256x512 per head, bf16 q/k/v, "
                        f"{args.decode_steps} chained steps",
            "steps_per_s": 1e3 * args.decode_steps / dec_ms,
            "us_per_step": dec_us_step,
            "kernel_us": dec_kernel_us,
            "roofline": {"bound": "hbm", "achieved": dec_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": dec_gbs / HBM_PEAK_GBS, "traffic": dec_traffic,
                         "algorithmic_bytes_per_launch": dec_bytes},
        },
    }
    out["continuation"] = {
        "workload": f"chunkwise fwd on {ct} new tokens per stream from a carried state, in place: batch 128, H=16, "
                    "fp32 state 256x512 per head, bf16 q/k/v",
        "tokens_per_s": dw.B * ct / (cont_us * 1e-6),
        "kernel_us": cont_us,
        "roofline": {"bound": "hbm", "achieved": cont_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": cont_gbs / HBM_PEAK_GBS, "traffic": cont_traffic,
                     "algorithmic_bytes_per_launch": cont_bytes},
    }
    out["backward"] = {
        "workload": "chunkwise backward (dQ, dK, dV, dS_in) of the layer1p3b workload: B=4 H=8 T=2048 dk=256 "
                    "dv=512 bf16 C=64, with state_in and grad_state_out, 3 rotating input sets",
        "tokens_per_s": tokens / (bwd_us * 1e-6),
        "kernel_us": bwd_us,
        "kernel_us_event_pairs": bwd_us_pairs,
        "roofline": {"bound": "hbm", "achieved": bwd_bytes / (bwd_us * 1e-6) / 1e9, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": bwd_bytes / (bwd_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                     "traffic": bwd_traffic, "algorithmic_bytes_per_launch": bwd_bytes,
                     "algorithmic_flops_per_launch": bwd_flops,
                     "mfma_tflops": bwd_flops / (bwd_us * 1e-6) / 1e12,
                     "mfma_frac": bwd_flops / (bwd_us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS},
    }
    out["group_norm"] = {
        "workload": "per-head GroupNorm of a layer1p3b output: [4,8,2048,512] bf16, affine weight/bias, 4 rotating inputs",
        "kernel_us": gn_us,
        "roofline": {"bound": "hbm", "achieved": gn_bytes / (gn_us * 1e-6) / 1e9, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": gn_bytes / (gn_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                     "traffic": gn_traffic, "algorithmic_bytes_per_launch": gn_bytes},
    }
    if not args.no_cpu_baseline:
        sample_B = int(os.environ.get("RET_CPU_SAMPLE_B", str(wl.B)))
        sample_T = int(os.environ.get("RET_CPU_SAMPLE_T", str(wl.T)))
        v_cpu, dt, cores = cpu_baseline_chunkwise(wl, sample_B, sample_T)
        out["cpu_baseline"] = {
            "value": v_cpu, "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 recurrent-form oracle on {sample_B} of {wl.B} batch elements x all {wl.H} heads x "
                      f"{sample_T} of {wl.T} tokens of the layer1p3b workload: {dt:.1f} s on {cores} threads "
                      f"of {host_cpu_model()}",
        }
        dsteps = int(os.environ.get("RET_CPU_DECODE_STEPS", "64"))
        dbatch = int(os.environ.get("RET_CPU_DECODE_BATCH", "16"))
        v_dec, ddt, _ = cpu_baseline_decode(dw, dsteps, dbatch)
        out["decode"]["cpu_baseline"] = {
            "value": v_dec, "unit": "steps/s", "cores": cores, "kind": "oracle",
            "sample": f"fp64 oracle decode steps, {dbatch} of {dw.B} sequences x {dw.H} heads, {dsteps} steps "
                      f"({ddt:.1f} s on {cores} threads of {host_cpu_model()}), scaled to the full batch",
        }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
