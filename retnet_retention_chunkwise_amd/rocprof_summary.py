"""Summaries of rocprofv3 CSV output for the libretention kernels.

    python -m retnet_retention_chunkwise_amd.rocprof_summary stats <kernel_stats.csv> [--cmd "..."]
    python -m retnet_retention_chunkwise_amd.rocprof_summary traffic --fetch <dir> --write <dir> \
        --kernel '<name substring>[|<substring>...]' --source <kernel .hip> --copy-mib <N> [--cmd "..."]
    python -m retnet_retention_chunkwise_amd.rocprof_summary mfma --pmc <dir> --stats <kernel_stats.csv> \
        --kernel '<name substring>' [--cmd "..."]

`stats` turns a `--kernel-trace --stats` kernel_stats.csv into a short text
table.  `traffic` turns two `--pmc FETCH_SIZE` / `--pmc WRITE_SIZE` runs into
HBM bytes per launch of one kernel (or per call of several kernels, one
dispatch of each, given as name substrings separated by '|', since template
argument lists hold commas), calibrated against a plain copy of
`--copy-mib` MiB measured in the same runs (bytes = counter * known copy bytes /
copy's counter), and records the sha256 of the kernel source so that a reader
can tell whether the figures still describe the current kernel.
`mfma` turns a `--pmc SQ_INSTS_VALU_MFMA_MOPS_BF16 SQ_VALU_MFMA_BUSY_CYCLES
GRBM_GUI_ACTIVE` run into the bf16 MFMA work a kernel executes per launch
(MOPS counts units of 512 flops) and, with its average duration from a kernel
trace, the executed MFMA rate against the 2.5 PFLOP/s dense bf16 peak, plus the
MFMA-busy share of SIMD cycles (busy cycles over the per-XCD active cycles x
1024 SIMDs; GRBM_GUI_ACTIVE sums the 8 XCDs, which the implied clock, active
cycles / 8 / duration, shows).
"""
from __future__ import annotations

import argparse
import collections
import csv
import glob
import hashlib
import os
import sys


def _short(name: str, width: int = 70) -> str:
    n = name.replace("(anonymous namespace)::", "")
    return n if len(n) <= width else n[: width - 3] + "..."


def stats_table(path: str, cmd: str = "") -> str:
    rows = list(csv.DictReader(open(path)))
    lines = []
    if cmd:
        lines.append(f"command: {cmd}")
    lines.append(f"{'kernel':72s} {'calls':>6s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} {'pct':>6s}")
    for r in rows:
        lines.append(f"{_short(r['Name'], 72):72s} {int(r['Calls']):6d} {float(r['AverageNs']) / 1e3:10.2f} "
                     f"{float(r['MinNs']) / 1e3:10.2f} {float(r['MaxNs']) / 1e3:10.2f} {float(r['Percentage']):6.2f}")
    return "\n".join(lines) + "\n"


def _per_dispatch(directory: str, counter: str):
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {directory}")
    acc = collections.defaultdict(float)
    names = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] != counter:
                continue
            key = (f, r["Dispatch_Id"])
            acc[key] += float(r["Counter_Value"])
            names[key] = r["Kernel_Name"]
    return [(names[k], v) for k, v in acc.items()]


def _mean_for(entries, substr):
    vals = [v for n, v in entries if substr in n]
    if not vals:
        raise ValueError(f"no dispatch of a kernel matching '{substr}'")
    return sum(vals) / len(vals), len(vals)


def _largest_for(entries, substr):
    vals = [v for n, v in entries if substr in n]
    if not vals:
        raise ValueError(f"no dispatch of a kernel matching '{substr}'")
    return max(vals)


def traffic(fetch_dir, write_dir, kernel, source, copy_mib, copy_substr="copy", cmd=""):
    f_entries = _per_dispatch(fetch_dir, "FETCH_SIZE")
    w_entries = _per_dispatch(write_dir, "WRITE_SIZE")
    # a call made of several kernels ('|'-separated substrings): one dispatch of each
    parts = [k for k in kernel.split("|") if k]
    k_fetch = k_write = 0.0
    n_f, n_w = [], []
    for part in parts:
        m, n = _mean_for(f_entries, part)
        k_fetch += m
        n_f.append(str(n))
        m, n = _mean_for(w_entries, part)
        k_write += m
        n_w.append(str(n))
    n_f, n_w = "+".join(n_f), "+".join(n_w)
    # the calibration copy is the largest dispatch of a copy kernel (small
    # runtime copies, e.g. device-to-host reads of a few bytes, also match)
    c_fetch = _largest_for(f_entries, copy_substr)
    c_write = _largest_for(w_entries, copy_substr)
    copy_bytes = copy_mib * 1024 * 1024
    f_scale = copy_bytes / (c_fetch * 1024.0)
    w_scale = copy_bytes / (c_write * 1024.0)
    rd = k_fetch * 1024.0 * f_scale
    wr = k_write * 1024.0 * w_scale
    sha = hashlib.sha256(open(source, "rb").read()).hexdigest()[:16]
    lines = []
    if cmd:
        lines.append(f"command: {cmd}")
    lines += [
        f"kernel: {kernel}",
        f"kernel_source: {os.path.basename(source)}",
        f"kernel_source_sha256_16: {sha}",
        f"dispatches_averaged: fetch {n_f}, write {n_w}",
        f"FETCH_SIZE_KiB_per_launch: {k_fetch:.1f}",
        f"WRITE_SIZE_KiB_per_launch: {k_write:.1f}",
        f"copy_calibration: {copy_mib} MiB copy read {c_fetch:.1f} KiB / wrote {c_write:.1f} KiB "
        f"-> factors read {f_scale:.4f}, write {w_scale:.4f}",
        f"read_bytes_per_launch: {rd:.0f}",
        f"write_bytes_per_launch: {wr:.0f}",
        f"traffic_bytes_per_launch: {rd + wr:.0f}",
    ]
    return "\n".join(lines) + "\n"


def _per_dispatch_all(directory: str):
    """{(file, dispatch): {counter: value}} and their kernel names."""
    files = glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {directory}")
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    names = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            key = (f, r["Dispatch_Id"])
            acc[key][r["Counter_Name"]] += float(r["Counter_Value"])
            names[key] = r["Kernel_Name"]
    return acc, names


def mfma(pmc_dir, stats_csv, kernel, cmd="", peak_tflops=2500.0, xcds=8, simds=1024, source=None):
    """MFMA work and busy share of one kernel from a counter run (and its
    steady-state duration from a kernel-trace stats file)."""
    files = glob.glob(os.path.join(pmc_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no counter_collection.csv under {pmc_dir}")
    acc = collections.defaultdict(lambda: collections.defaultdict(float))
    dur = {}
    for f in files:
        for r in csv.DictReader(open(f)):
            if kernel not in r["Kernel_Name"]:
                continue
            key = (f, r["Dispatch_Id"])
            acc[key][r["Counter_Name"]] += float(r["Counter_Value"])
            dur[key] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    if not acc:
        raise ValueError(f"no dispatch of a kernel matching '{kernel}'")
    keys = list(acc)
    mean = lambda c: sum(acc[k].get(c, 0.0) for k in keys) / len(keys)
    mops = mean("SQ_INSTS_VALU_MFMA_MOPS_BF16")
    busy = mean("SQ_VALU_MFMA_BUSY_CYCLES")
    active = mean("GRBM_GUI_ACTIVE")
    pmc_ns = sum(dur[k] for k in keys) / len(keys)
    rows = [r for r in csv.DictReader(open(stats_csv)) if kernel in r["Name"]]
    if not rows:
        raise ValueError(f"no kernel matching '{kernel}' in {stats_csv}")
    calls = sum(int(r["Calls"]) for r in rows)
    avg_ns = sum(float(r["AverageNs"]) * int(r["Calls"]) for r in rows) / calls
    flops = mops * 512.0
    tflops = flops / (avg_ns * 1e-9) / 1e12
    per_xcd = active / xcds
    lines = []
    if cmd:
        lines.append(f"command: {cmd}")
    lines.append(f"kernel: {kernel}")
    if source:
        lines += [f"kernel_source: {os.path.basename(source)}",
                  f"kernel_source_sha256_16: {hashlib.sha256(open(source, 'rb').read()).hexdigest()[:16]}"]
    lines += [
        f"dispatches_averaged: {len(keys)} (counters), {calls} (trace)",
        f"SQ_INSTS_VALU_MFMA_MOPS_BF16_per_launch: {mops:.0f}",
        f"SQ_VALU_MFMA_BUSY_CYCLES_per_launch: {busy:.0f}",
        f"GRBM_GUI_ACTIVE_per_launch: {active:.0f} (summed over {xcds} XCDs)",
        f"counter_run_kernel_us: {pmc_ns / 1e3:.2f} (clock {per_xcd / pmc_ns:.2f} GHz = GRBM_GUI_ACTIVE / {xcds} / duration)",
        f"kernel_avg_us (trace): {avg_ns / 1e3:.2f}",
        f"executed_bf16_mfma_flops_per_launch: {flops:.4e} (MOPS x 512)",
        f"executed_bf16_mfma_tflops: {tflops:.1f} (executed flops / trace average duration)",
        f"executed_mfma_frac_of_{peak_tflops:.0f}_tflops: {tflops / peak_tflops:.4f}",
        f"mfma_busy_frac: {busy / (per_xcd * simds):.4f} (busy cycles / (GRBM_GUI_ACTIVE / {xcds} x {simds} SIMDs))",
    ]
    return "\n".join(lines) + "\n"


def read_traffic_file(path: str):
    """Parse a `traffic` summary back into a dict (used by bench.py)."""
    out = {}
    for line in open(path):
        if ":" in line:
            k, v = line.split(":", 1)
            out[k.strip()] = v.strip()
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd_name", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--cmd", default="")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--source", required=True)
    t.add_argument("--copy-mib", type=float, required=True)
    t.add_argument("--copy-kernel", default="copy")
    t.add_argument("--cmd", default="")
    m = sub.add_parser("mfma")
    m.add_argument("--pmc", required=True)
    m.add_argument("--stats", required=True)
    m.add_argument("--kernel", required=True)
    m.add_argument("--source", default=None)
    m.add_argument("--cmd", default="")
    a = ap.parse_args(argv)
    if a.cmd_name == "stats":
        sys.stdout.write(stats_table(a.csv, a.cmd))
    elif a.cmd_name == "mfma":
        sys.stdout.write(mfma(a.pmc, a.stats, a.kernel, a.cmd, source=a.source))
    else:
        sys.stdout.write(traffic(a.fetch, a.write, a.kernel, a.source, a.copy_mib, a.copy_kernel, a.cmd))


if __name__ == "__main__":
    main()
