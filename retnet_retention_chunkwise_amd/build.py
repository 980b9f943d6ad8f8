"""Build libretention.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

    python -m retnet_retention_chunkwise_amd.build

Compiles every source under csrc/ to an object in _build/ (in parallel) and
links them into retnet_retention_chunkwise_amd/libretention.so.  It always
recompiles: it is the "does it build" check as well as the build.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libretention.so")

SOURCES = [
    "api.cpp",
    "recurrent_step.hip",
    "parallel_fwd.hip",
    "chunkwise_generic.hip",
    "chunkwise_mfma.hip",
    "state_copy.hip",
    "short_chunk.hip",
    "chunkwise_bwd.hip",
    "chunkwise_bwd_passes.cpp",
    "group_norm.hip",
    "chunkwise_f32_mfma.hip",
    "short_mfma.hip",
    "noalloc.hip",
    "short_bf16.hip",
]

ARCH = "gfx950"
# Packed-fp32 VALU instructions are kept off: hipcc would otherwise form them
# from ordinary float code.
# MFMA results go to arch VGPRs (not AGPRs), which avoids AGPR<->VGPR copies
# around the VALU work on accumulators (decay masks, state scaling).
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang",
          "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form=true", f"-I{INCLUDE}", f"-I{CSRC}", "-Wall",
          "-Wno-unused-function"]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libretention)")


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, jobs: int = 8) -> str:
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        out = _run([hipcc, *COMMON, *lang, "-c", os.path.join(CSRC, src), "-o", obj])
        if verbose and out.strip():
            print(out)
        return obj

    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(SOURCES)))) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([hipcc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
