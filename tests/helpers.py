"""Shared helpers for the GPU parity tests."""
import sys
import time

import torch

BF16_TOL = 2e-2   # rel-L2 bound for bf16 inputs
F32_TOL = 1e-4    # rel-L2 bound for fp32 inputs


def tol(dtype) -> float:
    return F32_TOL if dtype == torch.float32 else BF16_TOL


def rel_l2(got, want) -> float:
    """||got - want||_2 / ||want||_2 over the whole tensor, in float64 on the CPU."""
    g = got.detach().to("cpu", torch.float64)
    w = want.detach().to("cpu", torch.float64)
    den = float(w.norm())
    num = float((g - w).norm())
    if den == 0.0:
        return num
    return num / den


def say(*args):
    """Progress line that names the case, flushed before the GPU work starts."""
    print(f"[{time.strftime('%H:%M:%S')}]", *args, flush=True)
    sys.stdout.flush()
