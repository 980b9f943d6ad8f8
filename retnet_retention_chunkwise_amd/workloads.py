"""Seeded synthetic workloads for multi-scale retention.

This module only describes shapes and draws random inputs; it holds none of
the operator's arithmetic.  Both the GPU path's tests/benchmarks and the CPU
oracle's tests take their inputs from here, so the two sides always see the
same values.

Shapes follow the retention operator of "Retentive Networks — Microsoft
Propone l'Alternativa Architetturale ai Transformer" (section "Il meccanismo:
Multi-Scale Retention"): one decay gamma per head, queries/keys of head
dimension d_k, values of head dimension d_v (the state is d_k x d_v, as the
author rebuttal on the paperhub "Retentive Network: A Successor to Transformer
for Large Language Models" page states in its answer on inference cost).

Input recipe (all workloads): a CPU ``torch.Generator`` seeded with ``seed``
draws q, then k, then v (then the initial state for decode) as float32
standard normals; q, k, v are multiplied by 1/sqrt(d_k) and rounded
(round-to-nearest-even) to the workload dtype.  The decode state stays fp32.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Tuple

import torch

__all__ = ["Workload", "WORKLOADS", "make_inputs", "make_decode_inputs", "torch_dtype"]


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


@dataclass(frozen=True)
class Workload:
    """One synthetic retention workload.

    ``kind`` is "chunkwise" (a full-sequence forward) or "decode" (``steps``
    chained single-token recurrent steps on an fp32 state).
    """

    key: str
    kind: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    dtype: str
    gammas: Tuple[float, ...]
    C: Optional[int] = None
    steps: int = 0
    description: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def head_tokens(self) -> int:
        return self.B * self.H * self.T


def _sched(H: int, slope: float) -> Tuple[float, ...]:
    # gamma_h = 1 - 2^(-5 - slope*h), rounded to fp32 (the value the library sees)
    return tuple(float(torch.tensor(1.0 - 2.0 ** (-5.0 - slope * h), dtype=torch.float32)) for h in range(H))


WORKLOADS = {
    "tiny": Workload(
        key="tiny", kind="chunkwise", B=1, H=2, T=64, dk=16, dv=16, dtype="f32",
        gammas=tuple(float(torch.tensor(g, dtype=torch.float32)) for g in (0.9, 0.5)), C=16,
        description="tiny: B1 H2 T64 d16 fp32, gamma {0.9, 0.5}; parallel, recurrent and chunkwise (C=16)",
    ),
    "layer1p3b": Workload(
        key="layer1p3b", kind="chunkwise", B=4, H=8, T=2048, dk=256, dv=512, dtype="bf16",
        gammas=_sched(8, 1.0), C=64,
        description="1.3B-scale layer: B4 H8 T2048 dk256 dv512 bf16, gamma_h=1-2^(-5-h), C=64",
    ),
    "layer6p7b": Workload(
        key="layer6p7b", kind="chunkwise", B=2, H=16, T=8192, dk=256, dv=512, dtype="bf16",
        gammas=_sched(16, 0.5), C=128,
        description="6.7B-scale layer: B2 H16 T8192 dk256 dv512 bf16, gamma_h=1-2^(-5-h/2), C=128",
    ),
    "decode": Workload(
        key="decode", kind="decode", B=128, H=16, T=1, dk=256, dv=512, dtype="bf16",
        gammas=_sched(16, 0.5), steps=1000,
        description="recurrent decode: batch 128, H16, fp32 state 256x512, bf16 q/k/v, 1000 chained steps",
    ),
    "long64k": Workload(
        key="long64k", kind="chunkwise", B=1, H=8, T=65536, dk=256, dv=512, dtype="bf16",
        gammas=_sched(8, 1.0), C=128,
        description="long context: B1 H8 T65536 dk256 dv512 bf16, gamma_h=1-2^(-5-h), C=128",
    ),
}


def _draw(gen: torch.Generator, shape, scale: float, dtype: torch.dtype) -> torch.Tensor:
    x = torch.randn(*shape, generator=gen, dtype=torch.float32)
    if scale != 1.0:
        x.mul_(scale)
    return x.to(dtype)


def make_inputs(B: int, H: int, T: int, dk: int, dv: int, dtype: str = "bf16", seed: int = 0,
                with_state: bool = False):
    """Draw (q, k, v[, state_in]) on the CPU.

    q, k: [B,H,T,dk]; v: [B,H,T,dv], all in ``dtype`` after scaling by 1/sqrt(dk).
    state_in (optional): fp32 [B,H,dk,dv] standard normal, drawn after v.
    """
    gen = torch.Generator("cpu").manual_seed(seed)
    dt = torch_dtype(dtype)
    s = 1.0 / math.sqrt(dk)
    q = _draw(gen, (B, H, T, dk), s, dt)
    k = _draw(gen, (B, H, T, dk), s, dt)
    v = _draw(gen, (B, H, T, dv), s, dt)
    if with_state:
        st = _draw(gen, (B, H, dk, dv), 1.0, torch.float32)
        return q, k, v, st
    return q, k, v


def make_decode_inputs(B: int, H: int, dk: int, dv: int, steps: int, dtype: str = "bf16", seed: int = 0):
    """Draw a decode run on the CPU: q, k [steps,B,H,dk], v [steps,B,H,dv] in ``dtype``
    (scaled by 1/sqrt(dk)), then the fp32 initial state S0 [B,H,dk,dv] ~ N(0,1)."""
    gen = torch.Generator("cpu").manual_seed(seed)
    dt = torch_dtype(dtype)
    s = 1.0 / math.sqrt(dk)
    q = _draw(gen, (steps, B, H, dk), s, dt)
    k = _draw(gen, (steps, B, H, dk), s, dt)
    v = _draw(gen, (steps, B, H, dv), s, dt)
    s0 = _draw(gen, (B, H, dk, dv), 1.0, torch.float32)
    return q, k, v, s0


def gammas_tensor(wl: Workload) -> torch.Tensor:
    return torch.tensor(wl.gammas, dtype=torch.float32)
