"""Seeded synthetic workloads shared by the tests, the smoke check and the benchmark.

This module only draws random inputs and names shapes; it holds none of the
attention arithmetic, and both the HIP path and the CPU oracle consume what it
returns. Inputs follow the pages' own synthetic workload (page "Add Fused
Multi-Head Attention example": Q, K and V drawn i.i.d. from a standard normal):
q, k and v are drawn in that order as fp32 normals from one CPU generator seeded
per workload, multiplied by the workload's standard deviation and then rounded
to the storage dtype with round-to-nearest-even (torch's ``.to``). The oracle
reads the same rounded values upcast to fp64, so input quantisation is never
charged to the kernel.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, replace

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    dtype: str  # "f32" | "f16" | "bf16"
    causal: bool
    seed: int
    std: float = 1.0
    scale: float | None = None  # None -> 1/sqrt(d)

    @property
    def softmax_scale(self) -> float:
        return self.scale if self.scale is not None else 1.0 / math.sqrt(self.d)

    @property
    def flops(self) -> float:
        """Attention FLOP convention: 4*B*H*Nq*Nk*d, halved for causal."""
        f = 4.0 * self.B * self.H * self.Nq * self.Nk * self.d
        return f / 2 if self.causal else f

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    @property
    def io_bytes(self) -> int:
        """Algorithmic HBM bytes: Q, K, V read once, O written once, L (fp32) written once."""
        s = self.elem_bytes
        bh = self.B * self.H
        return bh * (self.Nq * self.d * s * 2 + self.Nk * self.d * s * 2 + self.Nq * 4)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads the method is specified on (the pages' benchmark shape is
# B=4, H=4, N=4096, d=64 fp32 non-causal); d128_bf16 and d128_bf16_causal share inputs.
WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_causal_f32", 1, 1, 256, 256, 64, "f32", True, seed=1, scale=1 / 8),
        Workload("pages_f32", 4, 4, 4096, 4096, 64, "f32", False, seed=2, scale=1 / 8),
        Workload("d128_bf16", 4, 16, 4096, 4096, 128, "bf16", False, seed=3),
        Workload("d128_bf16_causal", 4, 16, 4096, 4096, 128, "bf16", True, seed=3),
        Workload("long_causal_bf16", 1, 8, 16384, 16384, 64, "bf16", True, seed=4, scale=1 / 8),
        Workload("ragged_f16", 2, 12, 1000, 3001, 96, "f16", False, seed=5, std=0.5),
    ]
}


def make_inputs(w: Workload):
    """Returns CPU tensors (q, k, v) in the workload's storage dtype, [B,H,N,d] contiguous."""
    g = torch.Generator(device="cpu")
    g.manual_seed(w.seed)
    shapes = [(w.B, w.H, w.Nq, w.d), (w.B, w.H, w.Nk, w.d), (w.B, w.H, w.Nk, w.d)]
    out = []
    for shp in shapes:
        x = torch.randn(shp, generator=g, dtype=torch.float32)
        if w.std != 1.0:
            x = x * w.std
        out.append(x.to(DTYPES[w.dtype]).contiguous())
    return tuple(out)


def make_random(shape, dtype: str, seed: int, std: float = 1.0):
    """One seeded normal tensor (fp32 draw, scaled, rounded to dtype), for ad-hoc test shapes."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    x = torch.randn(shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(DTYPES[dtype]).contiguous()


def make_lengths(n: int, lo: int, hi: int, seed: int):
    """Seeded sequence lengths for packed batches: n integers drawn uniformly from [lo, hi]."""
    g = torch.Generator(device="cpu")
    g.manual_seed(seed)
    return [int(x) for x in torch.randint(lo, hi + 1, (n,), generator=g)]


def offsets(lengths):
    """B+1 int32 offsets (0, l0, l0+l1, ...) of back-to-back sequences."""
    out = [0]
    for n in lengths:
        out.append(out[-1] + int(n))
    return torch.tensor(out, dtype=torch.int32)
