"""Seeded synthetic inputs for the fused hidden-state projection.

This module only draws random numbers and names workload shapes: it holds
none of the projection's arithmetic, and both the HIP path's tests/benchmark
and the CPU oracle consume the bit patterns it returns.

Value distributions (taken as the plainest reading of the workloads):

* bf16 workloads: x ~ N(0, 1) and W ~ U(-1/sqrt(K), 1/sqrt(K)), drawn in
  float32 and rounded to bf16 (round-to-nearest-even, torch's conversion).
* fp32 indexer-style workload: x ~ N(0, 1), W ~ N(0, 0.02) (0.02 is the
  standard deviation).
* Draw order: W_0, ..., W_{P-1}, then x, all from one
  ``torch.Generator('cpu').manual_seed(seed)``.

Shapes follow the pages' projections: DeepSeek-V4.1 wq_a (5120 -> 1280) with
wkv (5120 -> 512) from "tinygemm2 for the DeepSeek-V4.1 hidden-state
projections" (TensorRT-LLM PR #20636), Description; the DS-V3.2 indexer
wk + weights_proj in FP32 from PR #12055 (dimensions not on the page:
K=7168 with [128, 64] rows is this build's reading); GLM's fused-A
(q_a 2048 + compressed KV + rope, hidden 6144) from the fused-A commit of
PR #20502, with the split [2048, 576, 128].
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    K: int
    N: tuple
    dtype: str           # "bf16" or "f32"
    w_dist: str          # "uniform_inv_sqrt_k" or "normal_0.02"
    Ms: tuple
    seeds: tuple = (0,)
    notes: str = ""

    @property
    def n_total(self) -> int:
        return int(sum(self.N))


# The five workload cells.
WORKLOADS = {
    "wq_a+wkv_m1": Workload("wq_a+wkv_m1", 5120, (1280, 512), "bf16",
                            "uniform_inv_sqrt_k", (1,), (0,),
                            "DeepSeek-V4.1 wq_a + wkv, one token"),
    "wq_a+wkv_m2_8": Workload("wq_a+wkv_m2_8", 5120, (1280, 512), "bf16",
                              "uniform_inv_sqrt_k", (2, 4, 8), (1, 2, 3),
                              "fused vs one call per projection"),
    "indexer_f32": Workload("indexer_f32", 7168, (128, 64), "f32",
                            "normal_0.02", (1, 4, 8), (0, 1, 2, 3),
                            "indexer wk + weights_proj, fp32 FMA, split-K"),
    "fused_a_3way": Workload("fused_a_3way", 6144, (2048, 576, 128), "bf16",
                             "uniform_inv_sqrt_k", (1, 2, 3, 4, 5, 6, 7, 8),
                             (0,), "q_a + compressed KV + indexer rows"),
    "crossover": Workload("crossover", 5120, (1280, 512), "bf16",
                          "uniform_inv_sqrt_k",
                          (1, 2, 4, 8, 9, 16, 32, 64, 128), (0,),
                          "M sweep, strided x, reload through views"),
}


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def draw_weights(K: int, N, dtype: str, w_dist: str, g: torch.Generator):
    """Float32 weights, one [N_i, K] tensor per projection, then rounded to
    the storage dtype.  Returned as CPU torch tensors of that dtype."""
    out = []
    for n in N:
        if w_dist == "uniform_inv_sqrt_k":
            a = 1.0 / math.sqrt(K)
            w = (torch.rand(int(n), K, generator=g, dtype=torch.float32) * 2.0 - 1.0) * a
        elif w_dist == "normal_0.02":
            w = torch.randn(int(n), K, generator=g, dtype=torch.float32) * 0.02
        elif w_dist == "int4":
            w = torch.randint(-4, 5, (int(n), K), generator=g).to(torch.float32)
        else:
            raise ValueError(w_dist)
        out.append(w.to(torch.bfloat16) if dtype == "bf16" else w)
    return out


def draw_x(M: int, K: int, dtype: str, g: torch.Generator, ldx: int | None = None,
           x_dist: str = "normal"):
    """x as a CPU tensor [M, ldx] of the storage dtype; columns K..ldx-1 are
    filled with a large sentinel so a kernel that reads past K is caught."""
    ldx = K if ldx is None else ldx
    if x_dist == "normal":
        x = torch.randn(M, K, generator=g, dtype=torch.float32)
    elif x_dist == "int4":
        x = torch.randint(-4, 5, (M, K), generator=g).to(torch.float32)
    else:
        raise ValueError(x_dist)
    full = torch.full((M, ldx), 1.0e4, dtype=torch.float32)
    full[:, :K] = x
    return full.to(torch.bfloat16) if dtype == "bf16" else full


def make_case(K: int, N, dtype: str, M: int, seed: int,
              w_dist: str = "uniform_inv_sqrt_k", ldx: int | None = None,
              x_dist: str = "normal"):
    """Weights then x from one seeded generator (draw order W_0..W_{P-1}, x)."""
    g = _gen(seed)
    ws = draw_weights(K, N, dtype, w_dist, g)
    x = draw_x(M, K, dtype, g, ldx=ldx, x_dist=x_dist)
    return x, ws


def workload_case(name: str, M: int, seed: int, ldx: int | None = None):
    w = WORKLOADS[name]
    return make_case(w.K, w.N, w.dtype, M, seed, w.w_dist, ldx=ldx)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a CPU tensor: uint16 for bf16, uint32 for fp32."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    raise TypeError(t.dtype)


def from_bits(b: np.ndarray) -> torch.Tensor:
    """Inverse of ``bits``."""
    b = np.ascontiguousarray(b)
    if b.dtype == np.uint16:
        return torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16)
    if b.dtype == np.uint32:
        return torch.from_numpy(b.view(np.int32).copy()).view(torch.float32)
    raise TypeError(b.dtype)
