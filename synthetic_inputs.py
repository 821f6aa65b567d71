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
K=7168 with [128, 64] rows is a reading, not a figure of the page); GLM's fused-A
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
    # Epilogue workloads.  Router GEMV: GLM-5's 256 expert logits at hidden
    # 6144 for 1-16 tokens, fp32 output (router commit of PR #20502).
    "router_f32out": Workload("router_f32out", 6144, (256,), "bf16",
                              "uniform_inv_sqrt_k", tuple(range(1, 17)), (0, 1),
                              "bf16 operands, fp32 logits"),
    # wq_a + wkv with q_norm / kv_norm gains (PR #20636's consumers)
    "q_kv_norm": Workload("q_kv_norm", 5120, (1280, 512), "bf16",
                          "uniform_inv_sqrt_k", (1, 2, 3, 4, 5, 6, 7, 8), (0, 1),
                          "fused projection + RMSNorm per projection"),
    # dense-MLP gate/up of one TP16 rank: [2 * 768, 6144] (PR #20502)
    "gate_up_swiglu": Workload("gate_up_swiglu", 6144, (768, 768), "bf16",
                               "uniform_inv_sqrt_k", (1, 2, 3, 4, 5, 6, 7, 8), (0, 1),
                               "gate rows over up rows, SwiGLU epilogue"),
}


# MXFP8 weights: wq_a + wkv stored as E4M3 codes with one E8M0 scale per 32
# elements along K, the DeepSeek-V4.1 projections' MXFP8 form named on the
# pages.  Packed rows: K codes, then the K/32 scales.
MXFP8_WORKLOADS = {
    "wq_a+wkv_mxfp8": Workload("wq_a+wkv_mxfp8", 5120, (1280, 512), "mxfp8",
                               "codes_uniform_scales_112_117", (1, 2, 3, 4, 5, 6, 7, 8),
                               (0, 1), "MXFP8 weights, bf16 x and y"),
}
E4M3_NAN = (0x7F, 0xFF)


def draw_mxfp8_weights(K: int, N, g: torch.Generator, scale_lo: int = 112,
                       scale_hi: int = 117):
    """One packed uint8 [N_i, K + K/32] tensor per projection: codes uniform
    over the 254 non-NaN E4M3 codes, scales uniform in [scale_lo, scale_hi]
    (2^-15 .. 2^-10, so the weights are of the order of 1/sqrt(K))."""
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    out = []
    for n in N:
        codes = torch.randint(0, 254, (int(n), K), generator=g, dtype=torch.int64)
        codes = codes + (codes >= 0x7F).to(torch.int64)  # skip 0x7F; 0xFF is never drawn
        scales = torch.randint(scale_lo, scale_hi + 1, (int(n), K // 32), generator=g,
                               dtype=torch.int64)
        out.append(torch.cat([codes, scales], dim=1).to(torch.uint8))
    return out


def draw_mxfp4_weights(K: int, N, g: torch.Generator, scale_lo: int = 116,
                       scale_hi: int = 121):
    """One packed uint8 [N_i, K/2 + K/32] tensor per projection: code bytes
    uniform over 0..255 (two E2M1 codes each, every code valid), scales
    uniform in [scale_lo, scale_hi] (weights of the order of 1/sqrt(K))."""
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    out = []
    for n in N:
        codes = torch.randint(0, 256, (int(n), K // 2), generator=g, dtype=torch.int64)
        scales = torch.randint(scale_lo, scale_hi + 1, (int(n), K // 32), generator=g,
                               dtype=torch.int64)
        out.append(torch.cat([codes, scales], dim=1).to(torch.uint8))
    return out


def draw_nvfp4_weights(K: int, N, g: torch.Generator, scale_lo: int = 0x28,
                       scale_hi: int = 0x40):
    """One packed uint8 [N_i, K/2 + K/16] tensor per projection (code bytes
    uniform over 0..255, every E2M1 code valid; E4M3 block scales uniform
    over the codes scale_lo..scale_hi, i.e. 0.25 .. 2), and one fp32 tensor
    scale per projection, 2^-7 * (1 + u) with u uniform in [0, 1) rounded to
    fp32 (not a power of two): weights of the order of 1/sqrt(K)."""
    if K % 16:
        raise ValueError("K must be a multiple of 16")
    out, gs = [], []
    for n in N:
        codes = torch.randint(0, 256, (int(n), K // 2), generator=g, dtype=torch.int64)
        scales = torch.randint(scale_lo, scale_hi + 1, (int(n), K // 16), generator=g,
                               dtype=torch.int64)
        out.append(torch.cat([codes, scales], dim=1).to(torch.uint8))
        u = float(torch.rand((), generator=g, dtype=torch.float64))
        gs.append(float(np.float32(2.0 ** -7 * (1.0 + u))))
    return out, gs


def nvfp4_case(M: int, seed: int, K: int = 5120, N=(1280, 512), ldx: int | None = None):
    """Packed NVFP4 weights, their fp32 tensor scales, then bf16 x from one
    seeded generator."""
    g = _gen(seed)
    ws, gs = draw_nvfp4_weights(K, N, g)
    x = draw_x(M, K, "bf16", g, ldx=ldx)
    return x, ws, gs


def mxfp4_case(M: int, seed: int, K: int = 5120, N=(1280, 512), ldx: int | None = None):
    """Packed MXFP4 weights then bf16 x from one seeded generator."""
    g = _gen(seed)
    ws = draw_mxfp4_weights(K, N, g)
    x = draw_x(M, K, "bf16", g, ldx=ldx)
    return x, ws


def mxfp8_case(M: int, seed: int, K: int = 5120, N=(1280, 512), ldx: int | None = None):
    """Packed MXFP8 weights then bf16 x from one seeded generator."""
    g = _gen(seed)
    ws = draw_mxfp8_weights(K, N, g)
    x = draw_x(M, K, "bf16", g, ldx=ldx)
    return x, ws


def draw_gamma(N: int, g: torch.Generator) -> torch.Tensor:
    """An RMSNorm gain of N entries near 1 (1 + 0.1 * N(0, 1), in bf16), drawn
    after the weights and x of the same seed."""
    return (1.0 + 0.1 * torch.randn(int(N), generator=g, dtype=torch.float32)).to(
        torch.bfloat16)


def norm_case(M: int, seed: int, ldx: int | None = None):
    """x, the two weights and their two gains of the q_kv_norm workload."""
    w = WORKLOADS["q_kv_norm"]
    g = _gen(seed)
    ws = draw_weights(w.K, w.N, w.dtype, w.w_dist, g)
    x = draw_x(M, w.K, w.dtype, g, ldx=ldx)
    gammas = [draw_gamma(n, g) for n in w.N]
    return x, ws, gammas


def sparse_int_case(K: int, N, M: int, seed: int, nnz: int = 4, x_den: float = 64.0):
    """Exact-arithmetic data: x on a 1/x_den grid in [-4, 4], each weight row
    with nnz integer entries in [-2, 2] at random columns (bf16 exact).  Every
    fp32 partial sum of a projection is then exact, so the GPU's sums equal
    the exact ones bit for bit before any rounding."""
    g = _gen(seed)
    ws = []
    for n in N:
        w = torch.zeros(int(n), K, dtype=torch.float32)
        for r in range(int(n)):
            cols = torch.randperm(K, generator=g)[:nnz]
            w[r, cols] = torch.randint(-2, 3, (nnz,), generator=g).to(torch.float32)
        ws.append(w.to(torch.bfloat16))
    lim = int(4 * x_den) - 1
    x = (torch.randint(-lim, lim + 1, (M, K), generator=g).to(torch.float32) / x_den)
    return x.to(torch.bfloat16), ws


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
    """Raw bit patterns of a CPU tensor: uint16 for bf16, uint32 for fp32,
    the bytes themselves for uint8 (packed MXFP8 rows)."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    if t.dtype == torch.float32:
        return t.view(torch.int32).numpy().view(np.uint32)
    if t.dtype == torch.uint8:
        return t.numpy()
    raise TypeError(t.dtype)


def from_bits(b: np.ndarray) -> torch.Tensor:
    """Inverse of ``bits``."""
    b = np.ascontiguousarray(b)
    if b.dtype == np.uint16:
        return torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16)
    if b.dtype == np.uint32:
        return torch.from_numpy(b.view(np.int32).copy()).view(torch.float32)
    raise TypeError(b.dtype)
