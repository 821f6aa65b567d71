"""Helpers shared by the GPU tests: run the HIP path through the C ABI and
compare it with the CPU oracle on the same seeded bit patterns."""
from __future__ import annotations

import numpy as np
import torch

import oracle
import synthetic_inputs as si

BF16 = torch.bfloat16
F32 = torch.float32


def device():
    return torch.device("cuda:0")


def to_gpu(t: torch.Tensor) -> torch.Tensor:
    return t.to(device())


def out_bits(ys) -> list:
    torch.cuda.synchronize()
    return [si.bits(y.cpu()) for y in ys]


def out_f64(ys) -> list:
    """Exact fp64 value of each output (bf16/fp32 widened exactly)."""
    res = []
    for b in out_bits(ys):
        if b.dtype == np.uint16:
            res.append(oracle.bf16_bits_to_f64(b))
        else:
            res.append(oracle.f32_bits_to_f64(b))
    return res


def oracle_dtype(t: torch.Tensor) -> int:
    return oracle.BF16 if t.dtype == BF16 else oracle.F32


def assert_matches_oracle(ys, x_cpu: torch.Tensor, ws_cpu, rows=None, K=None, label=""):
    """Compare every output element (or the token rows ``rows``) with the
    oracle's fp64 result under the acceptance bound of the dtype."""
    K = int(ws_cpu[0].shape[1]) if K is None else K
    xb = si.bits(x_cpu)
    if rows is not None:
        xb = xb[list(rows)]
    vals = out_f64(ys)
    dt = oracle_dtype(ws_cpu[0])
    for i, (w, v) in enumerate(zip(ws_cpu, vals)):
        y, s = oracle.linear(xb, si.bits(w), K=K)
        got = v if rows is None else v[list(rows)]
        ok, worst, idx = oracle.check_within_bound(got, y, s, dt)
        assert ok, "%s proj %d: worst |err|/bound = %.3g at %s (got %r, want %r)" % (
            label, i, worst, idx, float(got[idx]) if idx is not None else None,
            float(y[idx]) if idx is not None else None)


def assert_bitwise_equal(a, b, label=""):
    ba, bb = out_bits(a), out_bits(b)
    for i, (p, q) in enumerate(zip(ba, bb)):
        assert p.shape == q.shape, (label, i)
        if not np.array_equal(p, q):
            bad = np.argwhere(p != q)
            raise AssertionError("%s proj %d: %d elements differ, first at %s"
                                 % (label, i, len(bad), tuple(bad[0])))
