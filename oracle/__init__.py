"""CPU oracle of the fused decode-time hidden-state projection.

TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the benchmark's
``cpu_baseline`` leg are the only code allowed to import this package.  The
product library never imports it and shares no code with it: the oracle
decodes bf16 bit patterns, accumulates and rounds with its own code
(``oracle.c``, built with gcc, plus the pure-Python exact-rational version in
``exact.py``).

What it computes, per projection i, token row m and output row r::

    y_i[m, r] = sum_k X[m, k] * W_i[r, k]        (plain linear layer, no bias)
    S_i[m, r] = sum_k |X[m, k] * W_i[r, k]|      (scale of the error bound)

Sources (TensorRT-LLM pull-request pages):

* "tinygemm2 for the DeepSeek-V4.1 hidden-state projections" (PR #20636),
  Description: several projections reading the same activations are
  row-concatenated into one weight and computed by one GEMM whose parts are
  returned as dense [M, N_i] tensors; Test Coverage: compared against an
  F.linear reference.  The fusion is therefore exactly the per-projection
  linear layers.
* "Fuse indexer wk + weights_proj into single GEMM in TF32 for DS-V3.2"
  (PR #12055), Description: the FP32 variant of the same fusion.
* "Staircase: GLM-5.2 NVFP4 low-latency decode target for Rubin (TP16)"
  (PR #20502), router GEMV commit: checked against an FP64 reference.

Acceptance rule (error bound) for a GPU result compared with the unrounded
fp64 ``y``: bf16 outputs within ``2**-7 * S + 1e-6``, fp32 outputs within
``1e-5 * S + 1e-7``.  The bf16 bound covers one output rounding (at most
``2**-8 * |y| <= 2**-8 * S``) plus any fp32 summation order over K <= 8192
(at most ``K * 2**-24 * S`` < ``2**-9 * S``).

Parity pins: every function here is pinned in ``tests/test_oracle.py`` against
hand-worked values (``tests/golden``), identity and one-hot weights,
linearity on exact data, fused == split bookkeeping, integer data, a torch
fp64 matmul and exact rational arithmetic on tiny inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

BF16 = 0
F32 = 1

# Error-bound coefficients of the acceptance rule (relative-to-S, absolute).
TOLERANCE = {BF16: (2.0 ** -7, 1e-6), F32: (1e-5, 1e-7)}


def build(force: bool = True) -> str:
    """Compile ``liboracle.so`` with gcc (IEEE semantics: no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fno-fast-math",
             _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB_PATH):
                build(force=False)
            lib = ctypes.CDLL(_LIB_PATH)
            lib.oracle_linear.restype = ctypes.c_int
            lib.oracle_linear.argtypes = [
                ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                ctypes.c_void_p, ctypes.c_void_p]
            lib.oracle_round_bf16.restype = ctypes.c_uint16
            lib.oracle_round_bf16.argtypes = [ctypes.c_double]
            lib.oracle_round_bf16_array.restype = None
            lib.oracle_round_bf16_array.argtypes = [
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
            _lib = lib
    return _lib


def _dtype_of(bits: np.ndarray) -> int:
    if bits.dtype == np.uint16:
        return BF16
    if bits.dtype == np.uint32:
        return F32
    raise TypeError("bit patterns must be uint16 (bf16) or uint32 (fp32), got %s"
                    % bits.dtype)


def linear(x_bits: np.ndarray, w_bits: np.ndarray, M: int | None = None,
           K: int | None = None):
    """One projection.  ``x_bits`` is [M, ldx] (only the first K columns are
    read), ``w_bits`` is [N, K]; both hold raw bf16 (uint16) or fp32 (uint32)
    patterns.  Returns ``(y, S)`` as float64 [M, N] arrays."""
    dt = _dtype_of(x_bits)
    if _dtype_of(w_bits) != dt:
        raise TypeError("x and w must share one dtype")
    x = np.ascontiguousarray(x_bits)
    w = np.ascontiguousarray(w_bits)
    if x.ndim != 2 or w.ndim != 2:
        raise ValueError("x and w must be 2-D")
    N, Kw = w.shape
    K = Kw if K is None else K
    if K != Kw:
        raise ValueError("w has %d columns, K=%d" % (Kw, K))
    M = x.shape[0] if M is None else M
    ldx = x.shape[1]
    if ldx < K:
        raise ValueError("x row length %d < K=%d" % (ldx, K))
    y = np.zeros((M, N), dtype=np.float64)
    s = np.zeros((M, N), dtype=np.float64)
    rc = _load().oracle_linear(dt, M, N, K, ldx, x.ctypes.data, w.ctypes.data,
                               y.ctypes.data, s.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_linear rejected its arguments")
    return y, s


def fused_projection(x_bits: np.ndarray, weights: list):
    """The fused projection's result: one ``(y_i, S_i)`` per projection, each
    the plain linear layer of that projection's own weight (the fused GEMM
    must equal these; the concatenation is bookkeeping, not arithmetic)."""
    return [linear(x_bits, w) for w in weights]


def concat_rows(weights: list) -> np.ndarray:
    """The plan's concatenated weight: W_cat[off_i + r, :] = W_i[r, :] with
    off_0 = 0 and off_{i+1} = off_i + N_i (PR #20636, Description: one
    row-concatenated [1792, 5120] tensor from the [1280, 5120] and
    [512, 5120] weights)."""
    return np.concatenate([np.ascontiguousarray(w) for w in weights], axis=0)


def row_offsets(ns: list) -> list:
    """off_i of the concatenation above."""
    out, acc = [], 0
    for n in ns:
        out.append(acc)
        acc += int(n)
    return out


def round_bf16(v) -> np.ndarray:
    """Round float64 values to bf16 bit patterns (ties to even, gradual
    underflow, overflow to inf), computed in ``oracle.c``."""
    a = np.ascontiguousarray(np.asarray(v, dtype=np.float64))
    out = np.zeros(a.shape, dtype=np.uint16)
    _load().oracle_round_bf16_array(a.ctypes.data, out.ctypes.data, a.size)
    return out


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bf16 patterns (upper half of a binary32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f32_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)


def error_bound(S: np.ndarray, dtype: int) -> np.ndarray:
    """Allowed |y_gpu - y| per element for the acceptance rule above."""
    rel, ab = TOLERANCE[dtype]
    return rel * np.asarray(S, dtype=np.float64) + ab


def check_within_bound(y_out_f64: np.ndarray, y: np.ndarray, S: np.ndarray,
                       dtype: int):
    """Returns ``(ok, worst_ratio, index)`` where ``worst_ratio`` is the
    largest |err| / bound over all elements (ok means <= 1)."""
    err = np.abs(np.asarray(y_out_f64, dtype=np.float64) - y)
    bound = error_bound(S, dtype)
    ratio = err / bound
    if ratio.size == 0:
        return True, 0.0, None
    idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    worst = float(ratio[idx])
    ok = bool(np.all(np.isfinite(y_out_f64)) and worst <= 1.0)
    return ok, worst, idx
