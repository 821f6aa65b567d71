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

MXFP8 weights (``oracle.c``, ``linear_mxfp8``): E4M3 codes with one E8M0
scale per 32 elements along K, decoded from the open microscaling format's
definition (the pages name MXFP8 projections without defining them); the
sum is the same fp64 loop over the exact dequantised values, held to the
bf16 rule.  MXFP4 (``linear_mxfp4``): E2M1 codes, two per byte, with the
same block scales.

Epilogues (``oracle.c``), each applied with the pages' rounding points:

* RMSNorm of a projection's bf16 output with a bf16 gain (q_norm over the
  q_a columns, kv_norm over the kv columns: the consumers of the fused
  projection in PR #20636, Description)::

      out[m, j] = V[m, j] * G[j] / sqrt(mean_j V[m, j]^2 + eps)

* SwiGLU of row-concatenated gate/up projections, gate and up rounded to
  bf16 first (dense-MLP commit of PR #20502)::

      h[m, j] = silu(G[m, j]) * U[m, j],   silu(v) = v / (1 + exp(-v))

Their acceptance bounds (``rmsnorm_bound``, ``swiglu_bound``) are derived
from the GPU's fp32 steps and documented at each function; the router GEMV
(bf16 operands, fp32 logits, PR #20502) uses the fp32 rule below.

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
            ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared", "-fno-fast-math",
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
            lib.oracle_linear_omp.restype = ctypes.c_int
            lib.oracle_linear_omp.argtypes = lib.oracle_linear.argtypes
            lib.oracle_omp_threads.restype = ctypes.c_int
            lib.oracle_omp_threads.argtypes = []
            lib.oracle_round_bf16.restype = ctypes.c_uint16
            lib.oracle_round_bf16.argtypes = [ctypes.c_double]
            lib.oracle_round_bf16_array.restype = None
            lib.oracle_round_bf16_array.argtypes = [
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64]
            lib.oracle_e4m3_value.restype = ctypes.c_double
            lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
            lib.oracle_e8m0_value.restype = ctypes.c_double
            lib.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
            lib.oracle_linear_mxfp8.restype = ctypes.c_int
            lib.oracle_linear_mxfp8.argtypes = [
                ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
            lib.oracle_e2m1_value.restype = ctypes.c_double
            lib.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
            lib.oracle_linear_mxfp4.restype = ctypes.c_int
            lib.oracle_linear_mxfp4.argtypes = [
                ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
            lib.oracle_linear_nvfp4.restype = ctypes.c_int
            lib.oracle_linear_nvfp4.argtypes = [
                ctypes.c_int64, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64,
                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_void_p,
                ctypes.c_void_p]
            lib.oracle_rmsnorm_bf16.restype = ctypes.c_int
            lib.oracle_rmsnorm_bf16.argtypes = [
                ctypes.c_int64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                ctypes.c_double, ctypes.c_void_p, ctypes.c_void_p]
            lib.oracle_swiglu_bf16.restype = ctypes.c_int
            lib.oracle_swiglu_bf16.argtypes = [
                ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
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


def linear_omp(x_bits: np.ndarray, w_bits: np.ndarray):
    """``linear`` with the output elements spread over the host's threads
    (same per-element loop, bitwise equal results): the multi-core CPU
    baseline."""
    dt = _dtype_of(x_bits)
    x = np.ascontiguousarray(x_bits)
    w = np.ascontiguousarray(w_bits)
    N, K = w.shape
    M, ldx = x.shape
    y = np.zeros((M, N), dtype=np.float64)
    s = np.zeros((M, N), dtype=np.float64)
    rc = _load().oracle_linear_omp(dt, M, N, K, ldx, x.ctypes.data, w.ctypes.data,
                                   y.ctypes.data, s.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_linear_omp rejected its arguments")
    return y, s


def omp_threads() -> int:
    """Threads ``linear_omp`` uses."""
    return int(_load().oracle_omp_threads())


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


# ------------------------------------------------------------------ MXFP8
def e4m3_value(code: int) -> float:
    """Exact value of one E4M3 code (``oracle.c``; NaN for the NaN codes)."""
    return float(_load().oracle_e4m3_value(int(code) & 0xFF))


def e8m0_value(code: int) -> float:
    """Exact value of one E8M0 scale code, 2^(s - 127) (NaN for 255)."""
    return float(_load().oracle_e8m0_value(int(code) & 0xFF))


def linear_mxfp8(x_bits: np.ndarray, w_packed: np.ndarray, K: int):
    """One projection with MXFP8 weights (``oracle.c``).  ``x_bits`` is bf16
    [M, ldx] (first K columns read); ``w_packed`` is uint8 [N, K + K/32]:
    per row the K E4M3 codes, then the K/32 E8M0 scales of its 32-element
    blocks.  Returns ``(y, S)`` as float64 [M, N]."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    w = np.ascontiguousarray(w_packed, dtype=np.uint8)
    if x.ndim != 2 or w.ndim != 2 or K % 32 != 0 or w.shape[1] != K + K // 32:
        raise ValueError("x must be [M, ldx] bf16, w [N, K + K/32] uint8, K % 32 == 0")
    M, ldx = x.shape
    N = w.shape[0]
    y = np.zeros((M, N), dtype=np.float64)
    S = np.zeros((M, N), dtype=np.float64)
    rc = _load().oracle_linear_mxfp8(M, N, K, ldx, x.ctypes.data, w.ctypes.data,
                                     y.ctypes.data, S.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_linear_mxfp8 rejected its arguments")
    return y, S


def e2m1_value(code: int) -> float:
    """Exact value of one E2M1 (FP4) code, low 4 bits (``oracle.c``)."""
    return float(_load().oracle_e2m1_value(int(code) & 0xF))


def linear_mxfp4(x_bits: np.ndarray, w_packed: np.ndarray, K: int):
    """One projection with MXFP4 weights (``oracle.c``).  ``w_packed`` is
    uint8 [N, K/2 + K/32]: per row the K/2 code bytes (element 2i in the
    low nibble of byte i, 2i+1 in the high nibble), then the K/32 E8M0
    scales.  Returns ``(y, S)`` as float64 [M, N]."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    w = np.ascontiguousarray(w_packed, dtype=np.uint8)
    if x.ndim != 2 or w.ndim != 2 or K % 32 != 0 or w.shape[1] != K // 2 + K // 32:
        raise ValueError("x must be [M, ldx] bf16, w [N, K/2 + K/32] uint8, K % 32 == 0")
    M, ldx = x.shape
    N = w.shape[0]
    y = np.zeros((M, N), dtype=np.float64)
    S = np.zeros((M, N), dtype=np.float64)
    rc = _load().oracle_linear_mxfp4(M, N, K, ldx, x.ctypes.data, w.ctypes.data,
                                     y.ctypes.data, S.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_linear_mxfp4 rejected its arguments")
    return y, S


def linear_nvfp4(x_bits: np.ndarray, w_packed: np.ndarray, K: int, g: float):
    """One projection with NVFP4 weights (``oracle.c``).  ``w_packed`` is
    uint8 [N, K/2 + K/16]: per row the K/2 code bytes (element 2i in the
    low nibble of byte i), then the K/16 E4M3 scales of its 16-element
    blocks; ``g`` is the tensor's fp32 scale (taken as float32).  Returns
    ``(y, S)`` as float64 [M, N]."""
    x = np.ascontiguousarray(x_bits, dtype=np.uint16)
    w = np.ascontiguousarray(w_packed, dtype=np.uint8)
    if x.ndim != 2 or w.ndim != 2 or K % 16 != 0 or w.shape[1] != K // 2 + K // 16:
        raise ValueError("x must be [M, ldx] bf16, w [N, K/2 + K/16] uint8, K % 16 == 0")
    M, ldx = x.shape
    N = w.shape[0]
    y = np.zeros((M, N), dtype=np.float64)
    S = np.zeros((M, N), dtype=np.float64)
    rc = _load().oracle_linear_nvfp4(M, N, K, ldx, x.ctypes.data, w.ctypes.data,
                                     float(np.float32(g)), y.ctypes.data, S.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_linear_nvfp4 rejected its arguments")
    return y, S


# --------------------------------------------------------------- epilogues
# Longest chain of fp32 roundings any output's sum goes through in the GPU
# kernels (sequential adds plus tree levels; the matrix unit's 32-term step
# counted as 32): the fp32 sum of an output is then within FP32_SUM_DEPTH *
# 2^-24 * S of the exact sum.  The kernels stay far below it (at most a few
# hundred); it only enters the epilogue bounds below.
FP32_SUM_DEPTH = 1024
_U = 2.0 ** -24


def rmsnorm(v_bits: np.ndarray, gamma_bits: np.ndarray, eps: float):
    """RMSNorm of each row of bf16 ``v_bits`` [M, N] with bf16 gain
    ``gamma_bits`` [N] (``oracle.c``): returns ``(out, rinv)``, out the
    unrounded float64 [M, N] result and rinv[m] = 1 / sqrt(mean_j v^2 + eps).
    ``eps`` should be a value exact in fp32 (the GPU adds it in fp32)."""
    v = np.ascontiguousarray(v_bits, dtype=np.uint16)
    g = np.ascontiguousarray(gamma_bits, dtype=np.uint16)
    if v.ndim != 2 or g.ndim != 1 or g.shape[0] != v.shape[1]:
        raise ValueError("v must be [M, N] and gamma [N]")
    M, N = v.shape
    out = np.zeros((M, N), dtype=np.float64)
    rinv = np.zeros(M, dtype=np.float64)
    rc = _load().oracle_rmsnorm_bf16(M, N, v.ctypes.data, g.ctypes.data, float(eps),
                                     out.ctypes.data, rinv.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_rmsnorm_bf16 rejected its arguments")
    return out, rinv


def swiglu(g_bits: np.ndarray, u_bits: np.ndarray) -> np.ndarray:
    """silu(G) * U elementwise over bf16 patterns (``oracle.c``), unrounded
    float64 of the same shape."""
    g = np.ascontiguousarray(g_bits, dtype=np.uint16)
    u = np.ascontiguousarray(u_bits, dtype=np.uint16)
    if g.shape != u.shape:
        raise ValueError("gate and up shapes differ")
    h = np.zeros(g.shape, dtype=np.float64)
    rc = _load().oracle_swiglu_bf16(g.size, g.ctypes.data, u.ctypes.data, h.ctypes.data)
    if rc != 0:
        raise ValueError("oracle_swiglu_bf16 rejected its arguments")
    return h


def fused_rmsnorm(x_bits: np.ndarray, weights: list, gammas: list, eps: float):
    """The fused projection followed by a per-projection RMSNorm, with the
    rounding points of the unfused chain: y_i = x . W_i^T (exact), rounded
    once to bf16, then normalised (gamma_i None: projection left as is).
    Returns one dict per projection: y, S (exact sum and its scale), yb (the
    bf16 patterns of y), out (unrounded fp64 normalised result, or y when not
    normalised), rinv (per token, or None)."""
    res = []
    for w, gm in zip(weights, gammas):
        y, s = linear(x_bits, w)
        yb = round_bf16(y)
        if gm is None:
            res.append({"y": y, "S": s, "yb": yb, "out": y, "rinv": None})
            continue
        out, rinv = rmsnorm(yb, gm, eps)
        res.append({"y": y, "S": s, "yb": yb, "out": out, "rinv": rinv})
    return res


def fused_swiglu(x_bits: np.ndarray, w_gate: np.ndarray, w_up: np.ndarray):
    """Gate/up + SwiGLU with the pages' rounding points: g = x . Wg^T and
    u = x . Wu^T (exact), each rounded to bf16, h = silu(g_b) * u_b
    (unrounded fp64; the GPU rounds it once to bf16).  Returns a dict with
    g, Sg, u, Su, gb, ub, h."""
    g, sg = linear(x_bits, w_gate)
    u, su = linear(x_bits, w_up)
    gb = round_bf16(g)
    ub = round_bf16(u)
    return {"g": g, "Sg": sg, "u": u, "Su": su, "gb": gb, "ub": ub, "h": swiglu(gb, ub)}


def _bf16_pair_gap(y, S, exact_sums: bool):
    """Bound on |a - RNE(y)| for a = RNE(y') with y' an fp32 sum of the same
    products (|y' - y| <= FP32_SUM_DEPTH * 2^-24 * S): both roundings are
    within 2^-8 of their argument, so the gap is at most
    2^-7 |y| + (1 + 2^-8) * D * u * S (+1e-6 for values near zero).  With
    exact_sums (integer data: every fp32 partial sum exact) the two
    roundings coincide and the gap is 0."""
    if exact_sums:
        return np.zeros_like(np.asarray(y, dtype=np.float64))
    y = np.abs(np.asarray(y, dtype=np.float64))
    S = np.asarray(S, dtype=np.float64)
    return 2.0 ** -7 * y + (1 + 2.0 ** -8) * FP32_SUM_DEPTH * _U * S + 1e-6


def rmsnorm_bound(r: dict, gamma_bits: np.ndarray, eps: float, exact_sums: bool = False):
    """Allowed |out_gpu - out| per element for one normalised projection of
    ``fused_rmsnorm`` (GPU: bf16 projection output, fp32 sum of squares,
    rsqrt and products in fp32, one rounding to bf16).  Derived bound:
      D_j   = gap of the GPU's bf16 projection output to RNE(y_j) (above)
      dms   = (1/N) sum_j D_j (2|v_j| + D_j) + (N + 4) u (ms + that)
      er    = 0.5 * d / (1 - d) + 8u,   d = dms / (ms + eps)   (rsqrt)
      E_j   = |g_j| rinv (D_j + |v_j| er) (1 + 4u)
      tol_j = E_j + 2^-8 (|out_j| + E_j) + 1e-6                (output rounding)"""
    v = bf16_bits_to_f64(r["yb"])
    M, N = v.shape
    D = _bf16_pair_gap(r["y"], r["S"], exact_sums)
    ms = np.sum(v * v, axis=1) / N
    dms = np.sum(D * (2 * np.abs(v) + D), axis=1) / N
    dms = dms + (N + 4) * _U * (ms + dms)
    d = dms / (ms + eps)
    if np.any(d >= 0.5):
        raise ValueError("perturbation too large for the first-order rsqrt bound")
    er = 0.5 * d / (1 - d) + 8 * _U
    gam = np.abs(bf16_bits_to_f64(gamma_bits))[None, :]
    rinv = r["rinv"][:, None]
    E = gam * rinv * (D + np.abs(v) * er[:, None]) * (1 + 4 * _U)
    return E + 2.0 ** -8 * (np.abs(r["out"]) + E) + 1e-6


# relative error allowed for the GPU's fp32 silu (fast exp of -g and a
# reciprocal-based division): the exponent's own rounding grows with |g|
def _silu_rel(g):
    return 2.0 ** -20 * (np.abs(g) + 8.0)


def swiglu_bound(r: dict, exact_sums: bool = False):
    """Allowed |h_gpu - h| per element for ``fused_swiglu``'s h.  With Dg,
    Du the gaps of the GPU's bf16 gate/up values to RNE(g), RNE(u) (above),
    |silu'| <= 1.1 and a relative error s of the fp32 silu:
      E   = 1.1 Dg (|u_b| + Du) + |silu(g_b)| Du + s (|silu(g_b)| + 1.1 Dg)(|u_b| + Du)
      tol = E + 2^-8 (|h| + E) + 1e-6."""
    Dg = _bf16_pair_gap(r["g"], r["Sg"], exact_sums)
    Du = _bf16_pair_gap(r["u"], r["Su"], exact_sums)
    gb = bf16_bits_to_f64(r["gb"])
    ub = np.abs(bf16_bits_to_f64(r["ub"]))
    sil = np.abs(swiglu(r["gb"], round_bf16(np.ones(r["gb"].shape))))  # |silu(g_b)|
    s = _silu_rel(gb)
    E = 1.1 * Dg * (ub + Du) + sil * Du + s * (sil + 1.1 * Dg) * (ub + Du)
    return E + 2.0 ** -8 * (np.abs(r["h"]) + E) + 1e-6


def check_against(got_f64: np.ndarray, want: np.ndarray, bound: np.ndarray):
    """``(ok, worst_ratio, index)`` of |got - want| / bound (ok: <= 1, all
    finite)."""
    got = np.asarray(got_f64, dtype=np.float64)
    ratio = np.abs(got - want) / bound
    if ratio.size == 0:
        return True, 0.0, None
    idx = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
    worst = float(ratio[idx])
    return bool(np.all(np.isfinite(got)) and worst <= 1.0), worst, idx
