"""Pins of the oracle's epilogues: the RMSNorm that follows the projection
(q_norm / kv_norm) and the gate/up SwiGLU.

Each pin is independent of the oracle's own code: hand-worked values
(``tests/golden``, closed forms evaluated with 40-digit decimal arithmetic),
invariants of the definitions (unit mean square after normalisation with
eps = 0, scale invariance, silu(v) - silu(-v) = v), torch's fp64 library
routines, the rounding point of the pages (the norm and SwiGLU read the
bf16-rounded projection), and planted mistakes that the pins must catch.
The derived error bounds are checked against an fp32 simulation of the GPU's
steps (inside) and against the same simulation with a planted mistake
(outside).
"""
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _bf16(a):
    f = np.asarray(a, dtype=np.float32)
    b = f.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value not exact in bf16"
    return (b >> 16).astype(np.uint16)


def _f64(bits):
    return oracle.bf16_bits_to_f64(bits)


# ------------------------------------------------------------------ RMSNorm
def _load_rmsnorm_cases():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "rmsnorm_hand.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "case":
                cur = {"name": tok[1], "N": int(tok[3]), "eps": float(tok[5]), "v": [],
                       "g": None, "out": {}}
            elif tok[0] == "v":
                cur["v"].append([float(t) for t in tok[1:]])
            elif tok[0] == "g":
                cur["g"] = [float(t) for t in tok[1:]]
            elif tok[0] == "out":
                cur["out"][int(tok[1])] = [float(t) for t in tok[2:]]
            elif tok[0] == "end":
                cases.append(cur)
                cur = None
    return cases


RMS_CASES = _load_rmsnorm_cases()


@pytest.mark.parametrize("case", RMS_CASES, ids=[c["name"] for c in RMS_CASES])
def test_rmsnorm_hand_worked(case):
    out, rinv = oracle.rmsnorm(_bf16(case["v"]), _bf16(case["g"]), case["eps"])
    for m, want in case["out"].items():
        np.testing.assert_allclose(out[m], want, rtol=2e-16, atol=0)


def test_rmsnorm_unit_mean_square_with_zero_eps():
    rng = np.random.default_rng(5)
    v = oracle.round_bf16(rng.standard_normal((4, 1280)))
    g = oracle.round_bf16(1.0 + 0.1 * rng.standard_normal(1280))
    out, _ = oracle.rmsnorm(v, g, 0.0)
    ms = np.mean((out / _f64(g)) ** 2, axis=1)
    np.testing.assert_allclose(ms, 1.0, rtol=1e-13)


def test_rmsnorm_scale_invariance_exact():
    rng = np.random.default_rng(6)
    v = rng.standard_normal((3, 512))
    g = oracle.round_bf16(rng.uniform(0.5, 1.5, 512))
    a, _ = oracle.rmsnorm(oracle.round_bf16(v), g, 0.0)
    for k in (-3, 4):
        b, _ = oracle.rmsnorm(oracle.round_bf16(v * 2.0 ** k), g, 0.0)
        assert np.array_equal(a, b), k


def test_rmsnorm_matches_torch_fp64():
    rng = np.random.default_rng(7)
    vb = oracle.round_bf16(rng.standard_normal((5, 1280)) * 0.6)
    gb = oracle.round_bf16(1.0 + 0.2 * rng.standard_normal(1280))
    eps = float(np.float32(1e-6))
    out, _ = oracle.rmsnorm(vb, gb, eps)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(_f64(vb)), (1280,),
                                       weight=torch.from_numpy(_f64(gb)), eps=eps)
    np.testing.assert_allclose(out, ref.numpy(), rtol=1e-14, atol=1e-300)


def test_fused_rmsnorm_reads_the_bf16_rounded_projection():
    # y = (1 + 2^-9, 1): RNE to bf16 gives (1, 1), whose normalisation with
    # eps = 0 is exactly the gain; normalising y itself would not be.
    x = _bf16([[1.0, 2.0 ** -9]])
    w = _bf16([[1.0, 1.0], [1.0, 0.0]])
    g = _bf16([0.75, -2.0])
    (r,) = oracle.fused_rmsnorm(x, [w], [g], 0.0)
    assert r["y"][0, 0] == 1.0 + 2.0 ** -9
    assert np.array_equal(r["out"][0], [0.75, -2.0])


def test_fused_rmsnorm_without_gain_passes_through():
    x = _bf16([[1.0, 2.0, 3.0]])
    w = _bf16([[1.0, 0.0, -1.0]])
    (r,) = oracle.fused_rmsnorm(x, [w], [None], 1e-6)
    assert r["rinv"] is None and r["out"][0, 0] == -2.0


def _rmsnorm_restated(v, g, eps, mutation):
    """Restatement used only to plant mistakes (not the oracle's code)."""
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    n = v.shape[1]
    ss = np.sum(v * v, axis=1)
    if mutation == "n_minus_1":
        ms = ss / (n - 1)
    else:
        ms = ss / n
    if mutation == "eps_outside":
        r = 1.0 / np.sqrt(ms) + eps
    elif mutation == "no_sqrt":
        r = 1.0 / (ms + eps)
    else:
        r = 1.0 / np.sqrt(ms + eps)
    if mutation == "gain_shift":
        g = np.roll(g, 1)
    return v * r[:, None] * g[None, :]


@pytest.mark.parametrize("mutation", ["n_minus_1", "eps_outside", "no_sqrt", "gain_shift"])
def test_rmsnorm_pins_catch_planted_mistakes(mutation):
    caught = False
    for case in RMS_CASES:
        good = _rmsnorm_restated(case["v"], case["g"], case["eps"], None)
        bad = _rmsnorm_restated(case["v"], case["g"], case["eps"], mutation)
        want = np.asarray([case["out"][m] for m in range(len(case["v"]))])
        assert np.allclose(good, want, rtol=2e-16, atol=0)
        if not np.allclose(bad, want, rtol=1e-12, atol=0):
            caught = True
    assert caught, mutation


def _gpu_like_rmsnorm(x_bits, w_bits, g_bits, eps, mutation=None, seed=0):
    """fp32 simulation of the GPU steps (numpy float32): the projection sum in
    a shuffled order of 64-term partial sums, RNE to bf16, fp32 sum of
    squares, rsqrt, two fp32 products, RNE to bf16."""
    rng = np.random.default_rng(seed)
    x = _f64(x_bits).astype(np.float32)
    w = _f64(w_bits).astype(np.float32)
    M, K = x.shape
    N = w.shape[0]
    prods = (x[:, None, :] * w[None, :, :]).astype(np.float32)  # exact in fp32
    parts = prods.reshape(M, N, K // 64, 64).sum(axis=3, dtype=np.float32)
    perm = rng.permutation(K // 64)
    acc = np.zeros((M, N), dtype=np.float32)
    for p in perm:
        acc = (acc + parts[:, :, p]).astype(np.float32)
    yb = _f64(oracle.round_bf16(acc.astype(np.float64))).astype(np.float32)
    ss = np.zeros(M, dtype=np.float32)
    for j in range(N):
        ss = (ss + yb[:, j] * yb[:, j]).astype(np.float32)
    n = np.float32(N - 1 if mutation == "n_minus_1" else N)
    ms = (ss / n).astype(np.float32)
    e = np.float32(0.0 if mutation == "no_eps" else eps)
    r = (np.float32(1.0) / np.sqrt((ms + e).astype(np.float32))).astype(np.float32)
    g = _f64(g_bits).astype(np.float32)
    o = ((yb * r[:, None]).astype(np.float32) * g[None, :]).astype(np.float32)
    return _f64(oracle.round_bf16(o.astype(np.float64)))


@pytest.mark.parametrize("mutation", [None, "n_minus_1", "no_eps"])
def test_rmsnorm_bound_holds_for_fp32_steps_and_catches_mistakes(mutation):
    rng = np.random.default_rng(11)
    # few columns, so that an N-1 divisor moves every output by ~4 %
    K, N, M = 512, 12, 3
    x = oracle.round_bf16(rng.standard_normal((M, K)))
    w = oracle.round_bf16(rng.uniform(-1, 1, (N, K)) / math.sqrt(K))
    g = oracle.round_bf16(1.0 + 0.1 * rng.standard_normal(N))
    # a large eps relative to the mean square makes the "no_eps" mistake visible
    eps = float(np.float32(0.25))
    (r,) = oracle.fused_rmsnorm(x, [w], [g], eps)
    got = _gpu_like_rmsnorm(x, w, g, eps, mutation)
    ok, worst, _ = oracle.check_against(got, r["out"], oracle.rmsnorm_bound(r, g, eps))
    if mutation is None:
        assert ok, worst
    else:
        assert not ok, (mutation, worst)


def test_rmsnorm_bound_exact_sums_is_half_ulp_tight():
    # integer data: the bound with exact sums allows only the output rounding
    rng = np.random.default_rng(12)
    K, N = 64, 40
    x = oracle.round_bf16(rng.integers(-2, 3, (2, K)).astype(float))
    w = oracle.round_bf16(rng.integers(-1, 2, (N, K)).astype(float))
    g = oracle.round_bf16(rng.uniform(0.5, 2.0, N))
    (r,) = oracle.fused_rmsnorm(x, [w], [g], 1e-6)
    b = oracle.rmsnorm_bound(r, g, 1e-6, exact_sums=True)
    rounded = _f64(oracle.round_bf16(r["out"]))
    assert np.all(np.abs(rounded - r["out"]) <= b)
    assert np.all(b <= 2.0 ** -8 * np.abs(r["out"]) * (1 + 2.0 ** -10) + 2e-6)


# ------------------------------------------------------------------ SwiGLU
def _load_swiglu_values():
    rows = []
    with open(os.path.join(GOLDEN, "swiglu_hand.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                g, u, h = line.split()
                rows.append((float(g), float(u), float(h)))
    return rows


SWIGLU_VALUES = _load_swiglu_values()


def test_swiglu_hand_worked():
    g = _bf16([r[0] for r in SWIGLU_VALUES])
    u = _bf16([r[1] for r in SWIGLU_VALUES])
    h = oracle.swiglu(g, u)
    np.testing.assert_allclose(h, [r[2] for r in SWIGLU_VALUES], rtol=4e-16, atol=0)


def test_swiglu_matches_decimal_definition():
    getcontext().prec = 40
    rng = np.random.default_rng(3)
    gb = oracle.round_bf16(rng.uniform(-12, 12, 64))
    ub = oracle.round_bf16(rng.standard_normal(64))
    h = oracle.swiglu(gb, ub)
    for gv, uv, hv in zip(_f64(gb), _f64(ub), h):
        d = Decimal(float(gv))
        want = d / (1 + (-d).exp()) * Decimal(float(uv))
        assert abs(Decimal(float(hv)) - want) <= abs(want) * Decimal("4e-16") + Decimal("1e-300")


def test_silu_odd_part_identity():
    rng = np.random.default_rng(4)
    v = oracle.round_bf16(rng.uniform(-20, 20, 200))
    one = oracle.round_bf16(np.ones(200))
    neg = oracle.round_bf16(-_f64(v))
    d = oracle.swiglu(v, one) - oracle.swiglu(neg, one)
    np.testing.assert_allclose(d, _f64(v), rtol=4e-15, atol=1e-300)


def test_swiglu_matches_torch_fp64():
    rng = np.random.default_rng(8)
    gb = oracle.round_bf16(rng.standard_normal(512) * 3)
    ub = oracle.round_bf16(rng.standard_normal(512))
    ref = torch.nn.functional.silu(torch.from_numpy(_f64(gb))) * torch.from_numpy(_f64(ub))
    np.testing.assert_allclose(oracle.swiglu(gb, ub), ref.numpy(), rtol=1e-15, atol=1e-300)


def test_fused_swiglu_reads_bf16_rounded_gate_and_up():
    # gate sum 1 + 2^-9 rounds to 1, up sum 3 + 2^-7 rounds to 3
    x = _bf16([[1.0, 2.0 ** -9, 2.0 ** -7]])
    wg = _bf16([[1.0, 1.0, 0.0]])
    wu = _bf16([[3.0, 0.0, 1.0]])
    r = oracle.fused_swiglu(x, wg, wu)
    assert r["g"][0, 0] == 1.0 + 2.0 ** -9 and r["u"][0, 0] == 3.0 + 2.0 ** -7
    getcontext().prec = 40
    want = float(Decimal(1) / (1 + Decimal(-1).exp()) * 3)
    assert abs(r["h"][0, 0] - want) <= 4e-16 * abs(want)


def _swiglu_restated(g, u, mutation):
    g = np.asarray(g, dtype=np.float64)
    u = np.asarray(u, dtype=np.float64)
    if mutation == "sigmoid_sign":
        return g / (1 + np.exp(g)) * u
    if mutation == "drop_up":
        return g / (1 + np.exp(-g))
    if mutation == "swap":
        return u / (1 + np.exp(-u)) * g
    return g / (1 + np.exp(-g)) * u


@pytest.mark.parametrize("mutation", ["sigmoid_sign", "drop_up", "swap"])
def test_swiglu_pins_catch_planted_mistakes(mutation):
    g = [r[0] for r in SWIGLU_VALUES]
    u = [r[1] for r in SWIGLU_VALUES]
    want = [r[2] for r in SWIGLU_VALUES]
    assert np.allclose(_swiglu_restated(g, u, None), want, rtol=1e-15, atol=0)
    assert not np.allclose(_swiglu_restated(g, u, mutation), want, rtol=1e-6, atol=0)


def _gpu_like_swiglu(x_bits, wg_bits, wu_bits, mutation=None):
    """fp32 simulation of the GPU steps: fp32 sums of the exact products,
    RNE to bf16, silu with an fp32 exp and division, product, RNE."""
    x = _f64(x_bits).astype(np.float32)

    def proj(wb):
        w = _f64(wb).astype(np.float32)
        acc = np.zeros((x.shape[0], w.shape[0]), dtype=np.float32)
        for k in range(x.shape[1]):
            acc = (acc + (x[:, None, k] * w[None, :, k]).astype(np.float32)).astype(np.float32)
        return _f64(oracle.round_bf16(acc.astype(np.float64))).astype(np.float32)

    g = proj(wg_bits)
    u = proj(wu_bits)
    if mutation == "no_gate_rounding":
        xd = _f64(x_bits)
        g = (xd @ _f64(wg_bits).T).astype(np.float32)
    e = np.exp((-g).astype(np.float32)).astype(np.float32)
    s = (g / (np.float32(1.0) + e).astype(np.float32)).astype(np.float32)
    if mutation == "sigmoid_sign":
        s = (g / (np.float32(1.0) + np.exp(g).astype(np.float32))).astype(np.float32)
    h = (s * u).astype(np.float32)
    return _f64(oracle.round_bf16(h.astype(np.float64)))


@pytest.mark.parametrize("mutation", [None, "sigmoid_sign"])
def test_swiglu_bound_holds_for_fp32_steps_and_catches_mistakes(mutation):
    rng = np.random.default_rng(21)
    K, I, M = 256, 64, 3
    x = oracle.round_bf16(rng.standard_normal((M, K)))
    wg = oracle.round_bf16(rng.uniform(-1, 1, (I, K)) * 4 / math.sqrt(K))
    wu = oracle.round_bf16(rng.uniform(-1, 1, (I, K)) / math.sqrt(K))
    r = oracle.fused_swiglu(x, wg, wu)
    got = _gpu_like_swiglu(x, wg, wu, mutation)
    ok, worst, _ = oracle.check_against(got, r["h"], oracle.swiglu_bound(r))
    if mutation is None:
        assert ok, worst
    else:
        assert not ok, (mutation, worst)


def test_swiglu_bound_exact_sums_catches_a_missing_rounding_point():
    # sparse integer-valued weights with a fractional x: gate sums are exact
    # in fp32 but not in bf16, so skipping the rounding of g shows
    rng = np.random.default_rng(22)
    K, I = 64, 48
    # x on a 1/64 grid up to +-4: gate sums carry more significant bits than
    # bf16 holds, and negative gates (where silu is most sensitive) occur
    x = oracle.round_bf16((rng.integers(-255, 256, (2, K)) / 64.0))
    wg = np.zeros((I, K))
    wu = np.zeros((I, K))
    for i in range(I):
        wg[i, rng.choice(K, 4, replace=False)] = rng.integers(-2, 3, 4)
        wu[i, rng.choice(K, 4, replace=False)] = rng.integers(-2, 3, 4)
    wg, wu = oracle.round_bf16(wg), oracle.round_bf16(wu)
    r = oracle.fused_swiglu(x, wg, wu)
    b = oracle.swiglu_bound(r, exact_sums=True)
    ok, worst, _ = oracle.check_against(_gpu_like_swiglu(x, wg, wu), r["h"], b)
    assert ok, worst
    ok, worst, _ = oracle.check_against(_gpu_like_swiglu(x, wg, wu, "no_gate_rounding"),
                                        r["h"], b)
    assert not ok, worst
