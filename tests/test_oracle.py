"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each pin is independent of the oracle's own code path: hand-worked values
(``tests/golden``), identity and scaled-permutation weights (the result is a
copy/gather, known exactly), linearity on exact data, the concatenation
offsets printed on the pages, integer data checked with integer arithmetic,
a torch fp64 matmul, exact rational brute force, and the closed-form error
bound.  A final group plants plausible mistakes in a copy of the oracle's
definition (on the CPU) and checks that the pins catch every one.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import exact
import synthetic_inputs as si

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ----------------------------------------------------------------- helpers
def _f32_bits(a):
    return np.asarray(a, dtype=np.float32).view(np.uint32)


def _bf16_bits(a):
    # only used on values exact in bf16 (asserted)
    f = np.asarray(a, dtype=np.float32)
    b = f.view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value not exact in bf16"
    return (b >> 16).astype(np.uint16)


def _load_hand_cases():
    cases, cur = [], None
    with open(os.path.join(GOLDEN, "hand_worked_linear.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            tok = line.split()
            if tok[0] == "case":
                cur = {"name": tok[1], "K": int(tok[3]), "x": [], "w": {},
                       "y": {}, "s": {}}
            elif tok[0] == "x":
                cur["x"].append([float(v) for v in tok[1:]])
            elif tok[0] == "w":
                cur["w"].setdefault(int(tok[1]), []).append([float(v) for v in tok[2:]])
            elif tok[0] in ("y", "s"):
                cur[tok[0]].setdefault(int(tok[1]), {})[int(tok[2])] = [float(v) for v in tok[3:]]
            elif tok[0] == "end":
                cases.append(cur)
                cur = None
    return cases


HAND = _load_hand_cases()


def _as_bits(dt, a):
    return _bf16_bits(a) if dt == "bf16" else _f32_bits(a)


# ------------------------------------------------------ P-1: hand-worked
@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("case", HAND, ids=[c["name"] for c in HAND])
def test_hand_worked(case, dt):
    x = _as_bits(dt, case["x"])
    ws = [_as_bits(dt, case["w"][i]) for i in sorted(case["w"])]
    res = oracle.fused_projection(x, ws)
    for i, (y, s) in enumerate(res):
        for m, expect in case["y"][i].items():
            assert y[m].tolist() == expect, (case["name"], i, m)
        for m, expect in case["s"][i].items():
            assert s[m].tolist() == expect, (case["name"], i, m)


def test_hand_worked_strided_x():
    # the oracle must read only the first K columns of a row of length ldx
    case = HAND[1]
    x = np.asarray(case["x"], dtype=np.float32)
    padded = np.full((x.shape[0], x.shape[1] + 5), 777.0, dtype=np.float32)
    padded[:, :x.shape[1]] = x
    w = _f32_bits(case["w"][1])
    y, _ = oracle.linear(_f32_bits(padded), w, K=3)
    assert y.tolist() == [case["y"][1][0], case["y"][1][1]]


# ---------------------------------------------------- P-2: identity weight
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_identity_weight_copies_x(dt):
    g = torch.Generator().manual_seed(5)
    K = 48
    x = torch.randn(3, K, generator=g)
    xb = si.bits(x.to(torch.bfloat16) if dt == "bf16" else x)
    eye = np.eye(K, dtype=np.float32)
    split = [16, 8, 24]
    ws, off = [], 0
    for n in split:
        ws.append(_as_bits(dt, eye[off:off + n]))
        off += n
    res = oracle.fused_projection(xb, ws)
    xv = oracle.bf16_bits_to_f64(xb) if dt == "bf16" else oracle.f32_bits_to_f64(xb)
    off = 0
    for (y, s), n in zip(res, split):
        assert np.array_equal(y, xv[:, off:off + n])
        assert np.array_equal(s, np.abs(xv[:, off:off + n]))
        off += n


# ----------------------------------------- P-3: scaled permutation (gather)
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_scaled_permutation_is_a_gather(dt):
    rng = np.random.default_rng(11)
    K, N, M = 32, 20, 4
    perm = rng.permutation(K)[:N]
    expo = rng.integers(-6, 7, size=N)
    w = np.zeros((N, K), dtype=np.float32)
    for n in range(N):
        w[n, perm[n]] = 2.0 ** int(expo[n]) * (-1 if n % 3 == 0 else 1)
    g = torch.Generator().manual_seed(3)
    x = torch.randn(M, K, generator=g)
    xb = si.bits(x.to(torch.bfloat16) if dt == "bf16" else x)
    xv = oracle.bf16_bits_to_f64(xb) if dt == "bf16" else oracle.f32_bits_to_f64(xb)
    y, s = oracle.linear(xb, _as_bits(dt, w))
    for n in range(N):
        sc = 2.0 ** int(expo[n]) * (-1 if n % 3 == 0 else 1)
        assert np.array_equal(y[:, n], sc * xv[:, perm[n]])
        assert np.array_equal(s[:, n], abs(sc) * np.abs(xv[:, perm[n]]))


# --------------------------------------------- P-4: linearity on exact data
def test_linearity_exact():
    rng = np.random.default_rng(7)
    K, N, M = 64, 9, 3
    x1 = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    x2 = rng.integers(-8, 9, size=(M, K)).astype(np.float32)
    w = rng.integers(-8, 9, size=(N, K)).astype(np.float32) * 0.25
    a, b = 3.0, -0.5
    y1, _ = oracle.linear(_f32_bits(x1), _f32_bits(w))
    y2, _ = oracle.linear(_f32_bits(x2), _f32_bits(w))
    y12, _ = oracle.linear(_f32_bits(a * x1 + b * x2), _f32_bits(w))
    assert np.array_equal(y12, a * y1 + b * y2)
    # and in the weight argument
    w2 = rng.integers(-8, 9, size=(N, K)).astype(np.float32)
    yw, _ = oracle.linear(_f32_bits(x1), _f32_bits(w + 2 * w2))
    yw2, _ = oracle.linear(_f32_bits(x1), _f32_bits(w2))
    assert np.array_equal(yw, y1 + 2 * yw2)


# ------------------------------------- P-5: fused == split, page offsets
def _page_shapes():
    out = []
    with open(os.path.join(GOLDEN, "page_shapes.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            lhs, rhs = line.split("=")
            tok = lhs.split()
            out.append((tok[0], int(tok[1]), [int(v) for v in tok[2:]], int(rhs)))
    return out


@pytest.mark.parametrize("shape", _page_shapes(), ids=lambda s: s[0])
def test_page_concat_shapes(shape):
    name, K, rows, total = shape
    offs = oracle.row_offsets(rows)
    assert offs[0] == 0
    assert offs[-1] + rows[-1] == total
    # concatenation of row-index-tagged weights: row j of W_cat is row
    # (j - off_i) of projection i
    ws = [np.full((n, 2), i, dtype=np.uint32) for i, n in enumerate(rows)]
    for i, n in enumerate(rows):
        ws[i][:, 1] = np.arange(n, dtype=np.uint32)
    cat = oracle.concat_rows(ws)
    assert cat.shape == (total, 2)
    for i, (o, n) in enumerate(zip(offs, rows)):
        assert np.all(cat[o:o + n, 0] == i)
        assert np.array_equal(cat[o:o + n, 1], np.arange(n))


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_fused_equals_split(dt):
    x, ws = si.make_case(40, (7, 3, 5), dt, 3, seed=9,
                         w_dist="uniform_inv_sqrt_k" if dt == "bf16" else "normal_0.02")
    xb = si.bits(x)
    wb = [si.bits(w) for w in ws]
    ycat, scat = oracle.linear(xb, oracle.concat_rows(wb))
    for (y, s), o, w in zip(oracle.fused_projection(xb, wb),
                            oracle.row_offsets([w.shape[0] for w in wb]), wb):
        n = w.shape[0]
        assert np.array_equal(ycat[:, o:o + n], y)
        assert np.array_equal(scat[:, o:o + n], s)


# ------------------------------------------ P-6: integer data, exact sums
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_integer_data_exact(dt):
    x, ws = si.make_case(512, (33, 17), dt, 4, seed=2, w_dist="int4", x_dist="int4")
    xb = si.bits(x)
    xi = x.to(torch.float32).numpy().astype(np.int64)
    for w in ws:
        y, s = oracle.linear(xb, si.bits(w))
        wi = w.to(torch.float32).numpy().astype(np.int64)
        assert np.array_equal(y, (xi @ wi.T).astype(np.float64))
        assert np.array_equal(s, (np.abs(xi) @ np.abs(wi).T).astype(np.float64))


# ------------------------------------------ P-7: torch fp64 matmul (CPU)
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_matches_torch_fp64_matmul(dt):
    K = 5120 if dt == "bf16" else 7168
    x, ws = si.make_case(K, (64, 32), dt, 3, seed=4,
                         w_dist="uniform_inv_sqrt_k" if dt == "bf16" else "normal_0.02")
    xb = si.bits(x)
    for w in ws:
        y, s = oracle.linear(xb, si.bits(w))
        ref = (x.double() @ w.double().T).numpy()
        assert np.all(np.abs(y - ref) <= 2 * K * 2.0 ** -53 * s)


# ---------------------------------------- P-8: exact rationals, tiny inputs
@pytest.mark.parametrize("seed", range(6))
def test_exact_rational_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    K = int(rng.integers(1, 9))
    M, N = int(rng.integers(1, 4)), int(rng.integers(1, 5))
    # random bf16 patterns with biased exponents in [120, 136]: products
    # span at most 2^32 in magnitude with 16 significant bits each, so a sum
    # of <= 8 of them needs at most 32 + 16 + 3 < 53 bits and every fp64
    # partial sum of the oracle is exact
    def rand_bf16(shape):
        sign = rng.integers(0, 2, size=shape) << 15
        expo = rng.integers(120, 137, size=shape) << 7
        frac = rng.integers(0, 128, size=shape)
        return (sign | expo | frac).astype(np.uint16)
    x, w = rand_bf16((M, K)), rand_bf16((N, K))
    y, s = oracle.linear(x, w)
    ye, se = exact.linear_exact(x.tolist(), w.tolist(), 7)
    for m in range(M):
        for n in range(N):
            assert Fraction(y[m, n]) == ye[m][n]
            assert Fraction(s[m, n]) == se[m][n]


@pytest.mark.parametrize("seed", range(3))
def test_exact_rational_wide_range_within_fp64_bound(seed):
    # any finite exponents: the fp64 loop is within K * 2^-53 * S of exact
    rng = np.random.default_rng(200 + seed)
    K, M, N = 8, 2, 3
    def rand_bf16(shape):
        sign = rng.integers(0, 2, size=shape) << 15
        expo = rng.integers(1, 255, size=shape) << 7
        frac = rng.integers(0, 128, size=shape)
        return (sign | expo | frac).astype(np.uint16)
    x, w = rand_bf16((M, K)), rand_bf16((N, K))
    # keep products finite in fp64 (exponents up to 2^255 are fine)
    y, s = oracle.linear(x, w)
    ye, se = exact.linear_exact(x.tolist(), w.tolist(), 7)
    for m in range(M):
        for n in range(N):
            assert abs(Fraction(y[m, n]) - ye[m][n]) <= Fraction(K) * Fraction(2) ** -53 * se[m][n]


def test_exact_decode_matches_numpy_widening():
    rng = np.random.default_rng(1)
    pats = rng.integers(0, 1 << 16, size=2000).astype(np.uint16)
    pats = pats[((pats >> 7) & 0xFF) != 0xFF]  # finite only
    vals = oracle.bf16_bits_to_f64(pats)
    for p, v in zip(pats.tolist(), vals.tolist()):
        assert exact.decode_bf16(p) == Fraction(v)
    f32 = rng.integers(0, 1 << 32, size=2000, dtype=np.uint64).astype(np.uint32)
    f32 = f32[((f32 >> 23) & 0xFF) != 0xFF]
    for p, v in zip(f32.tolist(), oracle.f32_bits_to_f64(f32).tolist()):
        assert exact.decode_f32(p) == Fraction(v)


# --------------------------------------------------- bf16 rounding pins
def _golden_rounding():
    out = []
    with open(os.path.join(GOLDEN, "bf16_rounding.txt")) as fh:
        for line in fh:
            line = line.split("#", 1)[0].strip()
            if line:
                expr, hexv = line.split()
                out.append((expr, int(hexv, 16)))
    return out


@pytest.mark.parametrize("expr,pattern", _golden_rounding())
def test_round_bf16_golden(expr, pattern):
    v = float(eval(expr, {"__builtins__": {}}))  # arithmetic on literals only
    assert int(oracle.round_bf16([v])[0]) == pattern


def test_round_bf16_matches_torch_on_float32_values():
    # torch's float32 -> bfloat16 conversion is round-to-nearest-even; on
    # values that are exact float32 numbers it is a single rounding, as is
    # the oracle's rounding from the exact value.
    g = torch.Generator().manual_seed(0)
    f = torch.cat([torch.randn(20000, generator=g) * 10.0 ** e for e in range(-30, 31, 6)])
    bits = f.view(torch.int32)
    # add exact ties (lower 16 bits 0x8000) so ties-to-even is exercised
    ties = ((bits & ~0xFFFF) | 0x8000).view(torch.float32)
    f = torch.cat([f, ties])
    expect = si.bits(f.to(torch.bfloat16))
    got = oracle.round_bf16(f.double().numpy())
    assert np.array_equal(got, expect)


# ------------------------------------- P-9: the closed-form error bound
def test_fp32_accumulation_within_bound_and_errors_outside():
    # any fp32 summation order, rounded once to bf16, lies inside
    # 2^-7 S + 1e-6; a result with one term dropped or a 2^-6 relative
    # error lies outside it for at least one element.
    x, ws = si.make_case(5120, (64,), "bf16", 2, seed=12)
    xb, wb = si.bits(x), si.bits(ws[0])
    y, s = oracle.linear(xb, wb)
    xf = x.float().numpy()
    wf = ws[0].float().numpy()
    prods = (xf[:, None, :] * wf[None, :, :]).astype(np.float32)  # exact
    seq = np.cumsum(prods, axis=2, dtype=np.float32)[:, :, -1]       # sequential fp32
    rev = np.cumsum(prods[:, :, ::-1], axis=2, dtype=np.float32)[:, :, -1]
    for acc in (seq, rev):
        out = oracle.bf16_bits_to_f64(oracle.round_bf16(acc.astype(np.float64)))
        ok, worst, _ = oracle.check_within_bound(out, y, s, oracle.BF16)
        assert ok, worst
    dropped = prods[:, :, :-1].astype(np.float64).sum(axis=2)
    big = np.abs(prods[:, :, -1]) > 4 * (2.0 ** -7 * s + 1e-6)
    if big.any():
        ok, _, _ = oracle.check_within_bound(dropped, y, s, oracle.BF16)
        assert not ok
    ok, _, _ = oracle.check_within_bound(y + 2.0 ** -6 * s, y, s, oracle.BF16)
    assert not ok


def test_fp32_bound_holds_for_tree_order():
    x, ws = si.make_case(7168, (16,), "f32", 2, seed=3, w_dist="normal_0.02")
    xb, wb = si.bits(x), si.bits(ws[0])
    y, s = oracle.linear(xb, wb)
    p = (x.numpy()[:, None, :].astype(np.float32) * ws[0].numpy()[None, :, :]).astype(np.float32)
    # 64 interleaved fp32 partial sums then a pairwise tree (a GPU-like order)
    parts = p.reshape(2, 16, -1, 64).sum(axis=2, dtype=np.float32)
    while parts.shape[-1] > 1:
        parts = (parts[..., 0::2] + parts[..., 1::2]).astype(np.float32)
    ok, worst, _ = oracle.check_within_bound(parts[..., 0].astype(np.float64), y, s, oracle.F32)
    assert ok, worst


# ------------------------------ mutation sensitivity of the pins (CPU only)
def _definition(x, w, mutation=None):
    """Restatement of the oracle's definition used only to plant mistakes."""
    M, K = x.shape
    N = w.shape[0]
    y = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                if mutation == "drop_last" and k == K - 1:
                    continue
                xv = x[m, k]
                wv = w[n, k]
                if mutation == "sign" and k == 1:
                    wv = -wv
                if mutation == "transpose" and n < K and m < K:
                    wv = w[n, m] if m < w.shape[1] else wv
                if mutation == "index":
                    xv = x[m, (k + 1) % K]
                acc += xv * wv
            y[m, n] = acc
    return y


@pytest.mark.parametrize("mutation", ["drop_last", "sign", "transpose", "index"])
def test_pins_catch_planted_mistakes(mutation):
    caught = False
    for case in HAND:
        x = np.asarray(case["x"])
        for i, wl in case["w"].items():
            w = np.asarray(wl)
            good = _definition(x, w)
            bad = _definition(x, w, mutation)
            expect = np.asarray([case["y"][i][m] for m in range(x.shape[0])])
            assert np.array_equal(good, expect)
            if not np.array_equal(bad, expect):
                caught = True
    assert caught, mutation


def test_multicore_oracle_is_the_same_loop():
    # the OpenMP form spreads the output elements over threads; every
    # element is still the sequential k loop, so the results are bitwise
    # those of the single-threaded oracle (bf16 and fp32 patterns)
    rng = np.random.default_rng(21)
    for dt, mask in ((np.uint16, 0x3fff), (np.uint32, 0x3fffffff)):
        x = (rng.integers(0, 2 ** 31, (5, 300)) & mask).astype(dt)
        w = (rng.integers(0, 2 ** 31, (37, 288)) & mask).astype(dt)
        ya, sa = oracle.linear(x, w, K=288)
        yb, sb = oracle.linear_omp(np.ascontiguousarray(x[:, :288]), w)
        assert np.array_equal(ya, yb) and np.array_equal(sa, sb)
    assert oracle.omp_threads() >= 1
