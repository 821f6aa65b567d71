"""Pins of the oracle's MXFP8 projection (E4M3 codes, one E8M0 scale per 32
elements along K, packed rows of K codes then K/32 scales) and MXFP4
projection (E2M1 codes, two per byte, low nibble first, same scales).

The pages name MXFP8 projections for the DeepSeek-V4.1 wq_a / wkv weights
("tinygemm2 for the DeepSeek-V4.1 hidden-state projections", Description)
without defining the encoding; the reading is the open microscaling format.
Each pin is independent of ``oracle.c``: a table of code values worked by
hand from the format definition (``tests/golden/e4m3_e8m0.txt``), a second
decoder written from the definition in exact rationals (``oracle/exact.py``),
properties of the format (code order is magnitude order, 126 positive finite
values, 448 the largest), the already pinned bf16 projection on the exactly
dequantised weights (which has no scale blocks), power-of-two scale
linearity, and planted mistakes that the pins must catch.
"""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import exact
import synthetic_inputs as si

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "e4m3_e8m0.txt")


def _golden():
    e4, e8, e2 = [], [], []
    for line in open(GOLDEN):
        line = line.split("#", 1)[0].strip()
        if not line:
            continue
        kind, code, val = line.split()
        if kind == "e4m3":
            e4.append((int(code, 16), val))
        elif kind == "e2m1":
            e2.append((int(code, 16), val))
        else:
            e8.append((int(code), val))
    return e4, e8, e2


E4, E8, E2 = _golden()


def _parse(val):
    if val == "nan":
        return None
    if val == "-0":
        return Fraction(0)
    if val.startswith("2^"):
        return Fraction(2) ** int(val[2:])
    return Fraction(val)


@pytest.mark.parametrize("code,val", E4)
def test_e4m3_golden(code, val):
    want = _parse(val)
    got = oracle.e4m3_value(code)
    if want is None:
        assert np.isnan(got)
        with pytest.raises(ValueError):
            exact.decode_e4m3(code)
        return
    assert Fraction(got) == want
    assert exact.decode_e4m3(code) == want
    if val == "-0":
        assert np.signbit(got)


@pytest.mark.parametrize("code,val", E8)
def test_e8m0_golden(code, val):
    want = _parse(val)
    got = oracle.e8m0_value(code)
    if want is None:
        assert np.isnan(got)
        return
    assert Fraction(got) == want == exact.decode_e8m0(code)


def test_all_codes_two_decoders_and_format_properties():
    vals = []
    for c in range(256):
        v = oracle.e4m3_value(c)
        if c in (0x7F, 0xFF):
            assert np.isnan(v)
            continue
        assert Fraction(v) == exact.decode_e4m3(c), hex(c)
        vals.append(v)
    pos = [oracle.e4m3_value(c) for c in range(0x00, 0x7F)]
    # code order is magnitude order, sign is the top bit
    assert all(a < b for a, b in zip(pos, pos[1:]))
    assert all(oracle.e4m3_value(c | 0x80) == -oracle.e4m3_value(c) for c in range(0x7F))
    assert len([v for v in pos if v > 0]) == 126 and max(pos) == 448.0
    assert min(v for v in pos if v > 0) == 2.0 ** -9


def _dequant_bf16(w_packed, K):
    """Exactly dequantised weights as bf16 patterns (every E4M3 value times a
    power of two has at most 4 significant bits: exact in bf16 inside its
    exponent range)."""
    N = w_packed.shape[0]
    out = np.zeros((N, K), dtype=np.uint16)
    for r in range(N):
        for k in range(K):
            v = exact.decode_e4m3(int(w_packed[r, k])) * exact.decode_e8m0(
                int(w_packed[r, K + k // 32]))
            f = np.float32(float(v))
            assert Fraction(float(f)) == v
            out[r, k] = np.array([f], dtype=np.float32).view(np.uint32)[0] >> 16
            assert Fraction(float(np.array([int(out[r, k]) << 16], dtype=np.uint32)
                                  .view(np.float32)[0])) == v
    return out


def _case(M, K, N, seed):
    g = torch.Generator().manual_seed(seed)
    (w,) = si.draw_mxfp8_weights(K, (N,), g)
    x = si.draw_x(M, K, "bf16", g)
    return si.bits(x), si.bits(w)


@pytest.mark.parametrize("M,K,N,seed", [(1, 32, 3, 0), (3, 64, 5, 1), (2, 160, 4, 2)])
def test_mxfp8_equals_bf16_projection_of_dequantised_weights(M, K, N, seed):
    x, w = _case(M, K, N, seed)
    y, s = oracle.linear_mxfp8(x, w, K)
    yb, sb = oracle.linear(x, _dequant_bf16(w, K))
    # same exact products added in the same order in double: bitwise equal
    assert np.array_equal(y, yb) and np.array_equal(s, sb)


@pytest.mark.parametrize("M,K,N,seed", [(2, 32, 3, 3), (1, 64, 4, 4)])
def test_mxfp8_brute_force_rationals(M, K, N, seed):
    x, w = _case(M, K, N, seed)
    y, s = oracle.linear_mxfp8(x, w, K)
    ye, se = exact.linear_exact_mxfp8(x.tolist(), w.tolist(), K)
    for m in range(M):
        for r in range(N):
            tol = K * 2.0 ** -53 * float(se[m][r])
            assert abs(Fraction(y[m, r]) - ye[m][r]) <= tol
            assert abs(Fraction(s[m, r]) - se[m][r]) <= tol


def test_mxfp8_scale_is_a_power_of_two_per_block():
    x, w = _case(2, 96, 3, 5)
    y, _ = oracle.linear_mxfp8(x, w, 96)
    w2 = w.copy()
    w2[:, 96:] += 1  # every scale doubles
    y2, _ = oracle.linear_mxfp8(x, w2, 96)
    assert np.array_equal(y2, 2 * y)
    # one block's scale only: the change equals that block's contribution
    w3 = w.copy()
    w3[:, 96 + 1] += 1
    y3, _ = oracle.linear_mxfp8(x, w3, 96)
    blk = w.copy()
    blk[:, :32] = 0
    blk[:, 64:96] = 0
    yb, _ = oracle.linear_mxfp8(x, blk, 96)  # only block 1's terms
    np.testing.assert_allclose(y3 - y, yb, rtol=1e-12, atol=0)


def test_mxfp8_argument_checks():
    x, w = _case(1, 32, 2, 6)
    with pytest.raises(ValueError):
        oracle.linear_mxfp8(x, w[:, :32], 32)  # missing scale column
    with pytest.raises(ValueError):
        oracle.linear_mxfp8(x, w, 33)


# ----------------------------------------------------------- planted mistakes
def _decode_mut(code, mutation):
    code = int(code) & 0xFF
    sign = -1 if code >> 7 else 1
    e, m = (code >> 3) & 0xF, code & 7
    bias = 8 if mutation == "bias8" else 7
    if e == 0 and mutation != "no_subnormal":
        return sign * Fraction(m, 8) * Fraction(2) ** (1 - bias)
    return sign * (1 + Fraction(m, 8)) * Fraction(2) ** (e - bias)


@pytest.mark.parametrize("mutation", ["bias8", "no_subnormal"])
def test_planted_decode_mistakes_fail_the_golden_table(mutation):
    bad = 0
    for code, val in E4:
        want = _parse(val)
        if want is None:
            continue
        if _decode_mut(code, mutation) != want:
            bad += 1
    assert bad > 0


@pytest.mark.parametrize("mutation", ["block16", "block_shift"])
def test_planted_block_mistakes_fail_the_bf16_equivalence(mutation):
    M, K, N = 2, 96, 3
    x, w = _case(M, K, N, 7)
    yb, _ = oracle.linear(x, _dequant_bf16(w, K))
    xs = [[exact.decode(b, 7) for b in row] for row in x.tolist()]
    diff = False
    for m in range(M):
        for r in range(N):
            acc = Fraction(0)
            for k in range(K):
                if mutation == "block16":  # one scale per 16 elements
                    blk = min(k // 16, K // 32 - 1)
                else:  # block boundary off by one
                    blk = min(k // 32 + (k % 32 == 31), K // 32 - 1)
                acc += xs[m][k] * exact.decode_e4m3(int(w[r, k])) * exact.decode_e8m0(
                    int(w[r, K + blk]))
            diff |= abs(float(acc) - yb[m, r]) > 1e-12 * (1 + abs(yb[m, r]))
    assert diff


# ------------------------------------------------------------------- MXFP4
@pytest.mark.parametrize("code,val", E2)
def test_e2m1_golden(code, val):
    want = _parse(val)
    got = oracle.e2m1_value(code)
    assert Fraction(got) == want == exact.decode_e2m1(code)
    if val == "-0":
        assert np.signbit(got)
    # a byte holds two codes: the oracle reads only the nibble it is given
    assert oracle.e2m1_value(code | 0xF0) == got


def _dequant4_bf16(w_packed, K):
    N = w_packed.shape[0]
    out = np.zeros((N, K), dtype=np.uint16)
    for r in range(N):
        for k in range(K):
            byte = int(w_packed[r, k // 2])
            code = (byte >> 4) if k % 2 else (byte & 0xF)
            v = exact.decode_e2m1(code) * exact.decode_e8m0(int(w_packed[r, K // 2 + k // 32]))
            f = np.float32(float(v))
            assert Fraction(float(f)) == v
            out[r, k] = np.array([f], dtype=np.float32).view(np.uint32)[0] >> 16
    return out


def _case4(M, K, N, seed):
    g = torch.Generator().manual_seed(seed)
    (w,) = si.draw_mxfp4_weights(K, (N,), g)
    x = si.draw_x(M, K, "bf16", g)
    return si.bits(x), si.bits(w)


@pytest.mark.parametrize("M,K,N,seed", [(1, 32, 3, 10), (3, 64, 5, 11), (2, 160, 4, 12)])
def test_mxfp4_equals_bf16_projection_of_dequantised_weights(M, K, N, seed):
    x, w = _case4(M, K, N, seed)
    y, s = oracle.linear_mxfp4(x, w, K)
    yb, sb = oracle.linear(x, _dequant4_bf16(w, K))
    assert np.array_equal(y, yb) and np.array_equal(s, sb)


def test_mxfp4_brute_force_rationals():
    x, w = _case4(2, 64, 3, 13)
    y, _ = oracle.linear_mxfp4(x, w, 64)
    ye, se = exact.linear_exact_mxfp4(x.tolist(), w.tolist(), 64)
    for m in range(2):
        for r in range(3):
            assert abs(Fraction(y[m, r]) - ye[m][r]) <= 64 * 2.0 ** -53 * float(se[m][r])


def test_mxfp4_planted_nibble_swap_fails():
    # reading the high nibble first must change the result
    x, w = _case4(2, 64, 3, 14)
    y, _ = oracle.linear_mxfp4(x, w, 64)
    w2 = w.copy()
    w2[:, :32] = ((w[:, :32] >> 4) | (w[:, :32] << 4)) & 0xFF
    y2, _ = oracle.linear_mxfp4(x, w2, 64)
    assert not np.array_equal(y, y2)
    # and the bf16 equivalence pins the order: the swapped reading disagrees
    yb, _ = oracle.linear(x, _dequant4_bf16(w, 64))
    assert np.array_equal(y, yb) and not np.array_equal(y2, yb)


def test_mxfp4_argument_checks():
    x, w = _case4(1, 32, 2, 15)
    with pytest.raises(ValueError):
        oracle.linear_mxfp4(x, w[:, :16], 32)
