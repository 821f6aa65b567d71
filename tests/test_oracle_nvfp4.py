"""Pins of the oracle's NVFP4 projection: E2M1 codes two per byte (low
nibble first), one E4M3 scale per 16 elements along K, one fp32 scale per
tensor; packed rows of K/2 code bytes then K/16 scale bytes.

The pages' FP4 fused weight is the NVFP4 checkpoint of "Fuse QK down_proj
with indexer K + weight_proj for FP4 ckpt" (PR #8771, first titled as NVFP4
only) and of the GLM-5.2 NVFP4 target (PR #20502); they do not define the
encoding, read as the public two-level NVFP4 format.  Each pin is
independent of ``oracle.c``'s NVFP4 function: with a unit tensor scale the
result equals the already pinned bf16 projection of the weights dequantised
by the second decoder (``oracle/exact.py``: E2M1 times E4M3 has at most 6
significant bits, exact in bf16); a power-of-two tensor scale scales the
result exactly; any tensor scale agrees with exact rational arithmetic; one
block scale changes exactly its 16 elements; planted misreadings (a block of
32, the high nibble first, the tensor scale dropped) fail.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import exact
import synthetic_inputs as si


def _case(M, K, N, seed):
    g = torch.Generator().manual_seed(seed)
    (w,), (gs,) = si.draw_nvfp4_weights(K, (N,), g)
    x = si.draw_x(M, K, "bf16", g)
    return si.bits(x), si.bits(w), gs


def _dequant_bf16(w_packed, K, blk=16, swap=False):
    """Block-scaled E2M1 values (no tensor scale) as bf16 patterns, from the
    second decoder; asserts that each is exact in bf16."""
    N = w_packed.shape[0]
    out = np.zeros((N, K), dtype=np.uint16)
    for r in range(N):
        for k in range(K):
            byte = int(w_packed[r, k // 2])
            hi = (k % 2 == 1) != swap
            code = (byte >> 4) if hi else (byte & 0xF)
            sidx = min(k // blk, K // 16 - 1)
            v = exact.decode_e2m1(code) * exact.decode_e4m3(int(w_packed[r, K // 2 + sidx]))
            f = np.float32(float(v))
            assert Fraction(float(f)) == v
            b = int(np.array([f], dtype=np.float32).view(np.uint32)[0])
            assert b & 0xFFFF == 0, "not exact in bf16"
            out[r, k] = b >> 16
    return out


@pytest.mark.parametrize("M,K,N,seed", [(1, 16, 3, 0), (3, 64, 5, 1), (2, 160, 4, 2)])
def test_unit_tensor_scale_equals_bf16_projection_of_dequantised_weights(M, K, N, seed):
    x, w, _ = _case(M, K, N, seed)
    y, s = oracle.linear_nvfp4(x, w, K, 1.0)
    yb, sb = oracle.linear(x, _dequant_bf16(w, K))
    # the same exact products added in the same order in double
    assert np.array_equal(y, yb) and np.array_equal(s, sb)


def test_power_of_two_tensor_scale_is_exact():
    x, w, _ = _case(2, 96, 3, 3)
    y1, s1 = oracle.linear_nvfp4(x, w, 96, 1.0)
    for j in (-9, -1, 3):
        y, s = oracle.linear_nvfp4(x, w, 96, 2.0 ** j)
        assert np.array_equal(y, y1 * 2.0 ** j) and np.array_equal(s, s1 * 2.0 ** j)


@pytest.mark.parametrize("M,K,N,seed", [(2, 32, 3, 4), (1, 64, 4, 5)])
def test_brute_force_rationals_with_tensor_scale(M, K, N, seed):
    x, w, g = _case(M, K, N, seed)
    y, s = oracle.linear_nvfp4(x, w, K, g)
    ye, se = exact.linear_exact_nvfp4(x.tolist(), w.tolist(), K, Fraction(float(np.float32(g))))
    for m in range(M):
        for r in range(N):
            tol = K * 2.0 ** -53 * float(se[m][r])
            assert abs(Fraction(y[m, r]) - ye[m][r]) <= tol
            assert abs(Fraction(s[m, r]) - se[m][r]) <= tol


def test_hand_worked_row():
    # K = 16, one row: codes 1.0 (0x2) and -0.5 (0x9) alternating, block
    # scale 1.5 (E4M3 0x3C = 1.5 * 2^0), tensor scale 0.25; x = 1..16
    K = 16
    codes = np.array([0x2 | (0x9 << 4)] * 8, dtype=np.uint8)  # elements 1.0, -0.5, ...
    w = np.concatenate([codes, np.array([0x3C], dtype=np.uint8)])[None, :]
    xv = np.arange(1, 17, dtype=np.float32)
    x = (xv.view(np.uint32) >> 16).astype(np.uint16)[None, :]
    y, s = oracle.linear_nvfp4(x, w, K, 0.25)
    # sum over pairs (2i+1, 2i+2): (2i+1) * 1.0 - (2i+2) * 0.5 = i ... -> 0+1+..+7 = 28
    # times 1.5 * 0.25
    assert y[0, 0] == 28 * 1.5 * 0.25
    assert s[0, 0] == (sum(range(1, 17, 2)) * 1.0 + sum(range(2, 17, 2)) * 0.5) * 1.5 * 0.25


def test_one_block_scale_moves_exactly_its_16_elements():
    x, w, g = _case(2, 64, 3, 6)
    y, _ = oracle.linear_nvfp4(x, w, 64, g)
    w2 = w.copy()
    w2[:, 32 + 1] = 0x00  # block 1 (elements 16..31) scaled to zero
    y2, _ = oracle.linear_nvfp4(x, w2, 64, g)
    only = w.copy()
    only[:, :8] = 0       # codes of block 0
    only[:, 16:32] = 0    # codes of blocks 2, 3
    yb, _ = oracle.linear_nvfp4(x, only, 64, g)  # block 1's terms alone
    np.testing.assert_allclose(y - y2, yb, rtol=1e-12, atol=1e-300)


@pytest.mark.parametrize("mutation", ["block32", "nibble_swap", "no_tensor_scale"])
def test_planted_misreadings_fail(mutation):
    M, K, N = 2, 64, 3
    x, w, g = _case(M, K, N, 7)
    y, _ = oracle.linear_nvfp4(x, w, K, g)
    if mutation == "no_tensor_scale":
        yw, _ = oracle.linear(x, _dequant_bf16(w, K))
    elif mutation == "block32":
        yw, _ = oracle.linear(x, _dequant_bf16(w, K, blk=32))
        yw = yw * float(np.float32(g))
    else:
        yw, _ = oracle.linear(x, _dequant_bf16(w, K, swap=True))
        yw = yw * float(np.float32(g))
    assert not np.allclose(y, yw, rtol=1e-9, atol=0)
    # the right reading agrees
    yr, _ = oracle.linear(x, _dequant_bf16(w, K))
    np.testing.assert_allclose(y, yr * float(np.float32(g)), rtol=1e-13, atol=0)


def test_argument_checks():
    x, w, g = _case(1, 32, 2, 8)
    with pytest.raises(ValueError):
        oracle.linear_nvfp4(x, w[:, :16], 32, g)
    with pytest.raises(ValueError):
        oracle.linear_nvfp4(x, w, 24, g)
    with pytest.raises(ValueError):
        oracle.linear_nvfp4(x, w, 32, float("inf"))
