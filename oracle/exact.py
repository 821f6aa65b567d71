"""Exact-rational brute force of the projection, for tiny inputs.

TEST INFRASTRUCTURE ONLY (see the package docstring).  Decodes IEEE bit
patterns into ``fractions.Fraction`` from the format definition (sign,
biased exponent, fraction field; bias 127 for both bf16 and binary32, 7 and
23 fraction bits) and sums the products with no rounding at all.  It is an
independent check of ``oracle.c``'s fp64 loop: for K <= 8 bf16 inputs every
partial sum is exact in double too, so the two must agree exactly.
"""
from __future__ import annotations

from fractions import Fraction


def decode(bits: int, frac_bits: int) -> Fraction:
    """Value of an IEEE pattern with an 8-bit exponent (bias 127) and
    ``frac_bits`` fraction bits (7 for bf16, 23 for binary32).  Infinities
    and NaNs are rejected (they have no rational value)."""
    total = 1 + 8 + frac_bits
    bits = int(bits) & ((1 << total) - 1)
    sign = -1 if (bits >> (total - 1)) & 1 else 1
    exp = (bits >> frac_bits) & 0xFF
    frac = bits & ((1 << frac_bits) - 1)
    if exp == 0xFF:
        raise ValueError("inf/nan has no rational value")
    if exp == 0:  # subnormal: 0.frac * 2^(1-127)
        mant = Fraction(frac, 1 << frac_bits)
        e = 1 - 127
    else:
        mant = 1 + Fraction(frac, 1 << frac_bits)
        e = exp - 127
    scale = Fraction(2) ** e
    return sign * mant * scale


def decode_bf16(bits: int) -> Fraction:
    return decode(bits, 7)


def decode_f32(bits: int) -> Fraction:
    return decode(bits, 23)


def linear_exact(x_rows, w_rows, frac_bits: int):
    """``x_rows``: list of M lists of K patterns; ``w_rows``: N lists of K
    patterns.  Returns (y, S) as M x N lists of Fractions."""
    xs = [[decode(b, frac_bits) for b in row] for row in x_rows]
    ws = [[decode(b, frac_bits) for b in row] for row in w_rows]
    y, s = [], []
    for xr in xs:
        yr, sr = [], []
        for wr in ws:
            if len(wr) != len(xr):
                raise ValueError("row lengths differ")
            acc = Fraction(0)
            mag = Fraction(0)
            for a, b in zip(xr, wr):
                acc += a * b
                mag += abs(a * b)
            yr.append(acc)
            sr.append(mag)
        y.append(yr)
        s.append(sr)
    return y, s


def decode_e4m3(code: int) -> Fraction:
    """E4M3 from its definition: sign, 4 exponent bits (bias 7), 3 mantissa
    bits; exponent 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN."""
    code = int(code) & 0xFF
    sign = -1 if code >> 7 else 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 15 and m == 7:
        raise ValueError("NaN has no rational value")
    if e == 0:
        return sign * Fraction(m, 8) * Fraction(1, 2 ** 6)
    return sign * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def decode_e8m0(code: int) -> Fraction:
    code = int(code) & 0xFF
    if code == 255:
        raise ValueError("NaN has no rational value")
    return Fraction(2) ** (code - 127)


def linear_exact_mxfp8(x_rows, w_rows, K: int):
    """``x_rows``: M lists of >= K bf16 patterns; ``w_rows``: N packed rows
    (K E4M3 codes, then K/32 E8M0 scales).  Exact (y, S) as Fractions."""
    xs = [[decode(b, 7) for b in row[:K]] for row in x_rows]
    ws = []
    for row in w_rows:
        sc = [decode_e8m0(b) for b in row[K:K + K // 32]]
        ws.append([decode_e4m3(row[k]) * sc[k // 32] for k in range(K)])
    y, s = [], []
    for xr in xs:
        yr, sr = [], []
        for wr in ws:
            acc = sum((a * b for a, b in zip(xr, wr)), Fraction(0))
            mag = sum((abs(a * b) for a, b in zip(xr, wr)), Fraction(0))
            yr.append(acc)
            sr.append(mag)
        y.append(yr)
        s.append(sr)
    return y, s


def decode_e2m1(code: int) -> Fraction:
    """E2M1 (FP4) from its definition: sign, 2 exponent bits (bias 1), 1
    mantissa bit; exponent 0 is subnormal (m * 1/2); no NaN or infinity."""
    code = int(code) & 0xF
    sign = -1 if code >> 3 else 1
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        return sign * Fraction(m, 2)
    return sign * (1 + Fraction(m, 2)) * Fraction(2) ** (e - 1)


def linear_exact_mxfp4(x_rows, w_rows, K: int):
    """Packed MXFP4 rows (K/2 code bytes, low nibble first, then K/32
    scales); exact (y, S) as Fractions."""
    xs = [[decode(b, 7) for b in row[:K]] for row in x_rows]
    ws = []
    for row in w_rows:
        sc = [decode_e8m0(b) for b in row[K // 2:K // 2 + K // 32]]
        vals = []
        for k in range(K):
            byte = int(row[k // 2])
            code = (byte >> 4) if k % 2 else (byte & 0xF)
            vals.append(decode_e2m1(code) * sc[k // 32])
        ws.append(vals)
    y, s = [], []
    for xr in xs:
        y.append([sum((a * b for a, b in zip(xr, wr)), Fraction(0)) for wr in ws])
        s.append([sum((abs(a * b) for a, b in zip(xr, wr)), Fraction(0)) for wr in ws])
    return y, s


def linear_exact_nvfp4(x_rows, w_rows, K: int, g):
    """Packed NVFP4 rows (K/2 code bytes, low nibble first, then K/16 E4M3
    block scales), tensor scale ``g`` (a Fraction or an exactly
    representable float); exact (y, S) as Fractions."""
    g = Fraction(g)
    xs = [[decode(b, 7) for b in row[:K]] for row in x_rows]
    ws = []
    for row in w_rows:
        sc = [decode_e4m3(b) for b in row[K // 2:K // 2 + K // 16]]
        vals = []
        for k in range(K):
            byte = int(row[k // 2])
            code = (byte >> 4) if k % 2 else (byte & 0xF)
            vals.append(decode_e2m1(code) * sc[k // 16] * g)
        ws.append(vals)
    y, s = [], []
    for xr in xs:
        y.append([sum((a * b for a, b in zip(xr, wr)), Fraction(0)) for wr in ws])
        s.append([sum((abs(a * b) for a, b in zip(xr, wr)), Fraction(0)) for wr in ws])
    return y, s
