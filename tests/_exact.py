"""Exact-rational helpers for pinning the oracle (tests only).

Everything here works on ``fractions.Fraction`` and rounds by explicit
definition, independently of the C oracle and of the HIP library.
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

import numpy as np


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def frac_of_float(x: float) -> Fraction:
    return Fraction(x)  # exact for any finite binary float


def round_to_binary(q: Fraction, sig_bits: int, emin: int) -> Fraction:
    """Round a rational to the nearest value with ``sig_bits`` significand bits
    (including the hidden bit) and minimum normal exponent ``emin``, gradual
    underflow, ties to even, no overflow handling (callers stay in range)."""
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = math.floor(math.log2(a.numerator) - math.log2(a.denominator))
    # fix floating log2 error
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - (sig_bits - 1))
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum


def rn32(q: Fraction) -> Fraction:
    return round_to_binary(q, 24, -126)


def rn64(q: Fraction) -> Fraction:
    return round_to_binary(q, 53, -1022)


def rnbf16(q: Fraction) -> Fraction:
    return round_to_binary(q, 8, -126)


E2M1_MAGS = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
             Fraction(4), Fraction(6)]


def e4m3_values():
    """The 127 finite non-negative E4M3 values in byte order, from the layout:
    4 exponent bits (bias 7), 3 mantissa bits, exponent 0 subnormal, 0x7F NaN."""
    vals = []
    for b in range(127):
        e, m = b >> 3, b & 7
        if e == 0:
            vals.append(Fraction(m, 8) * Fraction(1, 2 ** 6))
        else:
            vals.append((1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))
    return vals


E4M3_VALS = e4m3_values()


def nearest_even(t: Fraction, table) -> int:
    """Index of the nearest table value; ties to the even index; saturate at top."""
    if t >= table[-1]:
        return len(table) - 1
    best = None
    for i, v in enumerate(table):
        dist = abs(t - v)
        if best is None or dist < best[0] or (dist == best[0] and i % 2 == 0):
            best = (dist, i)
    return best[1]


def quantize_row_exact(x):
    """Independent exact-arithmetic model of the row quantizer: inputs are
    binary32 values (as Python floats); each binary32 operation is an exact
    rational followed by ``rn32``; roundings onto E4M3/E2M1 are done by
    scanning the value tables.  Returns (codes list (0..15), scale bytes, d)."""
    xs = [Fraction(v) for v in x]
    A = max((abs(v) for v in xs), default=Fraction(0))
    d = rn32(A / 2688)
    n = len(xs)
    if d == 0:
        codes = [8 if math.copysign(1.0, v) < 0 else 0 for v in x]
        return codes, [0] * (n // 16), d
    D = rn32(6 * d)
    codes, scales = [], []
    for b in range(n // 16):
        blk = xs[16 * b:16 * b + 16]
        Ab = max(abs(v) for v in blk)
        t = rn32(Ab / D)
        sb = nearest_even(t, E4M3_VALS)
        scales.append(sb)
        S = rn32(E4M3_VALS[sb] * d)
        for j, v in enumerate(blk):
            mag = 0 if S == 0 else nearest_even(rn32(abs(v) / S), E2M1_MAGS)
            neg = math.copysign(1.0, x[16 * b + j]) < 0
            codes.append((8 if neg else 0) | mag)
    return codes, scales, d


def unpack_codes(packed: np.ndarray) -> np.ndarray:
    """[rows, cols/2] bytes -> [rows, cols] codes (element 2j = low nibble)."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = packed & 15
    out[..., 1::2] = packed >> 4
    return out


def pack_codes(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
