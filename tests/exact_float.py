"""Exact binary floating-point rounding in rational arithmetic, for pinning
the oracle's FP32 / FP16 step sequences without NumPy's float arithmetic.

Every value is a ``fractions.Fraction``.  ``round_binary`` rounds a rational
to the nearest value of an IEEE binary format with p significand bits and
minimum normal exponent emin (subnormals included), ties to even; results
beyond the largest finite value become +-inf.  The E2M1 and E4M3 decoders
evaluate the OCP bit-field formulas (sign, exponent, mantissa), not a table.
Test infrastructure only.
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

F32 = (24, -126, 127)
F16 = (11, -14, 15)


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_binary(q: Fraction, fmt, mode: str = "rne"):
    """Nearest value of the binary format fmt = (p, emin, emax) to q; mode
    'rne' (ties to even) or 'trunc' (toward zero).  Returns a Fraction, or a
    float +-inf on overflow."""
    p, emin, emax = fmt
    if q == 0:
        return Fraction(0)
    neg = q < 0
    a = -q if neg else q
    e = max(_floor_log2(a), emin)
    quantum = Fraction(2) ** (e - p + 1)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if mode == "rne" and (rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1)):
        fl += 1
    r = fl * quantum
    max_finite = (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax
    if r > max_finite:
        return -math.inf if neg else math.inf
    return -r if neg else r


def rnd32(q):
    return round_binary(q, F32)


def rnd16(q, mode="rne"):
    return round_binary(q, F16, mode)


def f16_bits(v) -> int:
    """Bit pattern of an FP16-representable rational (or inf)."""
    return int(np.array(float(v), dtype=np.float16).view(np.uint16))


def frac(x) -> Fraction:
    """Exact rational value of a finite float (any width)."""
    return Fraction(float(x))


def e2m1_value(code: int) -> Fraction:
    """OCP E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0;
    exponent field 0 is subnormal (m * 2^-1)."""
    s = -1 if code & 8 else 1
    e, m = (code >> 1) & 3, code & 1
    mag = Fraction(m, 2) if e == 0 else (1 + Fraction(m, 2)) * Fraction(2) ** (e - 1)
    return s * mag


def e4m3_value(byte: int) -> Fraction:
    """OCP FP8 E4M3 ("fn"): sign bit 7, exponent bits 6..3 (bias 7),
    mantissa bits 2..0; exponent field 0 is subnormal (m/8 * 2^-6)."""
    s = -1 if byte & 0x80 else 1
    e, m = (byte >> 3) & 0xF, byte & 7
    if e == 0xF and m == 7:
        raise ValueError("E4M3 NaN")
    mag = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return s * mag


def nvfp4_element(codes, scales, r: int, c: int) -> Fraction:
    """Exact e2m1 * e4m3 value (no tensor scale) of element (r, c) of a
    packed NVFP4 matrix (element 2j in the low nibble of byte j)."""
    byte = int(codes[r, c // 2])
    code = byte & 0xF if c % 2 == 0 else byte >> 4
    return e2m1_value(code) * e4m3_value(int(scales[r, c // 16]))
