"""Exact rational arithmetic rounded to an IEEE-754 binary format.

Written here from the IEEE-754 definition of roundTiesToEven, independently
of the oracle: a value is the exact rational result of an operation, and it
is rounded once to the nearest representable value of a format with a p-bit
significand (implicit bit included), minimum normal exponent emin and maximum
exponent emax; ties go to the even significand; subnormals keep the fixed
quantum 2^(emin-p+1); magnitudes at or past the overflow threshold give inf.
"""
from fractions import Fraction
import math
import struct

import numpy as np

BINARY32 = (24, -126, 127)
BINARY16 = (11, -14, 15)
BFLOAT16 = (8, -126, 127)


def f32_to_fraction(x) -> Fraction:
    x = float(np.float32(x))
    if not math.isfinite(x):
        raise ValueError("not finite")
    return Fraction(x)


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # now 2^(e-1) < a < 2^(e+1); settle the exact floor
    if Fraction(2) ** e > a:
        e -= 1
    return e


def round_rne(q: Fraction, fmt, zero_sign_negative: bool = False) -> float:
    """Round the exact rational q to the format; returns a Python float whose
    value is exactly representable in that format (or +-inf).  When q == 0
    the sign of the zero is taken from ``zero_sign_negative``."""
    p, emin, emax = fmt
    if q == 0:
        return -0.0 if zero_sign_negative else 0.0
    neg = q < 0
    a = -q if neg else q
    e = max(_floor_log2(a), emin)
    quantum = Fraction(2) ** (e - p + 1)
    m = a / quantum
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if r >= Fraction(2) ** (emax + 1):
        v = math.inf
    else:
        v = float(r)
    if v == 0.0:
        # underflow to zero keeps the sign of the exact result
        return -0.0 if neg else 0.0
    return -v if neg else v


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def f16_bits(x: float) -> int:
    return int(np.array([x], np.float16).view(np.uint16)[0])


def sqrt_rne(q: Fraction, fmt) -> float:
    """The square root of the exact non-negative rational q, rounded once to
    the format (roundTiesToEven).  With 4^k scaling chosen so that every
    rounding boundary of the result is an integer multiple of 2^-k, the
    integer root r = isqrt(floor(q * 4^k)) brackets sqrt(q) * 2^k in
    [r, r + 1); an inexact root lies strictly inside, where (2r + 1) / 2
    rounds the same way."""
    if q < 0:
        raise ValueError("negative")
    if q == 0:
        return 0.0
    p = fmt[0]
    k = p + 4 - _floor_log2(q) // 2
    s = q * Fraction(4) ** k if k >= 0 else q / Fraction(4) ** (-k)
    t = s.numerator // s.denominator
    r = math.isqrt(t)
    exact = s.denominator == 1 and r * r == t
    root = Fraction(r) if exact else Fraction(2 * r + 1, 2)
    root = root / Fraction(2) ** k if k >= 0 else root * Fraction(2) ** (-k)
    return round_rne(root, fmt)
