"""Exact rational helpers for pinning the oracle (test-only).

Everything here is written from the IEEE 754 definition of binary32
round-to-nearest-even, on Python Fractions, so it shares nothing with the C
oracle's floating-point arithmetic.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

EMIN = -126          # binary32 smallest normal exponent
PREC = 24            # binary32 significand bits


def floor_log2(a: Fraction) -> int:
    """Largest e with 2**e <= a, for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_half_even(v: Fraction) -> int:
    f = v.numerator // v.denominator
    rem = v - f
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and f % 2 == 1):
        f += 1
    return f


def to_f32(v: Fraction) -> Fraction:
    """Exact value of the binary32 nearest to v (ties to even), subnormals
    included.  Overflow is not modelled (not reachable in these tests)."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = max(floor_log2(a), EMIN)
    ulp = Fraction(2) ** (e - (PREC - 1))
    return sign * round_half_even(a / ulp) * ulp


def frac(x) -> Fraction:
    """Exact value of a binary32/binary64 number."""
    return Fraction(float(x))


def as_f32(v: Fraction) -> np.float32:
    f = np.float32(float(v))
    assert Fraction(float(f)) == v, "value is not a binary32"
    return f
