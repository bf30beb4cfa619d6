"""Exact rational helpers used to pin the oracle (no oracle code here).

``round_to_f32`` rounds an exact rational to the nearest IEEE-754 single with
ties to even, including the subnormal range and overflow to infinity.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def round_to_f32(q: Fraction) -> np.float32:
    q = Fraction(q)
    if q == 0:
        return np.float32(0.0)
    neg = q < 0
    a = -q if neg else q
    # e with 2**e <= a < 2**(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    qexp = max(e - 23, -149)           # weight of the last significand bit
    scaled = a / (Fraction(2) ** qexp)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = Fraction(n) * (Fraction(2) ** qexp)
    if val >= Fraction(2) ** 128 - Fraction(2) ** 103:   # rounds to infinity
        out = np.float32(np.inf)
    else:
        out = np.float32(float(val))   # exact: n <= 2**24, exponent in range
    return np.float32(-out) if neg else out


def f32_bits(x) -> int:
    return int(np.asarray(x, dtype=np.float32).view(np.uint32))
