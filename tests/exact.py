"""Exact rational helpers for pinning the oracle (test-only).

These decode stored formats and round rationals to fp32 independently of the
oracle's C code, so the oracle can be compared against exact arithmetic.
"""
from fractions import Fraction

import numpy as np


def f32_value(x) -> Fraction:
    """Exact value of an fp32 number."""
    return Fraction(float(np.float32(x)))


def f16_bits_value(h: int) -> Fraction:
    """Exact value of IEEE binary16 bits (finite only)."""
    h = int(h)
    sign = -1 if (h >> 15) & 1 else 1
    e = (h >> 10) & 0x1F
    m = h & 0x3FF
    assert e != 31
    if e == 0:
        return sign * Fraction(m, 1 << 24)
    return sign * Fraction(1024 + m, 1 << 10) * (Fraction(2) ** (e - 15))


def bf16_bits_value(h: int) -> Fraction:
    """Exact value of bfloat16 bits (finite only)."""
    h = int(h)
    sign = -1 if (h >> 15) & 1 else 1
    e = (h >> 7) & 0xFF
    m = h & 0x7F
    assert e != 255
    if e == 0:
        return sign * Fraction(m, 1 << 7) * (Fraction(2) ** -126)
    return sign * Fraction(128 + m, 128) * (Fraction(2) ** (e - 127))


def f32_rne(v: Fraction) -> Fraction:
    """Round an exact rational to the nearest fp32 value, ties to even."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (max(e, -126) - 23)
    q = a / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def exact_chain(x, a, b, relu_even, round_each_stage=False):
    """The K-stage chain in exact rational arithmetic (optionally rounding to
    fp32 after every stage, modelling one rounding per stage)."""
    v = f32_value(x)
    for s in range(len(a)):
        v = f32_value(a[s]) * v + f32_value(b[s])
        if round_each_stage:
            v = f32_rne(v)
        if relu_even and s % 2 == 0 and v < 0:
            v = Fraction(0)
    return v
