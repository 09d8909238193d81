"""Exact rational rounding used by the oracle's pins (independent of numpy's
float32 arithmetic): round a Fraction to a binary floating-point format with
round-to-nearest, ties to even, including subnormals."""

from fractions import Fraction

import numpy as np


def round_to_binary(x: Fraction, mant_bits: int, emin: int) -> Fraction:
    """Nearest value with ``mant_bits`` significand bits (hidden bit included)
    and minimum normal exponent ``emin``; ties to an even significand.  No
    overflow handling (callers stay in range)."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - mant_bits + 1)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum


def to_f32(x: Fraction) -> np.float32:
    return np.float32(float(round_to_binary(x, 24, -126)))


def to_bf16_value(x: Fraction) -> float:
    return float(round_to_binary(x, 8, -126))


def f32_bits(v) -> int:
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0])


def frac(v) -> Fraction:
    return Fraction(float(v))
