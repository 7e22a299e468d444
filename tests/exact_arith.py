"""Exact rational arithmetic used to pin the oracle.

IEEE-754 binary32 rounding and round-half-to-even written from their
definitions on Python Fractions, so a test can check a float32 computation
without repeating it in float32.
"""
from __future__ import annotations

from fractions import Fraction

F32_MIN_EXP = -126          # smallest normal exponent
F32_MANT = 23               # fraction bits
F32_MAX = (2 - Fraction(1, 2**23)) * Fraction(2) ** 127


def round_half_even(r: Fraction) -> int:
    fl = r.numerator // r.denominator
    rem = r - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 != 0):
        fl += 1
    return fl


def to_f32(r: Fraction) -> Fraction:
    """Nearest binary32 value to r (ties to even), subnormals kept.

    Raises OverflowError past the largest finite value.
    """
    if r == 0:
        return Fraction(0)
    sign = -1 if r < 0 else 1
    a = abs(r)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, F32_MIN_EXP)
    quantum = Fraction(2) ** (e - F32_MANT)
    v = round_half_even(a / quantum) * quantum
    if v > F32_MAX:
        raise OverflowError
    return sign * v


def f32_div(a: float, b: float) -> Fraction:
    """Correctly rounded binary32 quotient of two binary32 values."""
    return to_f32(Fraction(a) / Fraction(b))


def f32_mul(a: float, b: float) -> Fraction:
    return to_f32(Fraction(a) * Fraction(b))


def f32_add(a: float, b: float) -> Fraction:
    return to_f32(Fraction(a) + Fraction(b))


def to_bf16_bits(r: Fraction) -> int:
    """Nearest bfloat16 to r (ties to even), as its 16-bit pattern."""
    if r == 0:
        return 0
    sign = 0x8000 if r < 0 else 0
    a = abs(r)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, F32_MIN_EXP)
    quantum = Fraction(2) ** (e - 7)
    n = round_half_even(a / quantum)          # significand in units of quantum
    if n == 256:                               # carried into the next binade
        n = 128
        e += 1
    if e > 127:
        return sign | 0x7F80                   # infinity
    if n < 128:                                # subnormal (e == -126)
        return sign | n
    return sign | ((e + 127) << 7) | (n - 128)


F16_MIN_EXP = -14           # smallest normal exponent of binary16
F16_MANT = 10               # fraction bits of binary16


def to_f16_bits(r: Fraction) -> int:
    """Nearest IEEE binary16 to r (ties to even), as its 16-bit pattern.

    Rounds as if the exponent range were unbounded above, then a result past
    the largest finite value (65504) is infinity, which is the IEEE rule
    (everything from 65520 up overflows). Subnormals are kept.
    """
    if r == 0:
        return 0
    sign = 0x8000 if r < 0 else 0
    a = abs(r)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, F16_MIN_EXP)
    quantum = Fraction(2) ** (e - F16_MANT)
    n = round_half_even(a / quantum)          # significand in units of quantum
    if n == 2 * 2**F16_MANT:                   # carried into the next binade
        n = 2**F16_MANT
        e += 1
    if e > 15:
        return sign | 0x7C00                   # infinity
    if n < 2**F16_MANT:                        # subnormal (e == -14)
        return sign | n
    return sign | ((e + 15) << F16_MANT) | (n - 2**F16_MANT)
