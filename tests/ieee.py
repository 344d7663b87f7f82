"""Exact IEEE-754 binary32 rounding of rational numbers, from the standard's
definition (round to nearest, ties to even; gradual underflow).  Used by the
oracle pins as an implementation independent of both the C oracle and numpy's
float32 arithmetic: values are carried as exact Fractions and rounded once
per operation, as IEEE-754 prescribes for +, *, /.
"""
from fractions import Fraction
import math
import struct

EMIN = -126       # smallest normal exponent of binary32
P = 24            # significand bits of binary32


def rn32(v: Fraction) -> Fraction:
    """Round an exact rational to the nearest binary32 value (ties to even)."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, EMIN)
    ulp = Fraction(2) ** (e - (P - 1))
    m = a / ulp
    fl = math.floor(m)
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * ulp


def f32_bits_to_fraction(bits: int) -> Fraction:
    f = struct.unpack("<f", struct.pack("<I", bits & 0xFFFFFFFF))[0]
    return Fraction(f)


def bf16_bits_to_fraction(bits: int) -> Fraction:
    return f32_bits_to_fraction((bits & 0xFFFF) << 16)


def rne_int(v: Fraction) -> int:
    """Round a rational to the nearest integer, ties to even."""
    fl = math.floor(v)
    rem = v - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return int(fl)
