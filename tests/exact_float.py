"""Exact rational rounding to binary floating-point formats (IEEE round-to-nearest,
ties to even), used to check the oracle's fp32/fp16 steps by a route that never
touches numpy's float arithmetic."""
from fractions import Fraction

FP32 = (24, -126)   # significand bits (incl. hidden), minimum normal exponent
FP16 = (11, -14)


def round_float(x: Fraction, fmt) -> Fraction:
    p, emin = fmt
    x = Fraction(x)
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - (p - 1))
    return sign * round(a / ulp) * ulp      # Fraction.__round__ is half-to-even


def rne_int(x: Fraction) -> int:
    return round(Fraction(x))
