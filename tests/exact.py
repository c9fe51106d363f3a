"""Exact rational arithmetic used to pin the oracle.

Nothing here imports the oracle or the HIP path. Values are Python
``fractions.Fraction``; rounding to a binary floating-point format is done
from the definition (nearest representable value, ties to the even
significand), with subnormals, so the oracle's numpy float32 arithmetic can be
checked against an independent route.
"""
from __future__ import annotations

import math
from decimal import Decimal, getcontext
from fractions import Fraction

F32 = (24, -126)    # significand bits (with the implicit one), min normal exponent
BF16 = (8, -126)


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_to(fr: Fraction, fmt=F32) -> Fraction:
    """Round a rational to the nearest value of a binary format, ties to even."""
    p, emin = fmt
    fr = Fraction(fr)
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = -fr if fr < 0 else fr
    e = max(_floor_log2(a), emin)
    quantum = Fraction(2) ** (e - (p - 1))
    n = a / quantum
    k = n.numerator // n.denominator
    rem = n - k
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and k % 2 == 1):
        k += 1
    return sign * k * quantum


def f32(fr) -> Fraction:
    return round_to(Fraction(fr), F32)


def bf16(fr) -> Fraction:
    return round_to(Fraction(fr), BF16)


def bf16_value(bits: int) -> Fraction:
    """Decode BF16 bits from the field definition (sign, 8-bit exponent,
    7-bit fraction), independently of any float reinterpretation."""
    bits = int(bits) & 0xFFFF
    sign = -1 if bits & 0x8000 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0xFF:
        raise ValueError("inf/nan")
    if e == 0:
        return sign * Fraction(m) * Fraction(2) ** (-126 - 7)
    return sign * Fraction(128 + m) * Fraction(2) ** (e - 127 - 7)


def bf16_bits(v: Fraction) -> int:
    """Encode an exactly representable BF16 value as bits."""
    v = Fraction(v)
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = -v if v < 0 else v
    e = _floor_log2(a)
    if e < -126:
        m = a / Fraction(2) ** (-133)
        assert m.denominator == 1 and m < 128
        return sign | int(m)
    m = a / Fraction(2) ** (e - 7)
    assert m.denominator == 1 and 128 <= m < 256, v
    return sign | ((e + 127) << 7) | (int(m) - 128)


def round_half_even(v: Fraction) -> int:
    return round(Fraction(v))     # Fraction.__round__ rounds half to even


def quant_scale(amax: Fraction) -> Fraction:
    return f32(Fraction(amax) / 127)


def quant_code(x: Fraction, s: Fraction) -> int:
    if s == 0:
        return 0
    q = round_half_even(f32(Fraction(x) / s))
    return max(-127, min(127, q))


def inv_sqrt_f32(v: Fraction, digits: int = 60) -> Fraction:
    """fl32(1/sqrt(v)) for a positive rational v, via high-precision decimals
    (60 digits leave the fp32 rounding decision unambiguous except at exact
    ties, which a 1/sqrt of a rational cannot hit unless it is rational)."""
    getcontext().prec = digits
    d = Decimal(v.numerator) / Decimal(v.denominator)
    r = Decimal(1) / d.sqrt()
    return f32(Fraction(r))


def f32_value(x: float) -> Fraction:
    return Fraction(float(x))


def is_finite(x: float) -> bool:
    return math.isfinite(x)
