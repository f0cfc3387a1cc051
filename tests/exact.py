"""Exact rational arithmetic helpers for the oracle's pins.

An independent way to evaluate IEEE fp32 / fp16 rounding: values are held
as ``fractions.Fraction`` and rounded to the nearest representable number
(ties to even) by integer arithmetic, not by NumPy or the FPU.
"""
from __future__ import annotations

import struct
from fractions import Fraction


def _round_to_format(r: Fraction, mant_bits: int, emin: int) -> Fraction:
    """Round r to a binary format with ``mant_bits`` significand bits (incl. the
    hidden one) and minimum normal exponent ``emin``; ties to even, gradual underflow."""
    if r == 0:
        return Fraction(0)
    sign = -1 if r < 0 else 1
    a = abs(r)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - (mant_bits - 1))
    q = a / ulp
    n = q.numerator // q.denominator
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def f32(r) -> Fraction:
    """Nearest IEEE binary32 value (ties to even, subnormals kept)."""
    return _round_to_format(Fraction(r), 24, -126)


def f16(r) -> Fraction:
    """Nearest IEEE binary16 value (ties to even, subnormals kept)."""
    return _round_to_format(Fraction(r), 11, -14)


def fp16_bits_struct(v: float) -> int:
    """binary16 bits of a Python float via the struct module's own conversion."""
    return struct.unpack("<H", struct.pack("<e", v))[0]


def floor_frac(r: Fraction) -> int:
    return r.numerator // r.denominator
