"""Exact-arithmetic helpers for pinning the oracle (test code only).

Roundings are written from the IEEE 754 definition on exact rationals
(fractions.Fraction), independent of the oracle's bit manipulations.
"""
from __future__ import annotations

import math
from decimal import Decimal, localcontext
from fractions import Fraction

import numpy as np


def _round_half_even(q: Fraction) -> int:
    fl = math.floor(q)
    rem = q - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # adjust so that 2^e <= a < 2^(e+1)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_binary(q: Fraction, mant_bits: int, emin: int, emax: int) -> float:
    """Round a rational to the nearest value of a binary format with
    `mant_bits` significand bits (including the hidden bit), minimum normal
    exponent emin and maximum exponent emax; ties to even; overflow -> inf."""
    if q == 0:
        return 0.0
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    e = max(_floor_log2(a), emin)
    quantum = Fraction(2) ** (e - (mant_bits - 1))
    m = _round_half_even(a / quantum)
    v = m * quantum
    # largest finite: (2 - 2^(1-mant_bits)) * 2^emax
    maxf = (2 - Fraction(2) ** (1 - mant_bits)) * Fraction(2) ** emax
    if v > maxf:
        return sign * math.inf
    return sign * float(v)


def rn32(q: Fraction) -> float:
    return round_binary(q, 24, -126, 127)


def rnbf16(q: Fraction) -> float:
    return round_binary(q, 8, -126, 127)


def exp_decimal(x: Fraction, digits: int = 60) -> Fraction:
    """exp(x) to `digits` significant digits (decimal's exp is correctly
    rounded at the context precision), as an exact Fraction of that decimal."""
    with localcontext() as ctx:
        ctx.prec = digits
        ctx.Emax = 10 ** 6
        ctx.Emin = -10 ** 6
        d = (Decimal(x.numerator) / Decimal(x.denominator)).exp()
        return Fraction(d)


def bf16_bits_value(b: int) -> float:
    return float(np.array([b << 16], dtype=np.uint32).view(np.float32)[0])


def f32_bits(v: float) -> int:
    return int(np.array([v], dtype=np.float32).view(np.uint32)[0])
