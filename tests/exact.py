"""Exact-arithmetic helpers for the oracle pins (CPU, no numpy float ops).

Correct rounding of an exact rational to fp32 / fp16 / bf16 is done by
comparing the rational against neighbouring representable values, so these
helpers do not depend on the arithmetic they are used to check.
"""
from __future__ import annotations

import math
from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np


def _round_to_format(x: Fraction, mant_bits: int, emin: int, emax: int) -> Fraction:
    """Round x to the binary format with ``mant_bits`` fraction bits, minimum
    normal exponent ``emin`` and maximum exponent ``emax``, ties to even."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    # exponent e with 2**e <= a < 2**(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)  # subnormals share the minimum exponent
    ulp = Fraction(2) ** (e - mant_bits)
    n = a / ulp
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * ulp
    if r >= Fraction(2) ** (emax + 1):
        raise OverflowError
    return sign * r


def rn32(x: Fraction) -> np.float32:
    return np.float32(_as_float(_round_to_format(Fraction(x), 23, -126, 127)))


def rn16(x: Fraction) -> np.float16:
    return np.float16(_as_float(_round_to_format(Fraction(x), 10, -14, 15)))


def rnbf16(x: Fraction) -> float:
    return _as_float(_round_to_format(Fraction(x), 7, -126, 127))


def _as_float(fr: Fraction) -> float:
    f = float(fr)  # exact: fr has at most 24 significant bits here
    assert Fraction(f) == fr
    return f


def F(v) -> Fraction:
    """Exact rational value of a numpy / Python float."""
    return Fraction(float(v))


def decimal_pow_ratio(a: float, b: float, alpha: float, digits: int = 60) -> Decimal:
    """a**alpha / b**(1-alpha) to ``digits`` significant digits (decimal ln/exp)."""
    getcontext().prec = digits
    da, db, al = Decimal(a), Decimal(b), Decimal(alpha)
    return (al * da.ln() - (Decimal(1) - al) * db.ln()).exp()


def rn32_decimal(d: Decimal) -> tuple[np.float32, float]:
    """Correct fp32 rounding of a high-precision decimal, and the relative
    distance of d from the nearest fp32 rounding midpoint."""
    fr = Fraction(d)
    f = rn32(fr)
    lo = np.nextafter(f, np.float32(-np.inf))
    hi = np.nextafter(f, np.float32(np.inf))
    mids = [(F(lo) + F(f)) / 2, (F(f) + F(hi)) / 2]
    dist = min(abs(fr - m) for m in mids) / abs(fr)
    return f, float(dist)


def ulp32(v: np.float32) -> float:
    v = np.float32(abs(v))
    return float(np.nextafter(v, np.float32(np.inf)) - v)


def ulp_f16(v: float) -> float:
    v = np.float16(abs(v))
    return float(np.nextafter(v, np.float16(np.inf))) - float(v)


def ulp_bf16(v: float) -> float:
    v = abs(float(v))
    if v == 0:
        return 2.0 ** -133
    e = max(math.floor(math.log2(v)), -126)
    return 2.0 ** (e - 7)
