"""Exact rational arithmetic used to pin the oracle: an independent second derivation of every
rounding decision, written with ``fractions.Fraction`` and no numpy floating point."""
from __future__ import annotations

from fractions import Fraction


def round_to_binary(v: Fraction, mant_bits: int, min_exp: int) -> Fraction:
    """Round ``v`` to the nearest binary floating-point value with ``mant_bits`` fraction bits and
    smallest normal exponent ``min_exp`` (subnormals included), ties to an even last bit."""
    if v == 0:
        return Fraction(0)
    sign = -1 if v < 0 else 1
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, min_exp)
    ulp = Fraction(2) ** (e - mant_bits)
    m = a / ulp
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return sign * lo * ulp


def to_f32(v: Fraction) -> Fraction:
    return round_to_binary(v, 23, -126)


def to_bf16(v: Fraction) -> Fraction:
    return round_to_binary(v, 7, -126)


def nearest_index(r: Fraction, codes) -> int:
    """Index of the code nearest to ``r``; on an exact tie the lower index."""
    best_i, best_d = 0, None
    for i, c in enumerate(codes):
        d = abs(r - Fraction(c))
        if best_d is None or d < best_d:
            best_i, best_d = i, d
    return best_i
