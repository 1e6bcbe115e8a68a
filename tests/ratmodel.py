"""Exact-rational model of binary32 arithmetic, used only to pin the oracle.

It decides every rounding from the definitions (IEEE 754 binary32 round to
nearest, ties to even, including the subnormal grid) on exact fractions, so it
shares nothing with the oracle's C code or with numpy's float32 paths.
"""
from fractions import Fraction as F


def rne_int(fr: F) -> int:
    """Nearest integer to an exact rational, ties to even."""
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > F(1, 2):
        return fl + 1
    if rem < F(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def rnd32(fr: F) -> F:
    """The binary32 value nearest to fr (ties to even); finite range assumed."""
    if fr == 0:
        return F(0)
    sgn = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if F(2) ** e > a:
        e -= 1
    if F(2) ** (e + 1) <= a:
        e += 1
    e = max(e, -126)
    q = rne_int(a / F(2) ** (e - 23))
    return sgn * q * F(2) ** (e - 23)


def quantize(values, q_max=7):
    """eq. (1) with binary32 divisions: (s, codes) for a vector of exact rationals."""
    amax = max(abs(v) for v in values)
    s = rnd32(amax / q_max)
    if amax == 0:
        return s, [0] * len(values)
    return s, [max(-q_max, min(q_max, rne_int(rnd32(v / s)))) for v in values]
