"""Exact rational arithmetic for pinning the oracle (tests only).

Rounding to float32 and bfloat16 is written here from the IEEE-754
definition on Python Fractions: find the binade, scale to an integer
significand, round half to even.  Nothing here calls numpy's float32
arithmetic, so it is an independent check of the oracle's float32 steps.
"""
from __future__ import annotations

from fractions import Fraction


def _round_half_even(q: Fraction) -> int:
    n = q.numerator // q.denominator          # floor
    rem = q - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def round_float(x: Fraction, sig_bits: int, emin: int) -> Fraction:
    """Nearest value with `sig_bits` significant bits (normal exponent >=
    emin, gradual underflow below), ties to even.  No overflow handling."""
    if x == 0:
        return Fraction(0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # fix e so that 2**e <= a < 2**(e+1)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = Fraction(2) ** (e - (sig_bits - 1))
    return sign * _round_half_even(a / ulp) * ulp


def to_f32(x: Fraction) -> Fraction:
    return round_float(x, 24, -126)


def to_bf16(x: Fraction) -> Fraction:
    return round_float(x, 8, -126)


E2M1_MAGS = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
             Fraction(3), Fraction(4), Fraction(6)]


def e2m1_code_by_thresholds(v: Fraction, negative: bool) -> int:
    """E2M1 magnitude by the decision points of round-to-nearest-even on the
    grid: ties at 0.25, 1.25, 2.5 and 5 go down (to codes 0, 2, 4, 6) and
    ties at 0.75, 1.75 and 3.5 go up (to codes 2, 4, 6)."""
    a = abs(v)
    m = (int(a > Fraction(1, 4)) + int(a >= Fraction(3, 4)) + int(a > Fraction(5, 4))
         + int(a >= Fraction(7, 4)) + int(a > Fraction(5, 2)) + int(a >= Fraction(7, 2))
         + int(a > 5))
    return (8 if negative else 0) | m


def e4m3_values():
    """All non-negative finite E4M3 values, from the bit layout."""
    out = []
    for c in range(0x7F):
        e, f = c >> 3, c & 7
        out.append(Fraction(f, 8) * Fraction(2) ** -6 if e == 0
                   else (1 + Fraction(f, 8)) * Fraction(2) ** (e - 7))
    return out


def e4m3_round(u: Fraction) -> int:
    vals = e4m3_values()
    if u >= vals[-1]:
        return 0x7E
    best = min(range(len(vals)), key=lambda c: (abs(vals[c] - u), c % 2))
    return best


def quantize_block_exact(xs, A: Fraction):
    """One block through the scale recipe with every float32 step rounded
    explicitly.  xs: list of Fractions (bf16 values); A: tensor amax."""
    a_b = max(abs(x) for x in xs)
    u = to_f32(to_f32(a_b * 448) / A)
    sc = e4m3_round(u)
    s = e4m3_values()[sc]
    codes = []
    for x in xs:
        neg = x < 0 or (x == 0 and False)
        if s == 0:
            codes.append(8 if neg else 0)
            continue
        rho = to_f32(Fraction(2688) / to_f32(s * A))
        v = to_f32(x * rho)
        codes.append(e2m1_code_by_thresholds(v, neg))
    return codes, sc
