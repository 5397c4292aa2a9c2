"""Exact-rational arithmetic used to pin the oracle.

Nothing here calls numpy's floating-point arithmetic: values are Python
Fractions, and rounding to a binary float format is done by hand (round to
nearest, ties to even, gradual underflow).  An IEEE operation "fp32(a / b)" is
then round_f32(Fraction(a) / Fraction(b)), which is its definition.
"""
from fractions import Fraction

TWO = Fraction(2)


def _round_binary(r: Fraction, mant_bits: int, emin: int) -> Fraction:
    if r == 0:
        return Fraction(0)
    sign = -1 if r < 0 else 1
    a = abs(r)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while TWO ** e > a:
        e -= 1
    while TWO ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    ulp = TWO ** (e - (mant_bits - 1))
    n = round(a / ulp)          # Fraction.__round__: half to even
    return sign * n * ulp


def round_f32(r: Fraction) -> Fraction:
    return _round_binary(Fraction(r), 24, -126)


def round_f16(r: Fraction) -> Fraction:
    return _round_binary(Fraction(r), 11, -14)


def clamp(v: int, lo: int, hi: int) -> int:
    return max(lo, min(hi, v))


def quant_row(row):
    """Per-token int8 quantisation of one row of fp16 values, exactly.

    s = fp32(absmax / 127); q = clamp(rne(fp32(x / s)), -127, 127);
    a zero row gives s = 0 and q = 0.  Returns (list of int, Fraction s).
    """
    xs = [Fraction(float(v)) for v in row]
    a = max((abs(v) for v in xs), default=Fraction(0))
    if a == 0:
        return [0] * len(xs), Fraction(0)
    s = round_f32(a / 127)
    return [clamp(round(round_f32(v / s)), -127, 127) for v in xs], s


def quant_group(vals):
    """int8 table quantisation of one 128-value group, exactly.

    S = fp16(fp32(absmax / 127)); Q = clamp(rne(fp32(v / S)), -127, 127);
    S == 0 gives Q = 0.  Returns (list of int, Fraction S).
    """
    xs = [Fraction(float(v)) for v in vals]
    a = max(abs(v) for v in xs)
    S = round_f16(round_f32(a / 127))
    if S == 0:
        return [0] * len(xs), Fraction(0)
    return [clamp(round(round_f32(v / S)), -127, 127) for v in xs], S
