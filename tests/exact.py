"""Exact rational rounding helpers used only to pin the oracle.

Independent of ``oracle/``: rounding of an exact rational to a binary floating
format is written here from the IEEE definition (nearest representable value,
ties to the even significand), for any significand width and exponent range.
"""

from fractions import Fraction
import math


def round_to_format(q: Fraction, sig_bits: int, emin: int, max_finite: Fraction | None,
                    saturate: bool):
    """Nearest value of a binary format to the rational q, ties to even.

    sig_bits counts the implicit bit; emin is the exponent of the smallest
    normal binade; values below it use the fixed subnormal spacing
    2^(emin - sig_bits + 1).  Returns a Fraction, or +/-inf when the value
    overflows and saturate is False.
    """
    if q == 0:
        return Fraction(0)
    neg = q < 0
    a = -q if neg else q
    # binade exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    elif Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - sig_bits + 1)
    n = a / quantum
    fl = math.floor(n)
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    r = fl * quantum
    if max_finite is not None and r > max_finite:
        if saturate:
            r = max_finite
        else:
            return float("-inf") if neg else float("inf")
    return -r if neg else r


E4M3_MAX = Fraction(448)
F32_MAX = (2 - Fraction(2) ** -23) * Fraction(2) ** 127


def to_e4m3_value(q: Fraction) -> Fraction:
    return round_to_format(q, 4, -6, E4M3_MAX, saturate=True)


def to_f32_value(q: Fraction) -> Fraction:
    return round_to_format(q, 24, -126, F32_MAX, saturate=False)


def to_bf16_value(q: Fraction) -> Fraction:
    return round_to_format(q, 8, -126, (2 - Fraction(2) ** -7) * Fraction(2) ** 127,
                           saturate=False)


def e4m3_code_of_value(v: Fraction, negative_zero=False) -> int:
    """Code of a representable E4M3 value, from the format's field layout."""
    neg = v < 0 or (v == 0 and negative_zero)
    a = -v if v < 0 else v
    if a == 0:
        code = 0
    elif a < Fraction(2) ** -6:
        code = int(a / Fraction(2) ** -9)
    else:
        e = a.numerator.bit_length() - a.denominator.bit_length()
        if Fraction(2) ** e > a:
            e -= 1
        m = (a / Fraction(2) ** e - 1) * 8
        assert m.denominator == 1
        code = ((e + 7) << 3) | int(m)
    return code | (0x80 if neg else 0)


def e4m3_value_of_code(code: int) -> Fraction:
    """Exact value of a finite E4M3 code from its fields (NaN codes raise)."""
    s, e, m = (code >> 7) & 1, (code >> 3) & 0xF, code & 7
    if e == 0xF and m == 7:
        raise ValueError("NaN code")
    if e == 0:
        v = Fraction(m, 8) * Fraction(2) ** -6
    else:
        v = (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if s else v


def e4m3_int9(code: int) -> int:
    """The code's value times 2^9, an integer for every finite code."""
    v = e4m3_value_of_code(code) * 512
    assert v.denominator == 1
    return int(v)
