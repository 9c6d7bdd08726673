"""Exact rational arithmetic used to pin the oracle.

This is an independent route to the same numbers: Python Fractions and
integers, never the oracle's fp64 code.  round_fraction() implements
round-to-nearest-even into a binary format with p significand bits from
the exact rational value, by floor-and-compare on Fractions.
"""
import math
import struct
from fractions import Fraction

BF16 = dict(p=8, emin=-126, emax=127)
F32 = dict(p=24, emin=-126, emax=127)


def floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_fraction(r: Fraction, p: int, emin: int, emax: int):
    """Nearest representable value, ties to even, or +-inf on overflow.
    Returns a Fraction, or a float inf."""
    if r == 0:
        return Fraction(0)
    s = -1 if r < 0 else 1
    a = abs(r)
    e = max(floor_log2(a), emin)
    quantum = Fraction(2) ** (e - p + 1)
    q = a / quantum
    fl = math.floor(q)
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    res = fl * quantum
    max_finite = (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax
    if res > max_finite:
        return s * math.inf
    return s * res


def bf16_code_to_fraction(code: int):
    u = (int(code) & 0xFFFF) << 16
    f = struct.unpack("<f", struct.pack("<I", u))[0]
    if math.isnan(f) or math.isinf(f):
        return f
    return Fraction(f)


def f32_to_fraction(v):
    f = float(v)
    if math.isnan(f) or math.isinf(f):
        return f
    return Fraction(f)


def e4m3_code_to_fraction(code: int):
    """OCP e4m3fn from its bit fields (independent of the oracle's decoder)."""
    code = int(code) & 0xFF
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 15 and m == 7:
        return math.nan
    if e == 0:
        return s * Fraction(m, 8) * Fraction(2) ** -6
    return s * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def same(a, b) -> bool:
    """Equality that treats NaN == NaN and compares infinities."""
    if isinstance(a, float) and math.isnan(a):
        return isinstance(b, float) and math.isnan(b)
    return a == b


def fits_fp64(r: Fraction) -> bool:
    """True when r is exactly a finite binary64 value."""
    if r == 0:
        return True
    d = r.denominator
    if d & (d - 1):
        return False                      # not a dyadic rational
    n = abs(r.numerator)
    while n % 2 == 0:
        n //= 2
    if n.bit_length() > 53:
        return False
    lsb = floor_log2(abs(r)) - n.bit_length() + 1   # exponent of the last bit
    return lsb >= -1074 and floor_log2(abs(r)) <= 1023


def fp64_sum_bound(products):
    """Bound on |fl(sum) - sum| for a left-to-right fp64 sum of products that
    are each exact in fp64 (true for bf16 x bf16 and e4m3 x e4m3).  An
    addition whose exact result is a binary64 number is exact; any other
    rounds once, by at most 2^-53 of its result.  First-order bound with a
    factor 2 of slack."""
    bound = Fraction(0)
    partial = Fraction(0)
    for p in products:
        nxt = partial + p
        if not fits_fp64(nxt):
            bound += abs(nxt)
        partial = nxt
    return bound * Fraction(2, 2 ** 53)


def round_range(s: Fraction, bound: Fraction, fmt):
    """RNE is monotonic: every value in [s - bound, s + bound] rounds to a
    result between these two."""
    return round_fraction(s - bound, **fmt), round_fraction(s + bound, **fmt)
