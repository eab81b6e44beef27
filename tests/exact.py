"""Exact rational arithmetic for pinning the oracle.

Everything here works on ``fractions.Fraction`` values and rounds with its own
round-to-nearest-even routine, so it shares nothing with the C float operations
or libm that the oracle uses. ``exp`` comes from mpmath at high precision, with a
check that the rounding decision is certain.
"""

from __future__ import annotations

import math
import struct
from fractions import Fraction

import mpmath

F32 = (24, -126, 127)  # precision, minimum normal exponent, maximum exponent
BF16 = (8, -126, 127)
F16 = (11, -14, 15)


def _floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def round_nearest_even(q: Fraction, fmt=F32, negative_zero: bool = False) -> float:
    """Round an exact rational to the binary format ``fmt``; ties to even.

    Returns a Python float holding the rounded value exactly (or +-inf). A zero
    input returns -0.0 when ``negative_zero`` is set.
    """
    p, emin, emax = fmt
    if q == 0:
        return -0.0 if negative_zero else 0.0
    neg = q < 0
    a = -q if neg else q
    e = max(_floor_log2(a), emin)
    quantum = Fraction(2) ** (e - p + 1)
    m = a / quantum
    n = m.numerator // m.denominator
    r = m - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    val = n * quantum
    if val >= Fraction(2) ** (emax + 1):
        return -math.inf if neg else math.inf
    f = float(val)
    assert Fraction(f) == val
    if f == 0.0:
        return -0.0 if neg else 0.0
    return -f if neg else f


def rn32(q: Fraction) -> float:
    return round_nearest_even(q, F32)


def fma32(a: float, b: float, c: float) -> float:
    """Fused multiply-add of binary32 values, exact product and sum, one rounding."""
    prod = Fraction(a) * Fraction(b)
    s = prod + Fraction(c)
    if s == 0:
        prod_neg = (math.copysign(1.0, a) * math.copysign(1.0, b)) < 0
        if prod == 0 and c == 0:
            return -0.0 if (prod_neg and math.copysign(1.0, c) < 0) else 0.0
        return 0.0  # exact cancellation of nonzero terms gives +0 under round to nearest
    return rn32(s)


def add32(a: float, b: float) -> float:
    if math.isinf(a) or math.isinf(b):
        return a + b
    s = Fraction(a) + Fraction(b)
    if s == 0:
        return -0.0 if (math.copysign(1.0, a) < 0 and math.copysign(1.0, b) < 0) else 0.0
    return rn32(s)


def div32(a: float, b: float) -> float:
    if math.isinf(b):
        if math.isinf(a):
            return math.nan
        return math.copysign(0.0, a) * math.copysign(1.0, b)
    if math.isinf(a):
        return math.copysign(math.inf, a) * math.copysign(1.0, b)
    q = Fraction(a) / Fraction(b)
    neg = (math.copysign(1.0, a) * math.copysign(1.0, b)) < 0
    return round_nearest_even(q, F32, negative_zero=neg)


def _mpf_to_fraction(v: mpmath.mpf) -> Fraction:
    sign, man, exp, _ = v._mpf_
    f = Fraction(int(man)) * (Fraction(2) ** int(exp))
    return -f if sign else f


def exp32(x: float, prec: int = 200) -> float:
    """exp(x) correctly rounded to binary32, from an mpmath value at ``prec`` bits.

    The rounding is done on the value shifted down and up by a bound on mpmath's
    error; both must round the same way, else the case is reported as uncertain.
    """
    if math.isnan(x):
        return math.nan
    if math.isinf(x):
        return 0.0 if x < 0 else math.inf
    # exp(-200) is far below half the smallest subnormal (2^-150) and exp(200) far
    # above the largest binary32; keep mpmath away from huge arguments.
    if x < -200.0:
        return 0.0
    if x > 200.0:
        return math.inf
    with mpmath.workprec(prec):
        v = mpmath.exp(mpmath.mpf(x))
        q = _mpf_to_fraction(v)
    slack = q / (Fraction(2) ** (prec - 8))
    lo, hi = rn32(q - slack), rn32(q + slack)
    if lo != hi:
        raise ArithmeticError(f"exp({x!r}) too close to a binary32 midpoint at {prec} bits")
    return lo


def f32(x) -> float:
    """Round a Python number to the nearest binary32 value (via struct, exact for floats)."""
    return struct.unpack("<f", struct.pack("<f", x))[0]


def bits32(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def from_bits32(u: int) -> float:
    return struct.unpack("<f", struct.pack("<I", u & 0xFFFFFFFF))[0]


def bf16_word(y: float) -> int:
    """bf16 bit pattern of the binary32 value y rounded to bf16 (NaN -> 0x7FC0)."""
    if math.isnan(y):
        return 0x7FC0
    if math.isinf(y):
        return 0xFF80 if y < 0 else 0x7F80
    r = round_nearest_even(Fraction(y), BF16, negative_zero=math.copysign(1.0, y) < 0)
    return bits32(r) >> 16


def f16_word(y: float) -> int:
    """binary16 bit pattern of the binary32 value y rounded to binary16 (NaN -> 0x7E00).

    Rounds the exact rational value to 11 significant bits with binary16's exponent
    range (subnormals in steps of 2^-24, overflow to infinity); the encoding of the
    rounded value is struct's "e" format, exact for a representable value."""
    if math.isnan(y):
        return 0x7E00
    if math.isinf(y):
        return 0xFC00 if y < 0 else 0x7C00
    r = round_nearest_even(Fraction(y), F16, negative_zero=math.copysign(1.0, y) < 0)
    if math.isinf(r):
        return 0xFC00 if r < 0 else 0x7C00
    return struct.unpack("<H", struct.pack("<e", r))[0]


def f32_word(y: float) -> int:
    """The stored FP32 word of a binary32 value (NaN -> 0x7FC00000)."""
    return 0x7FC00000 if math.isnan(y) else bits32(y)


WORDS = {"bf16": bf16_word, "f16": f16_word, "f32": f32_word}


def silu32(a: float) -> float:
    """SiLU a / (1 + exp(-a)) with exp correctly rounded and each step rounded to binary32."""
    if math.isnan(a):
        return math.nan
    e = exp32(-a)
    d = add32(1.0, e)
    return div32(a, d)


def silu_word(a: float, fmt: str = "bf16") -> int:
    """The stored word (format fmt) for accumulator a with SiLU."""
    return WORDS[fmt](silu32(a))


def silu_bf16_word(a: float) -> int:
    """The stored word for accumulator a: SiLU a / (1 + exp(-a)) in binary32, then bf16."""
    return bf16_word(silu32(a))


def bf16_to_float(h: int) -> float:
    return from_bits32((h & 0xFFFF) << 16)


def f16_to_float(h: int) -> float:
    """Value of a binary16 number (not NaN), via struct's "e" format."""
    return struct.unpack("<e", struct.pack("<H", h & 0xFFFF))[0]
