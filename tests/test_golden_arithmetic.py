"""The binary32 golden files re-derived in exact rational arithmetic.

The quantiser and RMSNorm goldens state the binary32 value of every step.
This test recomputes those steps with Python fractions and a round-to-nearest-
even to 24 bits written here from the IEEE 754 definition, with no float32
arithmetic from numpy, the oracle or the library, so a slip in a golden file
cannot hide behind the code it pins.  CPU only.
"""
import json
import math
import os
import struct
from fractions import Fraction

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def rn32(q):
    """Nearest binary32 value of the rational q (ties to even), normal range."""
    q = Fraction(q)
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1)
    assert -126 <= e <= 127
    ulp = Fraction(2) ** (e - 23)
    m = a / ulp
    n = math.floor(m)
    r = m - n
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return sign * n * ulp


def sqrt32(a):
    """Correctly rounded binary32 square root of the binary32 value a > 0."""
    c = rn32(Fraction(math.sqrt(a)))
    # walk to the candidate whose rounding interval holds sqrt(a)
    for _ in range(4):
        e = c.numerator.bit_length() - c.denominator.bit_length()
        if Fraction(2) ** e > c:
            e -= 1
        half = Fraction(2) ** (e - 24)
        lo, hi = c - half, c + half
        if lo * lo > a:
            c = rn32(c - 2 * half)
        elif hi * hi < a:
            c = rn32(c + 2 * half)
        else:
            return c
    raise AssertionError("sqrt did not settle")


def round_half_away(q):
    return int(math.copysign(math.floor(abs(q) + Fraction(1, 2)), q))


def from_bits(s):
    return Fraction(struct.unpack("<f", struct.pack("<I", int(s, 16)))[0])


def to_bits(q):
    return hex(struct.unpack("<I", struct.pack("<f", float(q)))[0])


def quantise(v):
    """The page's quantiser on exact binary32 values: scale, reciprocal, codes."""
    amax = max(abs(a) for a in v)
    sc = rn32(amax / 127)
    inv = rn32(1 / sc) if sc > 0 else Fraction(0)
    xq = [max(-128, min(127, round_half_away(rn32(a * inv)))) for a in v]
    suma = [sum(xq[g * 64:(g + 1) * 64]) for g in range(len(v) // 64)]
    return sc, xq, suma


def rmsnorm(x, w, eps):
    ss = sum(a * a for a in x)          # exact, as a binary64 sum of these squares is
    ms = rn32(ss / len(x))
    inv = rn32(1 / sqrt32(rn32(ms + eps)))
    return [rn32(rn32(a * inv) * b) for a, b in zip(x, w)]


def test_act_quant_reciprocal_golden():
    g = _golden("act_quant_reciprocal.json")
    x = [from_bits(b) for b in g["x_head_bits"]] + [Fraction(0)] * (g["K"] - 2)
    sc, xq, suma = quantise(x)
    assert to_bits(sc) == g["act_scale_bits"]
    assert xq[:2] == g["xq_head"] and suma == g["suma"]
    # the slip this golden separates: a division by the scale gives 85
    assert round_half_away(rn32(x[1] / sc)) == 85


def test_rmsnorm_sum_of_squares_golden():
    g = _golden("rmsnorm_sum_of_squares.json")
    K = g["K"]
    x = [Fraction(4096)] + [Fraction(1)] * (K - 1)
    v = rmsnorm(x, [Fraction(1)] * K, Fraction(g["eps"]))
    sc, xq, suma = quantise(v)
    assert [to_bits(a) for a in v[:2]] == g["v_bits_head"]
    assert to_bits(sc) == g["act_scale_bits"]
    assert xq[:2] == g["xq_head"] and suma == g["suma"]
    # a binary32 running sum of squares loses every +1 and changes the scale
    s32 = Fraction(0)
    for a in x:
        s32 = rn32(s32 + a * a)
    assert s32 == 2 ** 24
    inv = rn32(1 / sqrt32(rn32(s32 / K)))
    assert to_bits(rn32(rn32(x[0] * inv) / 127)) == "0x3e810204"


def test_rmsnorm_product_order_golden():
    g = _golden("rmsnorm_product_order.json")
    K = g["K"]
    x = [Fraction(1), Fraction(7)] * (K // 2)
    w = [Fraction(1), Fraction(3, 2)] * (K // 2)
    v = rmsnorm(x, w, Fraction(g["eps"]))
    sc, xq, suma = quantise(v)
    assert [to_bits(a) for a in v[:2]] == g["v_bits_head"]
    assert to_bits(sc) == g["act_scale_bits"]
    assert xq[:2] == g["xq_head"] and suma == g["suma"]
    inv = rn32(Fraction(1, 5))
    assert to_bits(rn32(7 * rn32(inv * Fraction(3, 2)))) == "0x40066667"


def test_rn32_against_hardware_conversion():
    """The rounding helper agrees with the platform's binary64 -> binary32
    conversion (IEEE round to nearest even) on values that are exact in
    binary64, including ties."""
    cases = [Fraction(2 ** 24 + 1), Fraction(2 ** 24 + 3), Fraction(-(2 ** 25 + 6)),
             Fraction(16385) + Fraction(1, 1024), Fraction(123456789, 2 ** 40),
             Fraction(0x1fffffd, 2 ** 60), Fraction(-0x3ffffff, 2 ** 3)]
    for q in cases:
        assert float(rn32(q)) == struct.unpack("<f", struct.pack("<f", float(q)))[0], q
