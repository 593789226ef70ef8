"""Exact rational brute force -- TEST INFRASTRUCTURE ONLY.

An implementation of binary floating-point rounding from its definition, on
``fractions.Fraction`` values, with no use of hardware floating point.  It is
the second, independent formulation the C oracle is checked against on tiny
inputs: a value is decoded from its bit fields, sums are exact rationals, and
each rounding step picks the nearest representable value with ties to the
even significand (IEEE 754-2019, clause 4.3.1), subnormals included.
"""
from fractions import Fraction

# (significand bits incl. the implicit one, minimum normal exponent, maximum exponent)
BINARY32 = (24, -126, 127)
BFLOAT16 = (8, -126, 127)

INF = float("inf")


def decode(bits, fmt_bits):
    """Exact value of a float bit pattern.  fmt_bits = 32 (binary32) or 16 (bf16).
    Returns a Fraction, +-inf as float, or None for NaN."""
    bits = int(bits)
    man_bits = 23 if fmt_bits == 32 else 7
    exp_bits = 8
    sign = -1 if (bits >> (fmt_bits - 1)) & 1 else 1
    e = (bits >> man_bits) & ((1 << exp_bits) - 1)
    m = bits & ((1 << man_bits) - 1)
    if e == (1 << exp_bits) - 1:
        return None if m else sign * INF
    if e == 0:  # subnormal: 0.m * 2^(1 - bias)
        return sign * Fraction(m, 1 << man_bits) * Fraction(2) ** (1 - 127)
    return sign * (1 + Fraction(m, 1 << man_bits)) * Fraction(2) ** (e - 127)


def _floor_log2(q):
    """Largest e with 2^e <= q, for a positive Fraction q."""
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    while Fraction(2) ** (e + 1) <= q:
        e += 1
    return e


def round_nearest_even(q, fmt):
    """Round an exact value to the format (p, emin, emax); +-inf on overflow."""
    if q in (INF, -INF):
        return q
    if q == 0:
        return Fraction(0)
    p, emin, emax = fmt
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = max(_floor_log2(a), emin)
    quantum = Fraction(2) ** (e - p + 1)
    m = a / quantum
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    r = lo * quantum
    largest = (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax
    if r > largest:
        return sign * INF
    return sign * r


def encode(value, fmt_bits):
    """Bit pattern of an exactly representable value (Fraction or +-inf)."""
    man_bits = 23 if fmt_bits == 32 else 7
    if value in (INF, -INF):
        return ((1 << (fmt_bits - 1)) if value < 0 else 0) | (0xFF << man_bits)
    if value == 0:
        return 0
    sign = (1 << (fmt_bits - 1)) if value < 0 else 0
    a = abs(value)
    e = _floor_log2(a)
    if e < -126:  # subnormal
        m = a / (Fraction(2) ** (1 - 127)) * (1 << man_bits)
        assert m.denominator == 1
        return sign | int(m)
    m = (a / Fraction(2) ** e - 1) * (1 << man_bits)
    assert m.denominator == 1, "value not representable"
    return sign | ((e + 127) << man_bits) | int(m)


def fp32_fold(values, scale):
    """Left fold in binary32 (each add rounded), then one rounded multiply."""
    acc = values[0]
    for v in values[1:]:
        acc = round_nearest_even(acc + v, BINARY32)
    return round_nearest_even(acc * scale, BINARY32)


def reduce_bits(bit_lists, fmt_bits, scale):
    """Element-wise fp32 fold of several bit-pattern inputs, rounded to the
    buffer format; returns the output bit patterns.  Inputs must be finite."""
    out = []
    for elems in zip(*bit_lists):
        vals = [decode(b, fmt_bits) for b in elems]
        r = fp32_fold(vals, scale)
        if fmt_bits == 16:
            r = round_nearest_even(r, BFLOAT16)
        out.append(encode(r, fmt_bits))
    return out
