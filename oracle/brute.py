"""Brute-force reference for tiny inputs -- TEST INFRASTRUCTURE ONLY.

Independent of ``ring_oracle.c``: pure Python, exact rational arithmetic, and a
round-to-nearest-even written from the IEEE 754 definition.  It computes the
AllReduce result of one element position straight from the definition of the
ring result:

* The post "Why AllReduce = ReduceScatter + AllGather -- with NCCL Ring
  AllReduce" (loosp.cn), section 5, builds chunk k's sum by starting at the rank
  with the same index and adding each next rank around the ring (chunk 0:
  a0+b0, then +c0, then +d0; chunk 2: c2+d2, then +a2, then +b2).  So for an
  element of chunk c the result is the left fold over ranks c, c+1, ..., c+R-1
  (mod R), rounded to the storage format after every addition.
* Section 1 defines the target: every rank ends with that same value.

Values are Python ints for int32 (wrapped to 32 bits after each addition) and
``Fraction`` for floating point, so nothing here shares rounding behaviour with
the C oracle.

The other reductions follow the same fold: MAX keeps the running value unless
the next rank's compares greater, MIN unless it compares less; PROD multiplies
exactly and rounds once to the format (int32 wraps).
"""
from __future__ import annotations

import math
import struct
from fractions import Fraction

# (significant bits, minimum normal exponent, maximum exponent)
FORMATS = {"fp32": (24, -126, 127), "bf16": (8, -126, 127), "fp16": (11, -14, 15)}

INF = float("inf")


def fp32_bits_to_value(bits: int):
    """Decode binary32 bits: a Fraction, +-inf, nan, or a signed zero (float)."""
    x = struct.unpack("<f", struct.pack("<I", bits & 0xFFFFFFFF))[0]
    if math.isnan(x) or math.isinf(x) or x == 0.0:
        return x
    return Fraction(x)


def bf16_bits_to_value(bits: int):
    return fp32_bits_to_value((bits & 0xFFFF) << 16)


def fp16_bits_to_value(bits: int):
    x = struct.unpack("<e", struct.pack("<H", bits & 0xFFFF))[0]
    if math.isnan(x) or math.isinf(x) or x == 0.0:
        return x
    return Fraction(x)


def value_to_fp16_bits(v) -> int:
    if isinstance(v, float) and math.isnan(v):
        return 0x7E00
    if isinstance(v, Fraction):
        f = float(v)
        assert Fraction(f) == v
        v = f
    return struct.unpack("<H", struct.pack("<e", v))[0]


def value_to_fp32_bits(v) -> int:
    if isinstance(v, Fraction):
        v = float(v)  # exact: v is representable in binary32
    return struct.unpack("<I", struct.pack("<f", v))[0]


def value_to_bf16_bits(v) -> int:
    if isinstance(v, float) and math.isnan(v):
        return 0x7FC0
    bits = value_to_fp32_bits(v)
    assert bits & 0xFFFF == 0, "value is not a bfloat16"
    return bits >> 16


def round_nearest_even(x: Fraction, fmt: str):
    """Round an exact non-zero rational to the format, ties to even.

    Returns a Fraction, or +-inf on overflow.
    """
    p, emin, emax = FORMATS[fmt]
    sign = -1 if x < 0 else 1
    a = -x if x < 0 else x
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    if Fraction(2) ** (e + 1) <= a:
        e += 1
    quantum_exp = max(e, emin) - (p - 1)
    scaled = a / (Fraction(2) ** quantum_exp)
    n = scaled.numerator // scaled.denominator
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * Fraction(2) ** quantum_exp
    largest = (2 - Fraction(2) ** (1 - p)) * Fraction(2) ** emax
    if r > largest:
        return sign * INF
    return sign * r


def add(a, b, fmt: str):
    """One IEEE addition in the format: exact sum, then one rounding."""
    fa = isinstance(a, float)
    fb = isinstance(b, float)
    if (fa and math.isnan(a)) or (fb and math.isnan(b)):
        return math.nan
    if fa and math.isinf(a):
        if fb and math.isinf(b) and a != b:
            return math.nan
        return a
    if fb and math.isinf(b):
        return b
    if fa and fb:  # both zeros
        return -0.0 if (math.copysign(1, a) < 0 and math.copysign(1, b) < 0) else 0.0
    if fa:
        return b
    if fb:
        return a
    s = a + b
    if s == 0:
        return 0.0  # exact cancellation gives +0 under round to nearest
    return round_nearest_even(s, fmt)


def mul(a, b, fmt: str):
    """One IEEE multiplication in the format: exact product, then one rounding."""
    fa = isinstance(a, float)
    fb = isinstance(b, float)
    if (fa and math.isnan(a)) or (fb and math.isnan(b)):
        return math.nan
    sa = math.copysign(1, a) if fa else (1 if a > 0 else -1)
    sb = math.copysign(1, b) if fb else (1 if b > 0 else -1)
    sign = sa * sb
    a_inf = fa and math.isinf(a)
    b_inf = fb and math.isinf(b)
    a_zero = fa and a == 0.0
    b_zero = fb and b == 0.0
    if (a_inf and b_zero) or (b_inf and a_zero):
        return math.nan
    if a_inf or b_inf:
        return sign * INF
    if a_zero or b_zero:
        return math.copysign(0.0, sign)
    p = a * b
    r = round_nearest_even(p, fmt)
    if r == 0:
        return math.copysign(0.0, sign)
    return r


def ring_order(R: int, chunk: int):
    """Ranks in the order the ring folds an element of ``chunk``."""
    return [(chunk + i) % R for i in range(R)]


def allreduce_element(values, chunk: int, dtype: str, op: str):
    """Expected result at one position; ``values[r]`` is rank r's input bits/int."""
    R = len(values)
    order = ring_order(R, chunk)
    if dtype == "int32":
        xs = [int(values[r]) for r in order]
        if op == "max":
            return max(xs)
        if op == "min":
            return min(xs)
        acc = xs[0] & 0xFFFFFFFF
        for x in xs[1:]:
            acc = (acc * x if op == "prod" else acc + x) & 0xFFFFFFFF
        return acc - (1 << 32) if acc >= (1 << 31) else acc
    decode = {"fp32": fp32_bits_to_value, "bf16": bf16_bits_to_value,
              "fp16": fp16_bits_to_value}[dtype]
    encode = {"fp32": value_to_fp32_bits, "bf16": value_to_bf16_bits,
              "fp16": value_to_fp16_bits}[dtype]
    xs = [decode(int(values[r])) for r in order]
    if op in ("max", "min"):
        best = xs[0]
        for x in xs[1:]:
            if (x > best) if op == "max" else (x < best):
                best = x
        return encode(best)
    acc = xs[0]
    for x in xs[1:]:
        acc = add(acc, x, dtype) if op == "sum" else mul(acc, x, dtype)
    return encode(acc)
