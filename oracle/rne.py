"""Round-to-nearest-even conversions into binary16 and bfloat16 (test infrastructure only).

Written from the IEEE-754 format definitions, not from any library's code:

* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.  Normal
  values are 2^e * (1 + f/1024) for e in [-14, 15]; subnormals are f * 2^-24.
* bfloat16: the top 16 bits of binary32: 1 sign bit, 8 exponent bits
  (bias 127), 7 fraction bits.  Normals 2^e * (1 + f/128), e in [-126, 127];
  subnormals f * 2^-133.

Rounding is to the nearest representable value, ties to the one with an even
fraction field; magnitudes that round past the largest finite value become
infinity.  A fp64 input is rounded ONCE (never through binary32), which is
what the scales of both weight formats need: page [P1] section 3.1 stores the
ternary scale as fp16 and aligns everything on that fp16 value.

Two tiers:

* ``*_bits_exact``: pure Python on exact rationals (``float.as_integer_ratio``),
  the specification.
* ``f16_bits`` / ``bf16_bits``: numpy, for arrays.  ``f16_bits`` relies on
  numpy's float64 -> float16 cast; ``bf16_bits`` does the rounding on the
  binary32 bit pattern.  Both are pinned to the exact tier by tests.
"""

import math
from fractions import Fraction

import numpy as np


def _rne_bits_exact(x: float, frac_bits: int, bias: int, exp_field_max: int) -> int:
    """Bit pattern of the format nearest to ``x`` (ties to even)."""
    total_bits = 1 + (exp_field_max.bit_length()) + frac_bits
    sign_bit = 1 << (total_bits - 1)
    inf_bits = exp_field_max << frac_bits
    if x != x:  # NaN: the canonical quiet NaN
        return inf_bits | (1 << (frac_bits - 1))
    neg = math.copysign(1.0, x) < 0
    sign = sign_bit if neg else 0
    if x in (float("inf"), float("-inf")):
        return sign | inf_bits
    a = abs(Fraction(x))
    if a == 0:
        return sign
    # exponent e with 2^e <= a < 2^(e+1), computed exactly
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    emin = 1 - bias
    E = max(e, emin)
    quantum = Fraction(2) ** (E - frac_bits)
    r = round(a / quantum)  # Fraction.__round__ rounds half to even
    one = 1 << frac_bits
    if r == 2 * one:  # carried into the next binade
        E += 1
        r = one
    if E == emin:
        bits = r  # subnormal (r < one) or the smallest normal (r == one)
    else:
        bits = ((E + bias) << frac_bits) + (r - one)
    if (bits >> frac_bits) >= exp_field_max:
        return sign | inf_bits
    return sign | bits


def f16_bits_exact(x: float) -> int:
    """binary16 bit pattern of fp64 ``x`` rounded once, ties to even."""
    return _rne_bits_exact(float(x), 10, 15, 31)


def bf16_bits_exact(x: float) -> int:
    """bfloat16 bit pattern of ``x`` rounded once, ties to even."""
    return _rne_bits_exact(float(x), 7, 127, 255)


def f16_value_exact(bits: int) -> float:
    """Exact value of a binary16 bit pattern (decoded from the definition)."""
    bits &= 0xFFFF
    s = -1.0 if bits & 0x8000 else 1.0
    e = (bits >> 10) & 0x1F
    f = bits & 0x3FF
    if e == 31:
        return s * float("inf") if f == 0 else float("nan")
    if e == 0:
        return s * f * 2.0 ** -24
    return s * (1024 + f) * 2.0 ** (e - 25)


def bf16_value_exact(bits: int) -> float:
    """Exact value of a bfloat16 bit pattern."""
    bits &= 0xFFFF
    s = -1.0 if bits & 0x8000 else 1.0
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 255:
        return s * float("inf") if f == 0 else float("nan")
    if e == 0:
        return s * f * 2.0 ** -133
    return s * (128 + f) * 2.0 ** (e - 134)


# ----------------------------------------------------------------- numpy tier

def f16_bits(x) -> np.ndarray:
    """uint16 bit patterns of fp64 array ``x`` rounded once to binary16 (RNE)."""
    with np.errstate(over="ignore"):
        return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def f16_values(bits) -> np.ndarray:
    """fp64 values of uint16 binary16 bit patterns (exact)."""
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def bf16_bits(x) -> np.ndarray:
    """uint16 bfloat16 bit patterns of an array, rounded to nearest even.

    The input must be exactly representable in binary32 (fp16 and bf16 values,
    fp32 data); it is taken as binary32, and the low 16 bits are rounded away
    with ties to even.  NaNs become the canonical quiet NaN.
    """
    x32 = np.asarray(x, dtype=np.float64)
    f = x32.astype(np.float32)
    if not np.array_equal(f.astype(np.float64), x32, equal_nan=True):
        raise ValueError("bf16_bits: input is not exactly representable in binary32")
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint32)
    nan = np.isnan(f)
    r = np.where(nan, (((u >> 16) & 0x8000) | 0x7FC0).astype(np.uint32), r)
    return r.astype(np.uint16)


def bf16_values(bits) -> np.ndarray:
    """fp64 values of uint16 bfloat16 bit patterns (exact)."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)
