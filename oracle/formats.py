"""Exact conversions and round-to-nearest-even for the 16-bit activation formats.

Test infrastructure (see the package docstring).  The activations of the W4A16
layer stay in a 16-bit float format, FP16 (1 sign, 5 exponent, 10 mantissa
bits) or BF16 (1 sign, 8 exponent, 7 mantissa bits) (page
"推理优化中“用精度换性能“的核心技术：量化", §2.1 浮点格式).  NumPy has no bf16
type, so bf16 values travel as their uint16 bit patterns.

``round_to_format`` is the plain definition of IEEE round-to-nearest-even onto
a binary format with ``p`` significant bits and minimum normal exponent
``emin``: pick the quantum ``2^(max(e, emin) - p + 1)`` of the binade holding
``|v|``, divide (exact: a power of two), round half-to-even with ``np.rint``
(exact on float64), multiply back.  ``round_fraction_to_format`` is the same
rule on exact rationals, used to pin the float64 version.
"""

from __future__ import annotations

from dataclasses import dataclass
from fractions import Fraction

import numpy as np


@dataclass(frozen=True)
class Format:
    name: str
    p: int      # significant bits, including the implicit leading one
    emin: int   # exponent of the smallest normal number
    emax: int   # exponent of the largest finite binade


F16 = Format("fp16", 11, -14, 15)
BF16 = Format("bf16", 8, -126, 127)


def f16_to_f64(x) -> np.ndarray:
    """Exact widening of an fp16 array to float64."""
    return np.asarray(x, dtype=np.float16).astype(np.float64)


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns (uint16) to float64.

    A bf16 value is the upper half of the fp32 value with the same bits.
    """
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def round_to_format(v, fmt: Format) -> np.ndarray:
    """Round float64 values to ``fmt`` with round-to-nearest-even; returns float64.

    Overflow past the largest finite value rounds to +-inf as IEEE RNE does.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.empty_like(v)
    finite = np.isfinite(v)
    out[~finite] = v[~finite]
    a = np.abs(v[finite])
    nz = a != 0
    res = np.zeros_like(a)
    an = a[nz]
    _, E = np.frexp(an)            # an = f * 2^E with f in [0.5, 1)
    e = E.astype(np.int64) - 1     # an in [2^e, 2^(e+1))
    e = np.maximum(e, fmt.emin)
    q = np.ldexp(1.0, (e - fmt.p + 1).astype(np.int64))
    r = np.rint(an / q) * q
    limit = np.ldexp(1.0, fmt.emax + 1)
    r[r >= limit] = np.inf
    res[nz] = r
    out[finite] = np.copysign(res, v[finite])
    return out


def round_fraction_to_format(x: Fraction, fmt: Format) -> float:
    """Round an exact rational to ``fmt`` (RNE) and return it as a Python float."""
    if x == 0:
        return 0.0
    sign = -1.0 if x < 0 else 1.0
    a = abs(x)
    # exponent e with 2^e <= a < 2^(e+1)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, fmt.emin)
    quantum = Fraction(2) ** (e - fmt.p + 1)
    t = a / quantum
    n = t.numerator // t.denominator
    rem = t - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    r = n * quantum
    if r >= Fraction(2) ** (fmt.emax + 1):
        return sign * float("inf")
    return sign * float(r)


def round_to_f16(v) -> np.ndarray:
    """RNE of float64 values to fp16, returned as a NumPy float16 array."""
    return round_to_format(v, F16).astype(np.float16)


def round_to_bf16_bits(v) -> np.ndarray:
    """RNE of float64 values to bf16, returned as uint16 bit patterns."""
    r = round_to_format(v, BF16).astype(np.float32)   # exact: bf16 values fit in fp32
    return (r.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
