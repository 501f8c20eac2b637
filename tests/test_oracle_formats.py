"""Pins for the oracle's 16-bit format helpers (CPU only).

``round_to_format`` (float64 RNE by quantum scaling) is checked against
``round_fraction_to_format`` (exact rationals) and, for fp16, against NumPy's
own double->half conversion, an independent library routine.  The bf16 helpers
are checked against exact rationals and against the input generator's
independent fp32->bf16 bit trick.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle.formats import BF16, F16
from synth import f32_to_bf16_bits

FP32 = F.Format("fp32", 24, -126, 127)


def _random_f64(rng, n):
    # wide exponent spread, including fp16 subnormals and overflow territory
    mant = rng.uniform(1.0, 2.0, n)
    exp = rng.integers(-30, 20, n)
    sign = rng.choice([-1.0, 1.0], n)
    return sign * np.ldexp(mant, exp)


def _midpoints_f16(rng, n):
    # exact midpoints between adjacent fp16 values: ties must round to even
    bits = rng.integers(0, 0x7BFF, n).astype(np.uint16)
    lo = bits.view(np.float16).astype(np.float64)
    hi = (bits + 1).view(np.float16).astype(np.float64)
    return (lo + hi) / 2


def test_f16_rounding_matches_exact_rationals():
    rng = np.random.default_rng(1)
    v = np.concatenate([_random_f64(rng, 400), _midpoints_f16(rng, 200),
                        [0.0, -0.0, 65504.0, 65519.99, 65520.0, 2.0**-24, 2.0**-25, 3 * 2.0**-26]])
    got = F.round_to_format(v, F16)
    want = np.array([F.round_fraction_to_format(Fraction(float(x)), F16) for x in v])
    np.testing.assert_array_equal(got, want)


def test_f16_rounding_matches_numpy_cast():
    rng = np.random.default_rng(2)
    v = np.concatenate([_random_f64(rng, 20000), _midpoints_f16(rng, 5000)])
    got = F.round_to_f16(v)
    want = v.astype(np.float16)
    np.testing.assert_array_equal(got.view(np.uint16), want.view(np.uint16))


def test_midpoints_round_to_even_mantissa():
    rng = np.random.default_rng(3)
    v = _midpoints_f16(rng, 1000)
    bits = F.round_to_f16(v).view(np.uint16)
    assert np.all(bits % 2 == 0)


def test_bf16_rounding_matches_exact_rationals():
    rng = np.random.default_rng(4)
    mant = rng.uniform(1.0, 2.0, 300)
    exp = rng.integers(-140, 120, 300)
    v = np.ldexp(mant, exp) * rng.choice([-1.0, 1.0], 300)
    got = F.round_to_format(v, BF16)
    want = np.array([F.round_fraction_to_format(Fraction(float(x)), BF16) for x in v])
    np.testing.assert_array_equal(got, want)


def test_bf16_bits_roundtrip_and_known_patterns():
    assert F.bf16_bits_to_f64(np.array([0x3F80], np.uint16))[0] == 1.0
    assert F.bf16_bits_to_f64(np.array([0xC000], np.uint16))[0] == -2.0
    assert F.bf16_bits_to_f64(np.array([0x0001], np.uint16))[0] == 2.0**-133
    assert F.bf16_bits_to_f64(np.array([0x7F7F], np.uint16))[0] == (2 - 2.0**-7) * 2.0**127
    bits = np.arange(0, 0x7F80, 7, dtype=np.uint16)
    np.testing.assert_array_equal(F.round_to_bf16_bits(F.bf16_bits_to_f64(bits)), bits)


def test_bf16_oracle_agrees_with_generator_bit_trick():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(50000) * np.exp(rng.uniform(-20, 20, 50000))).astype(np.float32)
    np.testing.assert_array_equal(F.round_to_bf16_bits(x.astype(np.float64)), f32_to_bf16_bits(x))


def test_fp32_format_reproduces_hardware_fp32_ops():
    # the same RNE definition with p=24 must agree with NumPy's float32 arithmetic;
    # this pins the Format parameters used by the quantizer pins
    rng = np.random.default_rng(6)
    a = rng.standard_normal(2000).astype(np.float32)
    b = rng.standard_normal(2000).astype(np.float32)
    q = a / b
    want = np.array([F.round_fraction_to_format(Fraction(float(x)) / Fraction(float(y)), FP32)
                     for x, y in zip(a, b)])
    np.testing.assert_array_equal(q.astype(np.float64), want)


@pytest.mark.parametrize("fmt", [F16, BF16])
def test_overflow_and_signed_zero(fmt):
    big = np.ldexp(1.0, fmt.emax + 1)
    r = F.round_to_format(np.array([big, -big, 0.0, -0.0, np.inf, -np.inf]), fmt)
    assert r[0] == np.inf and r[1] == -np.inf
    assert r[2] == 0.0 and not np.signbit(r[2])
    assert r[3] == 0.0 and np.signbit(r[3])
    assert r[4] == np.inf and r[5] == -np.inf
