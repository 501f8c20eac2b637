"""Pins for the 8-bit weight oracle (CPU only): quantizer, byte packing, dequantization and
the W8A16 linear layer.

Each step is pinned by something other than the oracle itself: hand-worked vectors
(tests/golden/hand_vectors_w8.json), an exact-rational recomputation of every fp32
operation, a brute-force nearest-grid-point search over all 256 codes, the round-trip
bound, grid fixed points, invariances (power-of-two scaling, symmetric negation), the
per-channel case, and the linear layer against exact rationals.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

from oracle import formats as F
from oracle import w8a16 as W8
from synth import BF16, FP16, activations, weights

GOLD = os.path.join(os.path.dirname(__file__), "golden", "hand_vectors_w8.json")
FP32 = F.Format("fp32", 24, -126, 127)


def _vectors():
    with open(GOLD) as f:
        return json.load(f)["vectors"]


@pytest.mark.parametrize("vec", _vectors(), ids=lambda v: v["name"])
def test_hand_vectors(vec):
    x = np.array([vec["x"]], dtype=np.float32)
    scheme = W8.ASYM if vec["scheme"] == "asym" else W8.SYM
    codes, s, z = W8.quantize8(x, 8, scheme)
    assert codes.tolist() == [vec["codes"]]
    assert float(s[0, 0]) == vec["scale"]
    assert float(z[0, 0]) == vec["zero"]
    words = W8.pack8(codes)
    assert [int(w) for w in words.view(np.uint32)[0]] == [int(h, 16) for h in vec["words_hex"]]
    xhat = W8.dequantize8(words, s, z, 8)
    assert xhat[0].tolist() == vec["xhat"]
    if "signed_codes" in vec:
        assert (codes.astype(int) - 128).tolist() == [vec["signed_codes"]]
        np.testing.assert_array_equal(W8.dequantize8(words, s, None, 8), xhat)
    if "y_ones" in vec:
        y = W8.linear8_ref(np.ones((1, 8), dtype=np.float16), FP16, words, s, z, 8)
        assert float(y[0, 0]) == vec["y_ones"]


def test_fixed_words():
    w = np.array([[0x04030201, 0xFF00807F]], dtype=np.uint32).view(np.int32)
    assert W8.unpack8(w).tolist() == [[1, 2, 3, 4, 0x7F, 0x80, 0x00, 0xFF]]
    w2 = W8.pack8(np.array([[0, 0, 0, 255]], dtype=np.uint8))
    assert int(w2.view(np.uint32)[0, 0]) == 0xFF000000


@settings(max_examples=60, deadline=None)
@given(n=st.integers(1, 5), kw=st.integers(1, 6), seed=st.integers(0, 2**31))
def test_pack_unpack_identity(n, kw, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 256, (n, 4 * kw)).astype(np.uint8)
    words = W8.pack8(codes)
    assert words.dtype == np.int32 and words.shape == (n, kw)
    np.testing.assert_array_equal(W8.unpack8(words), codes)
    raw = rng.integers(0, 2**32, (n, kw), dtype=np.uint64).astype(np.uint32).view(np.int32)
    np.testing.assert_array_equal(W8.pack8(W8.unpack8(raw)), raw)


def _rne_int(t: Fraction) -> int:
    n = t.numerator // t.denominator
    rem = t - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def _rt32(x: Fraction) -> Fraction:
    return Fraction(F.round_fraction_to_format(x, FP32))


def _group_rational(xs, scheme):
    """Per-group recomputation with exact rationals: each fp32 operation is its exact
    result rounded once to fp32, integer rounding is half-to-even, the scale is rounded
    to fp16 (a zero scale becomes 1)."""
    fx = [Fraction(float(v)) for v in xs]
    if scheme == W8.ASYM:
        mn, mx = min(fx), max(fx)
        s32 = _rt32(_rt32(mx - mn) / 255)
    else:
        s32 = _rt32(max(abs(v) for v in fx) / 127)
    s = Fraction(F.round_fraction_to_format(s32, F.F16))
    if s == 0:
        s = Fraction(1)
    if scheme == W8.ASYM:
        z = _rne_int(_rt32(-mn / s))
        codes = [min(255, max(0, _rne_int(_rt32(v / s)) + z)) for v in fx]
    else:
        z = 128
        codes = [min(127, max(-128, _rne_int(_rt32(v / s)))) + 128 for v in fx]
    return codes, s, z


@pytest.mark.parametrize("scheme", [W8.ASYM, W8.SYM])
@pytest.mark.parametrize("g", [8, 32, 128])
def test_quantizer_matches_rational_recomputation(scheme, g):
    W = weights(5, 256, 0.02, seed=117, outlier_frac=0.01, outlier_mult=20.0)
    codes, s, z = W8.quantize8(W, g, scheme)
    for n in range(W.shape[0]):
        for j in range(W.shape[1] // g):
            c, sr, zr = _group_rational(W[n, j * g:(j + 1) * g], scheme)
            assert codes[n, j * g:(j + 1) * g].tolist() == c
            assert Fraction(float(s[n, j])) == sr
            assert float(z[n, j]) == zr


@pytest.mark.parametrize("scheme", [W8.ASYM, W8.SYM])
def test_codes_are_nearest_grid_points(scheme):
    # brute force over all 256 codes: away from exact ties RTN picks the nearest grid point
    W = weights(6, 256, 0.02, seed=123)
    codes, s, z = W8.quantize8(W, 64, scheme)
    sf = np.repeat(s.astype(np.float64), 64, axis=1)
    zf = np.repeat(z.astype(np.float64), 64, axis=1)
    grid = np.arange(256, dtype=np.float64)
    cand = sf[:, :, None] * (grid[None, None, :] - zf[:, :, None])
    dist = np.abs(W.astype(np.float64)[:, :, None] - cand)
    best = dist.argmin(axis=2)
    srt = np.sort(dist, axis=2)
    clear = (srt[:, :, 1] - srt[:, :, 0]) > 1e-6 * sf
    assert clear.mean() > 0.99
    np.testing.assert_array_equal(codes[clear], best[clear])


@pytest.mark.parametrize("scheme", [W8.ASYM, W8.SYM])
def test_roundtrip_error_bound(scheme):
    # |x - x_hat| <= s/2 up to the fp32 rounding of x/s; a code clamped at the top of the
    # asymmetric range (the stored fp16 scale may sit slightly below (max-min)/255) is off
    # by at most s*(1/2 + 255*2^-11 + 2^-20)
    W = weights(32, 1024, 0.02, seed=129, outlier_frac=0.001, outlier_mult=20.0)
    codes, s, z = W8.quantize8(W, 128, scheme)
    xhat = W8.dequantize8(W8.pack8(codes), s, z, 128)
    sf = np.repeat(s.astype(np.float64), 128, axis=1)
    err = np.abs(W.astype(np.float64) - xhat) / sf
    assert err.max() <= 0.5 + 255 * 2.0**-11 + 2.0**-20
    unclamped = (codes > 0) & (codes < 255)
    assert err[unclamped].max() <= 0.5 * (1 + 2.0**-20)
    if scheme == W8.SYM:
        assert err.max() <= 0.5 * (1 + 2.0**-20)


@pytest.mark.parametrize("scheme", [W8.ASYM, W8.SYM])
def test_grid_fixed_point(scheme):
    # weights already on a grid s*(q - z) with both extreme codes present come back exactly
    rng = np.random.default_rng(137)
    N, K, g = 12, 256, 32
    G = K // g
    s = (rng.uniform(0.5, 2.0, (N, G)) * 2.0**rng.integers(-14, -6, (N, G))).astype(np.float16)
    if scheme == W8.ASYM:
        z = rng.integers(0, 256, (N, G)).astype(np.float32)
        q = rng.integers(0, 256, (N, K))
        q[:, ::g] = 0
        q[:, 1::g] = 255
        signed = q - np.repeat(z, g, axis=1)
    else:
        z = np.full((N, G), 128.0, np.float32)
        signed = rng.integers(-127, 128, (N, K))
        signed[:, ::g] = -127
        signed[:, 1::g] = 127
        q = signed + 128
    W = (np.repeat(s.astype(np.float32), g, axis=1) * signed.astype(np.float32)).astype(np.float32)
    codes, s2, z2 = W8.quantize8(W, g, scheme)
    np.testing.assert_array_equal(codes, q)
    np.testing.assert_array_equal(s2.view(np.uint16), s.view(np.uint16))
    np.testing.assert_array_equal(z2.astype(np.float32), z)


@pytest.mark.parametrize("scheme", [W8.ASYM, W8.SYM])
def test_power_of_two_scaling_invariance(scheme):
    # holds while every scale stays a normal fp16 number (8-bit scales of N(0, 0.02) weights
    # are near 6e-4, so the scalings stay within [2^-14, 65504] after the shift)
    W = weights(6, 512, 0.02, seed=141)
    c1, s1, z1 = W8.quantize8(W, 128, scheme)
    for j in (-2, 4):
        assert s1.astype(np.float64).min() * 2.0**j >= 2.0**-14
        c2, s2, z2 = W8.quantize8((W * np.float32(2.0**j)).astype(np.float32), 128, scheme)
        np.testing.assert_array_equal(c2, c1)
        np.testing.assert_array_equal(s2.astype(np.float64), s1.astype(np.float64) * 2.0**j)
        np.testing.assert_array_equal(z2, z1)


def test_symmetric_negation():
    W = weights(6, 256, 0.02, seed=153)
    c1, s1, _ = W8.quantize_sym8(W, 128)
    c2, s2, _ = W8.quantize_sym8(-W, 128)
    np.testing.assert_array_equal(s2, s1)
    np.testing.assert_array_equal(c2.astype(int), 256 - c1.astype(int))


def test_symmetric_clamps_at_minus_128():
    # max|x| = 2 gives s = fp16(2/127); -2/s rounds to -127, so -128 is reached only by a
    # value beyond the absmax grid: the clamp keeps every stored code in [0, 255]
    x = np.array([[-2.0, 1.0, 0.5, 0.0, 0.25, -1.0, 1.5, 2.0]], dtype=np.float32)
    codes, s, _ = W8.quantize_sym8(x, 8)
    assert codes.min() >= 0 and codes.max() <= 255
    assert int(codes[0, 0]) - 128 == _rne_int(_rt32(Fraction(-2.0) / Fraction(float(s[0, 0]))))


def test_per_channel_is_one_group_per_row():
    W = weights(4, 384, 0.02, seed=159)
    _, s, z = W8.quantize_asym8(W, 384)
    assert s.shape == (4, 1) and z.shape == (4, 1)
    for n in range(4):
        s32 = np.float32((np.float32(W[n].max()) - np.float32(W[n].min())) / np.float32(255))
        assert float(s[n, 0]) == float(np.float16(s32))


def test_zero_point_out_of_range_raises():
    W = np.full((1, 8), 1000.0, dtype=np.float32)
    W[0, 0] = 1000.5
    with pytest.raises(ValueError):
        W8.quantize_asym8(W, 8)


def test_dequantize_layout_and_zero_none():
    rng = np.random.default_rng(161)
    codes = rng.integers(0, 256, (3, 64)).astype(np.uint8)
    s = rng.uniform(0.001, 0.01, (3, 2)).astype(np.float16)
    z = rng.integers(0, 256, (3, 2)).astype(np.float16)
    Wq = W8.pack8(codes)
    D = W8.dequantize8(Wq, s, z, 32)
    for n in range(3):
        for k in range(64):
            assert D[n, k] == float(s[n, k // 32]) * (int(codes[n, k]) - float(z[n, k // 32]))
    np.testing.assert_array_equal(W8.dequantize8(Wq, s, None, 32),
                                  W8.dequantize8(Wq, s, np.full_like(z, 128.0), 32))


@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("scheme", [W8.ASYM, W8.SYM])
def test_linear_matches_exact_rationals(dtype, scheme):
    M, N, K, g = 3, 5, 64, 32
    W = weights(N, K, 0.02, seed=171 + scheme)
    X = activations(M, K, dtype, seed=173 + dtype)
    codes, s, z = W8.quantize8(W, g, scheme)
    q = W8.pack8(codes)
    ref = W8.linear8_ref(X, dtype, q, s, z, g)
    ex = W8.linear8_exact(X, dtype, q, s, z, g)
    if dtype == FP16:
        np.testing.assert_array_equal(ref.view(np.uint16), ex.view(np.uint16))
    else:
        np.testing.assert_array_equal(ref, ex)


def test_linear_one_hot_reads_one_weight():
    # X = e_k picks column k of W_hat: the output is the dequantized weight rounded once
    N, K, g = 6, 64, 16
    W = weights(N, K, 0.02, seed=181)
    codes, s, z = W8.quantize_asym8(W, g)
    q = W8.pack8(codes)
    for k in (0, 17, 63):
        X = np.zeros((1, K), dtype=np.float16)
        X[0, k] = 1.0
        y = W8.linear8_ref(X, FP16, q, s, z, g)
        want = [float(s[n, k // g]) * (int(codes[n, k]) - float(z[n, k // g])) for n in range(N)]
        np.testing.assert_array_equal(y[0].astype(np.float64), np.float16(np.array(want)).astype(np.float64))
