"""Pins for the oracle quantizer, packing and dequantization (CPU only).

Every step Q1..Q5/Q6 of the quantizer and the pack/unpack layout is pinned by
something other than the oracle itself: hand-worked vectors, exact-rational
recomputation of each fp32 operation, a brute-force nearest-grid-point search,
a grid fixed point, invariances (power-of-two scaling, permutation within a
group, negation for the symmetric scheme) and the worst-case round-trip bound.
"""

import json
import os
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from oracle import formats as F
from synth import weights

GOLD = os.path.join(os.path.dirname(__file__), "golden", "hand_vectors.json")
FP32 = F.Format("fp32", 24, -126, 127)


def _vectors():
    with open(GOLD) as f:
        return json.load(f)["vectors"]


@pytest.mark.parametrize("vec", _vectors(), ids=lambda v: v["name"])
def test_hand_vectors(vec):
    x = np.array([vec["x"]], dtype=np.float32)
    scheme = oracle.ASYM if vec["scheme"] == "asym" else oracle.SYM
    codes, s, z = oracle.quantize(x, 8, scheme)
    assert codes.tolist() == [vec["codes"]]
    assert float(s[0, 0]) == vec["scale"]
    assert float(z[0, 0]) == vec["zero"]
    if "zero_bits_hex" in vec:
        assert int(z.view(np.uint16)[0, 0]) == int(vec["zero_bits_hex"], 16)
    words = oracle.pack(codes)
    assert int(words.view(np.uint32)[0, 0]) == int(vec["word_hex"], 16)
    xhat = oracle.dequantize(words, s, z, 8)
    assert xhat[0].tolist() == vec["xhat"]
    if "signed_codes" in vec:
        assert (codes.astype(int) - 8).tolist() == [vec["signed_codes"]]
        np.testing.assert_array_equal(oracle.dequantize(words, s, None, 8), xhat)
    if "y_ones" in vec:
        X = np.ones((1, 8), dtype=np.float16)
        y = oracle.linear_ref(X, 0, words, s, z, 8)
        assert float(y[0, 0]) == vec["y_ones"]


def test_fixed_words():
    assert oracle.unpack(np.array([[0x76543210]], dtype=np.uint32).view(np.int32)).tolist() == \
        [[0, 1, 2, 3, 4, 5, 6, 7]]
    assert oracle.unpack(np.array([[0x0000000F]], dtype=np.uint32).view(np.int32)).tolist() == \
        [[15, 0, 0, 0, 0, 0, 0, 0]]
    w = oracle.pack(np.array([[0, 0, 0, 0, 0, 0, 0, 15]], dtype=np.uint8))
    assert int(w[0, 0]) == np.int32(np.uint32(0xF0000000).view(np.int32))


@settings(max_examples=60, deadline=None)
@given(n=st.integers(1, 5), kw=st.integers(1, 6), seed=st.integers(0, 2**31))
def test_pack_unpack_identity(n, kw, seed):
    rng = np.random.default_rng(seed)
    codes = rng.integers(0, 16, (n, 8 * kw)).astype(np.uint8)
    words = oracle.pack(codes)
    assert words.dtype == np.int32 and words.shape == (n, kw)
    np.testing.assert_array_equal(oracle.unpack(words), codes)
    # and the other direction: any 32-bit pattern survives unpack -> pack
    raw = rng.integers(0, 2**32, (n, kw), dtype=np.uint64).astype(np.uint32).view(np.int32)
    np.testing.assert_array_equal(oracle.pack(oracle.unpack(raw)), raw)


def _rne_int_fraction(t: Fraction) -> int:
    n = t.numerator // t.denominator
    rem = t - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    return n


def _rt32(x: Fraction) -> Fraction:
    return Fraction(F.round_fraction_to_format(x, FP32))


def _quantize_group_rational(xs, scheme):
    """Independent per-group recomputation with exact rationals.

    Each fp32 operation of the quantizer is its exact result rounded once to
    fp32; rounding to integers is half-to-even; the scale is rounded to fp16.
    """
    fx = [Fraction(float(v)) for v in xs]
    if scheme == oracle.ASYM:
        mn, mx = min(fx), max(fx)
        s32 = _rt32(_rt32(mx - mn) / 15)
    else:
        s32 = _rt32(max(abs(v) for v in fx) / 7)
    s = Fraction(F.round_fraction_to_format(s32, F.F16))
    if s == 0:
        s = Fraction(1)
    if scheme == oracle.ASYM:
        z = _rne_int_fraction(_rt32(-mn / s))
        codes = [min(15, max(0, _rne_int_fraction(_rt32(v / s)) + z)) for v in fx]
    else:
        z = 8
        codes = [min(7, max(-8, _rne_int_fraction(_rt32(v / s)))) + 8 for v in fx]
    return codes, s, z


@pytest.mark.parametrize("scheme", [oracle.ASYM, oracle.SYM])
@pytest.mark.parametrize("g", [8, 32, 128])
def test_quantizer_matches_rational_recomputation(scheme, g):
    W = weights(6, 256, 0.02, seed=17, outlier_frac=0.01, outlier_mult=20.0)
    codes, s, z = oracle.quantize(W, g, scheme)
    for n in range(W.shape[0]):
        for j in range(W.shape[1] // g):
            c, sr, zr = _quantize_group_rational(W[n, j * g:(j + 1) * g], scheme)
            assert codes[n, j * g:(j + 1) * g].tolist() == c
            assert Fraction(float(s[n, j])) == sr
            assert float(z[n, j]) == zr


@pytest.mark.parametrize("scheme", [oracle.ASYM, oracle.SYM])
def test_codes_are_nearest_grid_points(scheme):
    # brute force: away from exact ties, RTN picks the grid point nearest to x
    W = weights(8, 512, 0.02, seed=23)
    codes, s, z = oracle.quantize(W, 64, scheme)
    sf = np.repeat(s.astype(np.float64), 64, axis=1)
    zf = np.repeat(z.astype(np.float64), 64, axis=1)
    grid = np.arange(16, dtype=np.float64)
    cand = sf[:, :, None] * (grid[None, None, :] - zf[:, :, None])     # [N, K, 16]
    dist = np.abs(W.astype(np.float64)[:, :, None] - cand)
    best = dist.argmin(axis=2)
    srt = np.sort(dist, axis=2)
    clear = (srt[:, :, 1] - srt[:, :, 0]) > 1e-6 * sf
    assert clear.mean() > 0.99
    np.testing.assert_array_equal(codes[clear], best[clear])


@pytest.mark.parametrize("scheme", [oracle.ASYM, oracle.SYM])
def test_roundtrip_error_bound(scheme):
    # |x - x_hat| <= s/2 up to the fp32 rounding of x/s; a code clamped at the
    # top of the asymmetric range (possible because the stored fp16 scale may
    # be slightly below (max-min)/15) is off by at most s*(1/2 + 15*2^-11 + 2^-20).
    W = weights(64, 1024, 0.02, seed=29, outlier_frac=0.001, outlier_mult=20.0)
    codes, s, z = oracle.quantize(W, 128, scheme)
    xhat = oracle.dequantize(oracle.pack(codes), s, z, 128)
    sf = np.repeat(s.astype(np.float64), 128, axis=1)
    err = np.abs(W.astype(np.float64) - xhat) / sf
    assert err.max() <= 0.5 + 15 * 2.0**-11 + 2.0**-20
    unclamped = (codes > 0) & (codes < 15)
    assert err[unclamped].max() <= 0.5 * (1 + 2.0**-20)
    if scheme == oracle.SYM:
        assert err.max() <= 0.5 * (1 + 2.0**-20)


def test_straddling_groups_have_zero_in_code_range():
    W = weights(32, 1024, 0.02, seed=31)
    _, _, z = oracle.quantize_asym(W, 128)
    assert np.all((z >= 0) & (z <= 15))


@pytest.mark.parametrize("scheme", [oracle.ASYM, oracle.SYM])
def test_grid_fixed_point(scheme):
    # weights that already lie on a grid s*(q - z) with the extreme codes
    # present come back as exactly (q, s, z)
    rng = np.random.default_rng(37)
    N, K, g = 16, 256, 32
    G = K // g
    s = (rng.uniform(0.5, 2.0, (N, G)) * 2.0**rng.integers(-12, -2, (N, G))).astype(np.float16)
    if scheme == oracle.ASYM:
        z = rng.integers(0, 16, (N, G)).astype(np.float32)
        q = rng.integers(0, 16, (N, K))
        q[:, ::g] = 0
        q[:, 1::g] = 15
        signed = q - np.repeat(z, g, axis=1)
    else:
        z = np.full((N, G), 8.0, np.float32)
        signed = rng.integers(-7, 8, (N, K))
        signed[:, ::g] = -7
        signed[:, 1::g] = 7
        q = signed + 8
    W = (np.repeat(s.astype(np.float32), g, axis=1) * signed.astype(np.float32)).astype(np.float32)
    codes, s2, z2 = oracle.quantize(W, g, scheme)
    np.testing.assert_array_equal(codes, q)
    np.testing.assert_array_equal(s2.view(np.uint16), s.view(np.uint16))
    np.testing.assert_array_equal(z2.astype(np.float32), z)


@pytest.mark.parametrize("scheme", [oracle.ASYM, oracle.SYM])
def test_power_of_two_scaling_invariance(scheme):
    W = weights(8, 512, 0.02, seed=41)
    c1, s1, z1 = oracle.quantize(W, 128, scheme)
    for j in (-3, 4):
        c2, s2, z2 = oracle.quantize((W * np.float32(2.0**j)).astype(np.float32), 128, scheme)
        np.testing.assert_array_equal(c2, c1)
        np.testing.assert_array_equal(s2.astype(np.float64), s1.astype(np.float64) * 2.0**j)
        np.testing.assert_array_equal(z2, z1)


@pytest.mark.parametrize("scheme", [oracle.ASYM, oracle.SYM])
def test_permutation_within_group(scheme):
    rng = np.random.default_rng(43)
    W = weights(4, 256, 0.02, seed=47)
    perm = rng.permutation(64)
    Wp = W.reshape(4, 4, 64)[:, :, perm].reshape(4, 256)
    c1, s1, z1 = oracle.quantize(W, 64, scheme)
    c2, s2, z2 = oracle.quantize(Wp, 64, scheme)
    np.testing.assert_array_equal(c2, c1.reshape(4, 4, 64)[:, :, perm].reshape(4, 256))
    np.testing.assert_array_equal(s2, s1)
    np.testing.assert_array_equal(z2, z1)


def test_symmetric_negation():
    W = weights(8, 256, 0.02, seed=53)
    c1, s1, _ = oracle.quantize_sym(W, 128)
    c2, s2, _ = oracle.quantize_sym(-W, 128)
    np.testing.assert_array_equal(s2, s1)
    np.testing.assert_array_equal(c2.astype(int), 16 - c1.astype(int))


def test_per_channel_is_one_group_per_row():
    W = weights(5, 384, 0.02, seed=59)
    c, s, z = oracle.quantize_asym(W, 384)
    assert s.shape == (5, 1) and z.shape == (5, 1)
    for n in range(5):
        mn, mx = float(W[n].min()), float(W[n].max())
        s32 = np.float32((np.float32(mx) - np.float32(mn)) / np.float32(15))
        assert float(s[n, 0]) == float(np.float16(s32))


def test_zero_point_out_of_range_raises():
    W = np.full((1, 8), 1000.0, dtype=np.float32)
    W[0, 0] = 1000.5
    with pytest.raises(ValueError):
        oracle.quantize_asym(W, 8)


def test_dequantize_layout_and_zero_none():
    rng = np.random.default_rng(61)
    codes = rng.integers(0, 16, (3, 64)).astype(np.uint8)
    s = rng.uniform(0.01, 0.1, (3, 2)).astype(np.float16)
    z = rng.integers(0, 16, (3, 2)).astype(np.float16)
    Wq = oracle.pack(codes)
    D = oracle.dequantize(Wq, s, z, 32)
    for n in range(3):
        for k in range(64):
            assert D[n, k] == float(s[n, k // 32]) * (int(codes[n, k]) - float(z[n, k // 32]))
    D8 = oracle.dequantize(Wq, s, None, 32)
    np.testing.assert_array_equal(D8, oracle.dequantize(Wq, s, np.full_like(z, 8.0), 32))
