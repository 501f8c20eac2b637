"""Pins for the W8A8 / SmoothQuant oracle (CPU only).

* smoothing factors against the closed form in fp64 (alpha = 1/2, 0, 1), dead channels;
* alpha = 1/2 balances the channel maxima of the smoothed operands
  (max|X_j| / s_j = s_j max|W_j|), which fails if the scaling direction is swapped;
* per-row INT8 round trip within half a step, the row maximum at +-127, zero rows;
* the integer product and epilogue against a brute-force loop;
* on activations with outlier channels smoothing lowers the layer error (its purpose).
"""

import numpy as np
import pytest

from oracle import w8a8 as Q
from oracle.linear import _x64
from synth import BF16, FP16, calibration, weights


def test_smooth_factors_closed_form():
    X = calibration(64, 96, FP16, seed=1, outlier_frac=0.05, outlier_mult=30.0)
    W = weights(40, 96, 0.02, seed=2)
    xmax = np.abs(X.astype(np.float64)).max(axis=0)
    wmax = np.abs(W.astype(np.float64)).max(axis=0)
    np.testing.assert_allclose(Q.smooth_factors(X, FP16, W, 2), np.sqrt(xmax) / np.sqrt(wmax), rtol=4e-7)
    np.testing.assert_allclose(Q.smooth_factors(X, FP16, W, 0), 1.0 / wmax, rtol=1e-6)
    np.testing.assert_allclose(Q.smooth_factors(X, FP16, W, 4), xmax, rtol=1e-6)
    np.testing.assert_allclose(Q.smooth_factors(X, FP16, W, 1), xmax ** 0.25 / wmax ** 0.75, rtol=1e-6)
    X2 = X.copy()
    X2[:, 3] = 0
    W2 = W.copy()
    W2[:, 5] = 0
    s = Q.smooth_factors(X2, FP16, W2, 2)
    assert s[3] == 1.0 and s[5] == 1.0


def test_half_alpha_balances_channel_maxima():
    X = calibration(128, 64, FP16, seed=3, outlier_frac=0.05, outlier_mult=50.0)
    W = weights(32, 64, 0.02, seed=4)
    s = Q.smooth_factors(X, FP16, W, 2).astype(np.float64)
    xm = np.abs(X.astype(np.float64)).max(axis=0) / s
    wm = np.abs(W.astype(np.float64)).max(axis=0) * s
    np.testing.assert_allclose(xm, wm, rtol=1e-6)
    # and the activation maxima are flattened
    raw = np.abs(X.astype(np.float64)).max(axis=0)
    assert xm.max() / xm.min() < 0.5 * raw.max() / raw.min()


@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_int8_round_trip(dtype):
    X = calibration(16, 128, dtype, seed=5, outlier_frac=0.02, outlier_mult=20.0)
    W = weights(24, 128, 0.02, seed=6)
    s = Q.smooth_factors(X, dtype, W, 2)
    qx, sx = Q.quantize_act(X, dtype, s)
    xp = _x64(X, dtype) / s.astype(np.float64)[None, :]
    assert np.all(np.abs(qx * sx.astype(np.float64)[:, None] - xp) <= 0.5 * sx[:, None] * (1 + 1e-6))
    assert np.all(np.abs(qx).max(axis=1) == 127)
    qw, sw = Q.quantize_weight(W, s)
    wp = W.astype(np.float64) * s.astype(np.float64)[None, :]
    assert np.all(np.abs(qw * sw.astype(np.float64)[:, None] - wp) <= 0.5 * sw[:, None] * (1 + 1e-6))
    assert np.all(np.abs(qw.astype(int)).max(axis=1) == 127)
    Z = np.zeros((2, 128), dtype=np.float16)
    qz, sz = Q.quantize_act(Z, FP16, np.ones(128, np.float32))
    assert np.all(qz == 0) and np.all(sz == 1.0)


def test_int_product_brute_force():
    rng = np.random.default_rng(7)
    qx = rng.integers(-128, 128, size=(3, 40)).astype(np.int8)
    qw = rng.integers(-128, 128, size=(5, 40)).astype(np.int8)
    sx = rng.random(3).astype(np.float32)
    sw = rng.random(5).astype(np.float32) * np.float32(1e-3)
    Y = Q.linear_int8(qx, sx, qw, sw, FP16)
    for m in range(3):
        for n in range(5):
            acc = sum(int(qx[m, k]) * int(qw[n, k]) for k in range(40))
            y = np.float32(np.float32(np.float32(acc) * sx[m]) * sw[n])
            assert Y[m, n] == np.float16(y)


def test_smoothing_lowers_layer_error():
    X = calibration(256, 512, FP16, seed=8, outlier_frac=0.01, outlier_mult=50.0)
    W = weights(64, 512, 0.02, seed=9)
    y_true = X.astype(np.float64) @ W.astype(np.float64).T
    s = Q.smooth_factors(X, FP16, W, 2)
    y_s = Q.w8a8_reference(X, FP16, W, s)[0].astype(np.float64)
    y_0 = Q.w8a8_reference(X, FP16, W, np.ones(512, np.float32))[0].astype(np.float64)
    e_s = np.sum((y_s - y_true) ** 2)
    e_0 = np.sum((y_0 - y_true) ** 2)
    assert e_s < 0.5 * e_0
