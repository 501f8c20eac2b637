"""Pins for the GPTQ oracle (CPU only).

* H proportional to the identity: no compensation, GPTQ is RTN bit for bit;
* optimality: after every column the still-free weights equal the least-squares
  optimum of the layer output error given the columns already fixed, computed by an
  independent library least-squares solve (this is what step 2c is for);
* K = 2 closed form of the single compensation step;
* the page's running-inverse form (gptq_obs) and the Cholesky form agree;
* the Cholesky factor reproduces H^-1; H = 2 X^T X by brute force;
* the layer output error is below RTN's on correlated calibration data.
"""

import numpy as np
import pytest

import oracle
from oracle import gptq as G
from synth import FP16, BF16, calibration, weights


def _dequant(codes, s, z, g):
    return oracle.dequantize(oracle.pack(codes), s, z, g)


def test_hessian_brute_force():
    X = calibration(7, 5, FP16, seed=1)
    H = G.hessian(X, FP16)
    x = X.astype(np.float64)
    ref = np.zeros((5, 5))
    for t in range(7):
        for a in range(5):
            for b in range(5):
                ref[a, b] += 2.0 * x[t, a] * x[t, b]
    np.testing.assert_allclose(H, ref, rtol=1e-14, atol=0)
    assert np.all(np.linalg.eigvalsh(H) > -1e-9)


def test_damping_adds_scaled_identity():
    H = np.array([[4.0, 1.0], [1.0, 2.0]])
    Hd = G.damp_hessian(H, 0.5)
    np.testing.assert_array_equal(Hd, [[5.5, 1.0], [1.0, 3.5]])      # mean(diag) = 3
    np.testing.assert_array_equal(G.damp_hessian(H, 0.0), H)


def test_inverse_cholesky_factor():
    X = calibration(64, 24, FP16, seed=2)
    H = G.hessian(X, FP16)
    U = G.inverse_cholesky_upper(H)
    assert np.all(np.tril(U, -1) == 0) and np.all(np.diag(U) > 0)
    np.testing.assert_allclose(U.T @ U @ H, np.eye(24), atol=1e-9)


@pytest.mark.parametrize("scheme", [oracle.ASYM, oracle.SYM])
@pytest.mark.parametrize("g", [8, 32])
def test_identity_hessian_is_rtn(scheme, g):
    K = 32
    X = (3.0 * np.eye(K)).astype(np.float16)             # H = 18 I
    W = weights(10, K, 0.02, seed=3, outlier_frac=0.05, outlier_mult=10.0)
    H = G.hessian(X, FP16)
    rtn = oracle.quantize(W, g, scheme)
    for res in (G.gptq_quantize(W, G.inverse_cholesky_upper(H), g, scheme), G.gptq_obs(W, H, g, scheme)):
        for a, b in zip(res, rtn):
            np.testing.assert_array_equal(a, b)


def test_two_column_closed_form():
    # one compensation step: w1' = w1 + (w0 - w0_hat) * H01 / H11
    W = np.array([[0.3, -0.7]], dtype=np.float32)
    H = np.array([[2.0, 0.6], [0.6, 1.5]])
    trace = []
    codes, s, z = G.gptq_obs(W, H, 2, oracle.ASYM, trace=trace)
    w0_hat = float(s[0, 0]) * (float(codes[0, 0]) - float(z[0, 0]))
    w0, w1 = float(W[0, 0]), float(W[0, 1])
    expect = w1 + (w0 - w0_hat) * 0.6 / 1.5
    assert trace[0][0, 1] == pytest.approx(expect, rel=1e-14)
    trace2 = []
    G.gptq_quantize(W, G.inverse_cholesky_upper(H), 2, oracle.ASYM, trace=trace2)
    assert trace2[0][0, 1] == pytest.approx(expect, rel=1e-12)


@pytest.mark.parametrize("form", ["obs", "chol"])
def test_free_columns_are_least_squares_optimal(form):
    # after fixing columns 0..i, the free columns minimize ||X (W' - W)^T||^2; solved here
    # by an independent least-squares routine, row by row
    n, K, N, g = 96, 16, 5, 8
    X = calibration(n, K, FP16, seed=4, n_factors=4)
    x = X.astype(np.float64)
    W = weights(N, K, 0.05, seed=5)
    H = G.hessian(X, FP16)
    trace = []
    if form == "obs":
        G.gptq_obs(W, H, g, oracle.ASYM, trace=trace)
    else:
        G.gptq_quantize(W, G.inverse_cholesky_upper(H), g, oracle.ASYM, trace=trace)
    W64 = W.astype(np.float64)
    for i in (0, 3, 7, 8, 12):
        cur = trace[i]
        d_fixed = cur[:, :i + 1] - W64[:, :i + 1]
        for r in range(N):
            rhs = -(x[:, :i + 1] @ d_fixed[r])
            sol, *_ = np.linalg.lstsq(x[:, i + 1:], rhs, rcond=None)
            np.testing.assert_allclose(cur[r, i + 1:] - W64[r, i + 1:], sol, rtol=1e-7, atol=1e-9)


@pytest.mark.parametrize("scheme", [oracle.ASYM, oracle.SYM])
@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_obs_and_cholesky_forms_agree(scheme, dtype):
    X = calibration(300, 64, dtype, seed=6)
    W = weights(12, 64, 0.02, seed=7, outlier_frac=0.01, outlier_mult=10.0)
    H = G.damp_hessian(G.hessian(X, dtype), 0.01)
    a = G.gptq_obs(W, H, 32, scheme)
    b = G.gptq_quantize(W, G.inverse_cholesky_upper(H), 32, scheme)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


@pytest.mark.parametrize("g", [32, 128])
def test_error_below_rtn(g):
    n, K, N = 512, 256, 48
    X = calibration(n, K, FP16, seed=8)
    W = weights(N, K, 0.02, seed=9, outlier_frac=0.002, outlier_mult=10.0)
    H = G.damp_hessian(G.hessian(X, FP16), 0.01)
    codes, s, z = G.gptq_quantize(W, G.inverse_cholesky_upper(H), g, oracle.ASYM)
    e_gptq = G.layer_error(X, FP16, W, _dequant(codes, s, z, g))
    rc, rs, rz = oracle.quantize(W, g, oracle.ASYM)
    e_rtn = G.layer_error(X, FP16, W, _dequant(rc, rs, rz, g))
    assert e_gptq < 0.8 * e_rtn


def test_group_start_parameters_cover_current_weights():
    # G2: the first column of a group lies inside the range its own parameters were
    # computed from, so its round trip is within half a step
    X = calibration(256, 64, FP16, seed=10)
    W = weights(16, 64, 0.02, seed=11)
    H = G.damp_hessian(G.hessian(X, FP16), 0.01)
    trace = []
    codes, s, z = G.gptq_quantize(W, G.inverse_cholesky_upper(H), 16, oracle.ASYM, trace=trace)
    for grp in range(4):
        i = 16 * grp
        before = (W.astype(np.float64) if i == 0 else trace[i - 1])[:, i].astype(np.float32)
        sc = s[:, grp].astype(np.float64)
        w_hat = sc * (codes[:, i].astype(np.float64) - z[:, grp].astype(np.float64))
        assert np.all(np.abs(before.astype(np.float64) - w_hat) <= 0.5 * sc * (1 + 1e-6))
