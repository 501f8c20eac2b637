"""Pins for the oracle linear layer (CPU only).

``linear_ref`` (float64 BLAS product, one rounding) is pinned against the
exact-rational brute force on tiny shapes, against one-hot activations (which
select a dequantized weight exactly), against power-of-two scaling, against a
group-factored evaluation order, against torch's CPU matmul (an independent
library routine) and against the a-priori quantization error bound.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.linear import BF16_DT, FP16
from synth import activations, weights


def _case(M, K, N, g, scheme, dtype, seed):
    W = weights(N, K, 0.05, seed)
    X = activations(M, K, dtype, seed + 1)
    codes, s, z = oracle.quantize(W, g, scheme)
    return W, X, oracle.pack(codes), s, z


def _bits(y, dtype):
    return y.view(np.uint16) if dtype == FP16 else y


@pytest.mark.parametrize("dtype", [FP16, BF16_DT])
@pytest.mark.parametrize("scheme", [oracle.ASYM, oracle.SYM])
@pytest.mark.parametrize("M,K,N,g", [(1, 16, 3, 8), (3, 32, 5, 16), (2, 64, 4, 32), (4, 48, 2, 48)])
def test_linear_ref_equals_exact_rational(dtype, scheme, M, K, N, g):
    _, X, Wq, s, z = _case(M, K, N, g, scheme, dtype, seed=100 + M * K + N)
    got = oracle.linear_ref(X, dtype, Wq, s, z, g)
    want = oracle.linear_exact(X, dtype, Wq, s, z, g)
    np.testing.assert_array_equal(_bits(got, dtype), _bits(want, dtype))


@pytest.mark.parametrize("dtype", [FP16, BF16_DT])
def test_one_hot_selects_dequantized_weight(dtype):
    K, N, g = 256, 40, 64
    _, _, Wq, s, z = _case(1, K, N, g, oracle.ASYM, dtype, seed=7)
    ks = [0, 1, 7, 8, 63, 64, 200, 255]
    X64 = np.zeros((len(ks), K))
    for m, k in enumerate(ks):
        X64[m, k] = 1.0
    X = X64.astype(np.float16) if dtype == FP16 else oracle.round_to_bf16_bits(X64)
    y = oracle.linear_ref(X, dtype, Wq, s, z, g)
    D = oracle.dequantize(Wq, s, z, g)
    want = D[:, ks].T
    want = oracle.round_to_f16(want) if dtype == FP16 else oracle.round_to_bf16_bits(want)
    np.testing.assert_array_equal(_bits(y, dtype), _bits(want, dtype))


def test_power_of_two_scaling_of_x():
    _, X, Wq, s, z = _case(4, 512, 16, 128, oracle.ASYM, FP16, seed=11)
    y1 = oracle.linear_ref(X, FP16, Wq, s, z, 128).astype(np.float64)
    X2 = (X.astype(np.float64) * 4.0).astype(np.float16)
    y2 = oracle.linear_ref(X2, FP16, Wq, s, z, 128).astype(np.float64)
    np.testing.assert_array_equal(y2, 4.0 * y1)


def test_group_factored_order_agrees():
    # sum_g s_g * sum_{k in g} x_k (u_k - z_g): same value, another evaluation order
    _, X, Wq, s, z = _case(3, 512, 24, 128, oracle.ASYM, FP16, seed=13)
    y = oracle.linear_ref_f64(X, FP16, Wq, s, z, 128)
    u = oracle.unpack(Wq).astype(np.float64)
    x = X.astype(np.float64)
    alt = np.zeros_like(y)
    for j in range(4):
        sl = slice(128 * j, 128 * (j + 1))
        part = x[:, sl] @ (u[:, sl] - z[:, j:j + 1].astype(np.float64)).T
        alt += part * s[:, j].astype(np.float64)[None, :]
    np.testing.assert_allclose(y, alt, rtol=1e-12, atol=1e-12)


def test_matches_torch_cpu_matmul():
    _, X, Wq, s, z = _case(5, 1024, 48, 128, oracle.ASYM, FP16, seed=17)
    y = oracle.linear_ref_f64(X, FP16, Wq, s, z, 128)
    D = torch.from_numpy(oracle.dequantize(Wq, s, z, 128))
    yt = torch.from_numpy(X.astype(np.float64)) @ D.T
    np.testing.assert_allclose(y, yt.numpy(), rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("scheme", [oracle.ASYM, oracle.SYM])
def test_quantized_output_within_error_bound(scheme):
    # |Y_q - X W^T| <= sum_k |x_k| * s * 0.5073 (per-element round-trip bound)
    W, X, Wq, s, z = _case(4, 1024, 64, 128, scheme, FP16, seed=19)
    yq = oracle.linear_ref_f64(X, FP16, Wq, s, z, 128)
    x = X.astype(np.float64)
    ytrue = x @ W.astype(np.float64).T
    sf = np.repeat(s.astype(np.float64), 128, axis=1)
    bound = np.abs(x) @ (0.5073 * sf).T
    assert np.all(np.abs(yq - ytrue) <= bound)
    # and the quantization actually perturbs the product (guards against a no-op)
    assert np.abs(yq - ytrue).max() > 0


def test_rectangular_orientation():
    # Y is [M, N]; W is [N, K]: a transposed operand cannot pass these shapes
    _, X, Wq, s, z = _case(3, 64, 5, 32, oracle.ASYM, FP16, seed=23)
    y = oracle.linear_ref(X, FP16, Wq, s, z, 32)
    assert y.shape == (3, 5)
    with pytest.raises(ValueError):
        oracle.linear_ref(X[:, :32], FP16, Wq, s, z, 32)
