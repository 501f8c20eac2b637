"""GPU parity of the W8A8 / SmoothQuant entry points against the CPU oracle, through the C
ABI.  Every step uses one fixed fp32 operation order on both sides, so everything is
compared bit for bit: smoothing factors, INT8 codes and fp32 scales of weights and
activations, and the output of the INT8 matrix-core product (ragged M and N, full-size
shapes on sampled rows).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import w4a16_dequant_gemm_amd as W4
from oracle import w8a8 as Q
from synth import BF16, FP16, calibration, weights
from tests.gpu_util import x_to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    W4.lib()


def _u16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _f32bits(t) -> np.ndarray:
    return (t.cpu().numpy() if isinstance(t, torch.Tensor) else t).astype(np.float32).view(np.uint32)


# K % 4 == 0 takes the 64-channel tile kernel (ragged last tile at 4100, rows not a
# multiple of the 512-row stride); K = 322 the one-thread-per-channel kernel
@pytest.mark.parametrize("dtype,a,n,N,K", [(FP16, 2, 200, 96, 320), (BF16, 1, 200, 96, 320), (FP16, 4, 200, 96, 320),
                                           (FP16, 0, 200, 96, 320), (FP16, 2, 90, 50, 322),
                                           (BF16, 2, 1000, 700, 4100), (FP16, 3, 3, 1, 64)])
def test_smooth_factors(dtype, a, n, N, K):
    X = calibration(n, K, dtype, seed=a + 1, outlier_frac=0.02, outlier_mult=40.0)
    W = weights(N, K, 0.02, seed=a + 2)
    W[:, 7] = 0.0
    s = W4.w8a8_smooth(x_to_torch(X, dtype), torch.from_numpy(W).cuda(), a)
    np.testing.assert_array_equal(_f32bits(s), _f32bits(Q.smooth_factors(X, dtype, W, a)))


@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("K", [640, 200, 11008, 16384])     # vectorized and scalar row kernels
def test_quantize_operands(dtype, K):
    X = calibration(77, K, dtype, seed=3, outlier_frac=0.02, outlier_mult=40.0)
    W = weights(130, K, 0.02, seed=4)
    s = Q.smooth_factors(X, dtype, W, 2)
    st = torch.from_numpy(s).cuda()
    qw, sw = W4.w8a8_quantize_weight(torch.from_numpy(W).cuda(), st)
    qx, sx = W4.w8a8_quantize_act(x_to_torch(X, dtype), st)
    rqw, rsw = Q.quantize_weight(W, s)
    rqx, rsx = Q.quantize_act(X, dtype, s)
    np.testing.assert_array_equal(qw.cpu().numpy(), rqw)
    np.testing.assert_array_equal(_f32bits(sw), _f32bits(rsw))
    np.testing.assert_array_equal(qx.cpu().numpy(), rqx)
    np.testing.assert_array_equal(_f32bits(sx), _f32bits(rsx))


LIN = [(1, 64, 128), (70, 300, 256), (256, 256, 512), (300, 257, 1024), (513, 700, 384), (33, 1, 128)]


@pytest.mark.parametrize("M,N,K", LIN)
@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_linear_bit_exact(M, N, K, dtype):
    rng = np.random.default_rng(M * 7 + N + K)
    qx = rng.integers(-128, 128, size=(M, K)).astype(np.int8)
    qw = rng.integers(-128, 128, size=(N, K)).astype(np.int8)
    sx = (rng.random(M) * 0.05 + 1e-3).astype(np.float32)
    sw = (rng.random(N) * 1e-3 + 1e-5).astype(np.float32)
    Y = W4.w8a8_linear(torch.from_numpy(qx).cuda(), torch.from_numpy(sx).cuda(), torch.from_numpy(qw).cuda(),
                       torch.from_numpy(sw).cuda(), torch.float16 if dtype == FP16 else torch.bfloat16)
    ref = Q.linear_int8(qx, sx, qw, sw, dtype)
    np.testing.assert_array_equal(_u16(Y), ref.view(np.uint16))


@pytest.mark.parametrize("K,N", [(4096, 11008), (11008, 4096)])
def test_full_size_sampled_rows(K, N):
    M = 4096
    X = calibration(M, K, FP16, seed=K, outlier_frac=0.01, outlier_mult=20.0)
    W = weights(N, K, 0.02, seed=N)
    Xt = x_to_torch(X, FP16)
    Wt = torch.from_numpy(W).cuda()
    s = W4.w8a8_smooth(Xt, Wt, 2)
    qw, sw = W4.w8a8_quantize_weight(Wt, s)
    qx, sx = W4.w8a8_quantize_act(Xt, s)
    Y = W4.w8a8_linear(qx, sx, qw, sw)
    torch.cuda.synchronize()
    s_ref = Q.smooth_factors(X, FP16, W, 2)
    np.testing.assert_array_equal(_f32bits(s), _f32bits(s_ref))
    rows = np.unique(np.concatenate([[0, M - 1], np.random.default_rng(1).choice(M, 14, replace=False)]))
    rqw, rsw = Q.quantize_weight(W, s_ref)
    rqx, rsx = Q.quantize_act(X[rows], FP16, s_ref)
    np.testing.assert_array_equal(qw.cpu().numpy(), rqw)
    np.testing.assert_array_equal(qx.cpu().numpy()[rows], rqx)
    ref = Q.linear_int8(rqx, rsx, rqw, rsw, FP16)
    np.testing.assert_array_equal(_u16(Y)[rows], ref.view(np.uint16))


def test_smoothing_beats_plain_w8a8_end_to_end():
    X = calibration(256, 1024, FP16, seed=9, outlier_frac=0.01, outlier_mult=50.0)
    W = weights(512, 1024, 0.02, seed=10)
    Xt, Wt = x_to_torch(X, FP16), torch.from_numpy(W).cuda()
    y_true = X.astype(np.float64) @ W.astype(np.float64).T
    errs = []
    for s in (W4.w8a8_smooth(Xt, Wt, 2), torch.ones(1024, dtype=torch.float32, device="cuda")):
        qw, sw = W4.w8a8_quantize_weight(Wt, s)
        qx, sx = W4.w8a8_quantize_act(Xt, s)
        Y = W4.w8a8_linear(qx, sx, qw, sw).cpu().numpy().astype(np.float64)
        errs.append(np.sum((Y - y_true) ** 2))
    assert errs[0] < 0.5 * errs[1]
