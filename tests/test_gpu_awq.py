"""GPU parity of the AWQ entry points against the CPU oracle, through the C ABI.

* statistic: fp32 mean |x| per channel within 1 ulp-scale relative error;
* search, fed the oracle's statistic: every candidate's loss within 1e-9 (fp64, summation
  order only), the same chosen candidate (or an equal loss), and for it bit-exact scales
  s, codes, group scales and zero points;
* activation scaling: bit-exact single rounding;
* end to end: the AWQ-quantized layer through w4a16_linear with scaled activations matches
  the oracle's product within the output tolerance, and beats RTN on held-out activations.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import w4a16_dequant_gemm_amd as W4
from oracle import awq as A
from oracle import gptq as G
from synth import ASYM, BF16, FP16, SYM, calibration, weights
from tests.gpu_util import assert_close, ref_to_f64, x_to_torch, y_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    W4.lib()


def _bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("n,K,dtype", [(100, 96, FP16), (513, 384, BF16), (64, 4096, FP16)])
def test_stats(n, K, dtype):
    X = calibration(n, K, dtype, seed=n + K, outlier_frac=0.01, outlier_mult=20.0)
    got = W4.awq_stats(x_to_torch(X, dtype)).cpu().numpy()
    np.testing.assert_allclose(got, A.channel_mean_abs(X, dtype), rtol=2e-7)


CASES = [(96, 512, 128, ASYM, FP16), (64, 256, 32, SYM, BF16), (50, 384, 384, ASYM, FP16),
         (33, 1024, 64, SYM, FP16), (1024, 4096, 128, ASYM, FP16)]


@pytest.mark.parametrize("N,K,g,scheme,dtype", CASES)
def test_search_against_oracle(N, K, g, scheme, dtype):
    n = 256
    X = calibration(n, K, dtype, seed=N + K, outlier_frac=0.01, outlier_mult=20.0)
    W = weights(N, K, 0.02, seed=N * 5 + K)
    xm = A.channel_mean_abs(X, dtype)
    qw, sc, z, s, losses, best = W4.awq_search(torch.from_numpy(W).cuda(), x_to_torch(X, dtype),
                                               torch.from_numpy(xm).cuda(), g, scheme)
    torch.cuda.synchronize()
    b_ref, l_ref, s_ref, c_ref, sc_ref, z_ref = A.awq_search(W, X, dtype, xm, g, scheme)
    lg = losses.cpu().numpy()
    np.testing.assert_allclose(lg, l_ref, rtol=1e-9)
    b = int(best.cpu().numpy()[0])
    assert b == b_ref or abs(l_ref[b] - l_ref[b_ref]) <= 1e-9 * l_ref[b_ref]
    s_b = A.candidate_scales(xm, A.GRID[b])
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint32), s_b.view(np.uint32))
    codes, s_h, z_h = oracle.quantize((W / s_b[None, :]).astype(np.float32), g, scheme)
    np.testing.assert_array_equal(qw.cpu().numpy(), oracle.pack(codes))
    np.testing.assert_array_equal(_bits(sc), s_h.view(np.uint16))
    np.testing.assert_array_equal(_bits(z), z_h.view(np.uint16))


@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_scale_activations_bit_exact(dtype):
    X = calibration(37, 640, dtype, seed=5, outlier_frac=0.02, outlier_mult=50.0)
    s = A.candidate_scales(A.channel_mean_abs(X, dtype), -3)
    got = W4.awq_scale(x_to_torch(X, dtype), torch.from_numpy(s).cuda())
    ref = A.scale_activations(X, dtype, s)
    np.testing.assert_array_equal(_bits(got), ref.view(np.uint16))


@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_end_to_end_linear(dtype):
    N, K, g = 256, 1024, 128
    Xall = calibration(320, K, dtype, seed=11, outlier_frac=0.01, outlier_mult=20.0)
    Xc, Xt = Xall[:256].copy(), Xall[256:].copy()          # calibration / held-out rows
    W = weights(N, K, 0.02, seed=12)
    xm_t = W4.awq_stats(x_to_torch(Xc, dtype))
    qw, sc, z, s, losses, best = W4.awq_search(torch.from_numpy(W).cuda(), x_to_torch(Xc, dtype), xm_t, g, ASYM)
    Xs = W4.awq_scale(x_to_torch(Xt, dtype), s)
    Y = W4.linear(Xs, qw, sc, z, g)
    torch.cuda.synchronize()
    s_np = s.cpu().numpy()
    Xs_ref = A.scale_activations(Xt, dtype, s_np)
    ref = oracle.linear_ref(Xs_ref, dtype, qw.cpu().numpy(), sc.cpu().numpy(), z.cpu().numpy(), g)
    assert_close(y_to_f64(Y), ref_to_f64(ref, dtype), "awq linear")
    # held-out error against the full-precision layer (unrounded products): below RTN's
    x = oracle.linear._x64(Xt, dtype)
    y_true = x @ W.astype(np.float64).T
    rc, rs, rz = oracle.quantize(W, g, ASYM)
    y_rtn = oracle.linear_ref_f64(Xt, dtype, oracle.pack(rc), rs, rz, g)
    y_awq = oracle.linear_ref_f64(Xs_ref, dtype, qw.cpu().numpy(), sc.cpu().numpy(), z.cpu().numpy(), g)
    e_awq = np.sum((y_awq - y_true) ** 2)
    e_rtn = np.sum((y_rtn - y_true) ** 2)
    assert e_awq < 0.8 * e_rtn, (e_awq, e_rtn, int(best.cpu()[0]))
