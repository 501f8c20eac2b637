"""GPU parity of the GPTQ entry points against the CPU oracle, through the C ABI.

* Hessian: fp64 lower triangle of 2 X^T X within 1e-12 (summation order only);
* factor: U against the oracle's library inverse + Cholesky, relative to max |U|;
* quantize with the oracle's own U uploaded: codes, scales and zero points bit-exact
  (both sides compensate in fp64 and decide codes by the same fp32 RTN arithmetic);
* the whole pipeline (GPU Hessian -> GPU factor -> GPU quantize) against the whole oracle
  pipeline: codes equal except where the oracle's value sits on a rounding tie to fp64
  precision (none expected), and the layer output error below RTN's;
* the full 4096 x 4096 layer of the benchmark on sampled rows (rows are independent given U).
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import w4a16_dequant_gemm_amd as W4
from oracle import gptq as G
from synth import ASYM, BF16, FP16, SYM, calibration, weights
from tests.gpu_util import x_to_torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    W4.lib()


def _lower(a):
    return np.tril(a)


@pytest.mark.parametrize("n,K,dtype", [(64, 96, FP16), (300, 256, BF16), (1000, 200, FP16)])
def test_hessian(n, K, dtype):
    X = calibration(n, K, dtype, seed=n + K)
    H = W4.gptq_hessian(x_to_torch(X, dtype)).cpu().numpy()
    ref = G.hessian(X, dtype)
    np.testing.assert_allclose(_lower(H), _lower(ref), rtol=1e-12, atol=1e-12 * np.abs(ref).max())
    # accumulation over two calibration batches
    H2 = W4.gptq_hessian(x_to_torch(X[: n // 2], dtype))
    W4.gptq_hessian(x_to_torch(X[n // 2:], dtype), H2)
    np.testing.assert_allclose(_lower(H2.cpu().numpy()), _lower(ref), rtol=1e-12,
                               atol=1e-12 * np.abs(ref).max())


@pytest.mark.parametrize("K,damp", [(64, 0.0), (200, 0.01), (512, 0.01), (1000, 0.1)])
def test_factor(K, damp):
    X = calibration(max(2 * K, 256), K, FP16, seed=K)
    Href = G.damp_hessian(G.hessian(X, FP16), damp)
    # only the lower triangle is read: NaN above the diagonal must not reach U
    Hl = np.tril(G.hessian(X, FP16))
    Hl[np.triu_indices(K, 1)] = np.nan
    H = torch.from_numpy(Hl).cuda()
    U = W4.gptq_factor(H, damp).cpu().numpy()
    ref = G.inverse_cholesky_upper(Href)
    assert np.all(np.tril(U, -1) == 0.0)
    err = np.abs(U - ref).max() / np.abs(ref).max()
    assert err < 1e-9, err


def _gpu_quant(W, U, g, scheme):
    qw, s, z = W4.gptq_quantize(torch.from_numpy(W).cuda(), torch.from_numpy(np.ascontiguousarray(U)).cuda(),
                                g, scheme)
    torch.cuda.synchronize()
    return qw.cpu().numpy(), s.cpu().numpy(), z.cpu().numpy()


@pytest.mark.parametrize("N,K,g,scheme", [(300, 512, 128, ASYM), (77, 256, 32, SYM), (64, 384, 384, ASYM),
                                          (130, 1024, 64, ASYM), (33, 96, 96, SYM)])
def test_quantize_with_oracle_factor(N, K, g, scheme):
    X = calibration(max(2 * K, 512), K, FP16, seed=N + K)
    W = weights(N, K, 0.02, seed=N * 3 + K, outlier_frac=0.002, outlier_mult=10.0)
    U = G.inverse_cholesky_upper(G.damp_hessian(G.hessian(X, FP16), 0.01))
    qn, sn, zn = _gpu_quant(W, U, g, scheme)
    codes, s_ref, z_ref = G.gptq_quantize(W, U, g, scheme)
    np.testing.assert_array_equal(qn, oracle.pack(codes))
    np.testing.assert_array_equal(sn.view(np.uint16), s_ref.view(np.uint16))
    np.testing.assert_array_equal(zn.view(np.uint16), z_ref.view(np.uint16))


def _compare_codes_allowing_ties(qn, sn, zn, W, U, g, scheme, rows=None):
    Wr = W if rows is None else W[rows]
    pre = np.zeros(Wr.shape, dtype=np.float64)
    codes, s_ref, z_ref = G.gptq_quantize(Wr, U, g, scheme, pre=pre)
    got = oracle.unpack(qn if rows is None else qn[rows])
    mism = np.argwhere(got != codes)
    for n, k in mism:
        s = np.float32(s_ref[n, k // g])
        t = np.float64(np.float32(pre[n, k])) / np.float64(s)
        assert abs(abs(t - np.floor(t)) - 0.5) < 1e-6, f"code mismatch off a tie at ({n}, {k})"
    assert len(mism) <= max(1, got.size // 100000)
    sg = sn if rows is None else sn[rows]
    same_groups = np.all(got.reshape(got.shape[0], -1, g) == codes.reshape(codes.shape[0], -1, g), axis=2)
    # where no code of the row differs before a group, its parameters must agree exactly
    ok_prefix = np.cumprod(np.concatenate([np.ones((got.shape[0], 1), bool), same_groups[:, :-1]], axis=1),
                           axis=1).astype(bool)
    np.testing.assert_array_equal(sg.view(np.uint16)[ok_prefix], s_ref.view(np.uint16)[ok_prefix])
    return codes, s_ref, z_ref


@pytest.mark.parametrize("dtype,scheme,g", [(FP16, ASYM, 128), (BF16, SYM, 64)])
def test_pipeline_against_oracle(dtype, scheme, g):
    n, K, N = 1024, 512, 200
    X = calibration(n, K, dtype, seed=21)
    W = weights(N, K, 0.02, seed=22, outlier_frac=0.002, outlier_mult=10.0)
    H = W4.gptq_hessian(x_to_torch(X, dtype))
    Ut = W4.gptq_factor(H, 0.01)
    qw, s, z = W4.gptq_quantize(torch.from_numpy(W).cuda(), Ut, g, scheme)
    torch.cuda.synchronize()
    qn, sn, zn = qw.cpu().numpy(), s.cpu().numpy(), z.cpu().numpy()
    U = G.inverse_cholesky_upper(G.damp_hessian(G.hessian(X, dtype), 0.01))
    _compare_codes_allowing_ties(qn, sn, zn, W, U, g, scheme)
    # the quantized layer beats RTN on the calibration data
    W_hat = oracle.dequantize(qn, sn, zn, g)
    rc, rs, rz = oracle.quantize(W, g, scheme)
    e_rtn = G.layer_error(X, dtype, W, oracle.dequantize(oracle.pack(rc), rs, rz, g))
    assert G.layer_error(X, dtype, W, W_hat) < 0.8 * e_rtn


def test_full_layer_sampled_rows():
    # the benchmark's layer: K = N = 4096, g = 128, 2048 calibration rows
    n, K, N, g = 2048, 4096, 4096, 128
    X = calibration(n, K, FP16, seed=31)
    W = weights(N, K, 0.02, seed=32)
    H = W4.gptq_hessian(x_to_torch(X, FP16))
    Ut = W4.gptq_factor(H, 0.01)
    qw, s, z = W4.gptq_quantize(torch.from_numpy(W).cuda(), Ut, g, ASYM)
    torch.cuda.synchronize()
    U = G.inverse_cholesky_upper(G.damp_hessian(G.hessian(X, FP16), 0.01))
    err = np.abs(Ut.cpu().numpy() - U).max() / np.abs(U).max()
    assert err < 1e-9, err
    rows = np.unique(np.concatenate([[0, N - 1], np.random.default_rng(33).choice(N, 14, replace=False)]))
    _compare_codes_allowing_ties(qw.cpu().numpy(), s.cpu().numpy(), z.cpu().numpy(), W, U, g, ASYM, rows)
