"""GPU parity of the workspace form of the linear call (split K over the idle CUs for the
prefill regime's tile-starved shapes), through the C ABI: the output against the fp64 oracle
within the output bar, including full-size layers on sampled rows and columns; identical
results on repeated calls; and without a workspace the call is w4a16_linear, bit for bit."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import w4a16_dequant_gemm_amd as W4
from synth import FP16, activations, weights
from tests.gpu_util import assert_close, upload_packed, x_to_torch, y_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    W4.lib()


def _setup(M, N, K, g, scheme, seed):
    W = weights(N, K, 0.02, seed=seed)
    X = activations(M, K, FP16, seed + 1, outlier_frac=0.01, outlier_mult=20.0)
    codes, s, z = oracle.quantize(W, g, scheme)
    qn = oracle.pack(codes)
    return X, qn, s, z


@pytest.mark.parametrize("M,N,K,g,scheme,zeros_none", [
    (40, 300, 2048, 128, oracle.ASYM, False), (100, 513, 4096, 64, oracle.ASYM, False),
    (300, 256, 8192, 128, oracle.SYM, True), (257, 700, 2176, 2176, oracle.ASYM, False),
    (64, 64, 11008, 128, oracle.SYM, False)])
def test_splitk_matches_oracle(M, N, K, g, scheme, zeros_none):
    assert W4.linear_workspace(M, N, K, g) > 0
    X, qn, s, z = _setup(M, N, K, g, scheme, seed=M + N + K)
    zz = None if zeros_none else z
    qw, st, zt = upload_packed(qn, s, zz)
    Xt = x_to_torch(X, FP16)
    Y = W4.linear_ws(Xt, qw, st, zt, g)
    ref = oracle.linear_ref(X, FP16, qn, s, zz, g)
    assert_close(y_to_f64(Y), ref.astype(np.float64), f"split-K M={M} N={N} K={K}")
    # deterministic: a second call gives the same bits
    Y2 = W4.linear_ws(Xt, qw, st, zt, g)
    assert torch.equal(Y.view(torch.int16), Y2.view(torch.int16))


def test_without_workspace_is_the_plain_call():
    M, N, K, g = 100, 300, 4096, 128
    X, qn, s, z = _setup(M, N, K, g, oracle.ASYM, seed=11)
    qw, st, zt = upload_packed(qn, s, z)
    Xt = x_to_torch(X, FP16)
    Y0 = W4.linear(Xt, qw, st, zt, g)
    small = torch.empty(16, dtype=torch.float32, device="cuda")       # too small: no split
    Y1 = W4.linear_ws(Xt, qw, st, zt, g, work=small)
    assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16))


@pytest.mark.parametrize("M,K,N", [(256, 11008, 4096), (1024, 11008, 4096), (256, 4096, 11008)])
def test_full_size_sampled(M, K, N):
    g = 128
    rng = np.random.default_rng(M + K)
    W = weights(N, K, 0.02, seed=21 + K)
    X = activations(M, K, FP16, seed=22 + M)
    qw, s, z = W4.quantize_pack(torch.from_numpy(W).cuda(), g, W4.ASYM)
    Y = W4.linear_ws(x_to_torch(X, FP16), qw, s, z, g)
    torch.cuda.synchronize()
    ns = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 1024, replace=False)]))
    ms = np.unique(np.concatenate([[0, M - 1], rng.choice(M, 64, replace=False)]))
    codes, s_ref, z_ref = oracle.quantize(W[ns], g, oracle.ASYM)
    qn = oracle.pack(codes)
    idx = torch.from_numpy(ns).cuda()
    np.testing.assert_array_equal(qw[idx].cpu().numpy(), qn)
    ref = oracle.linear_ref(X[ms], FP16, qn, s_ref, z_ref, g)
    y = y_to_f64(Y[torch.from_numpy(ms).cuda()][:, idx])
    assert_close(y, ref.astype(np.float64), f"split-K full M={M} K={K} N={N}")
