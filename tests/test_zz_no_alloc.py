"""GPU test of the entry point that allocates nothing, w4a16_linear_ws_noalloc, called
through the C ABI with raw device pointers.

Its output must be bit-identical to that of w4a16_linear_ws with a caller workspace (the
same kernels and split plan, only the workspace differs), on two calls in a row on one GPU,
the second with a smaller problem (the static buffer keeps the first call's partial tiles),
and again on a problem that does not split K (it then runs as w4a16_linear).  A sample of
each output is also held to the oracle's bar.
"""

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


def _problem(M, N, K, g, seed):
    W = weights(N, K, 0.02, seed=seed)
    X = activations(M, K, FP16, seed + 1)
    codes, s, z = oracle.quantize_asym(W, g)
    qn = oracle.pack(codes)
    qw, st, zt = upload_packed(qn, s, z)
    return X, qn, s, z, x_to_torch(X, FP16), qw, st, zt


def _noalloc(Xt, qw, st, zt, g):
    M, K = Xt.shape
    N = qw.shape[0]
    Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
    rc = W4.lib().w4a16_linear_ws_noalloc(Xt.data_ptr(), W4.F16, M, N, K, g, qw.data_ptr(), st.data_ptr(),
                                          zt.data_ptr(), Y.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, W4.lib().w4a16_strerror(rc)
    return Y


def test_noalloc_matches_workspace_form_on_consecutive_calls():
    g = 128
    # first call: the largest split of the prefill crossover (64 MiB of partial tiles), then a
    # smaller one (43 MB), then one that does not split K at all
    cases = [(1024, 4096, 11008), (256, 11008, 4096), (8, 1000, 4096)]
    outs = []
    for i, (M, N, K) in enumerate(cases):
        X, qn, s, z, Xt, qw, st, zt = _problem(M, N, K, g, seed=900 + i)
        need = W4.linear_workspace(M, N, K, g)
        assert (need > 0) == (i < 2)
        Y = _noalloc(Xt, qw, st, zt, g)
        outs.append((X, qn, s, z, Xt, qw, st, zt, Y))
    torch.cuda.synchronize()
    for (M, N, K), (X, qn, s, z, Xt, qw, st, zt, Y) in zip(cases, outs):
        want = W4.linear_ws(Xt, qw, st, zt, g)
        torch.cuda.synchronize()
        assert torch.equal(Y.view(torch.int16), want.view(torch.int16)), f"M={M} N={N} K={K}"
        rng = np.random.default_rng(M + N)
        ms = np.unique(np.r_[0, M - 1, rng.choice(M, min(M, 32), replace=False)])
        ref = oracle.linear_ref(X[ms], FP16, qn, s, z, g)
        assert_close(y_to_f64(Y[torch.from_numpy(ms).cuda()]), ref.astype(np.float64), f"noalloc M={M}")
    # the larger problem again after the smaller one: the stale partial tiles of the buffer
    # must not leak into the result
    X, qn, s, z, Xt, qw, st, zt, Y0 = outs[0]
    Y1 = _noalloc(Xt, qw, st, zt, g)
    torch.cuda.synchronize()
    assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16))
