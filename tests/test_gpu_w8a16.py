"""GPU parity of the W8A16 entry points against the CPU oracle, through the C ABI.

* quantize-pack: 8-bit codes (as packed words), fp16 scales and zeros bit-exact, both
  schemes, group sizes 32 .. K, outlier weights;
* linear: both kernels (the weight-streaming GEMV for M <= 16, one weight row per wave at
  M = 1 and two from M = 2 on; the tiled MFMA GEMM) against the fp64 oracle within the
  output bar (relative Frobenius <= 1e-3, max |d| <= 1e-2 max |ref|), fp16 and bf16 activations, ragged N and M, per-channel groups, symmetric with and
  without stored zero points, both kernels forced on the same problems;
* one-hot activations: each output is one dequantized weight, rounded once, bit-exact;
* full-size layers (the 7B-like shapes at M = 1 and 4, the prefill at M = 4096), sampled.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import w4a16_dequant_gemm_amd as W4
from oracle import w8a16 as W8
from synth import BF16, FP16, activations, weights
from tests.gpu_util import assert_close, ref_bits, ref_to_f64, x_to_torch, y_bits, y_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    W4.lib()


def _quantize_both(N, K, g, scheme, seed, outliers=True):
    W = weights(N, K, 0.02, seed=seed, outlier_frac=0.001 if outliers else 0.0, outlier_mult=20.0)
    qw, s, z = W4.w8a16_quantize_pack(torch.from_numpy(W).cuda(), g, scheme)
    codes, s_ref, z_ref = W8.quantize8(W, g, scheme)
    return W, (qw, s, z), (W8.pack8(codes), s_ref, z_ref)


@pytest.mark.parametrize("scheme", [W8.ASYM, W8.SYM])
@pytest.mark.parametrize("N,K,g", [(64, 128, 32), (37, 1024, 128), (100, 4096, 64), (13, 768, 768),
                                   (5, 11008, 11008), (300, 4096, 4096)])
def test_quantize_pack_bit_exact(N, K, g, scheme):
    _, (qw, s, z), (q_ref, s_ref, z_ref) = _quantize_both(N, K, g, scheme, seed=N + K + g + scheme)
    np.testing.assert_array_equal(qw.cpu().numpy(), q_ref)
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint16), s_ref.view(np.uint16))
    np.testing.assert_array_equal(z.cpu().numpy().view(np.uint16), z_ref.view(np.uint16))


def test_quantize_sym_without_zeros():
    W = weights(40, 512, 0.02, seed=404)
    qw, s, z = W4.w8a16_quantize_pack(torch.from_numpy(W).cuda(), 128, W8.SYM, write_zeros=False)
    assert z is None
    codes, s_ref, _ = W8.quantize_sym8(W, 128)
    np.testing.assert_array_equal(qw.cpu().numpy(), W8.pack8(codes))
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint16), s_ref.view(np.uint16))


def _linear_case(M, N, K, g, dtype, scheme, path, seed, zeros_none=False):
    W, (qw, s, z), (q_ref, s_ref, z_ref) = _quantize_both(N, K, g, scheme, seed)
    np.testing.assert_array_equal(qw.cpu().numpy(), q_ref)
    X = activations(M, K, dtype, seed=seed + 1, outlier_frac=0.01, outlier_mult=20.0)
    zz = None if zeros_none else z
    Y = W4.w8a16_linear(x_to_torch(X, dtype), qw, s, zz, g, path=path)
    ref = W8.linear8_ref(X, dtype, q_ref, s_ref, None if zeros_none else z_ref, g)
    assert_close(y_to_f64(Y), ref_to_f64(ref, dtype), f"w8a16 M={M} N={N} K={K} g={g} path={path}")
    return Y


GEMV_CASES = [(1, 4096, 4096, 128), (2, 300, 1024, 32), (3, 1000, 2048, 64), (4, 37, 4096, 128),
              (1, 11008, 4096, 128), (1, 4096, 11008, 128), (1, 1024, 28672, 128), (4, 129, 7168, 7168),
              (1, 8, 32, 32),
              # activations staged in K slices (M rows of K do not fit 64 KB): several slices, a
              # ragged last slice, per-channel groups spanning slices
              (4, 300, 11008, 128), (3, 70, 20480, 256), (1, 33, 32768, 32768), (2, 1000, 15360, 64),
              # up to 16 activation rows (several K slices from M = 8 on)
              (8, 500, 4096, 128), (16, 257, 4096, 64), (13, 130, 11008, 11008),
              # two rows per wave: odd N (the last wave's second row is past the end), odd M
              # over several K slices
              (15, 201, 4096, 128), (2, 1, 1024, 128), (3, 17, 2048, 32)]
PREFILL_CASES = [(5, 4096, 1024, 128), (64, 300, 2048, 64), (300, 1000, 1024, 128), (129, 257, 4096, 4096),
                 (4, 4096, 11008, 128), (1, 64, 128, 64), (512, 128, 640, 128),
                 # more groups per row than one LDS staging holds (fp16: staged in phases)
                 (200, 300, 8192, 64)]


@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("M,N,K,g", GEMV_CASES)
def test_linear_gemv(M, N, K, g, dtype):
    assert W4.w8a16_select_path(M, N, K, g, dtype) == W4.PATH_GEMV
    _linear_case(M, N, K, g, dtype, W8.ASYM, W4.PATH_GEMV, seed=1000 + M + N + K)


@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("M,N,K,g", PREFILL_CASES)
def test_linear_prefill(M, N, K, g, dtype):
    _linear_case(M, N, K, g, dtype, W8.ASYM, W4.PATH_PREFILL, seed=2000 + M + N + K)


@pytest.mark.parametrize("path", [W4.PATH_GEMV, W4.PATH_PREFILL])
@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("zeros_none", [False, True])
def test_linear_symmetric(path, dtype, zeros_none):
    _linear_case(3, 200, 1024, 128, dtype, W8.SYM, path, seed=3000 + path, zeros_none=zeros_none)


@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_both_kernels_on_the_same_problem(dtype):
    ys = [_linear_case(4, 513, 2048, 128, dtype, W8.ASYM, p, seed=4000) for p in (W4.PATH_GEMV, W4.PATH_PREFILL)]
    assert torch.isfinite(ys[0].float()).all() and torch.isfinite(ys[1].float()).all()


@pytest.mark.parametrize("path", [W4.PATH_GEMV, W4.PATH_PREFILL])
@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_one_hot_bit_exact(path, dtype):
    # X = e_k: every output is s (u - z) for one weight, formed exactly and rounded once
    N, K, g = 96, 1024, 128
    W, (qw, s, z), (q_ref, s_ref, z_ref) = _quantize_both(N, K, g, W8.ASYM, seed=5000)
    M = 4
    X = np.zeros((M, K), dtype=np.float16 if dtype == FP16 else np.uint16)
    one = np.float16(1.0) if dtype == FP16 else np.uint16(0x3F80)
    for m, k in enumerate((0, 127, 128, 1023)):
        X[m, k] = one
    Y = W4.w8a16_linear(x_to_torch(X, dtype), qw, s, z, g, path=path)
    ref = W8.linear8_ref(X, dtype, q_ref, s_ref, z_ref, g)
    np.testing.assert_array_equal(y_bits(Y), ref_bits(ref, dtype))


def test_graph_replay_matches_eager():
    N, K, g = 2048, 4096, 128
    _, (qw, s, z), _ = _quantize_both(N, K, g, W8.ASYM, seed=6000)
    Xs = [x_to_torch(activations(M, K, FP16, seed=6001 + M), FP16) for M in (1, 300)]
    refs = [W4.w8a16_linear(X, qw, s, z, g) for X in Xs]
    outs = [torch.empty_like(r) for r in refs]
    st = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        for X, o in zip(Xs, outs):
            W4.w8a16_linear(X, qw, s, z, g, out=o)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph, stream=st):
            for X, o in zip(Xs, outs):
                W4.w8a16_linear(X, qw, s, z, g, out=o)
    for _ in range(3):
        for o in outs:
            o.fill_(float("nan"))
        W4.w8a16_linear(Xs[0], qw, s, z, g)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, refs):
            assert torch.equal(o.view(torch.int16), r.view(torch.int16))


@pytest.mark.parametrize("M,K,N", [(1, 4096, 11008), (1, 11008, 4096), (4, 11008, 4096), (4096, 4096, 11008)])
def test_full_size_sampled(M, K, N):
    # the whole layer on the GPU; the oracle checks sampled output rows (and, for the prefill,
    # sampled activation rows) from the sampled weight rows' own quantization
    g = 128
    rng = np.random.default_rng(7000 + M + K)
    W = weights(N, K, 0.02, seed=7001 + K + N)
    X = activations(M, K, FP16, seed=7002 + M + K)
    qw, s, z = W4.w8a16_quantize_pack(torch.from_numpy(W).cuda(), g, W8.ASYM)
    Y = W4.w8a16_linear(x_to_torch(X, FP16), qw, s, z, g)
    torch.cuda.synchronize()
    ns = np.unique(np.concatenate([[0, N - 1], rng.choice(N, 1024, replace=False)]))
    ms = np.arange(M) if M <= 64 else np.unique(np.concatenate([[0, M - 1], rng.choice(M, 64, replace=False)]))
    codes, s_ref, z_ref = W8.quantize8(W[ns], g, W8.ASYM)
    q_ref = W8.pack8(codes)
    idx = torch.from_numpy(ns).cuda()
    np.testing.assert_array_equal(qw[idx].cpu().numpy(), q_ref)
    ref = W8.linear8_ref(X[ms], FP16, q_ref, s_ref, z_ref, g)
    y = y_to_f64(Y[torch.from_numpy(ms).cuda()][:, idx])
    assert_close(y, ref_to_f64(ref, FP16), f"w8a16 full M={M} K={K} N={N}")
