"""GPU parity: every HIP kernel against the CPU oracle, through the C ABI.

* quantize-pack: bit-exact (qweight words, fp16 scale and zero bits);
* dequantize: exact;
* linear, every kernel path: relative Frobenius error <= 1e-3 and
  max |dY| <= 1e-2 * max |Y_ref| against the oracle rounded to the output dtype,
  plus bit-exact one-hot activations (which select single dequantized weights);
* full-size problems of every workload family at the launch configuration the
  benchmark times, on sampled output rows/columns the oracle computes one by one.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import w4a16_dequant_gemm_amd as W4
from synth import ASYM, BF16, FP16, SYM, Case, activations, config_cases, weights
from tests.gpu_util import (assert_close, packed_from_torch, ref_bits, ref_to_f64, upload_packed,
                            x_to_torch, y_bits, y_to_f64)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    W4.lib()


def _quant_gpu(W: np.ndarray, g: int, scheme: int, write_zeros: bool = True):
    Wt = torch.from_numpy(W).cuda()
    return W4.quantize_pack(Wt, g, scheme, write_zeros=write_zeros)


def _check_quant(W, g, scheme):
    qw, s, z = _quant_gpu(W, g, scheme)
    torch.cuda.synchronize()
    qn, sn, zn = packed_from_torch(qw, s, z)
    codes, s_ref, z_ref = oracle.quantize(W, g, scheme)
    np.testing.assert_array_equal(qn, oracle.pack(codes))
    np.testing.assert_array_equal(sn.view(np.uint16), s_ref.view(np.uint16))
    np.testing.assert_array_equal(zn.view(np.uint16), z_ref.view(np.uint16))
    return qn, sn, zn


QCASES = [(64, 256, 32), (37, 512, 64), (100, 1024, 128), (13, 384, 384), (8, 4096, 4096),
          (300, 11008, 128), (50, 2048, 2048), (3, 96, 96)]


@pytest.mark.parametrize("scheme", [ASYM, SYM])
@pytest.mark.parametrize("N,K,g", QCASES)
def test_quantize_pack_bit_exact(N, K, g, scheme):
    W = weights(N, K, 0.02, seed=N * 7 + K, outlier_frac=0.001, outlier_mult=20.0)
    _check_quant(W, g, scheme)


def test_quantize_pack_special_groups():
    # constant group, hand vectors (ties, non-straddling group, symmetric) tiled to g = 32,
    # a group with -0.0 and +0.0, and tiny (fp16-subnormal) scales
    rows = [
        np.full(32, 0.5, np.float32),
        np.tile(np.array([-0.75, 3.0, 0.1, 1.3, -0.2, 2.2, 0.0, 0.55], np.float32), 4),
        np.tile(np.array([0.0, 3.75, 0.625, 0.875, 0, 0, 0, 0], np.float32), 4),
        np.tile(np.array([1.0, 4.75, 2.0, 3.125, 1.5, 2.625, 4.0, 1.875], np.float32), 4),
        np.tile(np.array([-0.0, 0.0, -0.0, 1.0, 0.0, -0.0, 0.25, 0.0], np.float32), 4),
        np.linspace(-1e-6, 2e-6, 32, dtype=np.float32),
        np.linspace(-3.0, -2.0, 32, dtype=np.float32),
        np.zeros(32, np.float32),
    ]
    W = np.stack(rows).astype(np.float32)
    for scheme in (ASYM, SYM):
        _check_quant(W, 32, scheme)


def test_quantize_sym_without_zeros():
    W = weights(16, 512, 0.02, seed=5)
    qw, s, z = _quant_gpu(W, 128, SYM, write_zeros=False)
    assert z is None
    codes, s_ref, _ = oracle.quantize_sym(W, 128)
    np.testing.assert_array_equal(qw.cpu().numpy(), oracle.pack(codes))
    np.testing.assert_array_equal(s.cpu().numpy().view(np.uint16), s_ref.view(np.uint16))


@pytest.mark.parametrize("N,K,g", [(64, 256, 32), (100, 1024, 128), (13, 384, 384)])
def test_dequantize_exact(N, K, g):
    W = weights(N, K, 0.02, seed=11)
    qw, s, z = _quant_gpu(W, g, ASYM)
    D = W4.dequantize(qw, s, z, g).cpu().numpy().astype(np.float64)
    qn, sn, zn = packed_from_torch(qw, s, z)
    np.testing.assert_array_equal(D, oracle.dequantize(qn, sn, zn, g))
    D8 = W4.dequantize(qw, s, None, g).cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(D8, oracle.dequantize(qn, sn, None, g))


# ------------------------------------------------------------------ linear
def _run_linear(M, N, K, g, scheme, dtype, path, seed, zeros_none=False, x_outliers=False):
    W = weights(N, K, 0.02, seed=seed)
    X = activations(M, K, dtype, seed + 1, *(0.01, 100.0) if x_outliers else (0.0, 1.0))
    codes, s, z = oracle.quantize(W, g, scheme)
    qw_np = oracle.pack(codes)
    zz = None if zeros_none else z
    qw, st, zt = upload_packed(qw_np, s, zz)
    Y = W4.linear(x_to_torch(X, dtype), qw, st, zt, g, path=path)
    torch.cuda.synchronize()
    ref = oracle.linear_ref(X, dtype, qw_np, s, zz, g)
    return Y, ref


GEMV_CASES = [(1, 64, 256, 32), (2, 130, 512, 128), (3, 77, 1024, 1024), (4, 256, 4096, 128),
              (1, 300, 11008, 128), (5, 100, 2048, 64), (8, 64, 4096, 128), (1, 33, 28672, 128),
              (2, 50, 11008, 11008), (7, 16, 1024, 256), (1, 1, 32, 32),
              (1, 9477, 4096, 128), (2, 5000, 2048, 64), (4, 3000, 1024, 1024), (3, 2600, 6144, 128),
              # grid-sizing boundaries of the streaming kernel: one row per wave up to N = 4096,
              # two rows up to N = 12288 (768 blocks), one persistent block per CU beyond
              (1, 4097, 1024, 128), (2, 12288, 256, 64), (1, 12289, 512, 128), (1, 4096, 12288, 128),
              # one-row layers with >= 4 chunks per lane: one row per wave at any N, rows up to
              # K = 28672 (more than 64 KB of LDS), and past the LDS budget (g = 32 at K = 28672)
              (1, 12400, 8192, 128), (1, 70, 28672, 28672), (1, 500, 16384, 64), (1, 9, 14336, 128),
              (1, 40, 28672, 32)]
SKINNY_CASES = [(1, 64, 128, 128), (5, 100, 1024, 128), (16, 256, 4096, 128), (17, 77, 2048, 256),
                (32, 300, 11008, 128), (31, 129, 1024, 1024), (8, 4096, 4096, 128), (2, 50, 11008, 11008),
                (12, 1000, 28672, 128),
                # M <= 4: the k-split decode kernel (1..4 tiles per block, short and long K)
                (1, 4096, 4096, 128), (2, 11008, 4096, 128), (3, 4096, 11008, 128),
                (4, 1000, 2048, 256), (1, 16000, 1024, 128), (1, 300, 28672, 128),
                (4, 700, 8192, 8192), (1, 50, 11008, 11008), (3, 17, 128, 128), (2, 5000, 1408, 128),
                # 5 <= M <= 16: activations streamed next to the weights (1..4 tiles per block)
                (5, 4100, 2048, 128), (16, 12300, 512, 128), (9, 8200, 1024, 256), (13, 33, 11008, 128),
                (16, 4096, 11008, 128), (7, 3000, 8192, 8192), (11, 1, 256, 128), (16, 17, 4352, 128),
                (4, 4096, 11008, 128), (3, 300, 28672, 128),
                # the LDS-ring kernel with 5, 7 and 8 tiles per block (ragged last blocks), short K
                (6, 20000, 512, 128), (9, 24600, 256, 256), (16, 40000, 256, 128), (5, 28672, 1024, 1024),
                # 32 < M <= 512: the grid also runs over 32-row chunks of M (ragged last chunk,
                # 64 weight rows per block in fp16), K split over the waves
                (33, 300, 1024, 128), (100, 257, 2048, 128), (256, 1000, 4096, 256), (512, 64, 1024, 1024),
                (130, 4096, 11008, 128),
                # more groups per row than the skinny kernel stages in LDS (> 96): loaded per k-block
                (24, 300, 16384, 128), (40, 130, 14336, 128)]
PREFILL_CASES = [(1, 64, 64, 64), (17, 200, 192, 64), (130, 129, 256, 128), (256, 384, 1024, 128),
                 (300, 256, 4096, 4096), (64, 128, 11008, 128), (129, 1, 128, 64),
                 # fp16: 128-row tiles with K split over two wave groups (K % 256 == 0), ragged M and
                 # N; then K % 256 != 0, which keeps one group
                 (1100, 4000, 768, 128), (1100, 4096, 640, 64),
                 # 64-row tiles, three-stage loop: 3 and 4 steps per wave group
                 (70, 520, 384, 128), (70, 520, 512, 64),
                 # more groups per row than one LDS staging holds (fp16: staged in phases of up to
                 # 95 groups): 172 groups, 64-row tiles with two wave groups; 128 groups, 128-row
                 # tiles with two wave groups; 130 groups, 64-row tiles three steps deep; g = 128
                 # (112 groups)
                 (64, 130, 11008, 64), (1100, 4000, 8192, 64), (200, 300, 8320, 64), (300, 260, 14336, 128)]
# fp16 prefill also takes K % 64 == 32 and g == 32 (bf16 prefill needs multiples of 64); the last
# case has 128 groups of 32 per row (staged in two phases)
PREFILL_F16_CASES = [(40, 150, 96, 32), (257, 300, 160, 32), (70, 64, 96, 96), (513, 260, 2080, 32),
                     (100, 260, 4096, 32)]


@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("M,N,K,g", GEMV_CASES)
def test_linear_gemv(M, N, K, g, dtype):
    Y, ref = _run_linear(M, N, K, g, ASYM, dtype, W4.PATH_GEMV, seed=M * 131 + N + K)
    assert_close(y_to_f64(Y), ref_to_f64(ref, dtype), f"gemv M={M} N={N} K={K} g={g}")


@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("M,N,K,g", SKINNY_CASES)
def test_linear_skinny(M, N, K, g, dtype):
    Y, ref = _run_linear(M, N, K, g, ASYM, dtype, W4.PATH_SKINNY, seed=M * 71 + N + K)
    assert_close(y_to_f64(Y), ref_to_f64(ref, dtype), f"skinny M={M} N={N} K={K} g={g}")


@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("M,N,K,g", PREFILL_CASES)
def test_linear_prefill(M, N, K, g, dtype):
    Y, ref = _run_linear(M, N, K, g, ASYM, dtype, W4.PATH_PREFILL, seed=M * 17 + N + K)
    assert_close(y_to_f64(Y), ref_to_f64(ref, dtype), f"prefill M={M} N={N} K={K} g={g}")


@pytest.mark.parametrize("M,N,K,g", PREFILL_F16_CASES)
def test_linear_prefill_f16_k32(M, N, K, g):
    Y, ref = _run_linear(M, N, K, g, ASYM, FP16, W4.PATH_PREFILL, seed=M * 19 + N + K)
    assert_close(y_to_f64(Y), ref_to_f64(ref, FP16), f"prefill f16 M={M} N={N} K={K} g={g}")


ALL_PATHS = [W4.PATH_GEMV, W4.PATH_SKINNY, W4.PATH_PREFILL]


@pytest.mark.parametrize("path", ALL_PATHS)
@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("offset", [1, 3])
def test_linear_unaligned_metadata(path, dtype, offset):
    # scales / zeros need only 2-byte alignment: pass views that start `offset` halves into
    # larger buffers (the kernels stage them with 16-byte loads from arbitrary offsets)
    N, K, g = 301, 1024, 128
    G = K // g
    W = weights(N, K, 0.02, seed=61)
    M = {W4.PATH_GEMV: 2, W4.PATH_SKINNY: 3, W4.PATH_PREFILL: 70}[path]
    X = activations(M, K, dtype, 62)

    def view_at_offset(a: np.ndarray) -> torch.Tensor:
        buf = torch.zeros(N * G + 2 * offset, dtype=torch.float16, device="cuda")
        buf[offset:offset + N * G] = torch.from_numpy(a.astype(np.float16).reshape(-1)).cuda()
        v = buf[offset:offset + N * G].view(N, G)
        assert v.data_ptr() % 16 != 0
        return v

    for scheme in (ASYM, SYM):
        codes, s, z = oracle.quantize(W, g, scheme)
        qw_np = oracle.pack(codes)
        zz = z if scheme == ASYM else None           # symmetric: NULL zeros (all 8)
        Y = W4.linear(x_to_torch(X, dtype), torch.from_numpy(qw_np).cuda(), view_at_offset(s),
                      view_at_offset(zz) if zz is not None else None, g, path=path)
        ref = oracle.linear_ref(X, dtype, qw_np, s, zz, g)
        assert_close(y_to_f64(Y), ref_to_f64(ref, dtype), f"unaligned metadata path={path} scheme={scheme}")


@pytest.mark.parametrize("path", ALL_PATHS)
@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_linear_offset_groups(path, dtype):
    # groups that do not straddle zero: asymmetric zero points far outside 0..15
    N, K, g = 192, 1024, 128
    W = weights(N, K, 0.01, seed=51)
    W[: N // 2] += 0.5
    W[N // 2:] -= 0.5
    codes, s, z = oracle.quantize_asym(W, g)
    assert z.min() < -60 and z.max() > 60 and np.abs(z).max() <= 480
    qw_np = oracle.pack(codes)
    qw, st, zt = upload_packed(qw_np, s, z)
    M = 4 if path == W4.PATH_GEMV else 24
    X = activations(M, K, dtype, 52)
    Y = W4.linear(x_to_torch(X, dtype), qw, st, zt, g, path=path)
    ref = oracle.linear_ref(X, dtype, qw_np, s, z, g)
    assert_close(y_to_f64(Y), ref_to_f64(ref, dtype), f"offset groups path={path}")


@pytest.mark.parametrize("path", ALL_PATHS)
@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_linear_symmetric_and_null_zeros(path, dtype):
    for M in (4, 9):
        if path == W4.PATH_GEMV and M > 8:
            continue
        for zeros_none in (False, True):
            Y, ref = _run_linear(M, 192, 1024, 128, SYM, dtype, path, seed=3, zeros_none=zeros_none)
            assert_close(y_to_f64(Y), ref_to_f64(ref, dtype),
                         f"sym M={M} path={path} zeros_none={zeros_none}")


@pytest.mark.parametrize("path", ALL_PATHS)
def test_linear_bf16_outlier_channels(path):
    for M, K in ((4, 8192), (4, 4096), (16, 8192)):
        if path == W4.PATH_GEMV and M > 8:
            continue
        Y, ref = _run_linear(M, 256, K, 128, ASYM, BF16, path, seed=9, x_outliers=True)
        assert_close(y_to_f64(Y), ref_to_f64(ref, BF16), f"bf16 outliers M={M} path={path} K={K}")


@pytest.mark.parametrize("path", ALL_PATHS)
@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_one_hot_bit_exact(path, dtype):
    # one-hot rows select single dequantized weights: Y[m, n] = round(W_hat[n, k_m]) exactly
    N, K, g = 200, 1024, 128
    W = weights(N, K, 0.05, seed=21)
    codes, s, z = oracle.quantize_asym(W, g)
    qw_np = oracle.pack(codes)
    ks = [0, 1, 4, 7, 8, 31, 32, 63, 64, 127, 128, 500, 777, 1023]
    X64 = np.zeros((len(ks), K))
    for m, k in enumerate(ks):
        X64[m, k] = 1.0
    X = X64.astype(np.float16) if dtype == FP16 else oracle.round_to_bf16_bits(X64)
    qw, st, zt = upload_packed(qw_np, s, z)
    ref = oracle.linear_ref(X, dtype, qw_np, s, z, g)
    # GEMV serves M <= 8; the MFMA decode kernels take M <= 16 (K % 256 == 0)
    sizes = {W4.PATH_GEMV: [4], W4.PATH_SKINNY: [4, 7, len(ks)]}.get(path, [len(ks)])
    for rows in sizes:
        for m0 in range(0, len(ks), rows):
            Y = W4.linear(x_to_torch(X[m0:m0 + rows], dtype), qw, st, zt, g, path=path)
            np.testing.assert_array_equal(y_bits(Y), ref_bits(ref[m0:m0 + rows], dtype))


def test_auto_dispatch_matches_forced_paths():
    for M in (1, 4, 16, 64, 300):
        Y, ref = _run_linear(M, 256, 2048, 128, ASYM, FP16, W4.PATH_AUTO, seed=M)
        assert_close(y_to_f64(Y), ref_to_f64(ref, FP16), f"auto M={M}")


def test_non_default_stream_no_intermediate_sync():
    W = weights(512, 4096, 0.02, seed=31)
    X = activations(2, 4096, FP16, 32)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        Wt = torch.from_numpy(W).to("cuda", non_blocking=False)
        Xt = x_to_torch(X, FP16)
        qw, sc, z = W4.quantize_pack(Wt, 128, ASYM)
        Y = W4.linear(Xt, qw, sc, z, 128)
    s.synchronize()
    codes, s_ref, z_ref = oracle.quantize_asym(W, 128)
    ref = oracle.linear_ref(X, FP16, oracle.pack(codes), s_ref, z_ref, 128)
    assert_close(y_to_f64(Y), ref_to_f64(ref, FP16), "stream")


def test_repeat_determinism():
    W = weights(256, 4096, 0.02, seed=41)
    X = activations(4, 4096, BF16, 42)
    Wt = torch.from_numpy(W).cuda()
    outs = []
    for _ in range(3):
        qw, sc, z = W4.quantize_pack(Wt, 128, ASYM)
        outs.append((qw.clone(), sc.clone(), z.clone(), W4.linear(x_to_torch(X, BF16), qw, sc, z, 128)))
    for o in outs[1:]:
        for a, b in zip(o, outs[0]):
            assert torch.equal(a.view(torch.int16) if a.dtype != torch.int32 else a,
                               b.view(torch.int16) if b.dtype != torch.int32 else b)


# ------------------------------------------------------- full-size workloads
def _full_size(case: Case, n_rows: int = 1024, m_rows: int | None = None):
    """Full-size problem: GPU quantizes and multiplies the whole layer; the oracle checks
    ``n_rows`` sampled output rows n (bit-exact packing and Y columns) and, for large M,
    sampled activation rows m."""
    W, X = case.make()
    Wt = torch.from_numpy(W).cuda()
    qw, sc, z = W4.quantize_pack(Wt, case.g, case.scheme)
    del Wt
    Y = W4.linear(x_to_torch(X, case.dtype), qw, sc, z, case.g)
    torch.cuda.synchronize()
    rng = np.random.default_rng(case.config * 1000 + case.M)
    ns = np.unique(np.concatenate([[0, case.N - 1], rng.choice(case.N, min(n_rows, case.N), replace=False)]))
    ms = np.arange(case.M) if m_rows is None or case.M <= m_rows else \
        np.unique(np.concatenate([[0, case.M - 1], rng.choice(case.M, m_rows, replace=False)]))
    codes, s_ref, z_ref = oracle.quantize(W[ns], case.g, case.scheme)
    qn = qw[torch.from_numpy(ns).cuda()].cpu().numpy()
    np.testing.assert_array_equal(qn, oracle.pack(codes))
    np.testing.assert_array_equal(sc[torch.from_numpy(ns).cuda()].cpu().numpy().view(np.uint16),
                                  s_ref.view(np.uint16))
    ref = oracle.linear_ref(X[ms], case.dtype, qn, s_ref, z_ref, case.g)
    y = y_to_f64(Y[torch.from_numpy(ms).cuda()][:, torch.from_numpy(ns).cuda()])
    assert_close(y, ref_to_f64(ref, case.dtype), case.name)


# every case of the single-layer workloads: the 7B-like decode sweep (M = 1..16), the
# 70B-like decode shapes with outlier channels and weights (bf16), and the prefill grid
# (M = 256 / 1024 / 4096, g = 64 / 128, symmetric and asymmetric), each checked before the
# benchmark times it, on 1024 output columns (all activation rows up to M = 64, else 64)
FULL = [c for cfg in (1, 2, 3, 4) for c in config_cases(cfg)]


@pytest.mark.parametrize("case", FULL, ids=lambda c: c.name)
def test_full_size_sampled(case):
    _full_size(case, m_rows=64)


# ------------------------------------------------------- beyond 32-bit offsets
@pytest.mark.parametrize("M", [1, 8, 300])
def test_packed_weights_over_2gib(M):
    """Packed weights of 2.15 GB (past every 32-bit byte offset): the dispatcher must route to
    kernels with 64-bit addressing.  Random packed words, scales and zero points (no fp32
    weight matrix of 17 GB is needed); sampled output columns against the oracle."""
    N, K, g = 65600, 65536, 128
    G = K // g
    gen = torch.Generator(device="cuda")
    gen.manual_seed(77 + M)
    qw = torch.randint(-2 ** 31, 2 ** 31, (N, K // 8), dtype=torch.int32, device="cuda", generator=gen)
    sc = (torch.rand((N, G), device="cuda", generator=gen) * 0.02 + 0.001).half()
    z = torch.randint(0, 16, (N, G), device="cuda", generator=gen).half()
    X = activations(M, K, FP16, seed=M + 5)
    Y = W4.linear(x_to_torch(X, FP16), qw, sc, z, g)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M)
    ns = np.unique(np.concatenate([[0, N - 1, N // 2], rng.choice(N, 21, replace=False)]))
    idx = torch.from_numpy(ns).cuda()
    ref = oracle.linear_ref(X, FP16, qw[idx].cpu().numpy(), sc[idx].cpu().numpy(), z[idx].cpu().numpy(), g)
    assert_close(y_to_f64(Y[:, idx]), ref_to_f64(ref, FP16), f"2 GiB+ weights M={M}")
    del qw, sc, z, Y
    torch.cuda.empty_cache()
