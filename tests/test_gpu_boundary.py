"""GPU tests of the C-ABI boundary itself.

* ``w4a16_linear`` and ``w4a16_w8a16_linear`` (the plain entry points, automatic dispatch)
  called directly through ctypes with raw device pointers, against the oracle;
* the whole zero-point range the quantizers emit, ``|z| <= 2048``, on every kernel path of
  both code widths: random codes with zero points spread over the range (including the
  points where ``u - z`` leaves the fp16 integers), against the oracle's exact ``s (u - z)``;
  one-hot activations bit-exact everywhere;
* the quantizers on groups far from 0 (large ``|z|``), bit-exact;
* the binding's argument checks on the workspace form and the output tensor.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import w4a16_dequant_gemm_amd as W4
from oracle import w8a16 as W8
from synth import ASYM, BF16, FP16, activations, weights
from tests.gpu_util import assert_close, ref_bits, ref_to_f64, upload_packed, x_to_torch, y_bits, y_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    W4.lib()


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


# ------------------------------------------------- the plain entry points, through ctypes
@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("M,N,K", [(1, 4096, 4096), (16, 1000, 11008), (4096, 512, 4096)])
def test_plain_linear_through_c_abi(M, N, K, dtype):
    g = 128
    W = weights(N, K, 0.02, seed=M + N + K)
    X = activations(M, K, dtype, seed=M + 7)
    codes, s, z = oracle.quantize_asym(W, g)
    qw_np = oracle.pack(codes)
    qw, st, zt = upload_packed(qw_np, s, z)
    Xt = x_to_torch(X, dtype)
    Y = torch.empty((M, N), dtype=Xt.dtype, device="cuda")
    rc = W4.lib().w4a16_linear(Xt.data_ptr(), dtype, M, N, K, g, qw.data_ptr(), st.data_ptr(),
                               zt.data_ptr(), Y.data_ptr(), _stream())
    assert rc == 0, W4.lib().w4a16_strerror(rc)
    torch.cuda.synchronize()
    rows = np.arange(M) if M <= 64 else np.unique(np.r_[0, M - 1, np.random.default_rng(M).choice(M, 64, False)])
    ref = oracle.linear_ref(X[rows], dtype, qw_np, s, z, g)
    assert_close(y_to_f64(Y[torch.from_numpy(rows).cuda()]), ref_to_f64(ref, dtype), f"w4a16_linear M={M}")


@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("M", [1, 16, 300])
def test_plain_w8a16_linear_through_c_abi(M, dtype):
    N, K, g = 700, 4096, 128
    W = weights(N, K, 0.02, seed=M + 3)
    X = activations(M, K, dtype, seed=M + 4)
    codes, s, z = W8.quantize8(W, g, W8.ASYM)
    qw_np = W8.pack8(codes)
    qw, st, zt = upload_packed(qw_np, s, z)
    Xt = x_to_torch(X, dtype)
    Y = torch.empty((M, N), dtype=Xt.dtype, device="cuda")
    rc = W4.lib().w4a16_w8a16_linear(Xt.data_ptr(), dtype, M, N, K, g, qw.data_ptr(), st.data_ptr(),
                                     zt.data_ptr(), Y.data_ptr(), _stream())
    assert rc == 0, W4.lib().w4a16_strerror(rc)
    torch.cuda.synchronize()
    ref = W8.linear8_ref(X, dtype, qw_np, s, z, g)
    assert_close(y_to_f64(Y), ref_to_f64(ref, dtype), f"w4a16_w8a16_linear M={M}")


# ------------------------------------------------------- the whole zero-point range
# zero points over [-2048, 2048]: both ends, +-480 and 512 (the edges of the exact range of an
# integer-add construction of 1536 + u - z on fp16 bits), multiples of 512 and their
# neighbours, and -2033 / -1793, below which u - z itself leaves the fp16 integers
Z_VALUES = [-2048, -2040, -2033, -2000, -1800, -1793, -1537, -1536, -1024, -777, -600, -513, -481,
            -480, -300, -8, 0, 7, 15, 100, 255, 300, 480, 481, 512, 513, 600, 765, 1023, 1024, 1280,
            1536, 1537, 2000, 2047, 2048]


def _wide_z_layer(N: int, K: int, g: int, bits: int, seed: int, zmin: int = -2048):
    """Random codes, fp16 scales in [1e-3, 2e-2] and zero points cycling through Z_VALUES
    (at least ``zmin``) per (row, group)."""
    rng = np.random.default_rng(seed)
    G = K // g
    umax = 15 if bits == 4 else 255
    codes = rng.integers(0, umax + 1, size=(N, K), dtype=np.int64)
    zs = np.array([v for v in Z_VALUES if v >= zmin], dtype=np.float64)
    z = zs[(np.arange(N * G) * 7 + seed) % len(zs)].reshape(N, G).astype(np.float16)
    s = (rng.random((N, G)) * 0.019 + 0.001).astype(np.float16)
    qw = oracle.pack(codes) if bits == 4 else W8.pack8(codes)
    return qw, s, z


def _linear_bits(bits: int, Xt, qw, st, zt, g: int, path: int):
    if bits == 4:
        return W4.linear(Xt, qw, st, zt, g, path=path)
    return W4.w8a16_linear(Xt, qw, st, zt, g, path=path)


def _ref_bits(bits: int, X, dtype: int, qw, s, z, g: int):
    if bits == 4:
        return oracle.linear_ref(X, dtype, qw, s, z, g)
    return W8.linear8_ref(X, dtype, qw, s, z, g)


# (bits, path, M, K, g): every kernel of both code widths -- the GEMV (M = 1, 3), the MFMA
# decode kernels (M = 4 staged, M = 12 streamed), the skinny kernel (M = 40), the fp16
# 256 x 256 GEMM (K % 128 == 0), the fp16 256 x 128 GEMM (K % 128 == 64) and the bf16
# 128 x 128 GEMM (both dtypes run every case)
WIDE_Z_CASES = [
    (4, W4.PATH_GEMV, 1, 1024, 64), (4, W4.PATH_GEMV, 3, 1024, 128), (4, W4.PATH_SKINNY, 4, 1024, 128),
    (4, W4.PATH_SKINNY, 12, 1024, 128), (4, W4.PATH_SKINNY, 40, 1024, 128), (4, W4.PATH_PREFILL, 300, 1024, 64),
    (4, W4.PATH_PREFILL, 70, 960, 64),
    (8, W4.PATH_GEMV, 1, 1024, 64), (8, W4.PATH_GEMV, 6, 1024, 128), (8, W4.PATH_PREFILL, 300, 1024, 64),
    (8, W4.PATH_PREFILL, 70, 960, 64),
]


@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("bits,path,M,K,g", WIDE_Z_CASES)
def test_linear_whole_zero_point_range(bits, path, M, K, g, dtype):
    N = 301
    qw_np, s, z = _wide_z_layer(N, K, g, bits, seed=M + K + bits)
    assert z.min() == -2048 and z.max() == 2048
    qw, st, zt = upload_packed(qw_np, s, z)
    X = activations(M, K, dtype, seed=M + 11)
    Y = _linear_bits(bits, x_to_torch(X, dtype), qw, st, zt, g, path)
    torch.cuda.synchronize()
    ref = _ref_bits(bits, X, dtype, qw_np, s, z, g)
    assert_close(y_to_f64(Y), ref_to_f64(ref, dtype), f"wide z bits={bits} path={path} M={M} K={K}")


@pytest.mark.parametrize("dtype", [FP16, BF16])
@pytest.mark.parametrize("bits,path,M,K,g", [c for c in WIDE_Z_CASES if c[1] != W4.PATH_GEMV or c[2] == 1])
def test_one_hot_whole_zero_point_range(bits, path, M, K, g, dtype):
    # one-hot rows select single weights s (u - z): every kernel rounds that product once
    # (the fp16 GEMMs from an exact fp32 s (u - z)), bit-exact against the oracle over the
    # whole zero-point range
    N = 150
    qw_np, s, z = _wide_z_layer(N, K, g, bits, seed=K + bits)
    qw, st, zt = upload_packed(qw_np, s, z)
    ks = np.unique(np.r_[0, 1, 5, 63, 64, 100, 127, 128, 129, 511, 512, K - 65, K - 1,
                         np.random.default_rng(5).choice(K, max(M, 16) - 13, replace=False)])[:max(M, 1)]
    rows = len(ks)
    X64 = np.zeros((rows, K))
    X64[np.arange(rows), ks] = 1.0
    X = X64.astype(np.float16) if dtype == FP16 else oracle.round_to_bf16_bits(X64)
    Y = _linear_bits(bits, x_to_torch(X, dtype), qw, st, zt, g, path)
    torch.cuda.synchronize()
    ref = _ref_bits(bits, X, dtype, qw_np, s, z, g)
    np.testing.assert_array_equal(y_bits(Y), ref_bits(ref, dtype))


def _far_groups(N: int, K: int, g: int, levels: int, seed: int) -> np.ndarray:
    """Groups of width ~0.05 at distance c from 0, c chosen so that the zero point
    -min / s ~ levels * c / width spreads over about [-1900, 1900] (the realised range of a
    group is up to ~15 % narrower than the width, which widens |z| accordingly)."""
    rng = np.random.default_rng(seed)
    W = np.empty((N, K), np.float32)
    width = 0.05
    for n in range(N):
        for j in range(K // g):
            c = -rng.uniform(-1650.0, 1650.0) * width / levels
            W[n, j * g:(j + 1) * g] = (c + width * rng.random(g)).astype(np.float32)
    return W


def test_quantizers_far_from_zero():
    N, K, g = 64, 512, 64
    W = _far_groups(N, K, g, 15, seed=99)
    codes, s, z = oracle.quantize_asym(W, g)
    assert np.abs(z.astype(np.float64)).max() > 1500
    qw, st, zt = W4.quantize_pack(torch.from_numpy(W).cuda(), g, ASYM)
    np.testing.assert_array_equal(qw.cpu().numpy(), oracle.pack(codes))
    np.testing.assert_array_equal(st.cpu().numpy().view(np.uint16), s.view(np.uint16))
    np.testing.assert_array_equal(zt.cpu().numpy().view(np.uint16), z.view(np.uint16))
    W8w = _far_groups(N, K, g, 255, seed=98)
    codes8, s8, z8 = W8.quantize8(W8w, g, W8.ASYM)
    assert np.abs(z8.astype(np.float64)).max() > 1500
    q8, s8t, z8t = W4.w8a16_quantize_pack(torch.from_numpy(W8w).cuda(), g, W8.ASYM)
    np.testing.assert_array_equal(q8.cpu().numpy(), W8.pack8(codes8))
    np.testing.assert_array_equal(s8t.cpu().numpy().view(np.uint16), s8.view(np.uint16))
    np.testing.assert_array_equal(z8t.cpu().numpy().view(np.uint16), z8.view(np.uint16))


# ------------------------------------------------------------ binding argument checks
def test_binding_rejects_bad_arguments():
    M, N, K, g = 64, 256, 1024, 128
    X = torch.zeros((M, K), dtype=torch.float16, device="cuda")
    qw = torch.zeros((N, K // 8), dtype=torch.int32, device="cuda")
    s = torch.ones((N, K // g), dtype=torch.float16, device="cuda")
    z = torch.zeros((N, K // g), dtype=torch.float16, device="cuda")
    bad = [
        dict(zeros=z[:, :4].contiguous()),                                        # zeros shape
        dict(zeros=z.cpu()),                                                      # zeros on the host
        dict(zeros=z.float()),                                                    # zeros dtype
        dict(zeros=torch.zeros((K // g, N), dtype=torch.float16, device="cuda").t()),   # not contiguous
        dict(out=torch.empty((M, N + 1), dtype=torch.float16, device="cuda")),    # out shape
        dict(out=torch.empty((M, N), dtype=torch.bfloat16, device="cuda")),       # out dtype
        dict(out=torch.empty((M, N), dtype=torch.float16)),                       # out on the host
        dict(out=torch.empty((N, M), dtype=torch.float16, device="cuda").t()),    # out not contiguous
        dict(group_size=0),
        dict(group_size=100),
    ]
    for kw in bad:
        args = dict(zeros=z, out=None, group_size=g)
        args.update(kw)
        for fn in (W4.linear, W4.linear_ws):
            with pytest.raises((TypeError, ValueError)):
                fn(X, qw, s, args["zeros"], args["group_size"], out=args["out"])
    work_bad = [torch.zeros(16, dtype=torch.float32), torch.zeros(16, dtype=torch.float64, device="cuda"),
                torch.zeros((8, 8), dtype=torch.float32, device="cuda").t()]
    for w in work_bad:
        with pytest.raises((TypeError, ValueError)):
            W4.linear_ws(X, qw, s, z, g, work=w)
    torch.cuda.synchronize()
