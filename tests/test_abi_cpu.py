"""Host-only checks of the C ABI (no GPU): the library loads, exports every function
declared in include/w4a16.h, and rejects invalid arguments with the documented status
before anything is enqueued (fake device pointers are never dereferenced)."""

import os
import re

import pytest

from w4a16_dequant_gemm_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")

A = 0x10000       # aligned fake pointers (never dereferenced on these paths)
B = 0x20000
C = 0x30000
D = 0x40000
MIS = 0x10002     # misaligned for 16-byte requirements


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:int|int64_t|const char\*)\s+(w4a16_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from w4a16_dequant_gemm_amd.build import build
        build()
    return L.lib()


def test_header_declares_the_boundary():
    names = _declared()
    for required in ("w4a16_quantize_pack", "w4a16_linear", "w4a16_linear_ex",
                     "w4a16_select_path", "w4a16_dequantize", "w4a16_strerror",
                     "w4a16_abi_version", "w4a16_gptq_hessian", "w4a16_gptq_factor",
                     "w4a16_gptq_quantize", "w4a16_awq_workspace", "w4a16_awq_stats",
                     "w4a16_awq_search", "w4a16_awq_scale", "w4a16_w8a8_smooth",
                     "w4a16_w8a8_quantize_weight", "w4a16_w8a8_quantize_act", "w4a16_w8a8_linear",
                     "w4a16_kv_quantize", "w4a16_kv_attention_workspace",
                     "w4a16_kv_attention_decode", "w4a16_kv_attention_batch_workspace",
                     "w4a16_kv_attention_decode_batch", "w4a16_w8a16_quantize_pack",
                     "w4a16_w8a16_linear", "w4a16_w8a16_linear_ex", "w4a16_w8a16_select_path"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    for name in _declared():
        assert hasattr(lib, name), name


def test_abi_version_and_strerror(lib):
    assert lib.w4a16_abi_version() == 1
    for st in range(-9, 1):
        assert lib.w4a16_strerror(st)
    assert lib.w4a16_strerror(-99) == b"unknown status"


def _lin(lib, X=A, dtype=0, M=1, N=64, K=128, g=128, qw=B, s=C, z=D, Y=A + 4096, path=1):
    return lib.w4a16_linear_ex(X, dtype, M, N, K, g, qw, s, z, Y, path, None)


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), L.ERR_NULL),
    (dict(qw=None), L.ERR_NULL),
    (dict(s=None), L.ERR_NULL),
    (dict(Y=None), L.ERR_NULL),
    (dict(dtype=2), L.ERR_DTYPE),
    (dict(M=0), L.ERR_SHAPE),
    (dict(N=0), L.ERR_SHAPE),
    (dict(K=0), L.ERR_SHAPE),
    (dict(K=48, g=48), L.ERR_SHAPE),           # K % 32 != 0
    (dict(K=192, g=48), L.ERR_GROUP),          # not a power of two, not K
    (dict(K=128, g=16), L.ERR_GROUP),          # below 32
    (dict(K=128, g=256), L.ERR_GROUP),         # larger than K
    (dict(K=384, g=256), L.ERR_GROUP),         # does not divide K
    (dict(X=MIS), L.ERR_ALIGN),
    (dict(qw=B + 8), L.ERR_ALIGN),
    (dict(s=C + 1), L.ERR_ALIGN),
    (dict(z=D + 1), L.ERR_ALIGN),
    (dict(Y=A + 4097), L.ERR_ALIGN),
    (dict(K=96, g=96, dtype=L.BF16, path=L.PATH_PREFILL), L.ERR_PATH),   # bf16: K % 64 != 0
    (dict(M=9, path=L.PATH_GEMV), L.ERR_PATH),             # GEMV handles M <= 8
    (dict(path=17), L.ERR_PATH),
])
def test_linear_rejects_invalid_arguments(lib, kw, status):
    assert _lin(lib, **kw) == status


@pytest.mark.parametrize("args,status", [
    ((None, 64, 128, 128, 0, B, C, D), L.ERR_NULL),
    ((A, 64, 128, 128, 5, B, C, D), L.ERR_SCHEME),
    ((A, 64, 128, 128, 0, B, C, None), L.ERR_NULL),      # asymmetric needs zeros
    ((A, 64, 100, 100, 0, B, C, D), L.ERR_SHAPE),
    ((A, 64, 128, 64 + 32, 0, B, C, D), L.ERR_GROUP),
    ((MIS, 64, 128, 128, 0, B, C, D), L.ERR_ALIGN),
    ((A, 64, 128, 128, 1, B + 4, C, None), L.ERR_ALIGN),
])
def test_quantize_pack_rejects_invalid_arguments(lib, args, status):
    assert lib.w4a16_quantize_pack(*args, None) == status


def test_dequantize_rejects_invalid_arguments(lib):
    assert lib.w4a16_dequantize(None, C, D, 4, 128, 128, A, None) == L.ERR_NULL
    assert lib.w4a16_dequantize(B, C, D, 4, 120, 120, A, None) == L.ERR_SHAPE
    assert lib.w4a16_dequantize(B, C, D, 4, 128, 128, A + 8, None) == L.ERR_ALIGN


@pytest.mark.parametrize("M,N,K,g,dtype,path", [
    (1, 4096, 4096, 128, 0, L.PATH_GEMV),
    (2, 11008, 4096, 128, 0, L.PATH_GEMV),
    (2, 4096, 11008, 128, 0, L.PATH_SKINNY),          # two rows, long K: MFMA decode
    (4, 11008, 4096, 128, 1, L.PATH_SKINNY),          # MFMA decode kernel
    (4, 4096, 11008, 128, 0, L.PATH_SKINNY),          # long K: activations streamed
    (3, 4096, 4096, 64, 0, L.PATH_GEMV),              # g = 64: the MFMA kernels need g % 128 == 0
    (16, 4096, 4096, 128, 0, L.PATH_SKINNY),
    (8, 4096, 11008, 128, 1, L.PATH_SKINNY),          # MFMA decode kernel, 5 <= M <= 16
    (17, 4096, 4096, 128, 0, L.PATH_SKINNY),
    (1, 8192, 28672, 128, 1, L.PATH_SKINNY),         # one row of K > 24576: the MFMA decode kernel
    (1, 8192, 24576, 128, 1, L.PATH_GEMV),
    (1, 28672, 8192, 128, 0, L.PATH_GEMV),
    (1, 8192, 28672, 64, 0, L.PATH_GEMV),             # g = 64: the MFMA decode kernel needs g % 128 == 0
    (4096, 11008, 4096, 128, 0, L.PATH_PREFILL),
    # fp16 between 32 and 512 rows, where the measured crossover lies: 4096 -> 11008 turns tiled
    # by M = 128, 11008 -> 4096 and 4096 -> 4096 past M = 256
    (64, 11008, 4096, 128, 0, L.PATH_SKINNY),
    (192, 11008, 4096, 128, 0, L.PATH_PREFILL),
    (256, 4096, 11008, 128, 0, L.PATH_SKINNY),
    (320, 4096, 11008, 128, 0, L.PATH_PREFILL),
    (256, 4096, 4096, 128, 0, L.PATH_SKINNY),
    (384, 4096, 4096, 128, 0, L.PATH_PREFILL),
    (1024, 4096, 11008, 64, 0, L.PATH_PREFILL),
    (1, 4096, 11008, 11008, 1, L.PATH_GEMV),          # per-channel
    # 32 < M <= 512: the K-split skinny kernel where the tiled GEMM would have few tiles
    (256, 4096, 11008, 128, 0, L.PATH_SKINNY),        # K = 11008, N = 4096: 16 tiles of 256 x 256
    (256, 11008, 4096, 128, 0, L.PATH_PREFILL),       # K = 4096: the K loop is short
    (64, 11008, 4096, 128, 1, L.PATH_SKINNY),
    (512, 4096, 11008, 128, 1, L.PATH_PREFILL),
    (128, 4096, 11008, 64, 0, L.PATH_PREFILL),        # g = 64: the skinny kernel needs g % 128 == 0
])
def test_dispatcher_choices(lib, M, N, K, g, dtype, path):
    assert lib.w4a16_select_path(M, N, K, g, dtype) == path


def test_dispatcher_rejects_invalid(lib):
    assert lib.w4a16_select_path(1, 64, 100, 100, 0) == L.ERR_SHAPE
    assert lib.w4a16_select_path(1, 64, 128, 128, 3) == L.ERR_DTYPE


def test_gptq_rejects_invalid_arguments(lib):
    assert lib.w4a16_gptq_hessian(None, 0, 16, 64, A, 0, None) == L.ERR_NULL
    assert lib.w4a16_gptq_hessian(A, 2, 16, 64, B, 0, None) == L.ERR_DTYPE
    assert lib.w4a16_gptq_hessian(A, 0, 0, 64, B, 0, None) == L.ERR_SHAPE
    assert lib.w4a16_gptq_hessian(A, 0, 16, 50000, B, 0, None) == L.ERR_SHAPE
    assert lib.w4a16_gptq_hessian(A + 1, 0, 16, 64, B, 0, None) == L.ERR_ALIGN
    assert lib.w4a16_gptq_factor(None, 64, 0.01, B, None) == L.ERR_NULL
    assert lib.w4a16_gptq_factor(A, 1, 0.01, B, None) == L.ERR_SHAPE
    assert lib.w4a16_gptq_factor(A, 64, -1.0, B, None) == L.ERR_SHAPE
    assert lib.w4a16_gptq_factor(A, 64, float("nan"), B, None) == L.ERR_SHAPE
    assert lib.w4a16_gptq_factor(A + 4, 64, 0.01, B, None) == L.ERR_ALIGN
    q = lambda **kw: lib.w4a16_gptq_quantize(kw.get("W", A), 64, kw.get("K", 128), kw.get("g", 128),
                                             kw.get("scheme", 0), kw.get("U", B), kw.get("work", C),
                                             kw.get("qw", D), kw.get("s", D + 4096), kw.get("z", D + 8192),
                                             None)
    assert q(W=None) == L.ERR_NULL
    assert q(work=None) == L.ERR_NULL
    assert q(z=None) == L.ERR_NULL                  # asymmetric needs zeros
    assert q(scheme=3) == L.ERR_SCHEME
    assert q(K=100, g=100) == L.ERR_SHAPE
    assert q(g=48) == L.ERR_GROUP
    assert q(U=B + 4) == L.ERR_ALIGN


def test_awq_workspace_and_invalid_arguments(lib):
    assert lib.w4a16_awq_workspace(64, 128, 32) >= 64 * 128 + 32 * 64 + 9 * 128 // 2
    assert lib.w4a16_awq_workspace(0, 128, 32) == L.ERR_SHAPE
    assert lib.w4a16_awq_stats(None, 0, 8, 64, A, None) == L.ERR_NULL
    assert lib.w4a16_awq_stats(A, 2, 8, 64, B, None) == L.ERR_DTYPE
    assert lib.w4a16_awq_stats(A, 0, 0, 64, B, None) == L.ERR_SHAPE
    assert lib.w4a16_awq_stats(A, 0, 8, 64, B + 2, None) == L.ERR_ALIGN
    s = lambda **kw: lib.w4a16_awq_search(kw.get("W", A), 64, kw.get("K", 128), kw.get("X", B), kw.get("dt", 0),
                                          32, kw.get("xm", C), kw.get("g", 128), kw.get("scheme", 0),
                                          kw.get("work", D), D + 0x100000, D + 0x200000, D + 0x300000,
                                          D + 0x400000, D + 0x500000, kw.get("z", D + 0x600000), None)
    assert s(W=None) == L.ERR_NULL
    assert s(xm=None) == L.ERR_NULL
    assert s(z=None) == L.ERR_NULL
    assert s(dt=5) == L.ERR_DTYPE
    assert s(scheme=2) == L.ERR_SCHEME
    assert s(K=100, g=100) == L.ERR_SHAPE
    assert s(g=96) == L.ERR_GROUP
    assert s(work=D + 4) == L.ERR_ALIGN
    assert lib.w4a16_awq_scale(A, 0, 4, 64, None, B, None) == L.ERR_NULL
    assert lib.w4a16_awq_scale(A, 0, 0, 64, C, B, None) == L.ERR_SHAPE
    assert lib.w4a16_awq_scale(A + 1, 0, 4, 64, C, B, None) == L.ERR_ALIGN


def test_w8a8_rejects_invalid_arguments(lib):
    assert lib.w4a16_w8a8_smooth(None, 0, 8, B, 16, 64, 2, C, None) == L.ERR_NULL
    assert lib.w4a16_w8a8_smooth(A, 0, 8, B, 16, 64, 5, C, None) == L.ERR_SHAPE
    assert lib.w4a16_w8a8_smooth(A, 3, 8, B, 16, 64, 2, C, None) == L.ERR_DTYPE
    assert lib.w4a16_w8a8_quantize_weight(A, 16, 64, None, B, C, None) == L.ERR_NULL
    assert lib.w4a16_w8a8_quantize_weight(A + 2, 16, 64, B, C, D, None) == L.ERR_ALIGN
    assert lib.w4a16_w8a8_quantize_act(A, 0, 0, 64, B, C, D, None) == L.ERR_SHAPE
    lin = lambda **kw: lib.w4a16_w8a8_linear(kw.get("qx", A), kw.get("sx", B), kw.get("M", 64), 64,
                                             kw.get("K", 256), kw.get("qw", C), kw.get("sw", D),
                                             kw.get("Y", D + 4096), kw.get("dt", 0), None)
    assert lin(qx=None) == L.ERR_NULL
    assert lin(K=200) == L.ERR_SHAPE                 # K % 128 != 0
    assert lin(M=1 << 24, K=1 << 8) == L.ERR_SHAPE   # M * K >= 2^31
    assert lin(qw=C + 8) == L.ERR_ALIGN
    assert lin(dt=4) == L.ERR_DTYPE


def test_kv_rejects_invalid_arguments(lib):
    assert lib.w4a16_kv_attention_workspace(32, 4096, 128) > 0
    assert lib.w4a16_kv_attention_workspace(32, 4096, 96) == L.ERR_SHAPE
    assert lib.w4a16_kv_quantize(None, 0, 2, 8, 128, 8, B, C, None, None) == L.ERR_NULL
    assert lib.w4a16_kv_quantize(A, 0, 2, 8, 128, 4, B, C, None, None) == L.ERR_NULL   # KV4 needs zeros
    assert lib.w4a16_kv_quantize(A, 0, 2, 8, 128, 6, B, C, D, None) == L.ERR_SCHEME
    assert lib.w4a16_kv_quantize(A, 0, 2, 8, 96, 8, B, C, None, None) == L.ERR_SHAPE
    assert lib.w4a16_kv_quantize(A + 8, 0, 2, 8, 128, 8, B, C, None, None) == L.ERR_ALIGN
    att = lambda **kw: lib.w4a16_kv_attention_decode(A, kw.get("dt", 0), kw.get("Hq", 8), kw.get("Hkv", 4),
                                                     kw.get("T", 16), kw.get("Tmax", 32), 128, kw.get("bits", 8),
                                                     B, C, None, B + 0x10000, C + 0x1000, None, D, D + 0x10000,
                                                     None)
    assert att(Hkv=3) == L.ERR_SHAPE             # Hq % Hkv != 0
    assert att(T=40) == L.ERR_SHAPE              # T > Tmax
    assert att(bits=4) == L.ERR_NULL             # KV4 needs zeros
    assert att(dt=7) == L.ERR_DTYPE


def test_kv_batch_rejects_invalid_arguments(lib):
    assert lib.w4a16_kv_attention_batch_workspace(16, 32, 4096, 128) > 0
    assert lib.w4a16_kv_attention_batch_workspace(0, 32, 4096, 128) == L.ERR_SHAPE
    assert lib.w4a16_kv_attention_batch_workspace(16, 32, 1 << 25, 128) == L.ERR_SHAPE
    att = lambda **kw: lib.w4a16_kv_attention_decode_batch(
        kw.get("q", A), kw.get("dt", 0), kw.get("B", 2), kw.get("Hq", 8), kw.get("Hkv", 4), kw.get("lens", C + 0x2000),
        kw.get("Tmax", 32), 128, kw.get("bits", 8), B, C, None, B + 0x10000, C + 0x1000, None, D, D + 0x10000, None)
    assert att(lens=None) == L.ERR_NULL
    assert att(bits=4) == L.ERR_NULL             # KV4 needs zeros
    assert att(dt=7) == L.ERR_DTYPE
    assert att(bits=5) == L.ERR_SCHEME
    assert att(B=0) == L.ERR_SHAPE
    assert att(B=70000) == L.ERR_SHAPE
    assert att(Hkv=3) == L.ERR_SHAPE             # Hq % Hkv != 0
    assert att(Tmax=1 << 25) == L.ERR_SHAPE
    assert att(q=A + 8) == L.ERR_ALIGN           # q must be 16-byte aligned
    assert att(lens=C + 0x2002) == L.ERR_ALIGN


# --------------------------------------------------------------------------- W8A16
def _lin8(lib, X=A, dtype=0, M=1, N=64, K=128, g=128, qw=B, s=C, z=D, Y=A + 4096, path=0):
    return lib.w4a16_w8a16_linear_ex(X, dtype, M, N, K, g, qw, s, z, Y, path, None)


@pytest.mark.parametrize("kw,status", [
    (dict(X=None), L.ERR_NULL),
    (dict(qw=None), L.ERR_NULL),
    (dict(s=None), L.ERR_NULL),
    (dict(Y=None), L.ERR_NULL),
    (dict(dtype=2), L.ERR_DTYPE),
    (dict(M=0), L.ERR_SHAPE),
    (dict(K=48, g=48), L.ERR_SHAPE),
    (dict(K=192, g=48), L.ERR_GROUP),
    (dict(X=MIS), L.ERR_ALIGN),
    (dict(qw=B + 8), L.ERR_ALIGN),
    (dict(z=D + 1), L.ERR_ALIGN),
    (dict(M=17, path=L.PATH_GEMV), L.ERR_PATH),                    # the 8-bit GEMV takes M <= 16
    (dict(M=17, K=128, g=32), L.ERR_PATH),                          # M > 16 needs g % 64 == 0
    (dict(K=96, g=32, path=L.PATH_PREFILL), L.ERR_PATH),            # the GEMM needs K % 64 == 0
    (dict(path=L.PATH_SKINNY), L.ERR_PATH),                         # no skinny kernel for 8 bits
    (dict(path=17), L.ERR_PATH),
])
def test_w8a16_linear_rejects_invalid_arguments(lib, kw, status):
    assert _lin8(lib, **kw) == status


@pytest.mark.parametrize("args,status", [
    ((None, 64, 128, 128, 0, B, C, D), L.ERR_NULL),
    ((A, 64, 128, 128, 5, B, C, D), L.ERR_SCHEME),
    ((A, 64, 128, 128, 0, B, C, None), L.ERR_NULL),
    ((A, 64, 100, 100, 0, B, C, D), L.ERR_SHAPE),
    ((A, 64, 128, 96, 0, B, C, D), L.ERR_GROUP),
    ((MIS, 64, 128, 128, 0, B, C, D), L.ERR_ALIGN),
    ((A, 64, 128, 128, 1, B + 4, C, None), L.ERR_ALIGN),
])
def test_w8a16_quantize_pack_rejects_invalid_arguments(lib, args, status):
    assert lib.w4a16_w8a16_quantize_pack(*args, None) == status


@pytest.mark.parametrize("M,N,K,g,dtype,path", [
    (1, 4096, 4096, 128, 0, L.PATH_GEMV),
    (4, 11008, 4096, 128, 1, L.PATH_GEMV),
    (4, 4096, 11008, 128, 0, L.PATH_GEMV),         # activations staged in K slices
    (1, 8192, 28672, 128, 1, L.PATH_GEMV),
    (16, 4096, 4096, 128, 0, L.PATH_GEMV),
    (17, 4096, 4096, 128, 0, L.PATH_PREFILL),
    (4096, 11008, 4096, 64, 0, L.PATH_PREFILL),
    (2, 4096, 4096, 32, 0, L.PATH_GEMV),           # g = 32: GEMV only
])
def test_w8a16_dispatcher_choices(lib, M, N, K, g, dtype, path):
    assert lib.w4a16_w8a16_select_path(M, N, K, g, dtype) == path


def test_linear_workspace_sizes(lib):
    assert lib.w4a16_linear_workspace(16, 4096, 4096, 128, 0) == 0         # decode: no split
    assert lib.w4a16_linear_workspace(4096, 4096, 11008, 128, 0) == 0      # enough tiles
    assert lib.w4a16_linear_workspace(256, 4096, 11008, 128, 1) == 0       # bf16: no split
    n = lib.w4a16_linear_workspace(256, 4096, 11008, 128, 0)
    assert n > 0 and n % (256 * 4096 * 4) == 0                              # S fp32 partial planes
    assert lib.w4a16_linear_workspace(256, 4096, 100, 100, 0) == L.ERR_SHAPE


def test_linear_ws_rejects_invalid_arguments(lib):
    assert lib.w4a16_linear_ws(None, 0, 256, 64, 128, 128, B, C, D, A, A, 0, None) == L.ERR_NULL
    assert lib.w4a16_linear_ws(A, 0, 256, 64, 128, 128, B, C, D, A + 4096, A + 4, 1 << 20, None) == L.ERR_ALIGN


def test_linear_ws_noalloc_rejects_invalid_arguments(lib):
    # host-side checks run before the scratch buffer is looked up (no GPU needed)
    f = lib.w4a16_linear_ws_noalloc
    assert f(None, 0, 256, 64, 128, 128, B, C, D, A, None) == L.ERR_NULL
    assert f(A, 0, 256, 64, 128, 128, B, C, D, None, None) == L.ERR_NULL
    assert f(A + 4, 0, 256, 64, 128, 128, B, C, D, A + 4096, None) == L.ERR_ALIGN
    assert f(A, 3, 256, 64, 128, 128, B, C, D, A + 4096, None) == L.ERR_DTYPE
    assert f(A, 0, 0, 64, 128, 128, B, C, D, A + 4096, None) == L.ERR_SHAPE
    assert f(A, 0, 256, 64, 100, 100, B, C, D, A + 4096, None) == L.ERR_SHAPE
    assert f(A, 0, 256, 64, 128, 48, B, C, D, A + 4096, None) == L.ERR_GROUP


def test_static_scratch_covers_every_split():
    # the no-allocation entry point's 64 MiB buffer holds the workspace of every split the
    # planner makes (at most 256 partial fp32 tiles of 256 x 256)
    lib = L.lib()
    worst = 0
    for M in (33, 100, 255, 256, 257, 511, 1024, 2047, 4096, 8192, 16384, 32512):
        for N in (1, 255, 256, 700, 2048, 4096, 11008, 28672):
            for K in (128, 2048, 4096, 8320, 11008, 28672):
                need = lib.w4a16_linear_workspace(M, N, K, 128, 0)
                assert need >= 0
                worst = max(worst, need)
    assert 0 < worst <= 64 * 2 ** 20


def test_linear_batch_rejects_invalid_arguments(lib):
    # every item is validated before anything is enqueued (no GPU needed)
    items = (L.LinearItem * 2)()
    items[0] = L.LinearItem(A, 1, 64, 128, 128, B, C, D, A + 4096)
    items[1] = L.LinearItem(A, 1, 64, 100, 100, B, C, D, A + 4096)       # K % 32 != 0
    assert lib.w4a16_linear_batch(items, 2, 0, None) == L.ERR_SHAPE
    items[1] = L.LinearItem(None, 1, 64, 128, 128, B, C, D, A + 4096)
    assert lib.w4a16_linear_batch(items, 2, 0, None) == L.ERR_NULL
    items[1] = L.LinearItem(A, 1, 64, 128, 48, B, C, D, A + 4096)        # group size
    assert lib.w4a16_linear_batch(items, 2, 0, None) == L.ERR_GROUP
    items[1] = L.LinearItem(A + 2, 1, 64, 128, 128, B, C, D, A + 4096)   # X alignment
    assert lib.w4a16_linear_batch(items, 2, 0, None) == L.ERR_ALIGN
    assert lib.w4a16_linear_batch(items, 2, 7, None) == L.ERR_DTYPE
    assert lib.w4a16_linear_batch(None, 1, 0, None) == L.ERR_NULL
    assert lib.w4a16_linear_batch(items, 0, 0, None) == L.ERR_SHAPE


def test_read_probe_library_loads_and_sizes_its_launch():
    """The benchmark's plain-read reference (libw4a16_probe.so, outside the W4A16 ABI) loads
    without a GPU and sizes its grid on the host: ceil(bytes / (per * 256 threads * 16 B))
    blocks, 0 for unsupported sizes."""
    import ctypes
    from w4a16_dequant_gemm_amd import build
    if not os.path.exists(build.PROBE_LIB):
        pytest.skip("libw4a16_probe.so not built")
    P = ctypes.CDLL(build.PROBE_LIB)
    P.w4a16_probe_blocks.restype = ctypes.c_longlong
    P.w4a16_probe_blocks.argtypes = [ctypes.c_longlong, ctypes.c_int]
    P.w4a16_probe_read.restype = ctypes.c_int
    P.w4a16_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p]
    assert P.w4a16_probe_blocks(56819712, 8) == -(-56819712 // (8 * 256 * 16))
    assert P.w4a16_probe_blocks(1, 16) == 1
    for bytes_, per in ((0, 8), (1 << 31, 8), (4096, 3), (4096, 32)):
        assert P.w4a16_probe_blocks(bytes_, per) == 0
    assert P.w4a16_probe_read(None, 4096, 8, None, None) == -1      # rejected before any launch
