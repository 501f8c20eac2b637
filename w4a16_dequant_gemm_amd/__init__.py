"""MI355X-native W4A16 weight-only linear layer: Python binding of ``libw4a16.so``.

The binding only marshals arguments: it checks dtypes, shapes and contiguity of torch
tensors, passes raw device pointers and the current HIP stream to the C ABI and turns
negative status codes into :class:`W4A16Error`.  Every step of the computation runs in
the library's HIP kernels; there is no CPU or PyTorch fallback.

``quantize_pack(W, group_size, scheme)`` -> ``(qweight, scales, zeros)``
    group-wise INT4 RTN quantization of an fp32 ``[N, K]`` CUDA tensor.
``linear(X, qweight, scales, zeros, group_size, path=PATH_AUTO)`` -> ``Y``
    ``Y = X . dequant(qweight)^T`` for fp16/bf16 ``X [M, K]``.
``linear_batch([(X, qweight, scales, zeros, group_size), ...])`` -> ``[Y, ...]``
    independent layers in one call; one-row layers share grouped launches.
``gptq_hessian(X, H=None)`` / ``gptq_factor(H, damp)`` / ``gptq_quantize(W, U, group_size, scheme)``
    GPTQ: ``H = 2 X^T X`` (fp64, lower triangle), the upper Cholesky factor ``U`` of the
    damped inverse, and the compensated column-wise quantization in the packed format.
``awq_stats(X)`` / ``awq_search(W, X, xmean, group_size, scheme)`` / ``awq_scale(X, s)``
    AWQ: per-channel activation statistic, grid search over channel scalings, and the
    activation side of the rescaling.
``w8a8_smooth`` / ``w8a8_quantize_weight`` / ``w8a8_quantize_act`` / ``w8a8_linear``
    W8A8 with SmoothQuant on the INT8 matrix cores.
``kv_quantize(x, bits)`` / ``kv_attention_decode(q, cache, T)``
    per-token KV8 / KV4 cache quantization and the decode attention over the quantized cache.
"""

from __future__ import annotations

import torch

from . import _lib as _lib_mod
from ._lib import (ASYM, BF16, F16, OK, PATH_AUTO, PATH_GEMV, PATH_NAMES, PATH_PREFILL,
                   PATH_SKINNY, SYM, W4A16Error, check, lib)

__all__ = [
    "ASYM", "SYM", "F16", "BF16", "PATH_AUTO", "PATH_GEMV", "PATH_SKINNY", "PATH_PREFILL",
    "PATH_NAMES", "W4A16Error", "quantize_pack", "linear", "linear_batch", "dequantize", "select_path",
    "w8a16_quantize_pack", "w8a16_linear", "w8a16_select_path", "linear_workspace", "linear_ws",
    "abi_version", "lib", "gptq_hessian", "gptq_factor", "gptq_quantize", "awq_stats",
    "awq_search", "awq_scale", "w8a8_smooth", "w8a8_quantize_weight", "w8a8_quantize_act",
    "w8a8_linear", "kv_quantize", "kv_attention_decode",
]


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _need(t: torch.Tensor, name: str, dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float16:
        return F16
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"activations must be float16 or bfloat16, got {t.dtype}")


def _check_linear(X, qweight, scales, zeros, group_size: int, codes_per_word: int):
    """Argument checks shared by the linear calls: dtypes, 2-D contiguous GPU tensors on the
    device of ``X``, ``qweight [N, K/codes_per_word]``, ``scales`` and ``zeros`` (if given)
    ``[N, K/group_size]``.  Returns ``(M, K, N)``."""
    _need(X, "X", X.dtype, 2)
    _need(qweight, "qweight", torch.int32, 2)
    _need(scales, "scales", torch.float16, 2)
    if zeros is not None:
        _need(zeros, "zeros", torch.float16, 2)
    M, K = X.shape
    N = qweight.shape[0]
    if qweight.shape[1] * codes_per_word != K:
        raise ValueError(f"qweight must be [N, K/{codes_per_word}]")
    if group_size <= 0 or K % group_size or tuple(scales.shape) != (N, K // group_size):
        raise ValueError("scales must be [N, K/group_size]")
    if zeros is not None and zeros.shape != scales.shape:
        raise ValueError("zeros must match scales")
    for t, name in ((qweight, "qweight"), (scales, "scales"), (zeros, "zeros")):
        if t is not None and t.device != X.device:
            raise ValueError(f"{name} must be on the device of X")
    return M, K, N


def _out(out, X, M: int, N: int) -> torch.Tensor:
    """The output tensor: allocated ``[M, N]`` in the dtype of ``X``, or a caller tensor
    checked for dtype, shape, device and contiguity."""
    if out is None:
        return torch.empty((M, N), dtype=X.dtype, device=X.device)
    _need(out, "out", X.dtype, 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out must be [M, N]")
    if out.device != X.device:
        raise ValueError("out must be on the device of X")
    return out


def abi_version() -> int:
    return lib().w4a16_abi_version()


def select_path(M: int, N: int, K: int, group_size: int, dtype: int = F16) -> int:
    """Kernel path the dispatcher picks (host only); raises on invalid arguments."""
    p = lib().w4a16_select_path(M, N, K, group_size, dtype)
    if p < 0:
        raise W4A16Error(p, "select_path")
    return p


def quantize_pack(W: torch.Tensor, group_size: int = 128, scheme: int = ASYM,
                  write_zeros: bool = True):
    """Quantize fp32 ``W [N, K]`` on the GPU.

    Returns ``(qweight int32 [N, K/8], scales fp16 [N, K/g], zeros fp16 [N, K/g] or None)``.
    ``zeros`` is None only for the symmetric scheme with ``write_zeros=False``.
    """
    _need(W, "W", torch.float32, 2)
    N, K = W.shape
    if K % 8 or group_size <= 0 or K % group_size:
        raise ValueError("K must be a multiple of 8 and of group_size")
    G = K // group_size
    qweight = torch.empty((N, K // 8), dtype=torch.int32, device=W.device)
    scales = torch.empty((N, G), dtype=torch.float16, device=W.device)
    zeros = None
    if scheme == ASYM or write_zeros:
        zeros = torch.empty((N, G), dtype=torch.float16, device=W.device)
    st = lib().w4a16_quantize_pack(W.data_ptr(), N, K, group_size, scheme, qweight.data_ptr(),
                                   scales.data_ptr(), zeros.data_ptr() if zeros is not None else None,
                                   _stream())
    check(st, "w4a16_quantize_pack")
    return qweight, scales, zeros


def linear(X: torch.Tensor, qweight: torch.Tensor, scales: torch.Tensor, zeros, group_size: int,
           path: int = PATH_AUTO, out: torch.Tensor | None = None) -> torch.Tensor:
    """``Y [M, N] = X [M, K] . dequant(qweight)^T`` in the dtype of ``X``."""
    dt = _dtype_code(X)
    M, K, N = _check_linear(X, qweight, scales, zeros, group_size, 8)
    out = _out(out, X, M, N)
    st = lib().w4a16_linear_ex(X.data_ptr(), dt, M, N, K, group_size, qweight.data_ptr(),
                               scales.data_ptr(), zeros.data_ptr() if zeros is not None else None,
                               out.data_ptr(), path, _stream())
    check(st, "w4a16_linear")
    return out


def linear_batch(layers, outs=None) -> list:
    """Several independent layers in one call: ``layers`` is a sequence of
    ``(X, qweight, scales, zeros, group_size)`` with one activation dtype; returns the outputs
    ``Y`` (``outs``, if given, supplies them).  One-row layers share grouped launches."""
    layers = list(layers)
    if not layers:
        raise ValueError("linear_batch needs at least one layer")
    dt = _dtype_code(layers[0][0])
    outs = list(outs) if outs is not None else [None] * len(layers)
    if len(outs) != len(layers):
        raise ValueError("outs must match layers")
    items = (_lib_mod.LinearItem * len(layers))()
    ys = []
    for i, ((X, qweight, scales, zeros, group_size), out) in enumerate(zip(layers, outs)):
        if _dtype_code(X) != dt:
            raise TypeError("all layers of a batch need the same activation dtype")
        M, K, N = _check_linear(X, qweight, scales, zeros, group_size, 8)
        if X.device != layers[0][0].device:
            raise ValueError("all layers of a batch must be on one device")
        y = _out(out, X, M, N)
        items[i] = _lib_mod.LinearItem(X.data_ptr(), M, N, K, group_size, qweight.data_ptr(), scales.data_ptr(),
                                       zeros.data_ptr() if zeros is not None else None, y.data_ptr())
        ys.append(y)
    check(lib().w4a16_linear_batch(items, len(layers), dt, _stream()), "w4a16_linear_batch")
    return ys


def linear_workspace(M: int, N: int, K: int, group_size: int, dtype: int = F16) -> int:
    """Bytes of fp32 workspace :func:`linear_ws` can use (0: it behaves as :func:`linear`)."""
    need = lib().w4a16_linear_workspace(M, N, K, group_size, dtype)
    if need < 0:
        raise W4A16Error(int(need), "w4a16_linear_workspace")
    return int(need)


def linear_ws(X: torch.Tensor, qweight: torch.Tensor, scales: torch.Tensor, zeros, group_size: int,
              work: torch.Tensor | None = None, out: torch.Tensor | None = None) -> torch.Tensor:
    """:func:`linear` with a workspace for the tile-starved prefill shapes (split K, partial
    tiles summed in fixed order).  ``work``: float32 device tensor (allocated here if None)."""
    dt = _dtype_code(X)
    M, K, N = _check_linear(X, qweight, scales, zeros, group_size, 8)
    need = linear_workspace(M, N, K, group_size, dt)
    if work is None and need > 0:
        work = torch.empty((need + 3) // 4, dtype=torch.float32, device=X.device)
    if work is not None:
        _need(work, "work", torch.float32, work.dim())
        if work.device != X.device:
            raise ValueError("work must be on the device of X")
    out = _out(out, X, M, N)
    st = lib().w4a16_linear_ws(X.data_ptr(), dt, M, N, K, group_size, qweight.data_ptr(), scales.data_ptr(),
                               zeros.data_ptr() if zeros is not None else None, out.data_ptr(),
                               work.data_ptr() if work is not None else None,
                               work.numel() * 4 if work is not None else 0, _stream())
    check(st, "w4a16_linear_ws")
    return out


def w8a16_quantize_pack(W: torch.Tensor, group_size: int = 128, scheme: int = ASYM,
                        write_zeros: bool = True):
    """8-bit codes: quantize fp32 ``W [N, K]`` on the GPU.  Returns ``(qweight int32 [N, K/4],
    scales fp16 [N, K/g], zeros fp16 [N, K/g] or None)``; ``zeros`` is None only for the
    symmetric scheme with ``write_zeros=False`` (implicit zero point 128)."""
    _need(W, "W", torch.float32, 2)
    N, K = W.shape
    if K % 4 or group_size <= 0 or K % group_size:
        raise ValueError("K must be a multiple of 4 and of group_size")
    G = K // group_size
    qweight = torch.empty((N, K // 4), dtype=torch.int32, device=W.device)
    scales = torch.empty((N, G), dtype=torch.float16, device=W.device)
    zeros = None
    if scheme == ASYM or write_zeros:
        zeros = torch.empty((N, G), dtype=torch.float16, device=W.device)
    st = lib().w4a16_w8a16_quantize_pack(W.data_ptr(), N, K, group_size, scheme, qweight.data_ptr(),
                                         scales.data_ptr(), zeros.data_ptr() if zeros is not None else None,
                                         _stream())
    check(st, "w4a16_w8a16_quantize_pack")
    return qweight, scales, zeros


def w8a16_select_path(M: int, N: int, K: int, group_size: int, dtype: int = F16) -> int:
    """Kernel the 8-bit dispatcher picks (host only): ``PATH_GEMV`` or ``PATH_PREFILL``."""
    p = lib().w4a16_w8a16_select_path(M, N, K, group_size, dtype)
    if p < 0:
        raise W4A16Error(p, "w8a16_select_path")
    return p


def w8a16_linear(X: torch.Tensor, qweight: torch.Tensor, scales: torch.Tensor, zeros, group_size: int,
                 path: int = PATH_AUTO, out: torch.Tensor | None = None) -> torch.Tensor:
    """``Y [M, N] = X [M, K] . dequant(qweight)^T`` with 8-bit codes ``qweight int32 [N, K/4]``
    (the weight-streaming GEMV for M <= 16, the tiled MFMA GEMM above)."""
    dt = _dtype_code(X)
    M, K, N = _check_linear(X, qweight, scales, zeros, group_size, 4)
    out = _out(out, X, M, N)
    st = lib().w4a16_w8a16_linear_ex(X.data_ptr(), dt, M, N, K, group_size, qweight.data_ptr(),
                                     scales.data_ptr(), zeros.data_ptr() if zeros is not None else None,
                                     out.data_ptr(), path, _stream())
    check(st, "w4a16_w8a16_linear")
    return out


def dequantize(qweight: torch.Tensor, scales: torch.Tensor, zeros, group_size: int) -> torch.Tensor:
    """Exact fp32 ``W_hat [N, K]`` (layout checks and tests)."""
    _need(qweight, "qweight", torch.int32, 2)
    _need(scales, "scales", torch.float16, 2)
    if zeros is not None:
        _need(zeros, "zeros", torch.float16, 2)
    N, KW = qweight.shape
    K = KW * 8
    out = torch.empty((N, K), dtype=torch.float32, device=qweight.device)
    st = lib().w4a16_dequantize(qweight.data_ptr(), scales.data_ptr(),
                                zeros.data_ptr() if zeros is not None else None, N, K, group_size,
                                out.data_ptr(), _stream())
    check(st, "w4a16_dequantize")
    return out


def gptq_hessian(X: torch.Tensor, H: torch.Tensor | None = None) -> torch.Tensor:
    """``H = 2 X^T X`` (``H += 2 X^T X`` when ``H`` is given) for fp16/bf16 calibration
    activations ``X [n, K]``; fp64 ``[K, K]``, lower triangle defined."""
    dt = _dtype_code(X)
    _need(X, "X", X.dtype, 2)
    n, K = X.shape
    acc = H is not None
    if H is None:
        H = torch.empty((K, K), dtype=torch.float64, device=X.device)
    else:
        _need(H, "H", torch.float64, 2)
        if tuple(H.shape) != (K, K):
            raise ValueError("H must be [K, K]")
    check(lib().w4a16_gptq_hessian(X.data_ptr(), dt, n, K, H.data_ptr(), 1 if acc else 0, _stream()),
          "w4a16_gptq_hessian")
    return H


def gptq_factor(H: torch.Tensor, damp: float = 0.01) -> torch.Tensor:
    """Upper ``U`` with ``(H + damp * mean(diag H) I)^-1 = U^T U``; ``H`` is overwritten."""
    _need(H, "H", torch.float64, 2)
    K = H.shape[0]
    if tuple(H.shape) != (K, K):
        raise ValueError("H must be square")
    U = torch.empty_like(H)
    check(lib().w4a16_gptq_factor(H.data_ptr(), K, float(damp), U.data_ptr(), _stream()),
          "w4a16_gptq_factor")
    return U


def gptq_quantize(W: torch.Tensor, U: torch.Tensor, group_size: int = 128, scheme: int = ASYM,
                  work: torch.Tensor | None = None):
    """GPTQ of fp32 ``W [N, K]`` with the factor ``U``; returns ``(qweight, scales, zeros)``
    in the layout of :func:`quantize_pack` (zeros all 8 for the symmetric scheme)."""
    _need(W, "W", torch.float32, 2)
    _need(U, "U", torch.float64, 2)
    N, K = W.shape
    if tuple(U.shape) != (K, K):
        raise ValueError("U must be [K, K]")
    if K % 8 or group_size <= 0 or K % group_size:
        raise ValueError("K must be a multiple of 8 and of group_size")
    need = N * K + 64 * N
    if work is None:
        work = torch.empty(need, dtype=torch.float64, device=W.device)
    elif work.dtype != torch.float64 or work.numel() < need or not work.is_contiguous():
        raise ValueError(f"work must be a contiguous fp64 tensor of >= {need} elements")
    G = K // group_size
    qweight = torch.empty((N, K // 8), dtype=torch.int32, device=W.device)
    scales = torch.empty((N, G), dtype=torch.float16, device=W.device)
    zeros = torch.empty((N, G), dtype=torch.float16, device=W.device)
    check(lib().w4a16_gptq_quantize(W.data_ptr(), N, K, group_size, scheme, U.data_ptr(),
                                    work.data_ptr(), qweight.data_ptr(), scales.data_ptr(),
                                    zeros.data_ptr(), _stream()), "w4a16_gptq_quantize")
    return qweight, scales, zeros


def awq_stats(X: torch.Tensor) -> torch.Tensor:
    """Mean ``|x|`` per input channel of calibration activations ``X [n, K]`` (fp32 ``[K]``)."""
    dt = _dtype_code(X)
    _need(X, "X", X.dtype, 2)
    n, K = X.shape
    out = torch.empty(K, dtype=torch.float32, device=X.device)
    check(lib().w4a16_awq_stats(X.data_ptr(), dt, n, K, out.data_ptr(), _stream()), "w4a16_awq_stats")
    return out


def awq_search(W: torch.Tensor, X: torch.Tensor, xmean: torch.Tensor, group_size: int = 128,
               scheme: int = ASYM):
    """Grid search of the channel scaling; returns ``(qweight, scales, zeros, s, losses,
    best)`` (``s`` fp32 ``[K]``, ``losses`` fp64 ``[9]``, ``best`` int32 ``[1]``, all on the
    GPU)."""
    _need(W, "W", torch.float32, 2)
    dt = _dtype_code(X)
    _need(X, "X", X.dtype, 2)
    _need(xmean, "xmean", torch.float32, 1)
    N, K = W.shape
    n = X.shape[0]
    if X.shape[1] != K or xmean.shape[0] != K:
        raise ValueError("X must be [n, K] and xmean [K]")
    if K % 8 or group_size <= 0 or K % group_size:
        raise ValueError("K must be a multiple of 8 and of group_size")
    L = lib()
    need = L.w4a16_awq_workspace(N, K, n)
    if need < 0:
        raise W4A16Error(int(need), "w4a16_awq_workspace")
    work = torch.empty(need, dtype=torch.float64, device=W.device)
    G = K // group_size
    qweight = torch.empty((N, K // 8), dtype=torch.int32, device=W.device)
    scales = torch.empty((N, G), dtype=torch.float16, device=W.device)
    zeros = torch.empty((N, G), dtype=torch.float16, device=W.device)
    s = torch.empty(K, dtype=torch.float32, device=W.device)
    losses = torch.empty(9, dtype=torch.float64, device=W.device)
    best = torch.empty(1, dtype=torch.int32, device=W.device)
    check(L.w4a16_awq_search(W.data_ptr(), N, K, X.data_ptr(), dt, n, xmean.data_ptr(), group_size,
                             scheme, work.data_ptr(), losses.data_ptr(), best.data_ptr(), s.data_ptr(),
                             qweight.data_ptr(), scales.data_ptr(), zeros.data_ptr(), _stream()),
          "w4a16_awq_search")
    return qweight, scales, zeros, s, losses, best


def awq_scale(X: torch.Tensor, s: torch.Tensor, out: torch.Tensor | None = None) -> torch.Tensor:
    """``X * s`` per input channel, rounded once to the dtype of ``X``."""
    dt = _dtype_code(X)
    _need(X, "X", X.dtype, 2)
    _need(s, "s", torch.float32, 1)
    M, K = X.shape
    if s.shape[0] != K:
        raise ValueError("s must be [K]")
    if out is None:
        out = torch.empty_like(X)
    else:
        _need(out, "out", X.dtype, 2)
    check(lib().w4a16_awq_scale(X.data_ptr(), dt, M, K, s.data_ptr(), out.data_ptr(), _stream()),
          "w4a16_awq_scale")
    return out


def w8a8_smooth(X: torch.Tensor, W: torch.Tensor, alpha_quarters: int = 2) -> torch.Tensor:
    """SmoothQuant factors ``s [K]`` from calibration activations ``X [n, K]`` and ``W [N, K]``."""
    dt = _dtype_code(X)
    _need(X, "X", X.dtype, 2)
    _need(W, "W", torch.float32, 2)
    n, K = X.shape
    N = W.shape[0]
    if W.shape[1] != K:
        raise ValueError("W must be [N, K]")
    s = torch.empty(K, dtype=torch.float32, device=X.device)
    check(lib().w4a16_w8a8_smooth(X.data_ptr(), dt, n, W.data_ptr(), N, K, alpha_quarters, s.data_ptr(),
                                  _stream()), "w4a16_w8a8_smooth")
    return s


def w8a8_quantize_weight(W: torch.Tensor, s: torch.Tensor):
    """``(qweight int8 [N, K], wscale fp32 [N])`` of the smoothed weights ``W * s``."""
    _need(W, "W", torch.float32, 2)
    _need(s, "s", torch.float32, 1)
    N, K = W.shape
    q = torch.empty((N, K), dtype=torch.int8, device=W.device)
    sw = torch.empty(N, dtype=torch.float32, device=W.device)
    check(lib().w4a16_w8a8_quantize_weight(W.data_ptr(), N, K, s.data_ptr(), q.data_ptr(), sw.data_ptr(),
                                           _stream()), "w4a16_w8a8_quantize_weight")
    return q, sw


def w8a8_quantize_act(X: torch.Tensor, s: torch.Tensor):
    """``(qx int8 [M, K], xscale fp32 [M])``: per-token INT8 of ``X / s``."""
    dt = _dtype_code(X)
    _need(X, "X", X.dtype, 2)
    _need(s, "s", torch.float32, 1)
    M, K = X.shape
    q = torch.empty((M, K), dtype=torch.int8, device=X.device)
    sx = torch.empty(M, dtype=torch.float32, device=X.device)
    check(lib().w4a16_w8a8_quantize_act(X.data_ptr(), dt, M, K, s.data_ptr(), q.data_ptr(), sx.data_ptr(),
                                        _stream()), "w4a16_w8a8_quantize_act")
    return q, sx


def w8a8_linear(qx: torch.Tensor, sx: torch.Tensor, qw: torch.Tensor, sw: torch.Tensor,
                dtype=torch.float16, out: torch.Tensor | None = None) -> torch.Tensor:
    """``Y [M, N]`` from INT8 operands and their fp32 scales, on the INT8 matrix cores."""
    _need(qx, "qx", torch.int8, 2)
    _need(qw, "qweight", torch.int8, 2)
    _need(sx, "xscale", torch.float32, 1)
    _need(sw, "wscale", torch.float32, 1)
    M, K = qx.shape
    N = qw.shape[0]
    if qw.shape[1] != K or sx.shape[0] != M or sw.shape[0] != N:
        raise ValueError("shape mismatch")
    if out is None:
        out = torch.empty((M, N), dtype=dtype, device=qx.device)
    dt = _dtype_code(out)
    check(lib().w4a16_w8a8_linear(qx.data_ptr(), sx.data_ptr(), M, N, K, qw.data_ptr(), sw.data_ptr(),
                                  out.data_ptr(), dt, _stream()), "w4a16_w8a8_linear")
    return out


def kv_quantize(x: torch.Tensor, bits: int = 8):
    """Quantize ``x [H, T, D]`` (fp16/bf16) into ``(codes, scales, zeros)``: codes int8
    ``[H, T, D]`` (KV8) or int32 ``[H, T, D/8]`` (KV4), scales / zeros fp16 ``[H, T]`` (zeros
    None for KV8)."""
    dt = _dtype_code(x)
    _need(x, "x", x.dtype, 3)
    H, T, D = x.shape
    if bits == 8:
        codes = torch.empty((H, T, D), dtype=torch.int8, device=x.device)
        zeros = None
    else:
        codes = torch.empty((H, T, D // 8), dtype=torch.int32, device=x.device)
        zeros = torch.empty((H, T), dtype=torch.float16, device=x.device)
    scales = torch.empty((H, T), dtype=torch.float16, device=x.device)
    check(lib().w4a16_kv_quantize(x.data_ptr(), dt, H, T, D, bits, codes.data_ptr(), scales.data_ptr(),
                                  zeros.data_ptr() if zeros is not None else None, _stream()),
          "w4a16_kv_quantize")
    return codes, scales, zeros


def kv_attention_workspace(Hq: int, T: int, D: int) -> int:
    """fp32 elements of the scratch buffer that :func:`kv_attention_decode` needs."""
    need = lib().w4a16_kv_attention_workspace(Hq, T, D)
    if need < 0:
        raise W4A16Error(int(need), "w4a16_kv_attention_workspace")
    return int(need)


def kv_attention_batch_workspace(B: int, Hq: int, Tmax: int, D: int) -> int:
    """fp32 elements of the scratch buffer that :func:`kv_attention_decode_batch` needs."""
    need = lib().w4a16_kv_attention_batch_workspace(B, Hq, Tmax, D)
    if need < 0:
        raise W4A16Error(int(need), "w4a16_kv_attention_batch_workspace")
    return int(need)


def kv_attention_decode_batch(q: torch.Tensor, kcache, vcache, lengths: torch.Tensor, bits: int = 8,
                              out: torch.Tensor | None = None, work: torch.Tensor | None = None) -> torch.Tensor:
    """Decode attention for ``B`` sequences in one call: ``q [B, Hq, D]``, caches
    ``(codes, scales, zeros)`` of shape ``[B, Hkv, Tmax, ...]`` (scales ``[B, Hkv, Tmax]``),
    ``lengths`` int32 ``[B]`` on the device."""
    dt = _dtype_code(q)
    _need(q, "q", q.dtype, 3)
    _need(lengths, "lengths", torch.int32, 1)
    B, Hq, D = q.shape
    kc, ks, kz = kcache
    vc, vs, vz = vcache
    if ks.dim() != 3 or ks.shape[0] != B or lengths.shape[0] != B:
        raise ValueError("caches must be [B, Hkv, Tmax, ...] and lengths [B]")
    _, Hkv, Tmax = ks.shape
    L = lib()
    need = kv_attention_batch_workspace(B, Hq, Tmax, D)
    if work is None:
        work = torch.empty(need, dtype=torch.float32, device=q.device)
    elif work.dtype != torch.float32 or not work.is_cuda or work.numel() < need:
        raise ValueError(f"work must be a float32 device tensor of at least {need} elements")
    if out is None:
        out = torch.empty_like(q)
    ptr = lambda t: t.data_ptr() if t is not None else None
    check(L.w4a16_kv_attention_decode_batch(q.data_ptr(), dt, B, Hq, Hkv, lengths.data_ptr(), Tmax, D, bits,
                                            kc.data_ptr(), ks.data_ptr(), ptr(kz), vc.data_ptr(), vs.data_ptr(),
                                            ptr(vz), work.data_ptr(), out.data_ptr(), _stream()),
          "w4a16_kv_attention_decode_batch")
    return out


def kv_attention_decode(q: torch.Tensor, kcache, vcache, T: int, bits: int = 8,
                        out: torch.Tensor | None = None, work: torch.Tensor | None = None) -> torch.Tensor:
    """``softmax(q K^T / sqrt(D)) V`` over the first ``T`` tokens of quantized caches
    ``(codes, scales, zeros)`` of shape ``[Hkv, Tmax, ...]``; ``q [Hq, D]``.  ``work`` is an
    optional fp32 device buffer of at least :func:`kv_attention_workspace` elements."""
    dt = _dtype_code(q)
    _need(q, "q", q.dtype, 2)
    Hq, D = q.shape
    kc, ks, kz = kcache
    vc, vs, vz = vcache
    Hkv, Tmax = ks.shape
    L = lib()
    need = kv_attention_workspace(Hq, T, D)
    if work is None:
        work = torch.empty(need, dtype=torch.float32, device=q.device)
    elif work.dtype != torch.float32 or not work.is_cuda or work.numel() < need:
        raise ValueError(f"work must be a float32 device tensor of at least {need} elements")
    if out is None:
        out = torch.empty_like(q)
    ptr = lambda t: t.data_ptr() if t is not None else None
    check(L.w4a16_kv_attention_decode(q.data_ptr(), dt, Hq, Hkv, T, Tmax, D, bits, kc.data_ptr(), ks.data_ptr(),
                                      ptr(kz), vc.data_ptr(), vs.data_ptr(), ptr(vz), work.data_ptr(),
                                      out.data_ptr(), _stream()), "w4a16_kv_attention_decode")
    return out
