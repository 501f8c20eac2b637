"""Group-wise INT8 weight quantizer, byte packing and the W8A16 linear layer (CPU oracle).

Test infrastructure (see the package docstring).

The 8-bit weight-only variant of the same method: the weights keep one 16-bit scale and
one 16-bit zero point per group of ``g`` input columns, the codes have 8 bits, and the
product runs against 16-bit activations after dequantization -- page
"大模型推理中 Weight-only、W8A8 和 FP8 量化有什么区别？如何选型？", §二 (weight-only INT8 /
INT4 with 16-bit activations); page "Quantization & Acceleration: 解释 W8A8 与 W4A16 的差异与
取舍" (W8A16 beside W4A16).  The parameter formulas are the pages' general-bit-width ones
with b = 8:

* asymmetric: ``s = (max - min)/(2^8 - 1) = (max - min)/255``, ``z = round(-min/s)``,
  ``q = round(x/s) + z`` in [0, 255] -- page "推理优化中“用精度换性能“的核心技术：量化",
  §3.3 (where the 8-bit divisor 255 is printed), §2.3 (core formulas);
* symmetric: ``s = max|x|/(2^7 - 1) = max|x|/127``, ``q = round(x/s)`` in [-128, 127] --
  page 4, §3.3; page "量化实战深入（GPTQ / AWQ / SmoothQuant / KV 量化）", §二 (absmax);
* dequantization ``x_hat = s (q - z)`` (page 3, §二; page 4, §2.3).

Readings (the 4-bit quantizer's R1, R2, R4, R5, R6 and R7 apply unchanged):

* W1 codes are clamped to [0, 255] (asymmetric) and [-128, 127] (symmetric).
* W2 symmetric codes are stored offset-binary, ``u = q + 128``, with a stored zero point
  of 128.0 (``zeros`` may be omitted: the implicit zero point is 128).
* W3 packing: element ``k`` of a row is byte ``k % 4`` (bits ``8*(k % 4)``) of the 32-bit
  word ``k // 4``; words are stored as int32 ``[N, K/4]``.
* W4 the linear layer is ``Y = X W_hat^T`` formed in float64 from the exact dequantized
  weights and rounded once to the activation dtype (the 4-bit layer's L-a and L-b).
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

from .formats import BF16, F16, round_fraction_to_format, round_to_bf16_bits, round_to_f16, round_to_format
from .linear import BF16_DT, FP16, _x64

ASYM = 0
SYM = 1
SYM_ZERO = 128.0
_F0 = np.float32(0.0)


def _check(W: np.ndarray, g: int) -> tuple[int, int, int]:
    if W.dtype != np.float32 or W.ndim != 2:
        raise TypeError("W must be a 2-D float32 array")
    N, K = W.shape
    if g <= 0 or K % g != 0:
        raise ValueError(f"group size {g} must divide K={K}")
    if not np.all(np.isfinite(W)):
        raise ValueError("W must be finite")
    return N, K, K // g


def _stored_scale(s32: np.ndarray) -> np.ndarray:
    """The fp32 scale rounded to fp16 (RNE); a zero scale becomes 1.0."""
    s_h = round_to_format(s32.astype(np.float64), F16)
    if np.any(np.isinf(s_h)):
        raise ValueError("group range too large: fp16 scale overflows")
    s_h = np.where(s_h == 0.0, 1.0, s_h)
    return s_h.astype(np.float16)


def quantize_asym8(W: np.ndarray, g: int):
    """Asymmetric 8-bit RTN of fp32 ``W [N, K]``: ``(codes uint8 [N, K] in [0, 255],
    scales fp16 [N, K/g], zeros fp16 [N, K/g])``."""
    N, K, G = _check(W, g)
    Wg = W.reshape(N, G, g)
    mn = Wg.min(axis=2)
    mx = Wg.max(axis=2)
    s32 = (mx - mn) / np.float32(255.0)            # one fp32 subtraction, one fp32 division
    s_h = _stored_scale(s32)
    s = s_h.astype(np.float32)
    z = np.rint((-mn) / s) + _F0                   # canonical +0.0
    if np.any(np.abs(z) > 2048):
        raise ValueError("zero point outside the exactly representable fp16 range")
    q = np.clip(np.rint(Wg / s[:, :, None]) + z[:, :, None], 0.0, 255.0)
    return q.astype(np.uint8).reshape(N, K), s_h, z.astype(np.float16)


def quantize_sym8(W: np.ndarray, g: int):
    """Symmetric 8-bit absmax RTN, codes stored offset-binary ``u = q + 128`` (W2):
    ``(codes uint8 [N, K], scales fp16 [N, K/g], zeros fp16 [N, K/g] all 128.0)``."""
    N, K, G = _check(W, g)
    Wg = W.reshape(N, G, g)
    amax = np.abs(Wg).max(axis=2)
    s32 = amax / np.float32(127.0)
    s_h = _stored_scale(s32)
    s = s_h.astype(np.float32)
    q = np.clip(np.rint(Wg / s[:, :, None]), -128.0, 127.0)
    codes = (q + np.float32(SYM_ZERO)).astype(np.uint8).reshape(N, K)
    return codes, s_h, np.full((N, G), SYM_ZERO, dtype=np.float16)


def quantize8(W: np.ndarray, g: int, scheme: int = ASYM):
    if scheme == ASYM:
        return quantize_asym8(W, g)
    if scheme == SYM:
        return quantize_sym8(W, g)
    raise ValueError(f"unknown scheme {scheme}")


def pack8(codes: np.ndarray) -> np.ndarray:
    """Codes ``[N, K]`` (0..255) -> int32 words ``[N, K/4]``, little-endian bytes (W3)."""
    codes = np.asarray(codes)
    N, K = codes.shape
    if K % 4 != 0:
        raise ValueError("K must be a multiple of 4")
    if codes.min(initial=0) < 0 or codes.max(initial=0) > 255:
        raise ValueError("codes must lie in [0, 255]")
    c = codes.astype(np.uint32).reshape(N, K // 4, 4)
    words = np.zeros((N, K // 4), dtype=np.uint32)
    for i in range(4):
        words |= c[:, :, i] << np.uint32(8 * i)
    return words.view(np.int32)


def unpack8(qweight: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack8`: int32 ``[N, K/4]`` -> codes uint8 ``[N, K]``."""
    w = np.ascontiguousarray(qweight).view(np.uint32)
    N, KW = w.shape
    out = np.empty((N, KW, 4), dtype=np.uint8)
    for i in range(4):
        out[:, :, i] = (w >> np.uint32(8 * i)) & np.uint32(0xFF)
    return out.reshape(N, KW * 4)


def dequantize8(qweight: np.ndarray, scales: np.ndarray, zeros, g: int) -> np.ndarray:
    """``W_hat[n, k] = s[n, k//g] (u[n, k] - z[n, k//g])`` in float64 (exact); ``zeros=None``
    is the symmetric implicit zero point 128 (W2)."""
    u = unpack8(qweight).astype(np.float64)
    N, K = u.shape
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    if s.shape != (N, K // g):
        raise ValueError("scales shape mismatch")
    z = (np.full_like(s, SYM_ZERO) if zeros is None
         else np.asarray(zeros, dtype=np.float16).astype(np.float64))
    if z.shape != s.shape:
        raise ValueError("zeros shape mismatch")
    return np.repeat(s, g, axis=1) * (u - np.repeat(z, g, axis=1))


def linear8_ref_f64(X, dtype: int, qweight, scales, zeros, g: int) -> np.ndarray:
    """Unrounded ``Y = X W_hat^T`` in float64 (W4)."""
    x = _x64(X, dtype)
    w = dequantize8(qweight, scales, zeros, g)
    if x.shape[1] != w.shape[1]:
        raise ValueError("K mismatch")
    return x @ w.T


def linear8_ref(X, dtype: int, qweight, scales, zeros, g: int) -> np.ndarray:
    """``Y`` rounded once to the activation dtype: fp16 array or bf16 bit patterns."""
    y = linear8_ref_f64(X, dtype, qweight, scales, zeros, g)
    return round_to_f16(y) if dtype == FP16 else round_to_bf16_bits(y)


def linear8_exact(X, dtype: int, qweight, scales, zeros, g: int) -> np.ndarray:
    """Exact-rational ``Y`` rounded once (tiny shapes only), per element from the codes."""
    x = _x64(X, dtype)
    u = unpack8(qweight)
    M, K = x.shape
    N = u.shape[0]
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    z = (np.full_like(s, SYM_ZERO) if zeros is None
         else np.asarray(zeros, dtype=np.float16).astype(np.float64))
    fmt = F16 if dtype == FP16 else BF16
    out = np.empty((M, N), dtype=np.float64)
    for m in range(M):
        xm = [Fraction(float(v)) for v in x[m]]
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += xm[k] * Fraction(float(s[n, k // g])) * (int(u[n, k]) - Fraction(float(z[n, k // g])))
            out[m, n] = round_fraction_to_format(acc, fmt)
    return out.astype(np.float16) if dtype == FP16 else round_to_bf16_bits(out)


__all__ = ["ASYM", "SYM", "SYM_ZERO", "quantize_asym8", "quantize_sym8", "quantize8", "pack8", "unpack8",
           "dequantize8", "linear8_ref", "linear8_ref_f64", "linear8_exact", "FP16", "BF16_DT"]
