"""Group-wise INT4 quantizer, nibble packing and dequantization (CPU oracle).

Test infrastructure (see the package docstring).

Method (restated from the pages):

* Affine map between a float ``x`` and an integer code ``q``: quantize with
  ``q = round(x/s) + z``, dequantize with ``x_hat = s * (q - z)`` -- page
  "量化实战深入（GPTQ / AWQ / SmoothQuant / KV 量化）", §二 量化的数学本质;
  page "推理优化中“用精度换性能“的核心技术：量化", §2.3 核心公式.
* Asymmetric (min/max) parameters: the scale is the range divided by the
  number of steps of the code grid, ``s = (max - min)/(2^b - 1)``, and the
  zero point is ``z = round(-min/s)`` so the grid spans [min, max] -- page 4,
  §3.3 (printed there for 8 bits, ``/255``; with the 4-bit unsigned range
  [0, 15] of §2.2 the divisor is 15).
* Symmetric (absmax) parameters: ``s = max|x| / (2^(b-1) - 1)`` (``/7`` for
  4 bits) and ``z = 0`` -- page 3, §二 (absmax); page 4, §3.3.
* Granularity: one scale and one optional zero point, each 16 bits, per group
  of ``g`` consecutive input columns of an output row; ``g = 128`` is the
  usual choice, giving 4 + 32/128 = 4.25 bits per weight; ``g = K`` is the
  per-channel case -- page 4, §3.4 量化粒度; page 3, §二 granularity table.

Readings where the pages leave a step open:

* R1 orientation: ``W`` is ``[N = d_out, K = d_in]``; groups run along K.
* R2 ``round`` is round-half-to-even (``np.rint``), the IEEE default.
* R3 codes are clamped to the code range ([0, 15] asymmetric, [-8, 7]
  symmetric); the pages give the ranges but no clamp.
* R4 the stored fp16 scale ``s_h`` (not the fp32 quotient) feeds ``z`` and
  ``q``, so the stored triple is self-consistent with dequantization.
* R5 all quantizer arithmetic is IEEE fp32 with round-to-nearest-even in the
  order Q1..Q5 below, so a GPU can reproduce the codes bit for bit.
* R6 a zero-range group (``s_h == 0``) uses ``s_h = 1.0``.
* R7 the zero point is ``rint(-min/s) + 0.0``: the ``+ 0.0`` turns -0.0 into
  +0.0 so its fp16 bits are unique.  ``|z| <= 2048`` is required (fp16 holds
  such integers exactly); a larger zero point raises.
* R8 symmetric codes are stored offset-binary, ``u = q + 8`` in [0, 15], with
  a stored zero point of 8.0, so one unpack path serves both schemes.
* R9 packing: element ``k`` of a row lives in bits ``4*(k % 8)`` of 32-bit
  word ``k // 8`` (little-endian nibbles); words are stored as int32.
"""

from __future__ import annotations

import numpy as np

from .formats import F16, round_to_format

ASYM = 0   # RTN asymmetric min/max, codes [0, 15]
SYM = 1    # RTN symmetric absmax, codes [-8, 7] stored as u = q + 8

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
    """Q3: round the fp32 scale to fp16 (RNE); a zero scale becomes 1.0 (R6)."""
    s_h = round_to_format(s32.astype(np.float64), F16)
    if np.any(np.isinf(s_h)):
        raise ValueError("group range too large: fp16 scale overflows")
    s_h = np.where(s_h == 0.0, 1.0, s_h)
    return s_h.astype(np.float16)


def quantize_asym(W: np.ndarray, g: int):
    """Asymmetric RTN quantization of fp32 ``W [N, K]`` with group size ``g``.

    Returns ``(codes uint8 [N, K] in [0, 15], scales fp16 [N, K/g],
    zeros fp16 [N, K/g])``.
    """
    N, K, G = _check(W, g)
    Wg = W.reshape(N, G, g)
    # Q1: exact group minimum and maximum.
    mn = Wg.min(axis=2)
    mx = Wg.max(axis=2)
    # Q2: s32 = (max - min) / 15, two fp32 RNE operations in this order.
    s32 = (mx - mn) / np.float32(15.0)
    # Q3: stored fp16 scale; everything below uses it (R4).
    s_h = _stored_scale(s32)
    s = s_h.astype(np.float32)
    # Q4: zero point z = rint(-min / s), canonical +0.0 (R7).
    z = np.rint((-mn) / s) + _F0
    if np.any(np.abs(z) > 2048):
        raise ValueError("zero point outside the exactly representable fp16 range")
    # Q5: codes q = clamp(rint(x / s) + z, 0, 15) (R2, R3).
    q = np.rint(Wg / s[:, :, None]) + z[:, :, None]
    q = np.clip(q, 0.0, 15.0)
    codes = q.astype(np.uint8).reshape(N, K)
    return codes, s_h, z.astype(np.float16)


def quantize_sym(W: np.ndarray, g: int):
    """Symmetric absmax RTN quantization, codes stored offset-binary (R8).

    Returns ``(codes uint8 [N, K] in [0, 15], scales fp16 [N, K/g],
    zeros fp16 [N, K/g] all 8.0)``; the signed code is ``codes - 8``.
    """
    N, K, G = _check(W, g)
    Wg = W.reshape(N, G, g)
    # Q6: s32 = max|x| / 7 in fp32, stored scale as in Q3.
    amax = np.abs(Wg).max(axis=2)
    s32 = amax / np.float32(7.0)
    s_h = _stored_scale(s32)
    s = s_h.astype(np.float32)
    q = np.clip(np.rint(Wg / s[:, :, None]), -8.0, 7.0)
    codes = (q + np.float32(8.0)).astype(np.uint8).reshape(N, K)
    zeros = np.full((N, G), 8.0, dtype=np.float16)
    return codes, s_h, zeros


def quantize(W: np.ndarray, g: int, scheme: int = ASYM):
    """Dispatch on the scheme constant (``ASYM`` or ``SYM``)."""
    if scheme == ASYM:
        return quantize_asym(W, g)
    if scheme == SYM:
        return quantize_sym(W, g)
    raise ValueError(f"unknown scheme {scheme}")


def pack(codes: np.ndarray) -> np.ndarray:
    """Pack codes ``[N, K]`` (values 0..15) into int32 words ``[N, K/8]`` (R9)."""
    codes = np.asarray(codes)
    N, K = codes.shape
    if K % 8 != 0:
        raise ValueError("K must be a multiple of 8")
    if codes.min(initial=0) < 0 or codes.max(initial=0) > 15:
        raise ValueError("codes must lie in [0, 15]")
    c = codes.astype(np.uint32).reshape(N, K // 8, 8)
    words = np.zeros((N, K // 8), dtype=np.uint32)
    for i in range(8):
        words |= c[:, :, i] << np.uint32(4 * i)
    return words.view(np.int32)


def unpack(qweight: np.ndarray) -> np.ndarray:
    """Inverse of :func:`pack`: int32 words ``[N, K/8]`` -> codes uint8 ``[N, K]``."""
    w = np.ascontiguousarray(qweight).view(np.uint32)
    N, KW = w.shape
    out = np.empty((N, KW, 8), dtype=np.uint8)
    for i in range(8):
        out[:, :, i] = (w >> np.uint32(4 * i)) & np.uint32(0xF)
    return out.reshape(N, KW * 8)


def dequantize(qweight: np.ndarray, scales: np.ndarray, zeros, g: int) -> np.ndarray:
    """``W_hat[n, k] = s[n, k//g] * (u[n, k] - z[n, k//g])`` in float64 (exact).

    ``zeros=None`` means the symmetric implicit zero point 8 (R8).
    """
    u = unpack(qweight).astype(np.float64)
    N, K = u.shape
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    if s.shape != (N, K // g):
        raise ValueError("scales shape mismatch")
    if zeros is None:
        z = np.full_like(s, 8.0)
    else:
        z = np.asarray(zeros, dtype=np.float16).astype(np.float64)
        if z.shape != s.shape:
            raise ValueError("zeros shape mismatch")
    s_full = np.repeat(s, g, axis=1)
    z_full = np.repeat(z, g, axis=1)
    return s_full * (u - z_full)
