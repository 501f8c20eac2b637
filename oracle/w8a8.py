"""W8A8 with SmoothQuant: INT8 weights and INT8 activations for the integer matrix units,
with the activations' outlier channels migrated into the weights (CPU oracle).  Test
infrastructure (see the package docstring).

Method (restated from the pages):

* W8A8 quantizes both operands to INT8 so the product runs on INT8 matrix units; the
  activations need per-token dynamic scales because their range changes from token to
  token (page "Quantization & Acceleration: 解释 W8A8 与 W4A16 的差异与取舍", 数学机理 (1)
  and 深度剖析 ④; page "大模型推理中 Weight-only、W8A8 和 FP8 量化有什么区别？如何选型？",
  section 三);
* SmoothQuant rescales every input channel exactly, ``Y = (X / s) (s W)`` (same page,
  section 三; page "推理优化中“用精度换性能“的核心技术：量化", 6.2), with
  ``s_j = max|X_j|^alpha / max|W_j|^(1 - alpha)`` and ``alpha = 0.5`` (6.2);
* weights use per-channel scales (one per output channel, 3.4), symmetric absmax INT8:
  ``s = max|x| / 127``, codes in [-128, 127] (3.3, 2.2); activations one symmetric scale
  per token (3.4 per-token).

Readings:

* Q8-1 orientation: ``W [N, K]`` with input channels along K, so ``s W`` scales column j of
  ``W`` by ``s_j`` and ``X / s`` divides activation column j (the pages' ``diag(s)^-1 x``).
* Q8-2 ``alpha = a / 4`` (a in 0..4, default 2): ``v^(a/4)`` is formed from fp32 square
  roots and products (as in ``awq.py``), so the smoothing factors are exact IEEE results;
  a channel whose activation or weight maximum is 0 gets ``s_j = 1``.
* Q8-3 fp32 arithmetic in this order: ``w' = fp32(w * s_j)``, ``x' = fp32(x / s_j)``;
  scales ``fp32(amax / 127)`` (1.0 when ``amax == 0``); codes ``clamp(rint(v / scale),
  -128, 127)``; scales are stored as fp32.
* Q8-4 the product accumulates exactly in int32; the output is
  ``out(fp32(fp32(acc) * sx[m]) * sw[n])`` (one rounding per multiply, then one rounding
  to the activation dtype).
"""

from __future__ import annotations

import numpy as np

from .formats import round_to_bf16_bits, round_to_f16
from .linear import _x64

__all__ = ["smooth_factors", "quantize_weight", "quantize_act", "linear_int8", "w8a8_reference"]

_F127 = np.float32(127.0)


def _pow_quarters(v: np.ndarray, a: int) -> np.ndarray:
    """``v ** (a/4)`` for a in 0..4 from fp32 square roots and left-to-right products."""
    v = np.asarray(v, dtype=np.float32)
    q = np.sqrt(np.sqrt(v))
    out = np.ones_like(v)
    for _ in range(a):
        out = (out * q).astype(np.float32)
    return out


def smooth_factors(X, dtype: int, W, alpha_quarters: int = 2) -> np.ndarray:
    """Q8-2: ``s_j = max|X_j|^alpha / max|W_:,j|^(1-alpha)`` (fp32)."""
    if not 0 <= alpha_quarters <= 4:
        raise ValueError("alpha_quarters must be in 0..4")
    xmax = np.abs(_x64(X, dtype)).max(axis=0).astype(np.float32)    # exact (fp16/bf16 values)
    wmax = np.abs(np.asarray(W, dtype=np.float32)).max(axis=0)
    num = _pow_quarters(xmax, alpha_quarters)
    den = _pow_quarters(wmax, 4 - alpha_quarters)
    s = (num / np.where(den == 0, np.float32(1.0), den)).astype(np.float32)
    dead = (xmax == 0) | (wmax == 0)
    return np.where(dead, np.float32(1.0), s).astype(np.float32)


def _sym_int8(v: np.ndarray):
    """Row-wise symmetric absmax INT8 of fp32 rows (Q8-3)."""
    amax = np.abs(v).max(axis=1)
    sc = (amax / _F127).astype(np.float32)
    sc = np.where(sc == 0, np.float32(1.0), sc).astype(np.float32)
    q = np.clip(np.rint(v / sc[:, None]), -128.0, 127.0).astype(np.int8)
    return q, sc


def quantize_weight(W, s) -> tuple[np.ndarray, np.ndarray]:
    """Smoothed per-output-channel INT8 weights: ``(q int8 [N, K], sw fp32 [N])``."""
    Wp = (np.asarray(W, dtype=np.float32) * np.asarray(s, dtype=np.float32)[None, :]).astype(np.float32)
    return _sym_int8(Wp)


def quantize_act(X, dtype: int, s) -> tuple[np.ndarray, np.ndarray]:
    """Smoothed per-token INT8 activations: ``(q int8 [M, K], sx fp32 [M])``."""
    x = _x64(X, dtype).astype(np.float32)                       # exact
    xp = (x / np.asarray(s, dtype=np.float32)[None, :]).astype(np.float32)
    return _sym_int8(xp)


def linear_int8(qx, sx, qw, sw, dtype: int) -> np.ndarray:
    """Q8-4: exact integer product, fp32 epilogue, one rounding to the output dtype."""
    acc = np.asarray(qx, dtype=np.int64) @ np.asarray(qw, dtype=np.int64).T
    if np.abs(acc).max(initial=0) >= 2 ** 31:
        raise ValueError("int32 accumulator overflow")
    y = (acc.astype(np.float32) * np.asarray(sx, np.float32)[:, None]).astype(np.float32)
    y = (y * np.asarray(sw, np.float32)[None, :]).astype(np.float32)
    return round_to_f16(y.astype(np.float64)) if dtype == 0 else round_to_bf16_bits(y.astype(np.float64))


def w8a8_reference(X, dtype: int, W, s):
    """The whole W8A8 layer for given smoothing factors: ``(Y, qx, sx, qw, sw)``."""
    qw, sw = quantize_weight(W, s)
    qx, sx = quantize_act(X, dtype, s)
    return linear_int8(qx, sx, qw, sw, dtype), qx, sx, qw, sw
