"""The W4A16 linear layer ``Y = X . dequant(Wq)^T`` on the CPU (oracle).

Test infrastructure (see the package docstring).

The pages describe weight-only quantization as: load the INT4 weights,
dequantize them back to a 16-bit float, and run the matrix product against
16-bit activations, so the arithmetic stays 16-bit floating point while the
weight bytes shrink (page "推理优化中“用精度换性能“的核心技术：量化", §3.2
Weight-only 量化; page "大模型推理中 Weight-only、W8A8 和 FP8 量化有什么区别？
如何选型？", §二; page "LLM 量化中 W4A16 表示什么，它在权重位宽和激活精度上有什么
取舍？", 性能取决于 kernel).  The product is therefore exactly (up to summation
order) ``Y = X W_hat^T`` with ``W_hat`` from :func:`oracle.quant.dequantize`.

Readings:

* L-a the output dtype equals the activation dtype; accumulation is wide and
  the result is rounded once, round-to-nearest-even, to that dtype.
* L-b ``linear_ref`` forms ``Y`` in float64 (exact dequantization, one BLAS
  product) and rounds once; ``linear_exact`` does the same with exact
  rationals and is the pin for ``linear_ref`` on tiny shapes.
"""

from __future__ import annotations

from fractions import Fraction

import numpy as np

from .formats import (BF16, F16, bf16_bits_to_f64, f16_to_f64, round_fraction_to_format,
                      round_to_bf16_bits, round_to_f16)
from .quant import dequantize, unpack

FP16 = 0
BF16_DT = 1


def _x64(X, dtype: int) -> np.ndarray:
    if dtype == FP16:
        return f16_to_f64(X)
    if dtype == BF16_DT:
        return bf16_bits_to_f64(X)
    raise ValueError(f"unknown dtype {dtype}")


def linear_ref_f64(X, dtype: int, qweight, scales, zeros, g: int) -> np.ndarray:
    """Unrounded ``Y = X W_hat^T`` in float64.  ``X`` is fp16 or bf16 bits ``[M, K]``."""
    x = _x64(X, dtype)
    w = dequantize(qweight, scales, zeros, g)
    if x.shape[1] != w.shape[1]:
        raise ValueError("K mismatch")
    return x @ w.T


def linear_ref(X, dtype: int, qweight, scales, zeros, g: int) -> np.ndarray:
    """``Y`` rounded once to the activation dtype: fp16 array or bf16 bit patterns."""
    y = linear_ref_f64(X, dtype, qweight, scales, zeros, g)
    return round_to_f16(y) if dtype == FP16 else round_to_bf16_bits(y)


def linear_exact(X, dtype: int, qweight, scales, zeros, g: int) -> np.ndarray:
    """Exact-rational ``Y`` rounded once (tiny shapes only); same return types."""
    x = _x64(X, dtype)
    u = unpack(qweight)
    M, K = x.shape
    N = u.shape[0]
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    z = (np.full_like(s, 8.0) if zeros is None
         else np.asarray(zeros, dtype=np.float16).astype(np.float64))
    fmt = F16 if dtype == FP16 else BF16
    out = np.empty((M, N), dtype=np.float64)
    for m in range(M):
        xm = [Fraction(float(v)) for v in x[m]]
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                w = Fraction(float(s[n, k // g])) * (int(u[n, k]) - Fraction(float(z[n, k // g])))
                acc += xm[k] * w
            out[m, n] = round_fraction_to_format(acc, fmt)
    if dtype == FP16:
        return out.astype(np.float16)
    return round_to_bf16_bits(out)   # already on the bf16 grid: exact
