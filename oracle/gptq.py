"""GPTQ: column-by-column INT4 quantization with second-order error compensation
(CPU oracle).  Test infrastructure (see the package docstring).

Method (restated from page "推理优化中“用精度换性能“的核心技术：量化", section 四
"GPTQ：逐列贪心补偿的 INT4 权重量化", 4.2 算法核心 and 4.4 激活顺序与分组; also page
"量化实战深入（GPTQ / AWQ / SmoothQuant / KV 量化）", 4.1 GPTQ):

* the calibration inputs ``X [n, K]`` of the layer give ``H = 2 X^T X`` (4.2 step 1,
  4.3);
* the columns ``i = 0 .. K-1`` of ``W [N, K]`` are quantized in their natural order
  (4.4); the quantization error of column ``i`` is ``dw = W[:, i] - W_hat[:, i]``;
* every not-yet-quantized column ``j > i`` is corrected by
  ``W[:, j] -= dw * Hinv[i, j] / Hinv[i, i]`` (4.2 step 2c), the optimal-brain-surgeon
  update that keeps the layer output error ``||X (W - W_hat)^T||`` minimal over the
  columns still free;
* group-wise scales and zero points (one per ``g`` columns of a row, 4.4) are those of
  the RTN quantizer (``quant.py``).

Readings where the pages leave a step open:

* G1 ``Hinv`` in step 2c is the inverse Hessian of the columns not yet quantized: after
  column ``i`` is fixed it is removed from the problem (``Hinv`` loses row and column
  ``i`` through the Schur-complement update
  ``Hinv -= Hinv[:, i] Hinv[i, :] / Hinv[i, i]``).  This is the optimal-brain-surgeon
  update the page names (4.2) and what the Cholesky factor it mentions (4.4) provides:
  with ``H^-1 = U^T U`` (``U`` upper triangular), ``U[i, j] / U[i, i]`` equals that
  running ``Hinv[i, j] / Hinv[i, i]``.  ``gptq_obs`` runs the update as written;
  ``gptq_quantize`` uses ``U`` (identical up to rounding; pinned against each other).
* G2 the group parameters are computed when the loop reaches the group's first column,
  from the group's current (already compensated) weights, rounded to fp32, with the RTN
  rules of ``quant.py``; every column of the group is then quantized with them.
* G3 the error uses the compensated fp64 weight: ``dw = W'[:, i] - s (q - z)``; the code
  itself follows the fp32 RTN arithmetic on ``fp32(W'[:, i])``.
* G4 an optional damping ``H += damp * mean(diag H) * I`` keeps ``H`` invertible when the
  calibration set is small; the pages do not mention it (``damp = 0`` reproduces them).
* G5 all compensation arithmetic is fp64.
"""

from __future__ import annotations

import numpy as np

from .linear import _x64
from .quant import ASYM, SYM, quantize

__all__ = ["hessian", "damp_hessian", "inverse_cholesky_upper", "gptq_quantize", "gptq_obs",
           "layer_error"]


def hessian(X, dtype: int) -> np.ndarray:
    """``H = 2 X^T X`` in fp64 from 16-bit activations ``X [n, K]`` (page 4, 4.2 step 1)."""
    x = _x64(X, dtype)
    return 2.0 * (x.T @ x)


def damp_hessian(H: np.ndarray, damp: float) -> np.ndarray:
    """G4: ``H + damp * mean(diag H) * I``."""
    H = np.array(H, dtype=np.float64, copy=True)
    if damp:
        H[np.diag_indices_from(H)] += damp * np.mean(np.diag(H))
    return H


def inverse_cholesky_upper(H: np.ndarray) -> np.ndarray:
    """Upper-triangular ``U`` with ``H^-1 = U^T U`` (G1; library inverse and Cholesky)."""
    Hinv = np.linalg.inv(H)
    Hinv = 0.5 * (Hinv + Hinv.T)
    return np.linalg.cholesky(Hinv).T


def _group_params(Wcur: np.ndarray, scheme: int):
    """G2: RTN parameters of one group from its current weights, rounded to fp32."""
    w32 = Wcur.astype(np.float32)
    _, s_h, z_h = quantize(w32, w32.shape[1], scheme)
    return s_h[:, 0], z_h[:, 0]


def _code(x64: np.ndarray, s_h: np.ndarray, z_h: np.ndarray, scheme: int) -> np.ndarray:
    """G3: the RTN code of ``fp32(x)`` with the stored group parameters (fp32 RNE)."""
    x = x64.astype(np.float32)
    s = s_h.astype(np.float32)
    if scheme == ASYM:
        q = np.clip(np.rint(x / s) + z_h.astype(np.float32), 0.0, 15.0)
    elif scheme == SYM:
        q = np.clip(np.rint(x / s), -8.0, 7.0) + np.float32(8.0)
    else:
        raise ValueError(f"unknown scheme {scheme}")
    return q.astype(np.uint8)


def _run(W, g: int, scheme: int, coef, trace=None, pre=None):
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    if g <= 0 or K % g:
        raise ValueError(f"group size {g} must divide K={K}")
    Wc = W.astype(np.float64)
    codes = np.zeros((N, K), dtype=np.uint8)
    scales = np.zeros((N, K // g), dtype=np.float16)
    zeros = np.zeros((N, K // g), dtype=np.float16)
    for i in range(K):
        if i % g == 0:
            s_h, z_h = _group_params(Wc[:, i:i + g], scheme)
            scales[:, i // g] = s_h
            zeros[:, i // g] = z_h
        if pre is not None:
            pre[:, i] = Wc[:, i]
        q = _code(Wc[:, i], s_h, z_h, scheme)
        codes[:, i] = q
        w_hat = s_h.astype(np.float64) * (q.astype(np.float64) - z_h.astype(np.float64))
        dw = Wc[:, i] - w_hat
        c = coef(i)                      # Hinv[i, i+1:] / Hinv[i, i]
        Wc[:, i + 1:] -= np.outer(dw, c)
        Wc[:, i] = w_hat
        if trace is not None:
            trace.append(Wc.copy())
    return codes, scales, zeros


def gptq_quantize(W, U: np.ndarray, g: int, scheme: int = ASYM, trace=None, pre=None):
    """GPTQ with the Cholesky factor ``U`` of ``H^-1`` (``H^-1 = U^T U``, G1).

    Returns ``(codes uint8 [N, K], scales fp16 [N, K/g], zeros fp16 [N, K/g])`` in the
    layout of ``quant.quantize`` (pack with ``quant.pack``).  ``trace``, if a list,
    receives the compensated weights after every column (with the quantized columns
    replaced by their dequantized values); ``pre``, if an fp64 ``[N, K]`` array, receives
    the value each weight had when it was quantized.  Rows are independent given ``U``.
    """
    U = np.asarray(U, dtype=np.float64)
    return _run(W, g, scheme, lambda i: U[i, i + 1:] / U[i, i], trace, pre)


def gptq_obs(W, H: np.ndarray, g: int, scheme: int = ASYM, trace=None):
    """GPTQ exactly as the page writes step 2c, with the running inverse Hessian of the
    columns still free (G1): O(K^3), for small problems."""
    Hinv = np.linalg.inv(np.asarray(H, dtype=np.float64))
    state = {"Hinv": Hinv}

    def coef(i):
        Hi = state["Hinv"]
        c = Hi[i, i + 1:] / Hi[i, i]
        # remove column i from the problem (Schur complement)
        state["Hinv"] = Hi - np.outer(Hi[:, i], Hi[i, :]) / Hi[i, i]
        return c

    return _run(W, g, scheme, coef, trace)


def layer_error(X, dtype: int, W, W_hat) -> float:
    """``||X (W - W_hat)^T||_F^2`` in fp64: the layer output error GPTQ minimizes."""
    x = _x64(X, dtype)
    d = np.asarray(W, dtype=np.float64) - np.asarray(W_hat, dtype=np.float64)
    return float(np.sum((x @ d.T) ** 2))
