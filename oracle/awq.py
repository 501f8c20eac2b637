"""AWQ: activation-aware per-input-channel scaling before group-wise INT4 RTN quantization
(CPU oracle).  Test infrastructure (see the package docstring).

Method (restated from page "推理优化中“用精度换性能“的核心技术：量化", section 五 AWQ:
5.1 channel salience, 5.2 channel scaling and grid search; page "量化实战深入（GPTQ / AWQ /
SmoothQuant / KV 量化）", 4.2):

* a channel's importance comes from its mean activation magnitude on calibration data
  (5.1: ``x_i`` is the mean of ``|x|`` over the calibration tokens of input channel ``i``);
* salient channels are protected by an exactly equivalent rescaling of the layer,
  ``W x = (W diag(1/s)) (diag(s) x)`` (5.2): the quantizer sees ``W diag(1/s)`` and the
  activations are multiplied by ``s`` (in practice folded into the previous operator);
* the scales are chosen by a grid search over candidates, keeping the one whose quantized
  layer has the smallest output error on the calibration data (5.2);
* the quantizer itself is the plain group-wise RTN of ``quant.py`` (5.3).

Readings where the pages leave a step open or contradict themselves:

* A1 candidates: ``s(a) = r ** (a / 4)`` for ``a = -4 .. 4`` (nine points, ``a = 0`` is plain
  RTN), ``r_i = xc_i / sqrt(max xc * min xc)`` with ``xc_i = max(x_i, 1e-6 * max x)``: every
  channel gets its own candidate value from one exponent shared by all channels (5.1 gives
  the importance as a power of the channel's activation magnitude), and the search picks
  the exponent whose quantized layer has the smallest output error.  5.2 also calls the
  search per-channel; a literal independent choice per channel (each channel alone, the
  others unscaled) is a different method, compared in the tests: the channels of a group
  share one quantization grid, so independently chosen values combine badly and keep only
  a small part of the error reduction (0.6-0.9 of RTN against 0.2-0.3 for the shared
  exponent on outlier data), and its cost (an output-error evaluation per channel and
  candidate) does not fit the page's "seconds for a 4096-channel layer".  The page says
  salient channels get ``s_i > 1`` (weights shrunk) but also that the error of the quantized
  layer picks the scale; the grid spans both directions (``a < 0`` enlarges the salient
  channels' weights) and the measured error decides.  Exponents are quarters so the
  candidates come from IEEE-exact fp32 operations only (square roots, products, one
  division), reproducible bit for bit.
* A2 the statistic is the activation magnitude alone (the weight factor of 5.1's salience
  formula does not enter the candidate scales).
* A3 ``W diag(1/s)`` is the fp32 quotient ``W / s`` (one rounding); the quantized layer's
  effective weight is ``s * s_g (q - z)``; the output error is
  ``||X W^T - X diag(s) (W_hat')^T||_F^2 = ||X E^T||_F^2`` with ``E = W - diag-scaled
  W_hat``, evaluated in fp64; ties between candidates go to the first in grid order.
* A4 activations for the quantized layer are ``fp16/bf16(x * s)`` (one rounding), as a
  preceding operator would produce them.
"""

from __future__ import annotations

import numpy as np

from .formats import round_to_bf16_bits, round_to_f16
from .linear import _x64
from .quant import quantize, dequantize, pack

__all__ = ["channel_mean_abs", "candidate_ratio", "candidate_scales", "GRID", "awq_search",
           "awq_loss", "scale_activations"]

GRID = tuple(range(-4, 5))           # exponents a / 4


def channel_mean_abs(X, dtype: int) -> np.ndarray:
    """5.1: mean ``|x|`` of every input channel over the calibration tokens (fp32 of the
    fp64 mean)."""
    x = _x64(X, dtype)
    return (np.abs(x).sum(axis=0) / x.shape[0]).astype(np.float32)


def candidate_ratio(xmean) -> np.ndarray:
    """A1: ``r_i = xc_i / sqrt(max xc * min xc)``, fp32, IEEE operations in this order."""
    x = np.asarray(xmean, dtype=np.float32)
    mx = np.float32(x.max())
    xc = np.maximum(x, np.float32(1e-6) * mx)
    norm = np.sqrt(np.float32(mx) * np.float32(xc.min()))
    return (xc / norm).astype(np.float32)


def candidate_scales(xmean, a: int) -> np.ndarray:
    """A1: ``s = r ** (a / 4)``: q = sqrt(sqrt(r)); |a| left-to-right products of q; a < 0
    takes the reciprocal; all fp32 with round-to-nearest-even."""
    r = candidate_ratio(xmean)
    q = np.sqrt(np.sqrt(r))
    s = np.ones_like(q)
    for _ in range(abs(a)):
        s = (s * q).astype(np.float32)
    if a < 0:
        s = (np.float32(1.0) / s).astype(np.float32)
    return s


def _quantize_scaled(W, s, g, scheme):
    Wp = (np.asarray(W, dtype=np.float32) / s[None, :]).astype(np.float32)     # A3
    return quantize(Wp, g, scheme)


def awq_loss(X, dtype: int, W, s, codes, scales, zeros, g: int) -> float:
    """A3: ``||X E^T||_F^2`` with ``E = W - s * dequant`` (fp64)."""
    w_hat = dequantize(pack(codes), scales, zeros, g) * np.asarray(s, dtype=np.float64)[None, :]
    E = np.asarray(W, dtype=np.float64) - w_hat
    x = _x64(X, dtype)
    return float(np.sum((x @ E.T) ** 2))


def awq_search(W, X, dtype: int, xmean, g: int, scheme: int):
    """Grid search (5.2).  Returns ``(best_index, losses[9], s_best fp32 [K], codes,
    scales, zeros)``; ``best_index`` indexes ``GRID``."""
    losses, results = [], []
    for a in GRID:
        s = candidate_scales(xmean, a)
        codes, sc, z = _quantize_scaled(W, s, g, scheme)
        losses.append(awq_loss(X, dtype, W, s, codes, sc, z, g))
        results.append((s, codes, sc, z))
    best = int(np.argmin(losses))               # first minimum
    s, codes, sc, z = results[best]
    return best, np.array(losses), s, codes, sc, z


def scale_activations(X, dtype: int, s) -> np.ndarray:
    """A4: ``x * s`` per channel, rounded once to the activation dtype (fp16 array or bf16
    bit patterns)."""
    # the fp64 product of a 16-bit value and an fp32 scale is exact: one rounding below
    x = _x64(X, dtype) * np.asarray(s, dtype=np.float32).astype(np.float64)[None, :]
    if dtype == 0:
        return round_to_f16(x)
    return round_to_bf16_bits(x)
