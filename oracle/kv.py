"""KV-cache quantization (KV8 / KV4, per token) and the decode attention that reads the
quantized cache (CPU oracle).  Test infrastructure (see the package docstring).

Method (restated from the pages):

* the KV cache can outgrow the weights at long context and high concurrency; quantizing
  it (KV8, KV4) raises the number of requests that fit; keys and values are quantized
  separately, usually per token or per channel (page "量化实战深入（GPTQ / AWQ / SmoothQuant /
  KV 量化）", 六 KV Cache 量化); it is the usual companion of W4A16 ("W4A16 + KV INT8", page
  "Quantization & Acceleration: 解释 W8A8 与 W4A16 的差异与取舍", 深度剖析 ③; page
  "LLM 量化中 W4A16 表示什么…", on W4A16 not shrinking the KV cache by itself);
* the quantizers are the affine ones of the pages (symmetric absmax for 8 bits,
  asymmetric min/max for 4 bits), as in ``quant.py``;
* the consumer is decode attention: one new query per head against the cached keys and
  values, ``softmax(q K^T / sqrt(D)) V``.

Readings:

* KV1 granularity: one scale (and for KV4 one zero point) per (head, token) row of ``D``
  values ("per token"); layout ``[H, T, D]`` (each head's tokens contiguous).
* KV2 KV8: ``s = fp16(fp32(max|x| / 127))`` (1.0 if 0), codes ``clamp(rint(x / s), -127,
  127)`` in int8 (fp32 arithmetic with the stored scale, as R4-R5 of ``quant.py``); KV4:
  the asymmetric RTN of ``quant.py`` with ``g = D`` (codes [0, 15] packed 8 per 32-bit word).
* KV3 attention: fp64 reference of ``softmax(q . k_t / sqrt(D)) v_t`` over the dequantized
  rows, query heads ``h`` reading kv head ``h // (Hq / Hkv)`` (grouped-query attention
  when ``Hq > Hkv``); output rounded once to the query dtype.
"""

from __future__ import annotations

import numpy as np

from .formats import F16, round_to_bf16_bits, round_to_f16, round_to_format
from .linear import _x64
from .quant import ASYM, dequantize, pack, quantize

__all__ = ["quantize_kv8", "quantize_kv4", "dequant_kv8", "dequant_kv4", "attention_decode_f64",
           "attention_decode"]


def quantize_kv8(x, dtype: int):
    """KV2: ``x [H, T, D]`` (fp16 / bf16 bits) -> ``(codes int8 [H, T, D], scales fp16 [H, T])``."""
    v = _x64(np.asarray(x).reshape(-1, np.asarray(x).shape[-1]), dtype).astype(np.float32)
    amax = np.abs(v).max(axis=1)
    s32 = (amax / np.float32(127.0)).astype(np.float32)
    s_h = round_to_format(s32.astype(np.float64), F16)
    s_h = np.where(s_h == 0.0, 1.0, s_h).astype(np.float16)
    s = s_h.astype(np.float32)
    q = np.clip(np.rint(v / s[:, None]), -127.0, 127.0).astype(np.int8)
    H, T, D = np.asarray(x).shape
    return q.reshape(H, T, D), s_h.reshape(H, T)


def quantize_kv4(x, dtype: int):
    """KV2: asymmetric RTN per row (``g = D``) -> ``(words int32 [H, T, D/8], scales fp16
    [H, T], zeros fp16 [H, T])``."""
    H, T, D = np.asarray(x).shape
    v = _x64(np.asarray(x).reshape(-1, D), dtype).astype(np.float32)
    codes, s, z = quantize(v, D, ASYM)
    return pack(codes).reshape(H, T, D // 8), s.reshape(H, T), z.reshape(H, T)


def dequant_kv8(codes, scales) -> np.ndarray:
    return np.asarray(codes, np.float64) * np.asarray(scales, np.float16).astype(np.float64)[..., None]


def dequant_kv4(words, scales, zeros) -> np.ndarray:
    H, T, DW = np.asarray(words).shape
    D = DW * 8
    w = dequantize(np.asarray(words).reshape(H * T, DW), np.asarray(scales).reshape(H * T, 1),
                   np.asarray(zeros).reshape(H * T, 1), D)
    return w.reshape(H, T, D)


def attention_decode_f64(q, dtype: int, Kd: np.ndarray, Vd: np.ndarray, T: int) -> np.ndarray:
    """KV3: ``out [Hq, D] = softmax(q K^T / sqrt(D)) V`` in fp64 over the first ``T`` tokens
    of the dequantized caches ``Kd, Vd [Hkv, Tmax, D]``."""
    qd = _x64(q, dtype)
    Hq, D = qd.shape
    Hkv = Kd.shape[0]
    grp = Hq // Hkv
    out = np.zeros((Hq, D))
    for h in range(Hq):
        k = Kd[h // grp, :T]
        v = Vd[h // grp, :T]
        sc = k @ qd[h] / np.sqrt(D)
        p = np.exp(sc - sc.max())
        out[h] = (p / p.sum()) @ v
    return out


def attention_decode(q, dtype: int, Kd, Vd, T: int) -> np.ndarray:
    """:func:`attention_decode_f64` rounded once to the query dtype."""
    o = attention_decode_f64(q, dtype, Kd, Vd, T)
    return round_to_f16(o) if dtype == 0 else round_to_bf16_bits(o)
