"""CPU oracle for the W4A16 weight-only linear layer -- TEST INFRASTRUCTURE ONLY.

This package is the correctness authority for the HIP library.  It is a plain,
slow, obviously-correct NumPy implementation written from the pages' statement
of the method.  It shares no code with the GPU path and never imports it; only
``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import or run anything in here.  The product path
(``w4a16_dequant_gemm_amd``) must never route through it.

What it computes (sources are the five pages on W4A16 quantization):

* the affine quantizer ``q = round(x/s) + z`` and its inverse ``x ~ s(q - z)``
  (page "量化实战深入（GPTQ / AWQ / SmoothQuant / KV 量化）", §二 量化的数学本质;
  page "推理优化中“用精度换性能“的核心技术：量化", §2.3 核心公式);
* asymmetric min/max scaling ``s = (max - min)/(2^b - 1)``, ``z = round(-min/s)``
  and symmetric absmax scaling ``s = max|x|/(2^(b-1) - 1)``, ``z = 0``
  (same page, §3.3 对称量化 vs 非对称量化; page 3 §二, absmax);
* group-wise granularity with one 16-bit scale and one 16-bit zero point per
  group of input columns (page 4, §3.4 量化粒度, group-wise);
* INT4 code ranges [0, 15] (unsigned) and [-8, 7] (signed) (page 4, §2.2);
* the weight-only linear layer: INT4 weights are dequantized and multiplied by
  16-bit activations (page 4, §3.2 Weight-only 量化; page
  "大模型推理中 Weight-only、W8A8 和 FP8 量化有什么区别？如何选型？", §二).

* GPTQ (``gptq.py``): ``H = 2 X^T X`` from calibration activations and the column-wise
  quantization with the optimal-brain-surgeon compensation of the columns still free
  (page 4, section 四 GPTQ; page "量化实战深入（GPTQ / AWQ / SmoothQuant / KV 量化）", 4.1).

* AWQ (``awq.py``): per-input-channel rescaling ``W x = (W diag(1/s)) (diag(s) x)`` with
  ``s`` from the channels' mean activation magnitude, chosen by a grid search on the
  quantized layer's output error (page 4, section 五 AWQ).

* W8A8 with SmoothQuant (``w8a8.py``): the smoothing ``Y = (X/s)(sW)`` with
  ``s_j = max|X_j|^alpha / max|W_j|^(1-alpha)``, per-channel INT8 weights, per-token dynamic
  INT8 activations and the integer product with a float epilogue (page 2, section 三;
  page 4, section 六; page 1 on per-token dynamic quantization).

* KV-cache quantization (``kv.py``): per-token KV8 / KV4 and the decode attention that
  reads the quantized cache (page 3, section 六 KV Cache 量化; page 1 on W4A16 + KV INT8).

* W8A16 (``w8a16.py``): the same group-wise weight-only layer with 8-bit codes, four per
  32-bit word (page 4, section 3.3 prints the 8-bit asymmetric divisor 255; page 2, section
  二 and page 1 on INT8 weight-only quantization).

Readings where the pages are silent (tie rule, clamping, which scale feeds the
zero point, nibble order, symmetric storage) are listed in the docstrings of
``quant.py``, ``linear.py``, ``gptq.py``, ``awq.py``, ``w8a8.py``, ``kv.py`` and ``w8a16.py``.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against hand-worked vectors, closed forms, exact rational arithmetic or an
independent library routine; none is "parity unpinned".
"""

from .formats import (
    bf16_bits_to_f64,
    f16_to_f64,
    round_to_bf16_bits,
    round_to_f16,
    round_to_format,
    round_fraction_to_format,
    F16,
    BF16,
)
from .quant import (
    ASYM,
    SYM,
    quantize,
    quantize_asym,
    quantize_sym,
    pack,
    unpack,
    dequantize,
)
from .linear import linear_ref, linear_ref_f64, linear_exact

__all__ = [
    "bf16_bits_to_f64", "f16_to_f64", "round_to_bf16_bits", "round_to_f16",
    "round_to_format", "round_fraction_to_format", "F16", "BF16",
    "ASYM", "SYM", "quantize", "quantize_asym", "quantize_sym", "pack", "unpack",
    "dequantize", "linear_ref", "linear_ref_f64", "linear_exact",
]
