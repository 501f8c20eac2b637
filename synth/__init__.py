"""Seeded synthetic inputs for the W4A16 linear layer.

This module only draws random numbers and casts them to the input formats; it
holds none of the layer's arithmetic (no quantization, packing or products).
Both the CPU oracle's callers and the GPU path's callers take their inputs from
here, so the two sides see identical bytes.

Workloads (shapes follow 7B- and 70B-class decoder layers; the pages reason
about Llama-2-70B decode and 7B/8B decode, see page
"推理优化中“用精度换性能“的核心技术：量化", §一, and page
"大模型推理中 Weight-only、W8A8 和 FP8 量化有什么区别？如何选型？", §六):

* weights ``W`` fp32 ~ N(0, sigma^2), optionally with a fraction of entries
  multiplied by a factor (weight outliers);
* activations ``X`` drawn fp32 ~ N(0, 1), optionally with a fraction of input
  channels (the same channels for every row) multiplied by a factor -- the
  pages describe fixed activation channels 10-100x larger than the rest
  (page 4, §6.1) -- then rounded to fp16 or bf16 (round-to-nearest-even).

Host generators use NumPy's PCG64 (``default_rng``); the device generators used
for large benchmark layers use torch's generator on the GPU and are a different
stream (parity at those sizes copies the device inputs back to the host).
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

FP16 = 0
BF16 = 1
ASYM = 0
SYM = 1


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest-even) and return the uint16 bit patterns."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounding = np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))
    return ((b + rounding) >> np.uint64(16)).astype(np.uint16)


def seeds(config: int, layer: int = 0) -> tuple[int, int]:
    """Fixed seeds: weights ``1000 + 10*config + layer``, activations that + 5."""
    sw = 1000 + 10 * config + layer
    return sw, sw + 5


def weights(N: int, K: int, sigma: float, seed: int,
            outlier_frac: float = 0.0, outlier_mult: float = 1.0) -> np.ndarray:
    """fp32 ``[N, K]`` ~ N(0, sigma^2); ``round(outlier_frac*N*K)`` entries,
    chosen without replacement, are multiplied by ``outlier_mult``."""
    rng = np.random.default_rng(seed)
    W = rng.standard_normal((N, K), dtype=np.float32) * np.float32(sigma)
    n_out = int(round(outlier_frac * N * K))
    if n_out:
        idx = rng.choice(N * K, size=n_out, replace=False)
        flat = W.reshape(-1)
        flat[idx] *= np.float32(outlier_mult)
    return W


def activations(M: int, K: int, dtype: int, seed: int,
                outlier_frac: float = 0.0, outlier_mult: float = 1.0) -> np.ndarray:
    """``[M, K]`` activations: fp16 array, or bf16 as uint16 bit patterns."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K), dtype=np.float32)
    n_ch = int(round(outlier_frac * K))
    if n_ch:
        ch = rng.choice(K, size=n_ch, replace=False)
        X[:, ch] *= np.float32(outlier_mult)
    if dtype == FP16:
        return X.astype(np.float16)
    if dtype == BF16:
        return f32_to_bf16_bits(X)
    raise ValueError(f"unknown dtype {dtype}")


def calibration(n: int, K: int, dtype: int, seed: int, n_factors: int = 16,
                factor_scale: float = 0.5, outlier_frac: float = 0.01,
                outlier_mult: float = 10.0) -> np.ndarray:
    """Calibration activations ``[n, K]`` with correlated channels: i.i.d. N(0, 1) plus
    ``n_factors`` shared Gaussian factors (loadings ~ N(0, factor_scale^2)); a fraction
    ``outlier_frac`` of the channels (at least one) is multiplied by ``outlier_mult``.
    fp16 array, or bf16 bit patterns."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((n, K), dtype=np.float32)
    F = rng.standard_normal((n, n_factors), dtype=np.float32)
    L = rng.standard_normal((n_factors, K), dtype=np.float32) * np.float32(factor_scale)
    X += F @ L
    n_ch = max(1, int(round(outlier_frac * K))) if outlier_frac > 0 else 0
    if n_ch:
        ch = rng.choice(K, size=n_ch, replace=False)
        X[:, ch] *= np.float32(outlier_mult)
    if dtype == FP16:
        return X.astype(np.float16)
    if dtype == BF16:
        return f32_to_bf16_bits(X)
    raise ValueError(f"unknown dtype {dtype}")


@dataclass(frozen=True)
class Case:
    """One W4A16 linear problem: shapes, dtype, group size, scheme, distributions."""
    config: int
    M: int
    K: int
    N: int
    g: int
    scheme: int = ASYM
    dtype: int = FP16
    w_sigma: float = 0.02
    w_outlier_frac: float = 0.0
    w_outlier_mult: float = 1.0
    x_outlier_frac: float = 0.0
    x_outlier_mult: float = 1.0
    layer: int = 0
    tags: tuple = field(default_factory=tuple)

    @property
    def name(self) -> str:
        dt = "f16" if self.dtype == FP16 else "bf16"
        sc = "asym" if self.scheme == ASYM else "sym"
        return f"C{self.config}_M{self.M}_K{self.K}_N{self.N}_g{self.g}_{sc}_{dt}"

    def make(self):
        """Host inputs ``(W fp32 [N, K], X [M, K])`` for this case."""
        sw, sx = seeds(self.config, self.layer)
        W = weights(self.N, self.K, self.w_sigma, sw, self.w_outlier_frac, self.w_outlier_mult)
        X = activations(self.M, self.K, self.dtype, sx, self.x_outlier_frac, self.x_outlier_mult)
        return W, X


SHAPES_7B = [(4096, 4096), (4096, 11008), (11008, 4096)]          # (K, N)
SHAPES_70B = [(8192, 8192), (8192, 28672), (28672, 8192)]          # (K, N)
LAYER_7B = [("q", 4096, 4096), ("k", 4096, 4096), ("v", 4096, 4096), ("o", 4096, 4096),
            ("gate", 4096, 11008), ("up", 4096, 11008), ("down", 11008, 4096)]  # (name, K, N)


def config_cases(config: int) -> list[Case]:
    """The single-layer problems of workload family ``config`` (1..4)."""
    if config == 1:     # single layer, M=1, 4096x4096, g=128 asym, fp16
        return [Case(1, 1, 4096, 4096, 128)]
    if config == 2:     # decode batch sweep on 7B-like shapes
        return [Case(2, M, K, N, 128) for M in (1, 2, 4, 8, 16) for (K, N) in SHAPES_7B]
    if config == 3:     # 70B-like decode, bf16 with activation and weight outliers
        return [Case(3, M, K, N, 128, ASYM, BF16, 0.015, 0.001, 20.0, 0.01, 100.0)
                for M in (1, 4, 16) for (K, N) in SHAPES_70B]
    if config == 4:     # prefill / compute-bound crossover
        return [Case(4, M, K, N, g, sc, FP16)
                for M in (256, 1024, 4096) for (K, N) in [(4096, 11008), (11008, 4096)]
                for g in (64, 128) for sc in (SYM, ASYM)]
    raise ValueError(f"no single-layer cases for config {config}")


def stack_cases(M: int, per_channel: bool) -> list[Case]:
    """The 224 linears of a 32-layer 7B-shaped decode step (bf16, asym)."""
    out = []
    for layer in range(32):
        for j, (_, K, N) in enumerate(LAYER_7B):
            out.append(Case(5, M, K, N, K if per_channel else 128, ASYM, BF16,
                            layer=layer * 7 + j))
    return out


# ---------------------------------------------------------------- device side
def weights_device(N: int, K: int, sigma: float, seed: int, device="cuda",
                   outlier_frac: float = 0.0, outlier_mult: float = 1.0):
    """fp32 ``[N, K]`` on the GPU from torch's seeded device generator."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    W = torch.randn((N, K), generator=gen, device=device, dtype=torch.float32)
    W.mul_(sigma)
    n_out = int(round(outlier_frac * N * K))
    if n_out:
        idx = torch.randperm(N * K, generator=gen, device=device)[:n_out]
        W.view(-1)[idx] *= outlier_mult
    return W


def calibration_device(n: int, K: int, dtype: int, seed: int, device="cuda", **kw):
    """:func:`calibration` uploaded as a torch tensor (fp16, or bf16 viewed from the bits)."""
    import torch
    X = calibration(n, K, dtype, seed, **kw)
    if dtype == FP16:
        return torch.from_numpy(X).to(device)
    return torch.from_numpy(X.view(np.int16)).to(device).view(torch.bfloat16)


def activations_device(M: int, K: int, dtype: int, seed: int, device="cuda",
                       outlier_frac: float = 0.0, outlier_mult: float = 1.0):
    """``[M, K]`` fp16 or bf16 activations on the GPU (torch's RNE casts)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    X = torch.randn((M, K), generator=gen, device=device, dtype=torch.float32)
    n_ch = int(round(outlier_frac * K))
    if n_ch:
        ch = torch.randperm(K, generator=gen, device=device)[:n_ch]
        X[:, ch] *= outlier_mult
    return X.to(torch.float16 if dtype == FP16 else torch.bfloat16)
