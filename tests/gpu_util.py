"""Helpers shared by the GPU parity tests (host <-> device marshalling, tolerances).

The oracle is the reference for every comparison; nothing here computes the method.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle
from synth import BF16, FP16

REL_FRO = 1e-3      # relative Frobenius error bound on Y
MAX_REL = 1e-2      # max |dY| <= MAX_REL * max |Y_ref|


def x_to_torch(X: np.ndarray, dtype: int) -> torch.Tensor:
    if dtype == FP16:
        return torch.from_numpy(np.ascontiguousarray(X)).cuda()
    t = torch.from_numpy(np.ascontiguousarray(X).view(np.int16)).cuda()
    return t.view(torch.bfloat16)


def y_to_f64(Y: torch.Tensor) -> np.ndarray:
    if Y.dtype == torch.float16:
        return Y.cpu().numpy().astype(np.float64)
    bits = Y.view(torch.int16).cpu().numpy().view(np.uint16)
    return oracle.bf16_bits_to_f64(bits)


def y_bits(Y: torch.Tensor) -> np.ndarray:
    return Y.view(torch.int16).cpu().numpy().view(np.uint16)


def ref_to_f64(Yref: np.ndarray, dtype: int) -> np.ndarray:
    return Yref.astype(np.float64) if dtype == FP16 else oracle.bf16_bits_to_f64(Yref)


def ref_bits(Yref: np.ndarray, dtype: int) -> np.ndarray:
    return Yref.view(np.uint16) if dtype == FP16 else Yref


def errors(y: np.ndarray, ref: np.ndarray) -> tuple[float, float]:
    d = y - ref
    fro = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.abs(d).max() / max(np.abs(ref).max(), 1e-300))
    return fro, mx


def assert_close(y: np.ndarray, ref: np.ndarray, what: str = "") -> None:
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    fro, mx = errors(y, ref)
    assert fro <= REL_FRO and mx <= MAX_REL, f"{what}: rel_fro={fro:.3e} max_rel={mx:.3e}"


def packed_from_torch(qw: torch.Tensor, s: torch.Tensor, z):
    qn = qw.cpu().numpy()
    sn = s.cpu().numpy()
    zn = None if z is None else z.cpu().numpy()
    return qn, sn, zn


def upload_packed(qweight: np.ndarray, scales: np.ndarray, zeros):
    qw = torch.from_numpy(np.ascontiguousarray(qweight)).cuda()
    s = torch.from_numpy(np.ascontiguousarray(scales.astype(np.float16))).cuda()
    z = None if zeros is None else torch.from_numpy(np.ascontiguousarray(zeros.astype(np.float16))).cuda()
    return qw, s, z
