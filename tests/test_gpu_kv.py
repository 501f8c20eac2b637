"""GPU parity of the KV-cache entry points against the CPU oracle, through the C ABI.

* quantization: KV8 / KV4 codes and fp16 scales (and zeros) bit-exact;
* decode attention over the quantized caches (one sequence, and a batch of sequences with
  their own lengths): the output dtype tolerance (relative
  Frobenius <= 1e-3, max |d| <= 1e-2 max |ref|) against the fp64 oracle over the oracle's own
  quantized caches, with one token (closed form: the value row), grouped heads, ragged T
  inside a larger cache, long contexts that need several splits, and the 7B-like decode.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import w4a16_dequant_gemm_amd as W4
from oracle import kv as KV
from synth import BF16, FP16, activations
from tests.gpu_util import assert_close, ref_to_f64, x_to_torch, y_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    W4.lib()


def _u16(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _cache_host(H, T, D, dtype, seed, outliers=True):
    x = activations(H * T, D, dtype, seed, outlier_frac=0.02 if outliers else 0.0, outlier_mult=8.0)
    return x.reshape(H, T, D)


def _to_dev(x, dtype):
    H, T, D = x.shape
    return x_to_torch(x.reshape(H * T, D), dtype).reshape(H, T, D)


@pytest.mark.parametrize("bits", [8, 4])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_quantize(bits, D, dtype):
    x = _cache_host(3, 37, D, dtype, seed=D + bits)
    c, s, z = W4.kv_quantize(_to_dev(x, dtype), bits)
    if bits == 8:
        rc, rs = KV.quantize_kv8(x, dtype)
        np.testing.assert_array_equal(c.cpu().numpy(), rc)
    else:
        rc, rs, rz = KV.quantize_kv4(x, dtype)
        np.testing.assert_array_equal(c.cpu().numpy(), rc)
        np.testing.assert_array_equal(_u16(z), rz.view(np.uint16))
    np.testing.assert_array_equal(_u16(s), rs.view(np.uint16))


CASES = [(8, 8, 1, 16, 128, 8, FP16), (32, 8, 1000, 1024, 128, 8, FP16), (4, 4, 4096, 4096, 64, 4, BF16),
         (16, 16, 77, 100, 128, 4, FP16), (2, 1, 20000, 20000, 128, 8, BF16), (6, 2, 333, 512, 64, 8, FP16),
         (32, 32, 4096, 4096, 128, 8, FP16), (32, 32, 4096, 4096, 128, 4, FP16)]


@pytest.mark.parametrize("Hq,Hkv,T,Tmax,D,bits,dtype", CASES)
def test_attention_decode(Hq, Hkv, T, Tmax, D, bits, dtype):
    k = _cache_host(Hkv, Tmax, D, dtype, seed=Hq + T)
    v = _cache_host(Hkv, Tmax, D, dtype, seed=Hq + T + 1, outliers=False)
    q = activations(Hq, D, dtype, seed=T)
    kc = W4.kv_quantize(_to_dev(k, dtype), bits)
    vc = W4.kv_quantize(_to_dev(v, dtype), bits)
    out = W4.kv_attention_decode(x_to_torch(q, dtype), kc, vc, T, bits)
    torch.cuda.synchronize()
    if bits == 8:
        Kd = KV.dequant_kv8(*KV.quantize_kv8(k, dtype))
        Vd = KV.dequant_kv8(*KV.quantize_kv8(v, dtype))
    else:
        Kd = KV.dequant_kv4(*KV.quantize_kv4(k, dtype))
        Vd = KV.dequant_kv4(*KV.quantize_kv4(v, dtype))
    ref = KV.attention_decode(q, dtype, Kd, Vd, T)
    assert_close(y_to_f64(out), ref_to_f64(ref, dtype), f"kv attention Hq={Hq} T={T} bits={bits}")
    if T == 1:       # one token: the (dequantized) value row, up to the output rounding
        grp = Hq // Hkv
        row = np.stack([Vd[h // grp, 0] for h in range(Hq)])
        assert_close(y_to_f64(out), row, "single token")


# Batched decode: B sequences with their own lengths in one call, against the single-sequence
# oracle per sequence.  Lengths 0 and > Tmax exercise the documented clamp into [1, Tmax].
BATCH_CASES = [(5, 8, 2, 300, 128, 8, FP16, [300, 1, 77, 256, 129]),
               (3, 32, 8, 1024, 128, 4, BF16, [1024, 513, 2]),
               (4, 4, 4, 200, 64, 8, BF16, [0, 200, 999, 64]),
               (16, 32, 32, 2048, 128, 8, FP16, [2048 - 97 * i for i in range(16)])]


@pytest.mark.parametrize("B,Hq,Hkv,Tmax,D,bits,dtype,lens", BATCH_CASES)
def test_attention_decode_batch(B, Hq, Hkv, Tmax, D, bits, dtype, lens):
    k = _cache_host(B * Hkv, Tmax, D, dtype, seed=B + Tmax)
    v = _cache_host(B * Hkv, Tmax, D, dtype, seed=B + Tmax + 1, outliers=False)
    q = activations(B * Hq, D, dtype, seed=Tmax + B)
    kc = W4.kv_quantize(_to_dev(k, dtype), bits)
    vc = W4.kv_quantize(_to_dev(v, dtype), bits)

    def batched(c):
        codes, s, z = c
        return (codes.view(B, Hkv, Tmax, -1), s.view(B, Hkv, Tmax), None if z is None else z.view(B, Hkv, Tmax))
    lt = torch.tensor(lens, dtype=torch.int32, device="cuda")
    qd = x_to_torch(q, dtype).view(B, Hq, D)
    out = W4.kv_attention_decode_batch(qd, batched(kc), batched(vc), lt, bits)
    torch.cuda.synchronize()
    if bits == 8:
        Kd = KV.dequant_kv8(*KV.quantize_kv8(k, dtype))
        Vd = KV.dequant_kv8(*KV.quantize_kv8(v, dtype))
    else:
        Kd = KV.dequant_kv4(*KV.quantize_kv4(k, dtype))
        Vd = KV.dequant_kv4(*KV.quantize_kv4(v, dtype))
    got = y_to_f64(out.view(B * Hq, D)).reshape(B, Hq, D)
    for b in range(B):
        T = min(max(lens[b], 1), Tmax)
        ref = KV.attention_decode(q[b * Hq:(b + 1) * Hq], dtype, Kd[b * Hkv:(b + 1) * Hkv],
                                  Vd[b * Hkv:(b + 1) * Hkv], T)
        assert_close(got[b], ref_to_f64(ref, dtype), f"batch seq {b} T={T}")
