"""Pins for the KV-cache oracle (CPU only).

* KV8 round trip within half a step, the row maximum at +-127, zero rows; KV4 is the pinned
  RTN quantizer with g = D;
* attention against closed forms: one token returns its value row; a zero query averages
  the value rows; token order does not matter; a brute-force pure-Python softmax on a tiny
  case; grouped heads read their kv head.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import kv as KV
from synth import BF16, FP16, activations


def _cache(H, T, D, dtype, seed):
    return activations(H * T, D, dtype, seed).reshape(H, T, D)


@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_kv8_round_trip(dtype):
    x = _cache(3, 17, 64, dtype, 1)
    q, s = KV.quantize_kv8(x, dtype)
    xd = oracle.linear._x64(x.reshape(-1, 64), dtype).reshape(3, 17, 64)
    err = np.abs(KV.dequant_kv8(q, s) - xd)
    assert np.all(err <= 0.5 * s.astype(np.float64)[..., None] * (1 + 1e-3) + 1e-7)
    assert np.all(np.abs(q.astype(int)).max(axis=2) >= 126)
    z = np.zeros((1, 2, 64), np.float16)
    qz, sz = KV.quantize_kv8(z, FP16)
    assert np.all(qz == 0) and np.all(sz == 1.0)


def test_kv4_is_rtn_per_row():
    x = _cache(2, 9, 128, FP16, 2)
    w, s, z = KV.quantize_kv4(x, FP16)
    codes, s2, z2 = oracle.quantize(x.reshape(-1, 128).astype(np.float32), 128, oracle.ASYM)
    np.testing.assert_array_equal(w.reshape(-1, 16), oracle.pack(codes))
    np.testing.assert_array_equal(s.reshape(-1), s2[:, 0])
    np.testing.assert_array_equal(z.reshape(-1), z2[:, 0])


def test_attention_closed_forms():
    H, T, D = 2, 5, 8
    rng = np.random.default_rng(3)
    Kd = rng.standard_normal((H, T, D))
    Vd = rng.standard_normal((H, T, D))
    q = activations(H, D, FP16, 4)
    np.testing.assert_allclose(KV.attention_decode_f64(q, FP16, Kd, Vd, 1), Vd[:, 0], rtol=1e-15)
    qz = np.zeros((H, D), np.float16)
    np.testing.assert_allclose(KV.attention_decode_f64(qz, FP16, Kd, Vd, T), Vd.mean(axis=1), rtol=1e-12)
    perm = rng.permutation(T)
    np.testing.assert_allclose(KV.attention_decode_f64(q, FP16, Kd[:, perm], Vd[:, perm], T),
                               KV.attention_decode_f64(q, FP16, Kd, Vd, T), rtol=1e-12)
    # brute force, head 1
    qf = [float(v) for v in q[1]]
    sc = [sum(qf[d] * Kd[1, t, d] for d in range(D)) / math.sqrt(D) for t in range(T)]
    m = max(sc)
    e = [math.exp(v - m) for v in sc]
    ref = [sum(e[t] * Vd[1, t, d] for t in range(T)) / sum(e) for d in range(D)]
    np.testing.assert_allclose(KV.attention_decode_f64(q, FP16, Kd, Vd, T)[1], ref, rtol=1e-12)


def test_grouped_heads():
    Hkv, G, T, D = 2, 3, 6, 16
    rng = np.random.default_rng(5)
    Kd = rng.standard_normal((Hkv, T, D))
    Vd = rng.standard_normal((Hkv, T, D))
    q = activations(Hkv * G, D, FP16, 6)
    out = KV.attention_decode_f64(q, FP16, Kd, Vd, T)
    for h in range(Hkv * G):
        one = KV.attention_decode_f64(q[h:h + 1], FP16, Kd[h // G:h // G + 1], Vd[h // G:h // G + 1], T)
        np.testing.assert_allclose(out[h], one[0], rtol=1e-15)
