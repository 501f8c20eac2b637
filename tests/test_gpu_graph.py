"""The entry points inside a captured HIP graph: every kernel path (GEMV, MFMA decode, MFMA
skinny, fp16 and bf16 prefill), the split-K workspace form, the W8A8 product and the batched
KV decode attention are captured once into one graph with preallocated outputs (the split-K
workspace too); the graph is then replayed several times with eager work between the
replays (other launches of the same kernels, outputs overwritten with NaN), and after every
replay each output must equal the eager launch of the same call bit for bit (the kernels
have a fixed reduction order).  The timed loops of the benchmark run the same way, so this
is also the check behind its numbers.
"""

from __future__ import annotations

import pytest
import torch

import w4a16_dequant_gemm_amd as W4
from synth import BF16, FP16, activations_device, weights_device

pytestmark = pytest.mark.gpu

TDT = {FP16: torch.float16, BF16: torch.bfloat16}

# (M, K, N, g, scheme, dtype, path)
LINEAR_CASES = [
    (1, 4096, 4096, 128, W4.ASYM, FP16, W4.PATH_GEMV),
    (1, 11008, 4096, 128, W4.ASYM, FP16, W4.PATH_GEMV),
    (2, 4096, 11008, 128, W4.SYM, BF16, W4.PATH_GEMV),
    (8, 4096, 4096, 128, W4.ASYM, FP16, W4.PATH_SKINNY),
    (16, 11008, 4096, 128, W4.ASYM, BF16, W4.PATH_SKINNY),
    (24, 4096, 1024, 128, W4.SYM, FP16, W4.PATH_SKINNY),
    (300, 4096, 1024, 128, W4.ASYM, FP16, W4.PATH_PREFILL),
    (300, 2048, 1024, 64, W4.ASYM, BF16, W4.PATH_PREFILL),
]


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    W4.lib()


def _same(a: torch.Tensor, b: torch.Tensor) -> bool:
    return torch.equal(a.view(torch.int16) if a.dtype != torch.float32 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype != torch.float32 else b.view(torch.int32))


def test_graph_replays_match_eager():
    calls = []        # (name, fn(out) launching the call into `out`, out for the graph)
    for i, (M, K, N, g, scheme, dt, path) in enumerate(LINEAR_CASES):
        W = weights_device(N, K, 0.02, 7000 + i)
        qw, s, z = W4.quantize_pack(W, g, scheme)
        del W
        X = activations_device(M, K, dt, 7100 + i)
        zz = z if scheme == W4.ASYM else None
        calls.append((f"linear M={M} K={K} N={N} g={g} path={W4.PATH_NAMES[path]}",
                      lambda out, X=X, qw=qw, s=s, zz=zz, g=g, path=path: W4.linear(X, qw, s, zz, g, path=path, out=out),
                      torch.empty((M, N), dtype=TDT[dt], device="cuda")))
    # the workspace form on a tile-starved prefill shape (split K with the fixed-order reduction)
    Xw = activations_device(256, 4096, FP16, 7150)
    Ww = weights_device(1024, 4096, 0.02, 7151)
    qww, sww, zww = W4.quantize_pack(Ww, 128, W4.ASYM)
    del Ww
    assert W4.linear_workspace(256, 1024, 4096, 128, FP16) > 0
    ws = torch.empty(W4.linear_workspace(256, 1024, 4096, 128, FP16) // 4, dtype=torch.float32, device="cuda")
    calls.append(("linear_ws split K M=256 K=4096 N=1024",
                  lambda out: W4.linear_ws(Xw, qww, sww, zww, 128, work=ws, out=out),
                  torch.empty((256, 1024), dtype=torch.float16, device="cuda")))
    # W8A8 product
    Xc = activations_device(256, 1024, FP16, 7200)
    Wc = weights_device(512, 1024, 0.02, 7201)
    sm = W4.w8a8_smooth(Xc, Wc, 2)
    qw8, sw8 = W4.w8a8_quantize_weight(Wc, sm)
    qx8, sx8 = W4.w8a8_quantize_act(Xc, sm)
    calls.append(("w8a8 M=256 K=1024 N=512",
                  lambda out: W4.w8a8_linear(qx8, sx8, qw8, sw8, out=out),
                  torch.empty((256, 512), dtype=torch.float16, device="cuda")))
    # batched KV8 decode attention, 3 sequences of different lengths
    B, Hq, Hkv, Tmax, D = 3, 8, 2, 700, 128
    k = activations_device(B * Hkv * Tmax, D, FP16, 7300).reshape(B * Hkv, Tmax, D)
    v = activations_device(B * Hkv * Tmax, D, FP16, 7301).reshape(B * Hkv, Tmax, D)
    kc, ks, kz = W4.kv_quantize(k, 8)
    vc, vs, vz = W4.kv_quantize(v, 8)
    kcache = (kc.reshape(B, Hkv, Tmax, D), ks.reshape(B, Hkv, Tmax), None)
    vcache = (vc.reshape(B, Hkv, Tmax, D), vs.reshape(B, Hkv, Tmax), None)
    q = activations_device(B * Hq, D, FP16, 7302).reshape(B, Hq, D)
    lengths = torch.tensor([700, 1, 333], dtype=torch.int32, device="cuda")
    work = torch.empty(W4.kv_attention_batch_workspace(B, Hq, Tmax, D), dtype=torch.float32, device="cuda")
    calls.append(("kv8 attention batch of 3",
                  lambda out: W4.kv_attention_decode_batch(q, kcache, vcache, lengths, 8, out=out, work=work),
                  torch.empty((B, Hq, D), dtype=torch.float16, device="cuda")))

    # eager references (separate outputs)
    refs = [fn(torch.empty_like(out)) for _, fn, out in calls]
    torch.cuda.synchronize()

    st = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(st):
        for _, fn, out in calls:          # warm-up on the capture stream
            fn(out)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=st):
            for _, fn, out in calls:
                fn(out)
    torch.cuda.synchronize()

    for rep in range(3):
        for _, _, out in calls:
            out.fill_(float("nan"))
        # eager launches of the same kernels between replays
        for _, fn, out in calls[::2]:
            fn(torch.empty_like(out))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for (name, _, out), ref in zip(calls, refs):
            assert _same(out, ref), f"replay {rep}: {name} differs from the eager launch"
