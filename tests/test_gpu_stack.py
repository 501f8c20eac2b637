"""GPU parity of a full decode step of a 32-layer 7B-shaped stack: per layer q, k, v, o
(4096 -> 4096), gate, up (4096 -> 11008) and down (11008 -> 4096), 224 linears and about 3.5 GB
of packed weights resident at once, bf16 activations, asymmetric uint4 with g = 128 and a
per-channel variant (g = K), M = 1 and M = 8, every linear launched back to back on one
stream through the C ABI.

Weights come from torch's seeded device generator (the host generator would take minutes
for 6.5 G values).  Packing is checked bit for bit on sampled output rows (their fp32
weights are copied back and quantized by the oracle).  The outputs are then checked per
linear at full width: the oracle takes the GPU-packed codes, scales and zero points of the
whole linear (the packing being pinned on its own) and computes all N outputs of both
activation batches; each linear must meet the output bar, relative Frobenius <= 1e-3 and
max |dY| <= 1e-2 max |Y_ref|.  The GPU work runs once per variant (a module fixture); the
checks are split by layer so that each test stays short.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import w4a16_dequant_gemm_amd as W4
from synth import BF16, seeds, stack_cases, activations, weights_device
from tests.gpu_util import assert_close, ref_to_f64, x_to_torch, y_to_f64

pytestmark = pytest.mark.gpu

MS = (1, 8)


@pytest.fixture(scope="module", params=[False, True], ids=["g128", "per_channel"])
def stack(request):
    """Quantize all 224 linears on the GPU (packing checked on sampled rows), run the step at
    M = 1 and M = 8 back to back, and keep the packed weights and outputs."""
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    W4.lib()
    per_channel = request.param
    cases = stack_cases(1, per_channel)
    assert len(cases) == 224
    rng = np.random.default_rng(5000 + int(per_channel))
    layers = []
    for c in cases:
        sw, _ = seeds(c.config, c.layer)
        Wd = weights_device(c.N, c.K, c.w_sigma, sw)
        qw, sc, z = W4.quantize_pack(Wd, c.g, c.scheme)
        ns = np.unique(np.concatenate([[0, c.N - 1], rng.choice(c.N, 62, replace=False)]))
        idx = torch.from_numpy(ns).cuda()
        Wn = Wd[idx].cpu().numpy()
        del Wd
        codes, s_ref, z_ref = oracle.quantize(Wn, c.g, c.scheme)
        np.testing.assert_array_equal(qw[idx].cpu().numpy(), oracle.pack(codes),
                                      err_msg=f"packing, linear {c.layer}")
        np.testing.assert_array_equal(sc[idx].cpu().numpy().view(np.uint16), s_ref.view(np.uint16))
        np.testing.assert_array_equal(z[idx].cpu().numpy().view(np.uint16), z_ref.view(np.uint16))
        layers.append((c, qw, sc, z))
    xs = {M: [activations(M, c.K, BF16, seeds(c.config, c.layer)[1] + 100 * M) for c, *_ in layers] for M in MS}
    ys = {}
    for M in MS:
        xd = [x_to_torch(x, BF16) for x in xs[M]]
        ys[M] = [W4.linear(x, qw, sc, z, c.g) for x, (c, qw, sc, z) in zip(xd, layers)]
    torch.cuda.synchronize()
    yield layers, xs, ys
    del layers, ys
    torch.cuda.empty_cache()


@pytest.mark.parametrize("layer", range(32))
def test_full_stack_decode_step(stack, layer):
    layers, xs, ys = stack
    for j in range(7):
        i = 7 * layer + j
        c, qw, sc, z = layers[i]
        # one dequantization serves both batches: the rows of M = 1 and M = 8 stacked
        X = np.concatenate([xs[M][i] for M in MS])
        ref = ref_to_f64(oracle.linear_ref(X, BF16, qw.cpu().numpy(), sc.cpu().numpy(), z.cpu().numpy(), c.g),
                         BF16)
        r0 = 0
        for M in MS:
            assert_close(y_to_f64(ys[M][i]), ref[r0:r0 + M],
                         f"stack linear {c.layer} (K={c.K}, N={c.N}, g={c.g}) M={M}, all {c.N} outputs")
            r0 += M
