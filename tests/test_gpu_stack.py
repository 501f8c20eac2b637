"""GPU parity of a full decode step of a 32-layer 7B-shaped stack: per layer q, k, v, o
(4096 -> 4096), gate, up (4096 -> 11008) and down (11008 -> 4096), 224 linears and about 3.5 GB
of packed weights resident at once, bf16 activations, asymmetric uint4 with g = 128 and a
per-channel variant (g = K), M = 1 and M = 8, every linear launched back to back on one
stream through the C ABI.

Weights come from torch's seeded device generator (the host generator would take minutes
for 6.5 G values); for every linear the sampled output rows' fp32 weights are copied back, so
the oracle checks their packing bit for bit and 64 sampled output columns per linear within
the output tolerance.  Activations are the host recipe's, uploaded.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import w4a16_dequant_gemm_amd as W4
from synth import BF16, seeds, stack_cases, activations, weights_device
from tests.gpu_util import MAX_REL, REL_FRO, errors, ref_to_f64, x_to_torch, y_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    W4.lib()


@pytest.mark.parametrize("per_channel", [False, True], ids=["g128", "per_channel"])
def test_full_stack_decode_step(per_channel):
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
        qn = qw[idx].cpu().numpy()
        np.testing.assert_array_equal(qn, oracle.pack(codes), err_msg=f"packing, linear {c.layer}")
        np.testing.assert_array_equal(sc[idx].cpu().numpy().view(np.uint16), s_ref.view(np.uint16))
        np.testing.assert_array_equal(z[idx].cpu().numpy().view(np.uint16), z_ref.view(np.uint16))
        layers.append((c, qw, sc, z, idx, qn, s_ref, z_ref))
    for M in (1, 8):
        xs = [activations(M, c.K, BF16, seeds(c.config, c.layer)[1] + 100 * M) for c, *_ in layers]
        xd = [x_to_torch(x, BF16) for x in xs]
        ys = [W4.linear(x, qw, sc, z, c.g) for x, (c, qw, sc, z, *_) in zip(xd, layers)]
        torch.cuda.synchronize()
        got, want = [], []
        for x, y, (c, _, _, _, idx, qn, s_ref, z_ref) in zip(xs, ys, layers):
            ref = ref_to_f64(oracle.linear_ref(x, BF16, qn, s_ref, z_ref, c.g), BF16)
            yv = y_to_f64(y[:, idx])
            what = f"stack linear {c.layer} (K={c.K}, N={c.N}, g={c.g}) M={M}"
            assert np.all(np.isfinite(yv)), what
            # Both sides are rounded to bf16, so an element either matches or sits one
            # output ulp away (fp32 against fp64 accumulation near a rounding boundary), up to
            # the fp32 accumulation error itself on outputs near zero (2^-16 of the largest
            # output is generous for it).  A 64-element sample with one such flip can exceed
            # the Frobenius bar by itself, so per linear the check is this per-element bound
            # and the max-error bar; the Frobenius bar applies to the step's whole sample.
            ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
            bad = np.abs(yv - ref) > ulp + np.abs(ref).max() * 2.0 ** -16
            assert not bad.any(), f"{what}: {yv[bad][:4]} vs {ref[bad][:4]} (max |ref| {np.abs(ref).max():.4g})"
            assert errors(yv, ref)[1] <= MAX_REL, what
            got.append(yv.ravel())
            want.append(ref.ravel())
        fro, mx = errors(np.concatenate(got), np.concatenate(want))
        assert fro <= REL_FRO, f"step M={M}: rel_fro={fro:.3e}"
    del layers
    torch.cuda.empty_cache()
