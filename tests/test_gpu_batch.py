"""GPU parity of w4a16_linear_batch, the call that runs several independent layers, with the
one-row layers sharing grouped launches (one grid over their weights) and layers of up to 8
rows sharing grouped launches of the ring decode kernel.

* grouped outputs equal w4a16_linear's bit for bit wherever that call takes the same
  weight-streaming kernel (the grouped kernel runs each layer's block with the layer's own
  arithmetic), and meet the oracle's output bar;
* mixed batches (one-row layers grouped, the others run as w4a16_linear), more than 16
  one-row layers (several grouped launches), ragged and per-channel layers, symmetric
  weights without zero points, both activation dtypes;
* a 70B-shaped one-row layer (random codes), against the oracle on sampled rows;
* the batch captured in a HIP graph and replayed, every replay equal to the eager result;
* ring-kernel groups (2 <= M <= 8): outputs equal the single call's bit for bit where that
  call runs the ring kernel (M >= 5), meet the oracle's bar everywhere (M <= 4 alone runs the
  activation-staging kernel), ragged and per-channel layers, more than 16 layers, a graph.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import w4a16_dequant_gemm_amd as W4
from synth import ASYM, BF16, FP16, SYM, activations, weights
from tests.gpu_util import assert_close, ref_to_f64, upload_packed, x_to_torch, y_to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _needs_gpu():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    W4.lib()


def _layer(M, N, K, g, dtype, seed, scheme=ASYM, zeros_none=False):
    W = weights(N, K, 0.02, seed=seed)
    X = activations(M, K, dtype, seed + 1)
    codes, s, z = oracle.quantize(W, g, scheme)
    qn = oracle.pack(codes)
    zz = None if zeros_none else z
    qw, st, zt = upload_packed(qn, s, zz)
    return dict(X=X, qn=qn, s=s, z=zz, g=g, dtype=dtype, t=(x_to_torch(X, dtype), qw, st, zt, g))


# (M, N, K, g, scheme, zeros_none): the three 7B-like layers, short and ragged rows, two rows
# per wave (N > 4096), per-channel groups, symmetric weights without zero points, N = 1, and
# every chunks-per-lane case of the grouped kernel (1 .. 6: K up to 2048, 4096, 6144, 8192,
# 10240, 12288), with a row whose last chunks per lane run past its end (K = 4352) and
# 32-column groups
ONE_ROW = [(1, 4096, 4096, 128, ASYM, False), (1, 11008, 4096, 128, ASYM, False),
           (1, 4096, 11008, 128, ASYM, False), (1, 300, 2048, 64, ASYM, False),
           (1, 4097, 1024, 128, ASYM, False), (1, 50, 11008, 11008, ASYM, False),
           (1, 192, 1024, 128, SYM, True), (1, 1, 32, 32, ASYM, False), (1, 777, 12288, 256, ASYM, False),
           (1, 1000, 6144, 128, ASYM, False), (1, 129, 4352, 128, ASYM, False),
           (1, 520, 5120, 32, SYM, True), (1, 3000, 8192, 128, ASYM, False),
           (1, 333, 10240, 64, ASYM, False)]


@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_grouped_equals_single_calls_and_oracle(dtype):
    layers = [_layer(M, N, K, g, dtype, seed=100 + i, scheme=sc, zeros_none=zn)
              for i, (M, N, K, g, sc, zn) in enumerate(ONE_ROW)]
    ys = W4.linear_batch([L["t"] for L in layers])
    singles = [W4.linear(*L["t"]) for L in layers]
    torch.cuda.synchronize()
    for L, y, y1, shape in zip(layers, ys, singles, ONE_ROW):
        assert torch.equal(y.view(torch.int16), y1.view(torch.int16)), f"grouped != single {shape}"
        ref = oracle.linear_ref(L["X"], dtype, L["qn"], L["s"], L["z"], L["g"])
        assert_close(y_to_f64(y), ref_to_f64(ref, dtype), f"grouped {shape}")


def test_mixed_batch_and_many_groups():
    shapes = ([(1, 1024 + 64 * i, 2048 if i % 2 else 4096, 128) for i in range(20)] +
              [(4, 1000, 4096, 128), (300, 500, 2048, 64), (2, 3000, 8192, 128), (1, 64, 16384, 128)])
    order = [0, 20, 1, 2, 21, 3, 22] + list(range(4, 20)) + [23]
    layers = [_layer(*shapes[j], FP16, seed=500 + j) for j in order]
    ys = W4.linear_batch([L["t"] for L in layers])
    singles = [W4.linear(*L["t"]) for L in layers]
    torch.cuda.synchronize()
    for j, L, y, y1 in zip(order, layers, ys, singles):
        ref = oracle.linear_ref(L["X"], FP16, L["qn"], L["s"], L["z"], L["g"])
        assert_close(y_to_f64(y), ref.astype(np.float64), f"batch item {shapes[j]}")
        if shapes[j][0] == 1 and shapes[j][2] <= 12288:
            assert torch.equal(y.view(torch.int16), y1.view(torch.int16)), f"grouped != single {shapes[j]}"


def test_70b_shaped_one_row_layer():
    # packed weights of the 70B up-projection shape: random codes, scales and zero points (no
    # fp32 weight matrix needed); the grouped kernel takes it with 8 rows per block
    N, K, g = 28672, 8192, 128
    gen = torch.Generator(device="cuda")
    gen.manual_seed(70)
    qw = torch.randint(-2 ** 31, 2 ** 31, (N, K // 8), dtype=torch.int32, device="cuda", generator=gen)
    sc = (torch.rand((N, K // g), device="cuda", generator=gen) * 0.02 + 0.001).half()
    z = torch.randint(0, 16, (N, K // g), device="cuda", generator=gen).half()
    X = activations(1, K, BF16, seed=71, outlier_frac=0.01, outlier_mult=100.0)
    Xt = x_to_torch(X, BF16)
    small = _layer(1, 512, 4096, 128, BF16, seed=72)
    y, _ = W4.linear_batch([(Xt, qw, sc, z, g), small["t"]])
    torch.cuda.synchronize()
    ns = np.unique(np.r_[0, N - 1, np.random.default_rng(7).choice(N, 1024, replace=False)])
    idx = torch.from_numpy(ns).cuda()
    ref = oracle.linear_ref(X, BF16, qw[idx].cpu().numpy(), sc[idx].cpu().numpy(), z[idx].cpu().numpy(), g)
    assert_close(y_to_f64(y[:, idx]), ref_to_f64(ref, BF16), "70B-shaped grouped layer")


def test_batch_graph_replay_matches_eager():
    layers = [_layer(1, N, K, 128, FP16, seed=800 + i) for i, (N, K) in
              enumerate([(4096, 4096), (11008, 4096), (4096, 11008)])]
    outs = [torch.empty((1, L["t"][1].shape[0]), dtype=torch.float16, device="cuda") for L in layers]
    W4.linear_batch([L["t"] for L in layers], outs=outs)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        W4.linear_batch([L["t"] for L in layers], outs=outs)
    for _ in range(3):
        for o in outs:
            o.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16))


# (M, N, K, g, scheme, zeros_none): layers the ring decode kernel takes in a group (M <= 8, N and K
# <= 12288, K % 256 == 0, g % 128 == 0): the 7B-like shapes, ragged N, per-channel groups,
# symmetric weights without zero points, two-row layers whose single call runs the GEMV
RING = [(8, 4096, 4096, 128, ASYM, False), (8, 11008, 4096, 128, ASYM, False),
        (8, 4096, 11008, 128, ASYM, False), (5, 1000, 2048, 128, ASYM, False),
        (7, 777, 4096, 4096, ASYM, False), (6, 300, 12288, 256, SYM, True), (4, 1040, 4096, 128, ASYM, False),
        (3, 500, 8192, 128, ASYM, False), (2, 2000, 6144, 128, SYM, True), (2, 4096, 4096, 128, ASYM, False),
        (2, 1100, 2048, 128, ASYM, False)]


@pytest.mark.parametrize("dtype", [FP16, BF16])
def test_ring_group_equals_ring_kernel_and_oracle(dtype):
    layers = [_layer(M, N, K, g, dtype, seed=900 + i, scheme=sc, zeros_none=zn)
              for i, (M, N, K, g, sc, zn) in enumerate(RING)]
    assert all(W4.select_path(M, N, K, g, dtype) == W4.PATH_SKINNY for M, N, K, g, _, _ in RING if M > 2)
    ys = W4.linear_batch([L["t"] for L in layers])
    singles = [W4.linear(*L["t"]) for L in layers]
    torch.cuda.synchronize()
    for L, y, y1, shape in zip(layers, ys, singles, RING):
        if shape[0] >= 5:          # alone, the ring kernel too
            assert torch.equal(y.view(torch.int16), y1.view(torch.int16)), f"ring group != single {shape}"
        ref = oracle.linear_ref(L["X"], dtype, L["qn"], L["s"], L["z"], L["g"])
        assert_close(y_to_f64(y), ref_to_f64(ref, dtype), f"ring group {shape}")


def test_ring_groups_of_more_than_16_layers():
    shapes = [(3 + i % 6, 256 + 48 * i, 2048 if i % 3 else 4096, 128) for i in range(22)]    # 16 + 6
    layers = [_layer(*sh, FP16, seed=1000 + i) for i, sh in enumerate(shapes)]
    ys = W4.linear_batch([L["t"] for L in layers])
    singles = [W4.linear(*L["t"]) for L in layers]
    torch.cuda.synchronize()
    for sh, L, y, y1 in zip(shapes, layers, ys, singles):
        if sh[0] >= 5:
            assert torch.equal(y.view(torch.int16), y1.view(torch.int16)), f"ring group != single {sh}"
        ref = oracle.linear_ref(L["X"], FP16, L["qn"], L["s"], L["z"], L["g"])
        assert_close(y_to_f64(y), ref.astype(np.float64), f"ring group item {sh}")


def test_ring_group_graph_replay_matches_eager():
    layers = [_layer(8, N, K, 128, FP16, seed=1100 + i) for i, (N, K) in
              enumerate([(4096, 4096), (11008, 4096), (4096, 11008)])]
    outs = [torch.empty((8, L["t"][1].shape[0]), dtype=torch.float16, device="cuda") for L in layers]
    W4.linear_batch([L["t"] for L in layers], outs=outs)
    torch.cuda.synchronize()
    eager = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        W4.linear_batch([L["t"] for L in layers], outs=outs)
    for _ in range(3):
        for o in outs:
            o.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, e in zip(outs, eager):
            assert torch.equal(o.view(torch.int16), e.view(torch.int16))
