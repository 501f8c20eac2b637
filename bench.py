#!/usr/bin/env python3
"""Benchmark of the W4A16 linear layer on one MI355X.

Workload (one "step"): the decode batch on 7B-like layer shapes at M = 1 -- one
W4A16 linear for each (K, N) in (4096, 4096), (4096, 11008), (11008, 4096), group size
128, asymmetric uint4, fp16 scales and zeros, fp16 activations ~ N(0, 1), weights
~ N(0, 0.02) quantized on the GPU by the library.  Launches cycle through distinct
copies of the packed weights totalling >= 1 GiB so the 256 MB last-level cache cannot
serve them: every step streams its weights from HBM.

Metric: effective weight-stream bandwidth = (packed bytes + scale/zero bytes) / time,
the bytes the method must move (4 bits + 32/g bits per weight).  Also reported: the
M sweep 1..16, prefill TFLOP/s at M = 4096, the roofline of the dominant kernel and the
CPU oracle timed on the host (reported baseline, not a target).

Prints ONE JSON line.  ``--gpus N`` with N > 1 is refused: the path runs on one GPU.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "W4A16 linear: weight-stream GB/s (% HBM peak) at M=1; TFLOP/s at M=4096"
HBM_PEAK_GBS = 8000.0
FP64_PEAK_TFLOPS = 78.6             # MI355X dense fp64
MFMA_F16_PEAK_TFLOPS = 2500.0
SHAPES = [(4096, 4096), (4096, 11008), (11008, 4096)]      # (K, N)
GROUP = 128


# Kernel instantiation serving each layer at M = 1 (fp16, g = 128), as rocprofv3 names it.
KERNEL_NAMES = {(4096, 4096): "gemv_stream_kernel<0, 1, 2, 1, 8, 0>",
                (4096, 11008): "gemv_stream_kernel<0, 1, 2, 2, 8, 0>",
                (11008, 4096): "gemv_stream_kernel<0, 1, 6, 1, 8, 0>",
                "step": "gemv_group_kernel<0>"}     # the whole M = 1 step in one grouped launch
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = [os.path.join(ROOT, "w4a16_dequant_gemm_amd", "csrc", f)
                  for f in ("gemv.hip", "common.h")]
COPY_MIB = 256          # calibration copy: reads and writes COPY_MIB MiB


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_hash() -> str:
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def traffic_file(shape) -> str:
    if shape == "step":
        return os.path.join(PROFILES, "traffic_gemv_group_m1_7b_step.json")
    K, N = shape
    return os.path.join(PROFILES, f"traffic_gemv_stream_m1_k{K}_n{N}.json")


def traffic_record(shape):
    """HBM bytes per launch from the committed counter summary of a layer (K, N) or of the
    grouped step ("step"), if it was taken on the current kernel source (else None)."""
    path = traffic_file(shape)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh)
    if rec.get("source_sha256") != source_hash():
        return None
    return {"bytes_per_launch": rec["traffic_bytes_per_launch"], "source": os.path.relpath(path, ROOT)}


def weight_bytes(N: int, K: int, g: int) -> int:
    return N * K // 2 + 4 * N * (K // g)


class Layer:
    """Rotating copies of one packed layer, resident in HBM."""

    def __init__(self, K, N, g, copies, seed, W4, synth, torch):
        self.K, self.N, self.g = K, N, g
        W = synth.weights_device(N, K, 0.02, seed)
        qw, s, z = W4.quantize_pack(W, g, W4.ASYM)
        self.W_sample_rows = None
        self.copies = [(qw, s, z)] + [(qw.clone(), s.clone(), z.clone()) for _ in range(copies - 1)]
        self.W = W      # kept until parity is checked
        self.bytes = weight_bytes(N, K, g)


def capture(fn, iters, torch):
    """HIP graph holding ``iters`` back-to-back calls fn(0..iters-1) (launch overhead of
    the Python binding is paid once, at capture)."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(iters):
            fn(i)
    torch.cuda.synchronize()
    return g


REPEATS = 5       # timed replays per measurement; the median is reported


def time_graph(g, iters, torch, repeats: int = REPEATS):
    """ms per iteration of a graph that holds ``iters`` iterations: one warm replay, then
    ``repeats`` replays, each bracketed by synchronize + events; the median replay."""
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    g.replay()                     # warm replay
    torch.cuda.synchronize()
    times = []
    for _ in range(repeats):
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / iters)
    return sorted(times)[len(times) // 2]


def time_loop(fn, iters, torch, graph=True, repeats: int = REPEATS):
    if graph:
        return time_graph(capture(fn, iters, torch), iters, torch, repeats)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for i in range(iters):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / iters   # ms per iteration


PROBE_LIB = os.path.join(ROOT, "w4a16_dequant_gemm_amd", "libw4a16_probe.so")


def read_ceiling(nbytes: int, torch) -> dict:
    """The fastest plain read of ``nbytes`` in one launch (libw4a16_probe.so: every thread
    issues 4, 8 or 16 16-byte loads at once, then XORs them; the best of the three), over
    rotating buffers of >= 1 GiB, 200 launches per graph replay, median of 5 replays: the
    rate one launch of that size reaches on this GPU, the practical ceiling of a kernel that
    streams those bytes."""
    import ctypes
    if not os.path.exists(PROBE_LIB):
        raise SystemExit(f"{PROBE_LIB} is missing: build with `python -m w4a16_dequant_gemm_amd.build`")
    L = ctypes.CDLL(PROBE_LIB)
    L.w4a16_probe_blocks.restype = ctypes.c_longlong
    L.w4a16_probe_blocks.argtypes = [ctypes.c_longlong, ctypes.c_int]
    L.w4a16_probe_read.restype = ctypes.c_int
    L.w4a16_probe_read.argtypes = [ctypes.c_void_p, ctypes.c_longlong, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p]
    copies = max(2, -(-(1 << 30) // nbytes))
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    best = None
    for per in (4, 8, 16):
        out = torch.empty(L.w4a16_probe_blocks(nbytes, per) * 256, dtype=torch.int32, device="cuda")

        def f(i, per=per, out=out):
            rc = L.w4a16_probe_read(bufs[i % copies].data_ptr(), nbytes, per, out.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)
            if rc != 0:
                raise RuntimeError(f"w4a16_probe_read failed ({rc})")
        f(0)
        torch.cuda.synchronize()
        us = time_loop(f, 200, torch) * 1e3
        if best is None or us < best["us"]:
            best = {"us": round(us, 3), "GBps": round(nbytes / us / 1e3, 1), "loads_per_thread": per}
    del bufs
    torch.cuda.empty_cache()
    best["bytes"] = nbytes
    return best


def check_samples(samples, oracle, np):
    """The oracle on the sampled rows of every timed extra configuration: packing bit-exact
    (codes, scales, zero points) and outputs within the bar (relative Frobenius <= 1e-3,
    max |dY| <= 1e-2 max |Y_ref|)."""
    out = {}
    for smp in samples:
        codes, s, z = oracle.quantize(smp["W"], smp["g"], smp["scheme"])
        qw = oracle.pack(codes)
        pk = bool(np.array_equal(qw, smp["qw"]) and np.array_equal(s.view(np.uint16), smp["s"].view(np.uint16)))
        if smp["z"] is not None:
            pk &= bool(np.array_equal(z.view(np.uint16), smp["z"].view(np.uint16)))
        ref = oracle.linear_ref(smp["X"], smp["dtype"], qw, s, smp["z"] if smp["z"] is not None else z, smp["g"])
        if smp["dtype"] == 0:
            r, y = ref.astype(np.float64), smp["Y"].view(np.float16).astype(np.float64)
        else:
            r, y = oracle.bf16_bits_to_f64(ref), oracle.bf16_bits_to_f64(smp["Y"])
        fro = float(np.linalg.norm(y - r) / np.linalg.norm(r))
        mx = float(np.abs(y - r).max() / np.abs(r).max())
        out[smp["name"]] = {"packing_bit_exact": pk, "rel_fro": fro, "max_rel": mx,
                            "ok": pk and fro <= 1e-3 and mx <= 1e-2}
    return out


def cpu_baseline(layers, w_host, xs_host, y_gpu, budget_s, np, torch, samples=()):
    """The oracle beside the GPU path, on the host cores: quantize each layer (checked
    bit-exact against the GPU packing on sampled rows), then time the oracle's linear
    (fp64 dequantize + BLAS product) on the same M = 1 workload and check the GPU
    outputs of the timed step against its result; then the sampled rows of every timed
    extra configuration against the oracle."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = len(os.sched_getaffinity(0))
    host = []
    packing_ok = True
    for L, W in zip(layers, w_host):
        codes, s, z = oracle.quantize_asym(W, GROUP)
        qw = oracle.pack(codes)
        rng = np.random.default_rng(L.N + L.K)
        ns = np.unique(np.concatenate([[0, L.N - 1], rng.choice(L.N, 64, replace=False)]))
        idx = torch.from_numpy(ns).cuda()
        qg, sg, zg = L.copies[0]
        packing_ok &= bool(np.array_equal(qg[idx].cpu().numpy(), qw[ns]))
        packing_ok &= bool(np.array_equal(sg[idx].cpu().numpy().view(np.uint16), s[ns].view(np.uint16)))
        packing_ok &= bool(np.array_equal(zg[idx].cpu().numpy().view(np.uint16), z[ns].view(np.uint16)))
        host.append((qw, s, z, L.bytes))
    total_bytes = 0
    refs = None
    t0 = time.perf_counter()
    steps = 0
    while True:
        ys = [oracle.linear_ref(X, 0, qw, s, z, GROUP) for X, (qw, s, z, _) in zip(xs_host, host)]
        total_bytes += sum(h[3] for h in host)
        refs = refs or ys
        steps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or steps >= 50:
            break
    fro, mx = [], []
    for y, r in zip(y_gpu, refs):
        y = y.float().cpu().numpy().astype(np.float64)
        r = r.astype(np.float64)
        fro.append(float(np.linalg.norm(y - r) / np.linalg.norm(r)))
        mx.append(float(np.abs(y - r).max() / np.abs(r).max()))
    extra = check_samples(samples, oracle, np)
    parity = {"packing_bit_exact_sampled_rows": packing_ok, "rel_fro": fro, "max_rel": mx,
              "extra_configs_checked": len(extra),
              "extra_configs_failed": {k: v for k, v in extra.items() if not v["ok"]},
              "ok": packing_ok and max(fro) <= 1e-3 and max(mx) <= 1e-2 and all(v["ok"] for v in extra.values())}
    # one host thread on the single 4096 x 4096 layer, and the 32-layer stack extrapolated
    # from one 7-linear layer (q, k, v, o 4096 -> 4096; gate, up 4096 -> 11008; down 11008 -> 4096)
    one_thread = None
    try:
        from threadpoolctl import threadpool_limits
        qw, s, z, nb = host[0]
        with threadpool_limits(1):
            t1 = time.perf_counter()
            oracle.linear_ref(xs_host[0], 0, qw, s, z, GROUP)
            one_thread = nb / (time.perf_counter() - t1) / 1e9
    except Exception:  # pragma: no cover - threadpoolctl missing
        pass
    by_shape = {(L.K, L.N): h for L, h in zip(layers, host)}
    t1 = time.perf_counter()
    for K, N in [(4096, 4096)] * 4 + [(4096, 11008)] * 2 + [(11008, 4096)]:
        qw, s, z, _ = by_shape[(K, N)]
        oracle.linear_ref(xs_host[0] if K == 4096 else xs_host[2], 0, qw, s, z, GROUP)
    layer_s = time.perf_counter() - t1
    return {"value": total_bytes / el / 1e9, "unit": "GB/s", "cores": int(threads),
            "host_cpus": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)),
            "blas_env": {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS")},
            "kind": "oracle",
            "sample": f"{steps} oracle step(s) of the same M=1 workload (3 layers, fp64 "
                      f"dequantize + BLAS matmul), {el:.1f} s",
            "parity_vs_gpu": parity,
            "one_thread_GBps_4096x4096": None if one_thread is None else round(one_thread, 4),
            "stack_32_layers_s_extrapolated": round(32 * layer_s, 2),
            "other_rows": cpu_baseline_rows(oracle, np)}


def cpu_baseline_rows(oracle, np):
    """The oracle of each further method on a bounded sample of its workload (a few seconds
    each on the host cores), in the unit its GPU leg reports: GPTQ and AWQ in fp64
    TFLOP/s of their algorithmic flops, W8A8 in TOP/s of the integer product, KV decode
    attention in GB/s of the quantized cache."""
    import synth
    from oracle import awq, gptq, kv, w8a8
    out = {}
    # GPTQ, one 1024 x 1024 layer from 512 calibration rows
    n, K, N = 512, 1024, 1024
    X = synth.calibration(n, K, synth.FP16, 11)
    W = synth.weights(N, K, 0.02, 12)
    t0 = time.perf_counter()
    U = gptq.inverse_cholesky_upper(gptq.damp_hessian(gptq.hessian(X, synth.FP16), 0.01))
    t1 = time.perf_counter()
    gptq.gptq_quantize(W, U, GROUP, oracle.ASYM)
    t2 = time.perf_counter()
    out["gptq"] = {"sample": f"K=N={K}, n={n}", "hessian_factor_s": round(t1 - t0, 3),
                   "quantize_s": round(t2 - t1, 3),
                   "quantize_fp64_TFLOPs": round(N * K * (K - 1) / (t2 - t1) / 1e12, 5)}
    # AWQ, one 1024 x 1024 layer from 256 calibration rows
    n = 256
    X = synth.calibration(n, K, synth.FP16, 13, outlier_frac=0.01, outlier_mult=20.0)
    t0 = time.perf_counter()
    awq.awq_search(W, X, synth.FP16, awq.channel_mean_abs(X, synth.FP16), GROUP, oracle.ASYM)
    t1 = time.perf_counter()
    out["awq"] = {"sample": f"K=N={K}, n={n}", "search_s": round(t1 - t0, 3),
                  "search_fp64_TFLOPs": round(9 * 2.0 * n * N * K / (t1 - t0) / 1e12, 5)}
    # W8A8 with SmoothQuant, M = 128, K = N = 1024
    M = 128
    X = synth.calibration(M, K, synth.FP16, 14, outlier_frac=0.01, outlier_mult=20.0)
    s = w8a8.smooth_factors(X, synth.FP16, W, 2)
    qw, sw = w8a8.quantize_weight(W, s)
    qx, sx = w8a8.quantize_act(X, synth.FP16, s)
    t0 = time.perf_counter()
    w8a8.linear_int8(qx, sx, qw, sw, synth.FP16)
    t1 = time.perf_counter()
    out["w8a8"] = {"sample": f"M={M}, K=N={K}", "product_s": round(t1 - t0, 3),
                   "TOPS": round(2.0 * M * N * K / (t1 - t0) / 1e12, 5)}
    # KV8 decode attention, 32 heads, D = 128, 2048 cached tokens
    H, D, T = 32, 128, 2048
    k = synth.activations(H * T, D, synth.FP16, 15).reshape(H, T, D)
    v = synth.activations(H * T, D, synth.FP16, 16).reshape(H, T, D)
    q = synth.activations(H, D, synth.FP16, 17)
    Kd = kv.dequant_kv8(*kv.quantize_kv8(k, synth.FP16))
    Vd = kv.dequant_kv8(*kv.quantize_kv8(v, synth.FP16))
    t0 = time.perf_counter()
    kv.attention_decode(q, synth.FP16, Kd, Vd, T)
    t1 = time.perf_counter()
    out["kv8_attention"] = {"sample": f"H={H}, D={D}, T={T}", "s": round(t1 - t0, 4),
                            "GBps": round(2 * H * T * (D + 2) / (t1 - t0) / 1e9, 3)}
    # W8A16 linear, M = 1 on one 4096 x 4096 layer (8-bit codes, g = 128)
    from oracle import w8a16
    W = synth.weights(4096, 4096, 0.02, 18)
    codes, sc, z = w8a16.quantize8(W, GROUP, w8a16.ASYM)
    q = w8a16.pack8(codes)
    X = synth.activations(1, 4096, synth.FP16, 19)
    t0 = time.perf_counter()
    w8a16.linear8_ref(X, synth.FP16, q, sc, z, GROUP)
    t1 = time.perf_counter()
    out["w8a16_linear"] = {"sample": "M=1, K=N=4096, g=128", "s": round(t1 - t0, 4),
                           "GBps": round((4096 * 4096 + 4 * 4096 * 4096 // GROUP) / (t1 - t0) / 1e9, 3)}
    return out


def traffic_run(shape, W4, synth, torch, np):
    """Workload for the two counter passes: a plain elementwise copy (y = -x) of COPY_MIB
    MiB (calibration: known bytes read and written) five times, then 20 launches of the
    layer's kernel at M = 1 (shape (K, N)) or of the grouped M = 1 step ("step") over
    rotating weight copies."""
    shapes = SHAPES if shape == "step" else [shape]
    nbytes = sum(weight_bytes(N, K, GROUP) for K, N in shapes)
    copies = max(2, int(np.ceil(2**30 / nbytes)))
    layers = [Layer(K, N, GROUP, copies, 1000 + 10 * 2 + SHAPES.index((K, N)), W4, synth, torch) for K, N in shapes]
    for L in layers:
        del L.W
    xs = {K: synth.activations_device(1, K, synth.FP16, 1015) for K in (4096, 11008)}
    ys = [torch.empty((1, L.N), dtype=torch.float16, device="cuda") for L in layers]

    def run(i):
        c = i % copies
        if shape == "step":
            W4.linear_batch([(xs[L.K], *L.copies[c], GROUP) for L in layers], outs=ys)
        else:
            W4.linear(xs[layers[0].K], *layers[0].copies[c], GROUP, out=ys[0])
    src = torch.ones(COPY_MIB << 19, dtype=torch.float16, device="cuda")
    dst = torch.empty_like(src)
    for i in range(3):
        run(i)
    torch.cuda.synchronize()
    for _ in range(5):
        torch.neg(src, out=dst)          # one elementwise kernel: reads and writes COPY_MIB MiB
    torch.cuda.synchronize()
    for i in range(20):
        run(i + 3)
    torch.cuda.synchronize()
    log(f"traffic run done: {shape}, {copies} weight copies, copy {COPY_MIB} MiB x5")


def profile_run(name: str, W4, synth, torch):
    """A short fixed workload for counter and trace runs of one further kernel family:
    `prefill` (M = 4096 on both prefill shapes, 5 launches each), `w8a8` (the INT8 product at
    M = 4096, both shapes, 5 launches each), `kv_batch` (batched KV8 and KV4 decode attention,
    16 sequences, 2 layers' caches, 2 launches each), `decode_m16` (M = 16 on the 7B shapes
    over 20 rotating weight copies, 20 launches each), `w8a16` (8-bit codes: M = 1 and 4 on the 7B
    shapes over 10 rotating copies, 20 launches each, and the M = 4096 prefill, 5 each), `c3`
    (the 70B-like bf16 decode shapes at M = 1, 4, 16 over 4 rotating copies, 20 launches each),
    `crossover` (the plain prefill call at M = 256 on (4096, 11008) and at M = 1024 on
    (11008, 4096), g = 128 asym, 5 launches each)."""
    if name == "crossover":
        for M, K, N in [(256, 4096, 11008), (1024, 11008, 4096)]:
            W = synth.weights_device(N, K, 0.02, 3100 + K)
            qw, s, z = W4.quantize_pack(W, GROUP, W4.ASYM)
            del W
            X = synth.activations_device(M, K, synth.FP16, 3101 + K)
            Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
            for _ in range(5):
                W4.linear(X, qw, s, z, GROUP, out=Y)
    elif name == "prefill":
        for K, N in [(4096, 11008), (11008, 4096)]:
            W = synth.weights_device(N, K, 0.02, 3000 + K)
            qw, s, z = W4.quantize_pack(W, GROUP, W4.ASYM)
            del W
            X = synth.activations_device(4096, K, synth.FP16, 3001 + K)
            Y = torch.empty((4096, N), dtype=torch.float16, device="cuda")
            for _ in range(5):
                W4.linear(X, qw, s, z, GROUP, out=Y)
    elif name == "w8a8":
        for K, N in [(4096, 11008), (11008, 4096)]:
            X = synth.calibration_device(4096, K, synth.FP16, 6000 + K, outlier_frac=0.01, outlier_mult=20.0)
            W = synth.weights_device(N, K, 0.02, 6001 + K)
            s = W4.w8a8_smooth(X, W, 2)
            qw, sw = W4.w8a8_quantize_weight(W, s)
            qx, sx = W4.w8a8_quantize_act(X, s)
            Y = torch.empty((4096, N), dtype=torch.float16, device="cuda")
            for _ in range(5):
                W4.w8a8_linear(qx, sx, qw, sw, out=Y)
    elif name == "kv_batch":
        run_kv_batch(W4, synth, torch, layers=2, timed=False)
    elif name == "w8a16":
        # 8-bit codes: M = 1 and 4 on the 7B shapes over 10 rotating copies (20 launches each), and
        # the prefill at M = 4096 on both shapes (5 launches each)
        for K, N in SHAPES:
            W = synth.weights_device(N, K, 0.02, 9000 + K + N)
            q = W4.w8a16_quantize_pack(W, GROUP, W4.ASYM)
            del W
            cs = [tuple(t.clone() for t in q) for _ in range(10)]
            for M in (1, 4):      # one weight row per wave at M = 1, two at M = 4
                X = synth.activations_device(M, K, synth.FP16, 9 + M)
                Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
                for i in range(20):
                    W4.w8a16_linear(X, *cs[i % 10], GROUP, out=Y)
            del cs
        for K, N in [(4096, 11008), (11008, 4096)]:
            W = synth.weights_device(N, K, 0.02, 9200 + K)
            q = W4.w8a16_quantize_pack(W, GROUP, W4.ASYM)
            del W
            X = synth.activations_device(4096, K, synth.FP16, 9201 + K)
            Y = torch.empty((4096, N), dtype=torch.float16, device="cuda")
            for _ in range(5):
                W4.w8a16_linear(X, *q, GROUP, out=Y)
    elif name == "c3":
        # the 70B-like decode shapes (bf16 with outlier channels and weights), M = 1, 4, 16,
        # over 4 rotating copies (>= 140 MB apart in HBM), 20 launches each
        for i, (K, N) in enumerate([(8192, 8192), (8192, 28672), (28672, 8192)]):
            W = synth.weights_device(N, K, 0.015, 1030 + i, outlier_frac=0.001, outlier_mult=20.0)
            q = W4.quantize_pack(W, GROUP, W4.ASYM)
            del W
            cs = [q] + [tuple(t.clone() for t in q) for _ in range(3)]
            for M in (1, 4, 16):
                X = synth.activations_device(M, K, synth.BF16, 1035 + M, outlier_frac=0.01, outlier_mult=100.0)
                Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
                for j in range(20):
                    W4.linear(X, *cs[j % 4], GROUP, out=Y)
            del cs, q
    elif name == "decode_m16":
        for K, N in SHAPES:
            W = synth.weights_device(N, K, 0.02, 1000 + K + N)
            qw, s, z = W4.quantize_pack(W, GROUP, W4.ASYM)
            del W
            cs = [(qw.clone(), s.clone(), z.clone()) for _ in range(20)]
            X = synth.activations_device(16, K, synth.FP16, 7)
            Y = torch.empty((16, N), dtype=torch.float16, device="cuda")
            for i in range(20):
                W4.linear(X, *cs[i], GROUP, out=Y)
            del cs
    else:
        raise SystemExit(f"unknown profile workload {name}")
    torch.cuda.synchronize()
    log(f"profile run done: {name}")


def _counter_means(run_dir: str, counter: str):
    """Mean per-dispatch value of `counter` for each kernel name in a rocprofv3 csv run."""
    import csv
    import glob
    files = glob.glob(os.path.join(run_dir, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {run_dir}")
    vals = {}
    for r in csv.DictReader(open(files[0])):
        if r.get("Counter_Name") != counter:
            continue
        vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return vals


def traffic_parse(fetch_dir: str, write_dir: str, shape, commands, out_path=None):
    """Turn the FETCH_SIZE / WRITE_SIZE passes of traffic_run into HBM bytes per launch
    of the layer's (or the grouped step's) kernel, scaled by what the counters read for the
    known-size copy."""
    kname = KERNEL_NAMES[shape]
    shapes = SHAPES if shape == "step" else [shape]
    out = {"kernel": kname, "M": 1, "layers_KN": shapes, "group_size": GROUP,
           "source_sha256": source_hash(), "copy_bytes": COPY_MIB << 20,
           "algorithmic_bytes_per_launch": sum(weight_bytes(N, K, GROUP) for K, N in shapes),
           "commands": commands}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        vals = _counter_means(d, counter)
        kv = [v for name, vs in vals.items() if kname in name for v in vs]
        cv = [v for name, vs in vals.items() if "neg_kernel" in name for v in vs]
        if not kv or not cv:
            raise SystemExit(f"{counter}: kernel or copy dispatches not found in {d}: {list(vals)}")
        kv = kv[3:] if len(kv) > 6 else kv          # the first dispatches are warm-up
        key = counter.split("_")[0].lower()
        out[f"{key}_kib_per_launch"] = sum(kv) / len(kv)
        out[f"copy_{key}_kib"] = sum(cv) / len(cv)
        out[f"factor_{key}"] = out["copy_bytes"] / (out[f"copy_{key}_kib"] * 1024.0)
    out["traffic_bytes_per_launch"] = round(out["fetch_kib_per_launch"] * 1024 * out["factor_fetch"] +
                                            out["write_kib_per_launch"] * 1024 * out["factor_write"])
    out["traffic_over_algorithmic"] = out["traffic_bytes_per_launch"] / out["algorithmic_bytes_per_launch"]
    out_path = out_path or traffic_file(shape)
    os.makedirs(os.path.dirname(out_path), exist_ok=True)
    with open(out_path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def _library_kernel(name: str) -> bool:
    """False for the framework's own helper kernels that a profiled workload launches while it
    sets up inputs (torch's random generators, sorts, casts): summaries leave them out."""
    return not (name.startswith("at::") or name.startswith("void at::") or "rocprim::" in name
                or "randperm" in name or name.startswith("(anonymous namespace)::elementwise")
                or name.startswith("void (anonymous namespace)::elementwise"))


def trace_summary(run_dir: str, out_path: str, header: str = ""):
    """Per-kernel duration statistics of a rocprofv3 --kernel-trace --stats run: calls, average,
    p10, median, p90, min, max and share of the total, from every dispatch's end - start in the
    run's kernel_trace csv (all csv files under run_dir); torch's setup kernels left out."""
    import csv
    import glob
    durs = {}
    for f in glob.glob(os.path.join(run_dir, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            for row in csv.DictReader(fh):
                name = row.get("Kernel_Name") or row.get("Name") or "?"
                if not _library_kernel(name):
                    continue
                d = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1000.0
                durs.setdefault(name, []).append(d)
    if not durs:
        raise SystemExit(f"no kernel_trace csv under {run_dir}")
    total = sum(sum(v) for v in durs.values())

    def short(n):
        n = n.split("(")[0] if "(" in n and not n.startswith("void") else n
        n = n.replace("w4a16::(anonymous namespace)::", "").replace("void ", "")
        return n[:92]

    def pct(v, q):
        v = sorted(v)
        return v[min(len(v) - 1, int(q * (len(v) - 1) + 0.5))]
    lines = [header.rstrip("\n")] if header else []
    lines.append(f"{'kernel':<92} {'calls':>6} {'avg_us':>8} {'p10_us':>8} {'med_us':>8} {'p90_us':>8} "
                 f"{'min_us':>8} {'max_us':>8} {'pct':>6}")
    for name, v in sorted(durs.items(), key=lambda kv: -sum(kv[1])):
        lines.append(f"{short(name):<92} {len(v):>6} {sum(v) / len(v):>8.2f} {pct(v, 0.1):>8.2f} "
                     f"{pct(v, 0.5):>8.2f} {pct(v, 0.9):>8.2f} {min(v):>8.2f} {max(v):>8.2f} "
                     f"{100 * sum(v) / total:>6.2f}")
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines[:40]))


def counter_summary(run_dirs, out_path: str, header: str = ""):
    """Per-kernel means of the counters of one or more rocprofv3 --pmc runs (each run's
    counter_collection csv), with derived figures: matrix-core busy share, L2 hit rate and
    miss bytes, instructions per wave, the share of wave cycles spent waiting, LDS bank
    conflict cycles, address-unit busy share and L1 requests to L2 per L1 access.  Counter
    values are means per dispatch."""
    import csv
    import glob
    sums, grid = {}, {}
    for d in run_dirs:
        for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if not _library_kernel(r["Kernel_Name"]):
                        continue
                    k = (r["Kernel_Name"], r.get("Grid_Size") or "?")     # one entry per launch shape
                    sums.setdefault(k, {}).setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
                    grid[k] = k[1]
    if not sums:
        raise SystemExit(f"no counter_collection csv under {run_dirs}")

    def short(n):
        return n.replace("w4a16::(anonymous namespace)::", "").replace("void ", "").split("(unsigned")[0][:90]

    lines = [header.rstrip("\n")] if header else []
    for k in sorted(sums, key=lambda k: -max(sum(v) for v in sums[k].values())):
        c = {n: sum(v) / len(v) for n, v in sums[k].items()}
        lines.append(f"{short(k[0])}  (grid {grid.get(k, '?')} threads)")
        lines.append("  raw: " + ", ".join(f"{n}={c[n]:.0f}" for n in sorted(c)))
        d = []
        if "SQ_VALU_MFMA_BUSY_CYCLES" in c and c.get("GRBM_GUI_ACTIVE"):
            d.append(f"MFMA busy {100 * (c['SQ_VALU_MFMA_BUSY_CYCLES'] / 1024) / (c['GRBM_GUI_ACTIVE'] / 8):.1f} %")
        if "TCC_HIT_sum" in c and "TCC_MISS_sum" in c:
            t = c["TCC_HIT_sum"] + c["TCC_MISS_sum"]
            d.append(f"L2 hit rate {100 * c['TCC_HIT_sum'] / max(t, 1):.1f} %, miss bytes "
                     f"{c['TCC_MISS_sum'] * 128 / 1e6:.1f} MB")
        w = c.get("SQ_WAVES")
        if w:
            per = [f"{c[n] / w:.0f} {lab}" for n, lab in (("SQ_INSTS_VALU", "VALU"), ("SQ_INSTS_MFMA", "MFMA"),
                                                           ("SQ_INSTS_VMEM_RD", "VMEM reads"), ("SQ_INSTS_LDS", "LDS"),
                                                           ("SQ_INSTS_SALU", "SALU")) if n in c]
            if per:
                d.append("per wave: " + ", ".join(per))
        wc = c.get("SQ_WAVE_CYCLES")
        if wc:
            fr = [f"{lab} {100 * c[n] / wc:.0f} %" for n, lab in (("SQ_WAIT_ANY", "any"),
                                                                  ("SQ_WAIT_INST_ANY", "on instruction dependencies"))
                  if n in c]
            if fr:
                d.append("waiting: " + ", ".join(fr))
        if "SQ_LDS_BANK_CONFLICT" in c:
            d.append(f"LDS bank conflict cycles {c['SQ_LDS_BANK_CONFLICT']:.0f}")
        if "TA_BUSY_avr" in c and c.get("GRBM_GUI_ACTIVE"):
            d.append(f"address unit (TA) busy {100 * c['TA_BUSY_avr'] / (c['GRBM_GUI_ACTIVE'] / 8):.0f} %")
        if "TCP_TCC_READ_REQ_sum" in c and c.get("TCP_TOTAL_CACHE_ACCESSES_sum"):
            d.append(f"L1 read requests to L2 per L1 access {c['TCP_TCC_READ_REQ_sum'] / c['TCP_TOTAL_CACHE_ACCESSES_sum']:.2f}")
        lines.append("  derived: " + "; ".join(d))
    with open(out_path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    print("\n".join(lines[:60]))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--rotate-gib", type=float, default=1.0)
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extras", action="store_true")
    ap.add_argument("--traffic-run", nargs="+", metavar="K N | step",
                    help="counter workload: calibration copy + the layer's kernel at M = 1, or the "
                         "grouped M = 1 step")
    ap.add_argument("--traffic-parse", nargs="+", metavar="FETCH_DIR WRITE_DIR K N | step",
                    help="write profiles/traffic_*.json from the two counter passes")
    ap.add_argument("--traffic-commands", nargs="*", default=[],
                    help="the profiler command lines, recorded in the traffic file")
    ap.add_argument("--traffic-out", default=None, help="output path of --traffic-parse")
    ap.add_argument("--trace-summary", nargs=2, metavar=("RUN_DIR", "OUT"),
                    help="per-kernel duration statistics of a rocprofv3 --kernel-trace run")
    ap.add_argument("--trace-header", default="", help="text put above the --trace-summary table")
    ap.add_argument("--counter-summary", nargs="+", metavar="RUN_DIR... OUT",
                    help="per-kernel counter means and derived figures of rocprofv3 --pmc runs")
    ap.add_argument("--profile-run", choices=["prefill", "crossover", "w8a8", "kv_batch", "decode_m16", "w8a16", "c3"],
                    help="a short fixed workload of one kernel family, for counter runs")
    args = ap.parse_args()
    if args.trace_summary:
        trace_summary(args.trace_summary[0], args.trace_summary[1], args.trace_header)
        return
    if args.counter_summary:
        if len(args.counter_summary) < 2:
            raise SystemExit("--counter-summary needs at least one run directory and an output path")
        counter_summary(args.counter_summary[:-1], args.counter_summary[-1], args.trace_header)
        return

    def shape_arg(v):
        return "step" if v == ["step"] else (int(v[0]), int(v[1]))
    if args.traffic_parse:
        f, w = args.traffic_parse[:2]
        traffic_parse(f, w, shape_arg(args.traffic_parse[2:]), args.traffic_commands, args.traffic_out)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the W4A16 layer is benchmarked on a single "
              "MI355X (multi-GPU sharding is a design note, not a measured path).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import w4a16_dequant_gemm_amd as W4

    W4.lib()
    torch.cuda.set_device(0)
    if args.traffic_run:
        traffic_run(shape_arg(args.traffic_run), W4, synth, torch, np)
        return
    if args.profile_run:
        profile_run(args.profile_run, W4, synth, torch)
        return
    step_bytes = sum(weight_bytes(N, K, GROUP) for K, N in SHAPES)
    copies = max(2, int(np.ceil(args.rotate_gib * 2**30 / step_bytes)))
    log(f"setup: {len(SHAPES)} layers x {copies} copies ({copies * step_bytes / 2**30:.2f} GiB)")

    X_host = synth.activations(1, 4096, synth.FP16, 1015)
    X_host_k2 = synth.activations(1, 11008, synth.FP16, 1016)
    layers, xs_host, xs_dev = [], [], []
    for i, (K, N) in enumerate(SHAPES):
        layers.append(Layer(K, N, GROUP, copies, 1000 + 10 * 2 + i, W4, synth, torch))
        xh = X_host if K == 4096 else X_host_k2
        xs_host.append(xh)
        xs_dev.append(torch.from_numpy(xh).cuda())

    # host copies of the weights for the oracle leg (the oracle runs after the timing)
    w_host = [L.W.cpu().numpy() for L in layers] if not args.no_cpu else None
    for L in layers:
        del L.W
    torch.cuda.empty_cache()

    outs = [torch.empty((1, L.N), dtype=torch.float16, device="cuda") for L in layers]

    # The step: the three layers are independent, so they run as one w4a16_linear_batch call,
    # one grouped launch that streams all of their weights.  For comparison the same step with
    # one w4a16_linear launch per layer.
    def step(i):
        c = i % copies
        W4.linear_batch([(xd, *L.copies[c], GROUP) for L, xd in zip(layers, xs_dev)], outs=outs)

    def step_separate(i):
        c = i % copies
        for L, xd, o in zip(layers, xs_dev, outs):
            qw, s, z = L.copies[c]
            W4.linear(xd, qw, s, z, GROUP, out=o)

    for i in range(args.warmup):
        step(i)
    # The timed region is a replay of a graph holding exactly `steps` steps, bracketed by
    # synchronize + events; warm-up steps run eagerly and as one warm graph replay.  The
    # replay is timed REPEATS times and the median replay is reported.
    g_main = capture(lambda i: step(i + args.warmup), args.steps, torch)
    ms = time_graph(g_main, args.steps, torch)
    value = step_bytes / (ms * 1e-3) / 1e9
    log(f"step: {ms * 1e3:.1f} us, {value:.1f} GB/s (median of {REPEATS} replays of {args.steps} steps)")
    # the graph replays must reproduce the eager result of the last step, and the grouped
    # launch the per-layer launches, bit for bit
    last = [o.clone() for o in outs]
    step(args.warmup + args.steps - 1)
    torch.cuda.synchronize()
    if not all(torch.equal(a, b) for a, b in zip(last, outs)):
        print(json.dumps({"metric": METRIC, "error": "graph replay differs from eager launch"}))
        sys.exit(1)
    step_separate(args.warmup + args.steps - 1)
    torch.cuda.synchronize()
    if not all(torch.equal(a, b) for a, b in zip(last, outs)):
        print(json.dumps({"metric": METRIC, "error": "grouped launch differs from per-layer launches"}))
        sys.exit(1)
    # steady state: the grouped step is one launch, so >= 200 steps per replay; its per-step
    # time is the grouped kernel's average launch duration (the dominant and only kernel)
    ss_steps = max(args.steps, 200)
    ms_ss = time_loop(lambda i: step(i + args.warmup), ss_steps, torch)
    log(f"steady state: {ms_ss * 1e3:.2f} us per grouped launch over {ss_steps} launches")
    ms_sep = time_loop(lambda i: step_separate(i + args.warmup), max(args.steps, 67), torch)
    log(f"separate launches: {ms_sep * 1e3:.1f} us per step")

    # per-layer launch durations (back-to-back launches of one kernel over the copies)
    per_layer = []
    for L, xd, o in zip(layers, xs_dev, outs):
        def one(i, L=L, xd=xd, o=o):
            qw, s, z = L.copies[i % copies]
            W4.linear(xd, qw, s, z, GROUP, out=o)
        for i in range(10):
            one(i)
        t = time_loop(one, max(args.steps, 200), torch)
        per_layer.append({"K": L.K, "N": L.N, "us": t * 1e3, "bytes": L.bytes,
                          "GBps": L.bytes / (t * 1e-3) / 1e9,
                          "path": W4.PATH_NAMES[W4.select_path(1, L.N, L.K, GROUP)],
                          "kernel": KERNEL_NAMES.get((L.K, L.N), "?")})
        log(f"  layer K={L.K} N={L.N}: {t * 1e3:.2f} us/launch {per_layer[-1]['GBps']:.0f} GB/s")
    achieved = step_bytes / (ms_ss * 1e-3) / 1e9
    traffic = traffic_record("step")
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic["bytes_per_launch"] if traffic else None,
                "kernel": f"{KERNEL_NAMES['step']} (M=1, the three layers in one launch)",
                "avg_launch_us": round(ms_ss * 1e3, 3), "bytes_per_launch": step_bytes,
                "launches_timed": ss_steps}
    if traffic:
        roofline["traffic_source"] = traffic["source"]
    ceiling = read_ceiling(step_bytes, torch)
    roofline["read_ceiling"] = dict(ceiling, frac_of_ceiling=round(achieved / ceiling["GBps"], 4))
    log(f"plain read of the step's bytes in one launch: {ceiling['us']} us, {ceiling['GBps']} GB/s; "
        f"the grouped kernel reaches {achieved / ceiling['GBps']:.1%} of it")

    extras = {"per_layer_m1": per_layer}
    samples = []
    if not args.no_extras:
        extras["comparators"] = run_comparators(W4, synth, torch, ms)
        extras.update(run_extras(layers, copies, W4, synth, torch, np, samples))

    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(layers, w_host, xs_host, last, args.cpu_budget, np, torch, samples)
        log(f"cpu oracle: {cpu['value']:.3f} GB/s on {cpu['cores']} threads; "
            f"parity vs GPU: {cpu['parity_vs_gpu']}")
        if not cpu["parity_vs_gpu"]["ok"]:
            print(json.dumps({"metric": METRIC, "error": "GPU output differs from the oracle",
                              "parity": cpu["parity_vs_gpu"]}))
            sys.exit(1)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 6),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": "decode M=1 on 7B-like layers (K,N) = (4096,4096), "
                               "(4096,11008), (11008,4096), independent; g=128 asym uint4; fp16 activations",
                   "M": 1, "group_size": GROUP, "scheme": "asym", "rotating_copies": copies,
                   "bytes_per_step": step_bytes, "pct_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
                   "launch": "one w4a16_linear_batch call per step (one grouped launch over the three layers)",
                   "timing": f"median of {REPEATS} graph replays of the {args.steps} timed steps",
                   "steady_state": {"launches_per_replay": ss_steps, "us_per_step": round(ms_ss * 1e3, 3),
                                    "GBps": round(step_bytes / (ms_ss * 1e-3) / 1e9, 1)},
                   "separate_launches": {"us_per_step": round(ms_sep * 1e3, 3),
                                         "GBps": round(step_bytes / (ms_sep * 1e-3) / 1e9, 1)}},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "extras": extras,
    }
    print(json.dumps(line), flush=True)


def run_comparators(W4, synth, torch, w4_step_ms):
    """Context for the M = 1 step and the M = 4096 prefill: (1) the same three layers as
    dense fp16 weights through torch.matmul (hipBLASLt), rotating >= 1 GiB of weight copies,
    and the W4A16 step's speedup over it; (2) the unfused path the fused kernels replace:
    dequantize to fp32, cast to fp16, then torch.matmul, at M = 1 and M = 4096; (3) the launch
    gap: back-to-back one-element kernels in a graph, the floor under any short launch."""
    res = {}
    Xs = {K: synth.activations_device(1, K, synth.FP16, 9100 + K) for K in (4096, 11008)}
    per_copy = sum(2 * N * K for K, N in SHAPES)
    ncopy = max(2, -(-(1 << 30) // per_copy))
    Wd = [[torch.randn(N, K, dtype=torch.float16, device="cuda") for K, N in SHAPES] for _ in range(ncopy)]
    Ys = [torch.empty((1, N), dtype=torch.float16, device="cuda") for _, N in SHAPES]

    def dense(i):
        for (K, N), W, Y in zip(SHAPES, Wd[i % ncopy], Ys):
            torch.matmul(Xs[K], W.t(), out=Y)
    for i in range(3):
        dense(i)
    ms = time_loop(dense, 50, torch)
    res["dense_fp16_m1_step"] = {"us": round(ms * 1e3, 2), "GBps_fp16_weights": round(per_copy / (ms * 1e-3) / 1e9, 1),
                                 "w4a16_speedup": round(ms / w4_step_ms, 3)}
    log(f"  dense fp16 M=1 step (torch.matmul): {res['dense_fp16_m1_step']}")
    del Wd
    torch.cuda.empty_cache()
    # unfused: dequantize (fp32) -> fp16 -> matmul
    packed = []
    for K, N in SHAPES:
        W = synth.weights_device(N, K, 0.02, 9200 + K + N)
        packed.append((K, N) + tuple(W4.quantize_pack(W, GROUP, W4.ASYM)))
        del W

    def unfused(i):
        for (K, N, qw, s, z), Y in zip(packed, Ys):
            torch.matmul(Xs[K], W4.dequantize(qw, s, z, GROUP).half().t(), out=Y)
    for i in range(2):
        unfused(i)
    ms_u = time_loop(unfused, 10, torch, graph=False)
    res["unfused_dequant_then_matmul_m1_step"] = {"us": round(ms_u * 1e3, 1), "fused_speedup": round(ms_u / w4_step_ms, 2)}
    log(f"  unfused dequantize + matmul, M=1 step: {res['unfused_dequant_then_matmul_m1_step']}")
    pf = {}
    for K, N, qw, s, z in packed[1:]:
        X = synth.activations_device(4096, K, synth.FP16, 9300 + K)
        Y = torch.empty((4096, N), dtype=torch.float16, device="cuda")
        f_fused = lambda i: W4.linear(X, qw, s, z, GROUP, out=Y)
        f_unf = lambda i: torch.matmul(X, W4.dequantize(qw, s, z, GROUP).half().t(), out=Y)
        for f in (f_fused, f_unf):
            f(0)
        t_f = time_loop(f_fused, 5, torch)
        t_u = time_loop(f_unf, 5, torch)
        pf[f"K{K}_N{N}"] = {"fused_us": round(t_f * 1e3, 1), "unfused_us": round(t_u * 1e3, 1),
                            "fused_speedup": round(t_u / t_f, 2)}
        del X, Y
    res["prefill_m4096_fused_vs_unfused"] = pf
    log(f"  prefill M=4096 fused vs unfused: {pf}")
    del packed
    torch.cuda.empty_cache()
    # read ceilings at the sizes of single layers: 7B-like (8.9 and 24.0 MB) and 70B-like (35.7 and
    # 124.8 MB) packed weights with their scales and zeros
    res["read_ceiling_by_size"] = [read_ceiling(weight_bytes(N, K, GROUP), torch)
                                   for K, N in ((4096, 4096), (4096, 11008), (8192, 8192), (8192, 28672))]
    log(f"  plain-read ceilings: {res['read_ceiling_by_size']}")
    # launch gap
    one = torch.zeros(1, dtype=torch.float32, device="cuda")
    ms_l = time_loop(lambda i: one.add_(1.0), 200, torch)
    res["launch_gap_us"] = round(ms_l * 1e3, 3)
    log(f"  back-to-back one-element kernels: {res['launch_gap_us']} us each")
    return res


def run_extras(layers, copies, W4, synth, torch, np, samples):
    out = {}
    # decode sweep M in 2..16 on the same rotating layers
    sweep = {}
    for M in (2, 4, 8, 16):
        xs = {K: synth.activations_device(M, K, synth.FP16, 2000 + M) for K in (4096, 11008)}
        outs = [torch.empty((M, L.N), dtype=torch.float16, device="cuda") for L in layers]
        nbytes = sum(L.bytes for L in layers)

        def step(i):
            c = i % copies
            for L, o in zip(layers, outs):
                qw, s, z = L.copies[c]
                W4.linear(xs[L.K], qw, s, z, GROUP, out=o)

        def step_batch(i):
            c = i % copies
            W4.linear_batch([(xs[L.K], *L.copies[c], GROUP) for L in layers], outs=outs)
        for i in range(5):
            step(i)
            step_batch(i)
        ms = time_loop(step, 50, torch)
        ms_b = time_loop(step_batch, 50, torch)
        sweep[f"M{M}"] = {"GBps": round(nbytes / (ms * 1e-3) / 1e9, 1), "us_per_step": round(ms * 1e3, 2),
                          "paths": [W4.PATH_NAMES[W4.select_path(M, L.N, L.K, GROUP)] for L in layers],
                          "batch_call": {"GBps": round(nbytes / (ms_b * 1e-3) / 1e9, 1),
                                         "us_per_step": round(ms_b * 1e3, 2)}}
        log(f"  sweep M={M}: {sweep[f'M{M}']}")
    out["decode_sweep_fp16_g128"] = sweep
    # each kernel path forced, per M (same layers, same rotation)
    per_path = {}
    for M in (1, 2, 4, 8, 16):
        xs = {K: synth.activations_device(M, K, synth.FP16, 2100 + M) for K in (4096, 11008)}
        outs = [torch.empty((M, L.N), dtype=torch.float16, device="cuda") for L in layers]
        nbytes = sum(L.bytes for L in layers)
        for path in (W4.PATH_GEMV, W4.PATH_SKINNY):
            if path == W4.PATH_GEMV and M > 8:
                continue

            def step(i, path=path):
                c = i % copies
                for L, o in zip(layers, outs):
                    qw, s, z = L.copies[c]
                    W4.linear(xs[L.K], qw, s, z, GROUP, path=path, out=o)
            for i in range(3):
                step(i)
            ms = time_loop(step, 50, torch)
            per_path[f"M{M}_{W4.PATH_NAMES[path]}"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    log(f"  per-path GB/s: {per_path}")
    out["decode_per_path_GBps"] = per_path
    out["c3_decode_70b_bf16_outliers"] = run_c3(W4, synth, torch, np, samples)
    out["c4_prefill_crossover_fp16"] = run_c4(W4, synth, torch, np, samples)
    out["gptq_4096x4096_g128"] = run_gptq(W4, synth, torch)
    out["awq_4096x4096_g128"] = run_awq(W4, synth, torch)
    out["w8a8_m4096"] = run_w8a8(W4, synth, torch)
    out["kv_decode_attention_h32_d128_t4096"] = run_kv(W4, synth, torch)
    out["full_stack_7b_32_layers"] = run_stack(W4, synth, torch, np, samples)
    out["w8a16_g128"] = run_w8a16(W4, synth, torch)
    return out


def parity_sample(name, case_dtype, g, scheme, Wd, qw, s, z, X, Y, torch, np, n_cols=128, m_rows=16):
    """Sampled inputs and GPU results of a timed configuration for the oracle leg: the fp32
    weights, packed rows, scales and zero points of ``n_cols`` output columns, ``m_rows``
    activation rows and the matching outputs (host copies).  Nothing is computed here."""
    N, M = qw.shape[0], X.shape[0]
    rng = np.random.default_rng(N + M + g)
    ns = np.unique(np.concatenate([[0, N - 1], rng.choice(N, min(n_cols, N), replace=False)]))
    ms = np.unique(np.concatenate([[0, M - 1], rng.choice(M, min(m_rows, M), replace=False)]))
    ni, mi = torch.from_numpy(ns).cuda(), torch.from_numpy(ms).cuda()
    xh = X[mi].view(torch.int16).cpu().numpy()
    return {"name": name, "dtype": case_dtype, "g": g, "scheme": scheme,
            "W": Wd[ni].cpu().numpy(), "qw": qw[ni].cpu().numpy(),
            "s": s[ni].cpu().numpy(), "z": None if z is None else z[ni].cpu().numpy(),
            "X": xh.view(np.float16) if case_dtype == 0 else xh.view(np.uint16),
            "Y": Y[mi][:, ni].view(torch.int16).cpu().numpy().view(np.uint16)}


def run_c3(W4, synth, torch, np, samples):
    """The 70B-like decode shapes: M in {1, 4, 16} on (K, N) = (8192, 8192), (8192, 28672),
    (28672, 8192), g = 128 asymmetric, bf16 activations ~ N(0, 1) with 1 % of the channels
    x100, weights ~ N(0, 0.015) with 0.1 % of the entries x20.  Each layer rotates through
    >= 1 GiB of weight copies; >= 200 back-to-back launches per replay (graph), median of 5
    replays; effective weight-stream GB/s = (packed + scale/zero bytes) / launch time."""
    res = {}
    shapes = [(8192, 8192), (8192, 28672), (28672, 8192)]
    for i, (K, N) in enumerate(shapes):
        sw, sx = synth.seeds(3, i)
        Wd = synth.weights_device(N, K, 0.015, sw, outlier_frac=0.001, outlier_mult=20.0)
        q = W4.quantize_pack(Wd, GROUP, W4.ASYM)
        nbytes = weight_bytes(N, K, GROUP)
        copies = max(2, -(-2**30 // nbytes))
        cs = [q] + [tuple(t.clone() for t in q) for _ in range(copies - 1)]
        for M in (1, 4, 16):
            X = synth.activations_device(M, K, synth.BF16, sx + M, outlier_frac=0.01, outlier_mult=100.0)
            Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

            def one(j, X=X, Y=Y, cs=cs):
                qw, sc, z = cs[j % copies]
                W4.linear(X, qw, sc, z, GROUP, out=Y)
            for j in range(5):
                one(j)
            t = time_loop(one, 200, torch)
            gbps = nbytes / (t * 1e-3) / 1e9
            key = f"M{M}_K{K}_N{N}"
            res[key] = {"us": round(t * 1e3, 2), "GBps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBS, 4),
                        "bytes_per_launch": nbytes, "rotating_copies": copies,
                        "path": W4.PATH_NAMES[W4.select_path(M, N, K, GROUP, W4.BF16)]}
            log(f"  C3 {key}: {res[key]}")
            one(0)
            samples.append(parity_sample(f"C3_{key}", 1, GROUP, W4.ASYM, Wd, *cs[0], X, Y, torch, np))
        del Wd, cs, q
        torch.cuda.empty_cache()
    return res


def run_c4(W4, synth, torch, np, samples):
    """The prefill / compute-bound crossover: M in {256, 1024, 4096} on (K, N) = (4096, 11008)
    and (11008, 4096), g in {64, 128}, symmetric absmax and asymmetric uint4, fp16
    activations; TFLOP/s = 2 M N K / launch time (graph of 10 launches, median of 5 replays),
    the kernel the dispatcher took, the workspace form where it splits K, and a dense fp16
    GEMM of the same shape with fp16 weights (torch.matmul / hipBLASLt) as context."""
    res = {}
    for (K, N) in [(4096, 11008), (11008, 4096)]:
        X = synth.activations_device(4096, K, synth.FP16, 3001 + K)
        Y = torch.empty((4096, N), dtype=torch.float16, device="cuda")
        Wd16 = torch.randn(N, K, dtype=torch.float16, device="cuda")
        for g in (64, 128):
            for scheme in (W4.SYM, W4.ASYM):
                Wd = synth.weights_device(N, K, 0.02, 3000 + K + g + scheme)
                qw, s, z = W4.quantize_pack(Wd, g, scheme)
                sname = "asym" if scheme == W4.ASYM else "sym"
                for M in (256, 1024, 4096):
                    Xs, Ys = X[:M], Y[:M]
                    for _ in range(3):
                        W4.linear(Xs, qw, s, z, g, out=Ys)
                    t = time_loop(lambda i: W4.linear(Xs, qw, s, z, g, out=Ys), 10, torch)
                    tf = 2.0 * M * N * K / (t * 1e-3) / 1e12
                    key = f"M{M}_K{K}_N{N}_g{g}_{sname}"
                    rec = {"TFLOPs": round(tf, 1), "us": round(t * 1e3, 1),
                           "frac_mfma_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4),
                           "path": W4.PATH_NAMES[W4.select_path(M, N, K, g)]}
                    need = W4.linear_workspace(M, N, K, g)
                    if need > 0:   # the workspace form: K split over the idle CUs
                        work = torch.empty((need + 3) // 4, dtype=torch.float32, device="cuda")
                        for _ in range(3):
                            W4.linear_ws(Xs, qw, s, z, g, work=work, out=Ys)
                        tw = time_loop(lambda i: W4.linear_ws(Xs, qw, s, z, g, work=work, out=Ys), 10, torch)
                        rec["split_k_workspace"] = {"us": round(tw * 1e3, 1),
                                                    "TFLOPs": round(2.0 * M * N * K / (tw * 1e-3) / 1e12, 1),
                                                    "workspace_MB": round(need / 2**20, 1)}
                        del work
                    if g == 128 and scheme == W4.ASYM:
                        for _ in range(3):
                            torch.matmul(Xs, Wd16.t(), out=Ys)
                        td = time_loop(lambda i: torch.matmul(Xs, Wd16.t(), out=Ys), 10, torch, graph=False)
                        rec["dense_fp16_torch_TFLOPs"] = round(2.0 * M * N * K / (td * 1e-3) / 1e12, 1)
                    res[key] = rec
                    log(f"  C4 {key}: {rec}")
                    W4.linear(Xs, qw, s, z, g, out=Ys)
                    samples.append(parity_sample(f"C4_{key}", 0, g, scheme, Wd, qw, s, z, Xs, Ys, torch, np))
                del Wd, qw, s, z
        del X, Y, Wd16
        torch.cuda.empty_cache()
    return res


def run_w8a16(W4, synth, torch):
    """W8A16 (8-bit codes, g = 128 asym, fp16): the M = 1 step on the three 7B-like layers
    (graph-captured, rotating >= 1 GiB of weight copies; bytes = N K + 4 N K / g per layer)
    and each layer at M = 4, and the prefill at M = 4096 on both shapes (TFLOP/s)."""
    res = {}
    shapes = SHAPES
    per_copy = sum(N * K + 4 * N * K // GROUP for K, N in shapes)
    copies = max(2, int(-(-2**30 // per_copy)))
    layers = []
    for i, (K, N) in enumerate(shapes):
        W = synth.weights_device(N, K, 0.02, 9000 + i)
        q = W4.w8a16_quantize_pack(W, GROUP, W4.ASYM)
        del W
        layers.append((K, N, [q] + [tuple(t.clone() for t in q) for _ in range(copies - 1)]))
    for M in (1, 4):
        xs = {K: synth.activations_device(M, K, synth.FP16, 9100 + K + M) for K in (4096, 11008)}
        ys = [torch.empty((M, N), dtype=torch.float16, device="cuda") for K, N, _ in layers]

        def step(i, xs=xs, ys=ys):
            for (K, N, cs), y in zip(layers, ys):
                qw, sc, z = cs[i % copies]
                W4.w8a16_linear(xs[K], qw, sc, z, GROUP, out=y)
        for i in range(3):
            step(i)
        ms = time_loop(step, 50, torch)
        gbps = per_copy / (ms * 1e-3) / 1e9
        res[f"step_M{M}"] = {"us": round(ms * 1e3, 2), "GBps": round(gbps, 1), "frac_hbm_peak": round(gbps / HBM_PEAK_GBS, 4),
                             "paths": [W4.PATH_NAMES[W4.w8a16_select_path(M, N, K, GROUP)] for K, N, _ in layers]}
        log(f"  w8a16 step M={M}: {res[f'step_M{M}']}")
    del layers
    torch.cuda.empty_cache()
    pre = {}
    for (K, N) in [(4096, 11008), (11008, 4096)]:
        W = synth.weights_device(N, K, 0.02, 9200 + K)
        qw, sc, z = W4.w8a16_quantize_pack(W, GROUP, W4.ASYM)
        del W
        X = synth.activations_device(4096, K, synth.FP16, 9201 + K)
        Y = torch.empty((4096, N), dtype=torch.float16, device="cuda")
        for _ in range(3):
            W4.w8a16_linear(X, qw, sc, z, GROUP, out=Y)
        ms = time_loop(lambda i: W4.w8a16_linear(X, qw, sc, z, GROUP, out=Y), 10, torch)
        tf = 2.0 * 4096 * N * K / (ms * 1e-3) / 1e12
        pre[f"K{K}_N{N}"] = {"TFLOPs": round(tf, 1), "us": round(ms * 1e3, 1),
                             "frac_mfma_peak": round(tf / MFMA_F16_PEAK_TFLOPS, 4)}
        log(f"  w8a16 prefill M=4096 K={K} N={N}: {pre[f'K{K}_N{N}']}")
        del qw, sc, z, X, Y
    res["prefill_m4096"] = pre
    return res


def run_stack(W4, synth, torch, np, samples):
    """The full decode step of a 32-layer 7B-shaped stack: 224 linears (q, k, v, o, gate, up,
    down per layer), about 3.5 GB of packed weights, bf16 activations, launched back to back on
    one stream (graph-captured); g = 128 and the per-channel variant (g = K), each at M = 1 and
    M = 8.  Bytes: every linear's packed weights and metadata."""
    res = {}
    for per_channel in (False, True):
        layers = []
        for c in synth.stack_cases(1, per_channel):
            W = synth.weights_device(c.N, c.K, c.w_sigma, synth.seeds(c.config, c.layer)[0])
            qw, s, z = W4.quantize_pack(W, c.g, c.scheme)
            del W
            layers.append((c, qw, s, z))
        nbytes = sum(weight_bytes(c.N, c.K, c.g) for c, *_ in layers)
        for M in (1, 8):
            xs = {K: synth.activations_device(M, K, synth.BF16, 8000 + K + M) for K in (4096, 11008)}
            ys = [torch.empty((M, c.N), dtype=torch.bfloat16, device="cuda") for c, *_ in layers]

            def step(i, xs=xs, ys=ys, layers=layers):
                for (c, qw, s, z), y in zip(layers, ys):
                    W4.linear(xs[c.K], qw, s, z, c.g, out=y)
            for i in range(2):
                step(i)
            ms = time_loop(step, 5, torch)
            gbps = nbytes / (ms * 1e-3) / 1e9
            key = f"{'per_channel' if per_channel else 'g128'}_M{M}"
            res[key] = {"ms_per_step": round(ms, 3), "GBps": round(gbps, 1),
                        "frac_hbm_peak": round(gbps / HBM_PEAK_GBS, 4), "weight_GB": round(nbytes / 1e9, 3)}
            log(f"  full stack {key}: {res[key]}")
            # the same step with each transformer layer's independent projections batched:
            # w4a16_linear_batch over (q, k, v) and over (gate, up), then o and down alone
            # (4 launches per layer instead of 7; the dependencies of a real layer kept;
            # M = 1: the grouped GEMV, M = 8: the grouped ring decode kernel)
            def step_b(i, xs=xs, ys=ys, layers=layers):
                for l0 in range(0, len(layers), 7):
                    grp = [(xs[c.K], qw, s, z, c.g) for c, qw, s, z in layers[l0:l0 + 7]]
                    out = ys[l0:l0 + 7]
                    W4.linear_batch(grp[0:3], outs=out[0:3])
                    W4.linear(*grp[3], out=out[3])
                    W4.linear_batch(grp[4:6], outs=out[4:6])
                    W4.linear(*grp[6], out=out[6])
            for i in range(2):
                step_b(i)
            msb = time_loop(step_b, 5, torch)
            gb = nbytes / (msb * 1e-3) / 1e9
            res[key + "_batched_qkv_gateup"] = {"ms_per_step": round(msb, 3), "GBps": round(gb, 1),
                                                "frac_hbm_peak": round(gb / HBM_PEAK_GBS, 4),
                                                "launches_per_step": 128}
            log(f"  full stack {key}, q/k/v and gate/up batched: {res[key + '_batched_qkv_gateup']}")
            c, qw, s, z = layers[-1]          # the last layer's down projection
            step(0)
            Wd = synth.weights_device(c.N, c.K, c.w_sigma, synth.seeds(c.config, c.layer)[0])
            samples.append(parity_sample(f"C5_{key}_down", 1, c.g, c.scheme, Wd, qw, s, z, xs[c.K], ys[-1], torch, np))
            del ys, xs, Wd
        del layers
        torch.cuda.empty_cache()
    # context: the same step with q, k, v and gate, up concatenated along N (one launch each,
    # the usual serving layout; the same kernels at N = 12288 and N = 22016), g = 128, M = 1
    fused = [(4096, 12288), (4096, 4096), (4096, 22016), (11008, 4096)]
    layers = []
    for layer in range(32):
        for j, (K, N) in enumerate(fused):
            W = synth.weights_device(N, K, 0.02, 9000 + 4 * layer + j)
            layers.append((K, N) + tuple(W4.quantize_pack(W, GROUP, W4.ASYM)))
            del W
    nbytes = sum(weight_bytes(N, K, GROUP) for K, N, *_ in layers)
    xs = {K: synth.activations_device(1, K, synth.BF16, 8100 + K) for K in (4096, 11008)}
    ys = [torch.empty((1, N), dtype=torch.bfloat16, device="cuda") for _, N, *_ in layers]

    def step_fused(i):
        for (K, N, qw, s, z), y in zip(layers, ys):
            W4.linear(xs[K], qw, s, z, GROUP, out=y)
    for i in range(2):
        step_fused(i)
    ms = time_loop(step_fused, 5, torch)
    gbps = nbytes / (ms * 1e-3) / 1e9
    res["g128_M1_fused_qkv_gateup"] = {"ms_per_step": round(ms, 3), "GBps": round(gbps, 1),
                                       "frac_hbm_peak": round(gbps / HBM_PEAK_GBS, 4),
                                       "weight_GB": round(nbytes / 1e9, 3)}
    log(f"  full stack fused q/k/v and gate/up, M=1: {res['g128_M1_fused_qkv_gateup']}")
    del layers, ys
    torch.cuda.empty_cache()
    return res


def run_kv(W4, synth, torch, H=32, D=128, T=4096, layers=32):
    """Decode attention of a 32-head, head-dim-128 model over a 4096-token quantized cache,
    one query per head, across 32 layers (a different cache each, 0.5-1.1 GB in all, so no
    layer's cache stays in the last-level cache).  Roofline: HBM, algorithmic bytes = the
    codes and per-token parameters of K and V plus q and the output.  The per-token
    quantization of a whole 4096-token cache is timed beside it (bytes: fp16 in, codes and
    parameters out)."""
    res = {}
    q = synth.activations_device(H, D, synth.FP16, 7000)
    out = torch.empty_like(q)
    work = torch.empty(W4.kv_attention_workspace(H, T, D), dtype=torch.float32, device="cuda")
    for bits in (8, 4):
        caches = []
        for l in range(layers):
            k = synth.activations_device(H * T, D, synth.FP16, 7100 + 2 * l).view(H, T, D)
            v = synth.activations_device(H * T, D, synth.FP16, 7101 + 2 * l).view(H, T, D)
            caches.append((W4.kv_quantize(k, bits), W4.kv_quantize(v, bits)))
            del v
        row = D * bits // 8 + (2 if bits == 8 else 4)
        nbytes = layers * (2 * H * T * row + 2 * 2 * H * D)

        def step(i, bits=bits, caches=caches):
            for kc, vc in caches:
                W4.kv_attention_decode(q, kc, vc, T, bits, out=out, work=work)
        for i in range(3):
            step(i)
        ms = time_loop(step, 20, torch)
        gbps = nbytes / (ms * 1e-3) / 1e9
        ms_q = time_loop(lambda i, k=k, bits=bits: W4.kv_quantize(k, bits), 20, torch, graph=False)
        qbytes = H * T * (2 * D + row)
        entry = {"attention_us_per_layer": round(ms * 1e3 / layers, 2), "attention_GBps": round(gbps, 1),
                 "frac_hbm_peak": round(gbps / HBM_PEAK_GBS, 4),
                 "quantize_us": round(ms_q * 1e3, 1), "quantize_GBps": round(qbytes / (ms_q * 1e-3) / 1e9, 1)}
        res[f"kv{bits}"] = entry
        log(f"  kv{bits} decode attention H={H} D={D} T={T}: {entry}")
        del caches, k
    res["batch16"] = run_kv_batch(W4, synth, torch, H=H, D=D)
    return res


def run_kv_batch(W4, synth, torch, B=16, H=32, D=128, Tmax=4096, layers=4, timed=True):
    """Decode attention for a batch of 16 sequences in one call (the serving case the cache
    quantization is for), lengths drawn uniformly from [1024, 4096] (seeded), 4 layers'
    caches in rotation (1.4-2.2 GB).  Bytes: each sequence's codes and per-token parameters
    over its own length, plus q and the output."""
    import numpy as np
    lens = np.random.default_rng(7300).integers(1024, Tmax + 1, size=B).astype(np.int32)
    lt = torch.from_numpy(lens).cuda()
    q = synth.activations_device(B * H, D, synth.FP16, 7301).view(B, H, D)
    out = torch.empty_like(q)
    work = torch.empty(W4.kv_attention_batch_workspace(B, H, Tmax, D), dtype=torch.float32, device="cuda")
    res = {"lengths": [int(x) for x in lens]}
    for bits in (8, 4):
        caches = []
        for l in range(layers):
            pair = []
            for j in range(2):
                x = synth.activations_device(B * H * Tmax, D, synth.FP16, 7400 + 2 * l + j).view(B * H, Tmax, D)
                c, s, z = W4.kv_quantize(x, bits)
                del x
                pair.append((c.view(B, H, Tmax, -1), s.view(B, H, Tmax), None if z is None else z.view(B, H, Tmax)))
            caches.append(pair)
        row = D * bits // 8 + (2 if bits == 8 else 4)
        nbytes = layers * (2 * H * int(lens.sum()) * row + 2 * 2 * B * H * D)

        def step(i, bits=bits, caches=caches):
            for kc, vc in caches:
                W4.kv_attention_decode_batch(q, kc, vc, lt, bits, out=out, work=work)
        for i in range(3 if timed else 2):
            step(i)
        if not timed:
            del caches
            continue
        ms = time_loop(step, 10, torch)
        gbps = nbytes / (ms * 1e-3) / 1e9
        entry = {"us_per_layer": round(ms * 1e3 / layers, 2), "GBps": round(gbps, 1),
                 "frac_hbm_peak": round(gbps / HBM_PEAK_GBS, 4), "cache_MB_per_layer": round(nbytes / layers / 1e6, 1)}
        res[f"kv{bits}"] = entry
        log(f"  kv{bits} decode attention, batch of {B} (T 1024-4096), H={H} D={D}: {entry}")
        del caches
        torch.cuda.empty_cache()
    return res


INT8_PEAK_TOPS = 5000.0              # MI355X dense int8 MFMA


def run_w8a8(W4, synth, torch, M=4096):
    """W8A8 + SmoothQuant at M = 4096 on the two prefill shapes: the INT8 product (roofline:
    int8 MFMA peak, 2 M N K ops) and the per-token activation quantization (HBM: 3 M K bytes
    read + written)."""
    res = {}
    for (K, N) in [(4096, 11008), (11008, 4096)]:
        X = synth.calibration_device(M, K, synth.FP16, 6000 + K, outlier_frac=0.01, outlier_mult=20.0)
        W = synth.weights_device(N, K, 0.02, 6001 + K)
        s = W4.w8a8_smooth(X, W, 2)
        qw, sw = W4.w8a8_quantize_weight(W, s)
        qx, sx = W4.w8a8_quantize_act(X, s)
        Y = torch.empty((M, N), dtype=torch.float16, device="cuda")
        for _ in range(3):
            W4.w8a8_linear(qx, sx, qw, sw, out=Y)
        ms = time_loop(lambda i: W4.w8a8_linear(qx, sx, qw, sw, out=Y), 20, torch)
        tops = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        ms_q = time_loop(lambda i: W4.w8a8_quantize_act(X, s), 20, torch, graph=False)
        entry = {"gemm_us": round(ms * 1e3, 1), "TOPS": round(tops, 1), "frac_int8_peak": round(tops / INT8_PEAK_TOPS, 4),
                 "quant_act_us": round(ms_q * 1e3, 1),
                 "quant_act_GBps": round(3.0 * M * K / (ms_q * 1e-3) / 1e9, 1)}
        try:   # context: the library int8 GEMM behind torch._int_mm, where the installed torch has one
            a = qx
            b = qw.t()
            for _ in range(2):
                torch._int_mm(a, b)
            ms_t = time_loop(lambda i: torch._int_mm(a, b), 10, torch, graph=False)
            entry["torch_int_mm_TOPS"] = round(2.0 * M * N * K / (ms_t * 1e-3) / 1e12, 1)
        except Exception as e:       # noqa: BLE001 - comparator only
            entry["torch_int_mm_TOPS"] = None
        res[f"K{K}_N{N}"] = entry
        log(f"  w8a8 M={M} K={K} N={N}: {entry}")
        del X, W, qw, sw, qx, sx, Y, s
    return res


def run_awq(W4, synth, torch, n=512, K=4096, N=4096, reps=3):
    """AWQ of one 4096 x 4096 layer from 512 calibration rows with outlier channels: the
    statistic and the nine-candidate search timed with events; algorithmic fp64 flops of the
    search are its nine output-error products, 9 * 2 n N K."""
    X = synth.calibration_device(n, K, synth.FP16, 5001, outlier_frac=0.01, outlier_mult=20.0)
    W = synth.weights_device(N, K, 0.02, 5002)
    best_ms = {"stats": None, "search": None}
    res = None
    for _ in range(reps):
        torch.cuda.synchronize()
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record()
        xm = W4.awq_stats(X)
        e[1].record()
        res = W4.awq_search(W, X, xm, GROUP, W4.ASYM)
        e[2].record()
        torch.cuda.synchronize()
        for k, (a, b) in (("stats", (0, 1)), ("search", (1, 2))):
            ms = e[a].elapsed_time(e[b])
            best_ms[k] = ms if best_ms[k] is None else min(best_ms[k], ms)
    losses = res[4].cpu().numpy()
    best = int(res[5].cpu().numpy()[0])
    flops = 9 * 2.0 * n * N * K
    tf = flops / (best_ms["search"] * 1e-3) / 1e12
    out = {"stats_ms": round(best_ms["stats"], 3), "search_ms": round(best_ms["search"], 3),
           "search_fp64_TFLOPs": round(tf, 2), "frac_fp64_peak": round(tf / FP64_PEAK_TFLOPS, 4),
           "best_exponent_quarters": best - 4,
           "loss_vs_rtn": round(float(losses[best] / losses[4]), 4)}
    log(f"  awq 4096x4096 (n=512): {out}")
    del X, W, res
    return out


def run_gptq(W4, synth, torch, n=2048, K=4096, N=4096, reps=3):
    """GPTQ of one 4096 x 4096 layer from 2048 calibration rows: each entry point timed with
    events on its own; algorithmic fp64 flops: Hessian lower triangle n K (K + 1), factor
    (Cholesky + triangular inverse) 2 K^3 / 3, column compensation N K (K - 1)."""
    X = synth.activations_device(n, K, synth.FP16, 4001)
    W = synth.weights_device(N, K, 0.02, 4002)

    def timed(fn, prep=None):
        best = None
        for _ in range(reps):
            arg = prep() if prep else None
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            r = fn(arg)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        return best, r

    ms_h, H = timed(lambda _: W4.gptq_hessian(X))
    ms_f, U = timed(lambda Hc: W4.gptq_factor(Hc, 0.01), prep=lambda: H.clone())
    work = torch.empty(N * K + 64 * N, dtype=torch.float64, device="cuda")
    ms_q, _ = timed(lambda _: W4.gptq_quantize(W, U, GROUP, W4.ASYM, work=work))
    res = {}
    for name, ms, flops in (("hessian", ms_h, n * K * (K + 1)), ("factor", ms_f, 2 * K ** 3 / 3),
                            ("quantize", ms_q, N * K * (K - 1))):
        tf = flops / (ms * 1e-3) / 1e12
        res[name] = {"ms": round(ms, 3), "fp64_TFLOPs": round(tf, 2),
                     "frac_fp64_peak": round(tf / FP64_PEAK_TFLOPS, 4)}
    res["total_ms"] = round(ms_h + ms_f + ms_q, 3)
    log(f"  gptq 4096x4096 (n=2048): {res}")
    del X, W, H, U, work
    return res


if __name__ == "__main__":
    main()
