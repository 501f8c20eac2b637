"""Build ``libw4a16.so`` for gfx950 in-tree with hipcc (no torch involvement).

``python -m w4a16_dequant_gemm_amd.build`` or ``build()`` from Python.  Every source is
compiled to its own object in parallel (no device code crosses files: each file holds its
kernels and their host launchers), then the objects are linked into one shared library
written next to this file, so it travels with the source tree.  A second small library,
``libw4a16_probe.so`` (``csrc/probe.hip``), holds the plain-read reference kernel that the
benchmark times beside the weight-streaming kernels; it is not part of the W4A16 C ABI.
"""

from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libw4a16.so")
# read-rate reference timed by the benchmark beside the weight-streaming kernels (its own
# library: not part of the W4A16 C ABI)
PROBE_LIB = os.path.join(HERE, "libw4a16_probe.so")
PROBE_SOURCE = "probe.hip"
OBJDIR = os.path.join(HERE, "_build")
SOURCES = ["api.cpp", "quantize.hip", "gemv.hip", "skinny.hip", "decode.hip", "prefill.hip", "gptq.hip",
           "awq.hip", "w8a8.hip", "kv.hip", "w8a16.hip", "scratch.hip"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-ffp-contract=fast",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
]


def _jobs() -> int:
    for var in ("MAX_JOBS", "CMAKE_BUILD_PARALLEL_LEVEL"):
        v = os.environ.get(var, "")
        if v.isdigit() and int(v) > 0:
            return min(int(v), 16)
    return max(1, min(len(SOURCES), os.cpu_count() or 1, 16))


def build(verbose: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    os.makedirs(OBJDIR, exist_ok=True)

    def compile_one(src: str):
        obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *HIPCC_FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        return obj, subprocess.run(cmd, capture_output=True, text=True)

    with ThreadPoolExecutor(max_workers=_jobs()) as pool:
        results = list(pool.map(compile_one, SOURCES))
    failed = [r for _, r in results if r.returncode != 0]
    for r in failed:
        sys.stderr.write(r.stdout + r.stderr)
    if failed:
        raise RuntimeError("hipcc failed compiling libw4a16.so sources")
    tmp = LIB + ".tmp"
    cmd = [hipcc, "--offload-arch=gfx950", "-shared", "-fPIC", *[o for o, _ in results], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed linking libw4a16.so")
    os.replace(tmp, LIB)
    probe_tmp = PROBE_LIB + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, "-shared", "-x", "hip", os.path.join(CSRC, PROBE_SOURCE), "-o", probe_tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libw4a16_probe.so")
    os.replace(probe_tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
