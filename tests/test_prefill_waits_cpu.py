"""The wide prefill kernel's step ends wait for their activation tiles explicitly (CPU; needs hipcc).

The kernel loads each activation tile straight into LDS (buffer loads with the LDS destination)
a step ahead and ends a step with a barrier, after which every wave reads the tile.  Each wave
must therefore wait (s_waitcnt vmcnt) for its own loads into that tile before the barrier.  In
an earlier build the compiler, left to track those loads itself, emitted one step end of the
three-step pipeline with no vmcnt wait at all (the loop was rotated around loads it issued in a
waterfall loop), and a step now and then computed on the previous tile.  This test compiles
``prefill.hip`` for gfx950 and checks, in every instantiation of the wide kernel, that each
``s_barrier`` that follows vector-memory loads has a vmcnt wait after the loads of its segment
(in straight-line order of the assembly, which holds every loop body and step end in
sequence).  Run against the assembly of the earlier build, the rule flags the three-step
kernels, among them the phased one whose step end had no wait.
"""

import os
import re
import shutil
import subprocess

import pytest

from w4a16_dequant_gemm_amd import build

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def _assembly(tmp_path) -> str:
    if not os.path.exists(HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path / "prefill.s"
    cmd = [HIPCC, *build.HIPCC_FLAGS, "-x", "hip", "-S", "--cuda-device-only",
           os.path.join(build.CSRC, "prefill.hip"), "-o", str(out)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr[-2000:]
    return out.read_text()


def _wide_kernels(asm: str):
    """(name, instruction lines) of every wide-kernel instantiation."""
    funcs, name, body = [], None, []
    for line in asm.splitlines():
        m = re.match(r"^(_Z\S*prefill_f16_wide_kernel\S*):", line)
        if m:
            name, body = m.group(1), []
            continue
        if name is None:
            continue
        if line.startswith(".Lfunc_end"):
            funcs.append((name, body))
            name = None
            continue
        s = line.split(";")[0].strip()
        if s and not s.startswith("."):
            body.append(s)
    return funcs


def _unwaited_barriers(body):
    """Indices of s_barrier instructions whose segment (the instructions since the previous
    barrier, in the assembly's order) issues vector-memory loads with no vmcnt wait after the
    last of them.  A step end issues the loads of a later step and then waits for its tile; a
    barrier after loads with no wait at all is the failure described above (in the rotated
    loop the tile's own loads sat in another segment, so the rule looks at any load)."""
    bad, seg = [], []
    for i, ins in enumerate(body):
        if ins.startswith("s_barrier"):
            loads = [j for j, x in enumerate(seg) if x.startswith("buffer_load")]
            if loads and not any(x.startswith("s_waitcnt") and "vmcnt(" in x for x in seg[loads[-1] + 1:]):
                bad.append(i)
            seg = []
        else:
            seg.append(ins)
    return bad


def test_every_step_end_waits_for_its_tile(tmp_path):
    funcs = _wide_kernels(_assembly(tmp_path))
    assert len(funcs) >= 10, "wide-kernel instantiations not found in the assembly"
    with_dma = 0
    for name, body in funcs:
        if not any(ins.startswith("buffer_load") and ins.endswith(" lds") for ins in body):
            continue
        with_dma += 1
        bad = _unwaited_barriers(body)
        assert not bad, f"{name}: s_barrier without a vmcnt wait after LDS-destination loads at {bad[:3]}"
    assert with_dma >= 10
