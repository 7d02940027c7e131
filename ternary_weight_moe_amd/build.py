"""Builds libternary_moe.so in-tree for gfx950 (hipcc).  ``python -m ternary_weight_moe_amd.build``.

The host-side argument checks (tw_host.cpp) are compiled by the host compiler as plain C++; the
kernels (tw_kernels.hip) by hipcc for gfx950 only.  Flags that matter for the numerics:
-ffp-contract=off (no fused multiply-add: every fp32 step of the int8 path is one rounding) and
correctly rounded fp32 division and square root.  Packed-fp32 instructions are disabled.
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(os.path.dirname(HERE), "include")
LIB = os.path.join(HERE, "libternary_moe.so")
ARCH = "gfx950"
HIP_SOURCES = ("tw_kernels.hip", "tw_persist.hip", "tw_prefill.hip", "tw_base3.hip", "tw_attn.hip",
               "tw_head.hip", "tw_static.hip")

HIP_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-rdc",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-I" + INCLUDE,
]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build step failed: " + " ".join(cmd))
    return r


# The measurement build: the same sources with -DTW_PHASE_TIMES, whose stacked decode kernel also
# stores per-layer phase timestamps into its workspace (read by phase_times.py).
PHASES_LIB = os.path.join(HERE, "libternary_moe_phases.so")


def build(verbose: bool = False, phases: bool = False) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    bdir = os.path.join(HERE, "_build_phases" if phases else "_build")
    out = PHASES_LIB if phases else LIB
    extra = ["-DTW_PHASE_TIMES"] if phases else []
    os.makedirs(bdir, exist_ok=True)
    host_o = os.path.join(bdir, "tw_host.o")
    _run(["g++", "-O2", "-std=c++17", "-fPIC", "-Wall", "-I" + INCLUDE] + extra +
         ["-c", os.path.join(CSRC, "tw_host.cpp"), "-o", host_o])
    objs = [os.path.join(bdir, src.replace(".hip", ".o")) for src in HIP_SOURCES]
    jobs = [[hipcc] + HIP_FLAGS + extra + ["-c", os.path.join(CSRC, src), "-o", o]
            for src, o in zip(HIP_SOURCES, objs)]
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 8))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        list(ex.map(_run, jobs))
    objs = [host_o] + objs
    tmp = out + ".tmp%d" % os.getpid()
    _run([hipcc, "--offload-arch=" + ARCH, "-shared", "-fPIC"] + objs + ["-o", tmp])
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    build(verbose=True, phases=True)
