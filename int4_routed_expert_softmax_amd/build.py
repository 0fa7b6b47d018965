"""Builds libmoe.so (the gfx950 HIP library behind include/moe.h) in-tree,
and libmoe_trace.so: the same sources with the phase trace compiled in
(MOE_PHASE_TRACE; moe_trace_read in include/moe.h), for measurement only.

    python -m int4_routed_expert_softmax_amd.build [--trace]
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "lib", "libmoe.so")
TRACE_LIB = os.path.join(PKG, "lib", "libmoe_trace.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU ops are disabled for all device code.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17",
                "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def sources():
    csrc = os.path.join(PKG, "csrc")
    return sorted(glob.glob(os.path.join(csrc, "*.hip"))) + [os.path.join(csrc, "moe_abi.cpp")]


def build(verbose: bool = False, trace: bool = False) -> str:
    out = TRACE_LIB if trace else LIB
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    cmd = [HIPCC, *DEVICE_FLAGS, *(["-DMOE_PHASE_TRACE"] if trace else []), "-fPIC", "-shared",
           "-fvisibility=hidden", "-I", os.path.join(ROOT, "include"), "-o", tmp, *sources()]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, trace="--trace" in sys.argv))
