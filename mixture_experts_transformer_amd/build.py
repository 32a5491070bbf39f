"""Build the gfx950 shared library ``libmoe.so`` in-tree with hipcc.

    python -m mixture_experts_transformer_amd.build [--verbose]

Every HIP source under ``csrc/`` is compiled for gfx950 only.  Packed-fp32 VALU
instructions are disabled for device code (``-packed-fp32-ops``); the host pass prints a
harmless warning that it does not know the feature.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmoe.so")
SOURCES = ["route.hip", "gemm.hip", "moe_api.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    root = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(root, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def build(verbose: bool = False) -> str:
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-Wall", "-Wno-unused-function", "-Wno-unused-variable",
           "-I", os.path.join(os.path.dirname(HERE), "include"),
           "-o", tmp] + srcs
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    msgs = "\n".join(l for l in (r.stdout + r.stderr).splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed ({r.returncode}):\n{msgs}")
    if msgs.strip() and verbose:
        print(msgs)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
