"""Build the gfx950 shared library ``libmoe.so`` in-tree with hipcc.

    python -m mixture_experts_transformer_amd.build [--verbose]
    python -m mixture_experts_transformer_amd.build --host-sanitized <out.so>

Every HIP source under ``csrc/`` is compiled for gfx950 only.  The copies of the grouped GEMM
load M0 in inline assembly; the build checks the generated assembly (``check_m0``) and fails
rather than ship a library in which anything else uses M0.  Packed-fp32 VALU
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
SOURCES = ["route.hip", "gemm.hip", "backward.hip", "moe_api.hip"]
# bench.py's matrix-core rate calibration (not part of the MoE block), its own small library
CALIB_SRC = os.path.join(HERE, "calib", "mfma_rate.hip")
CALIB_LIB = os.path.join(HERE, "calib", "libmoe_calib.so")
ARCH = "gfx950"


def hipcc() -> str:
    root = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(root, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def device_asm(src: str) -> str:
    """gfx950 assembly of one HIP source (device code only), compiled as the library is."""
    import tempfile
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-S", "--cuda-device-only",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(os.path.dirname(HERE), "include"), os.path.join(CSRC, src), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc -S {src} failed ({r.returncode}):\n{r.stderr[-4000:]}")
        return open(out).read()


# Sources whose kernels issue the direct global->LDS copies (inline assembly that loads M0
# without the compiler preserving it).
M0_SOURCES = ["gemm.hip"]


def check_m0(src: str) -> int:
    """The LDS copies load M0 in inline assembly that the compiler does not preserve; that is
    sound only while nothing else in the generated code uses M0.  Raise if any use of M0 in
    the gfx950 assembly of `src` is not 's_mov_b32 m0, <scalar register>' (sN, or vcc_lo / vcc_hi
    where the compiler puts the copy's LDS address there) directly followed by 's_nop 0' and
    a global_load_lds copy.  Returns the number of copies checked."""
    import re
    lines = [l.split(";")[0].strip() for l in device_asm(src).splitlines()]
    lines = [l for l in lines if l and not l.startswith(".")]
    uses = [i for i, l in enumerate(lines) if re.search(r"\bm0\b", l)]
    if not uses:
        raise RuntimeError(f"{src}: expected the LDS copies to set M0")
    for i in uses:
        if not re.fullmatch(r"s_mov_b32 m0, (s\d+|vcc_lo|vcc_hi)", lines[i]):
            raise RuntimeError(f"{src}: M0 used other than by an LDS copy: {lines[i]!r}")
        nxt = lines[i + 1:i + 3]
        if len(nxt) < 2 or nxt[0] != "s_nop 0" or not nxt[1].startswith("global_load_lds_dword"):
            raise RuntimeError(f"{src}: M0 set but not consumed by a copy: {lines[i:i + 3]!r}")
    return len(uses)


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
    # the library ships only if the copies' M0 handling holds in the code just generated
    for s in M0_SOURCES:
        n = check_m0(s)
        if verbose:
            print(f"M0 check {s}: {n} copies, no other use", flush=True)
    os.replace(tmp, LIB)
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-o", CALIB_LIB + ".tmp", CALIB_SRC]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc (calibration kernel) failed ({r.returncode}):\n{r.stderr[-4000:]}")
    os.replace(CALIB_LIB + ".tmp", CALIB_LIB)
    return LIB


def build_host_sanitized(out: str) -> str:
    """A copy of the library whose host code (argument checks, workspace and stream handling,
    error strings, profiling) is built with AddressSanitizer and UndefinedBehaviorSanitizer,
    for exercising the C ABI on a machine without a GPU.  The device code is built as usual
    (the sanitizers apply to the host pass only); a program that loads this copy must itself
    be linked with the same compiler's sanitizer runtime (clang -fsanitize=address,undefined)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", "-shared",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-fno-omit-frame-pointer",
           "-Xarch_host", "-fsanitize=address",
           "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined",
           "-I", os.path.join(os.path.dirname(HERE), "include"), "-o", out] + srcs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized host build failed ({r.returncode}):\n{r.stderr[-4000:]}")
    return out


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv:
        print(build_host_sanitized(sys.argv[sys.argv.index("--host-sanitized") + 1]))
    else:
        print(build(verbose="--verbose" in sys.argv))
