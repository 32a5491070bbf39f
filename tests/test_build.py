"""Generated-code invariants of the HIP sources (CPU only: hipcc cross-compiles gfx950).

The grouped GEMM issues its direct global->LDS copies as inline assembly that loads M0
without the compiler preserving it; that is sound only while nothing else in the kernels
uses M0.  This test compiles the source to gfx950 assembly and checks that every use of M0
is one of those copies."""
import os
import re
import shutil
import subprocess
import tempfile

import pytest

from mixture_experts_transformer_amd import build as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def device_asm(src: str) -> str:
    hipcc = b.hipcc()
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        cmd = [hipcc, f"--offload-arch={b.ARCH}", "-O3", "-std=c++17", "-S", "--cuda-device-only",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include"), os.path.join(b.CSRC, src), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return open(out).read()


def test_m0_only_carries_lds_copy_destinations():
    lines = [l.split(";")[0].strip() for l in device_asm("gemm.hip").splitlines()]
    lines = [l for l in lines if l and not l.startswith(".")]
    uses = [i for i, l in enumerate(lines) if re.search(r"\bm0\b", l)]
    assert uses, "expected the LDS copies to set M0"
    for i in uses:
        assert re.fullmatch(r"s_mov_b32 m0, s\d+", lines[i]), f"other use of M0: {lines[i]}"
        nxt = lines[i + 1:i + 3]
        assert nxt[0] == "s_nop 0" and nxt[1].startswith("global_load_lds_dword"), \
            f"M0 set but not consumed by a copy: {lines[i:i + 3]}"
