"""Generated-code invariants of the HIP sources (CPU only: hipcc cross-compiles gfx950).

The grouped GEMM issues its direct global->LDS copies as inline assembly that loads M0
without the compiler preserving it; that is sound only while nothing else in the kernels
uses M0.  This test compiles the source to gfx950 assembly and checks that every use of M0
is one of those copies."""
import os
import shutil

import pytest

from mixture_experts_transformer_amd import build as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_m0_only_carries_lds_copy_destinations():
    hipcc = b.hipcc()
    if not (os.path.exists(hipcc) or shutil.which(hipcc)):
        pytest.skip("hipcc not available")
    for src in b.M0_SOURCES:
        assert b.check_m0(src) > 0


def test_m0_check_rejects_other_uses(monkeypatch):
    """The check itself: assembly with M0 set for anything but a copy must fail it."""
    good = "s_mov_b32 m0, s4\ns_nop 0\nglobal_load_lds_dwordx4 v1, s[2:3]\n"
    monkeypatch.setattr(b, "device_asm", lambda src: good)
    assert b.check_m0("x.hip") == 1
    vcc = "s_mov_b32 m0, vcc_lo\ns_nop 0\nglobal_load_lds_dwordx4 v1, s[2:3]\n"
    monkeypatch.setattr(b, "device_asm", lambda src: good + vcc)
    assert b.check_m0("x.hip") == 2
    for bad in ("s_mov_b32 m0, s4\ns_nop 0\nds_read_b32 v1, v2\n",
                good + "s_mov_b32 m0, -1\nds_write_b32 v1, v2\n",
                good + "v_readlane_b32 s5, v1, m0\n",
                good + "s_mov_b32 m0, v1\ns_nop 0\nglobal_load_lds_dwordx4 v1, s[2:3]\n"):
        monkeypatch.setattr(b, "device_asm", lambda src, t=bad: t)
        with pytest.raises(RuntimeError):
            b.check_m0("x.hip")
