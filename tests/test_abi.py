"""The C ABI without a GPU: the library loads, exports every function the header declares,
and rejects invalid arguments in host code before any HIP call (no compute call is made)."""
import ctypes
import os
import re

import pytest

import mixture_experts_transformer_amd as moe
from mixture_experts_transformer_amd.moe import _SIGNATURES

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")

MOE_OK, MOE_EINVAL, MOE_EFMT, MOE_EALIGN = 0, -1, -2, -3


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = moe.lib()
    names = declared_functions()
    assert {"moe_forward", "moe_route", "moe_experts"} <= set(names)
    for n in names:
        assert hasattr(lib, n), f"{n} declared in moe.h but not exported"
    assert set(names) == set(_SIGNATURES), "binding signatures and header disagree"


def test_header_constants_match_binding():
    src = open(HEADER).read()
    assert re.search(r"#define MOE_FMT_BF16 0\b", src) and re.search(r"#define MOE_FMT_MXFP4 1\b", src)
    assert re.search(r"#define MOE_FMT_MXFP8 2\b", src)
    assert moe.FMT == {"bf16": 0, "mxfp4": 1, "mxfp8": 2}
    assert "#define MOE_SWIGLU_ALPHA 1.702f" in src and "#define MOE_SWIGLU_LIMIT 7.0f" in src
    assert re.search(r"#define MOE_NUM_STAGES 8\b", src) and len(moe.STAGES) == 8


def test_version_string():
    assert "gfx950" in moe.version()


# fake, 16-byte aligned device addresses: only ever passed to calls that must fail validation
P = 0x10000
BAD = 0x10008


def fwd(T=8, D=64, E=4, k=2, F=64, fmt=0, ptrs=None):
    p = ptrs or [P] * 8
    return moe.lib().moe_forward(p[0], p[1], p[2], p[3], p[4], p[5], p[6], T, D, E, k, F, fmt, p[7])


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), MOE_EINVAL), (dict(D=0), MOE_EINVAL), (dict(D=96), MOE_EINVAL), (dict(F=32), MOE_EINVAL),
    (dict(E=0), MOE_EINVAL), (dict(E=257, k=2), MOE_EINVAL), (dict(k=0), MOE_EINVAL), (dict(k=5, E=4), MOE_EINVAL),
    (dict(T=2**30, k=2), MOE_EINVAL), (dict(fmt=3), MOE_EFMT), (dict(fmt=-1), MOE_EFMT),
    (dict(T=2**24, D=64), MOE_EINVAL), (dict(T=2**22, D=64, k=4, E=4, F=64), MOE_EINVAL),
    (dict(D=2**15, F=2**15, T=1), MOE_EINVAL),
])
def test_forward_rejects_bad_shapes(kw, code):
    assert fwd(**kw) == code
    assert moe.lib().moe_last_error().decode() != ""


@pytest.mark.parametrize("which", range(8))
def test_forward_rejects_null_and_misaligned_pointers(which):
    ptrs = [P] * 8
    ptrs[which] = None
    assert fwd(ptrs=ptrs) == MOE_EINVAL
    assert "NULL" in moe.lib().moe_last_error().decode()
    ptrs[which] = BAD
    assert fwd(ptrs=ptrs) == MOE_EALIGN
    assert "aligned" in moe.lib().moe_last_error().decode()


def test_zero_tokens_is_a_no_op():
    # T = 0 returns before any pointer is looked at or any launch is made
    assert fwd(T=0, ptrs=[None] * 8) == MOE_OK
    assert moe.lib().moe_route(None, None, None, 0, 64, 4, 2, None, None, None, None, None, None) == MOE_OK
    assert moe.lib().moe_experts(None, None, None, None, None, None, None, None, 0, 64, 4, 2, 64, 0, None) == MOE_OK


def test_route_and_experts_validate():
    lib = moe.lib()
    # logits may be NULL; other outputs may not
    assert lib.moe_route(P, P, P, 8, 64, 4, 2, None, None, P, P, P, P) == MOE_EINVAL
    assert lib.moe_route(P, P, P, 8, 64, 4, 5, None, P, P, P, P, P) == MOE_EINVAL
    assert lib.moe_route(P, P, P, 8, 64, 4, 2, BAD, P, P, P, P, P) == MOE_EALIGN
    assert lib.moe_experts(P, P, P, P, P, P, P, None, 8, 64, 4, 2, 64, 0, P) == MOE_EINVAL
    assert lib.moe_experts(P, P, P, P, P, P, P, P, 8, 64, 4, 2, 64, 7, P) == MOE_EFMT
    assert lib.moe_experts(P, P, P, P, P, P, P, P, 8, 64, 4, 2, 64, 3, P) == MOE_EFMT


def test_biased_entry_points_validate_the_bias():
    lib = moe.lib()
    rb = lambda eb, T=8: lib.moe_route_biased(P, P, P, eb, T, 64, 4, 2, None, P, P, P, P, P)
    fb = lambda eb, T=8: lib.moe_forward_biased(P, P, P, eb, P, P, P, P, T, 64, 4, 2, 64, 0, P)
    for call in (rb, fb):
        assert call(None) == MOE_EINVAL
        assert "expert_bias" in lib.moe_last_error().decode()
        assert call(BAD) == MOE_EALIGN
        assert "expert_bias" in lib.moe_last_error().decode()
        assert call(None, T=0) == MOE_OK
    # the shape checks come first, as in the unbiased calls
    assert lib.moe_route_biased(P, P, P, P, 8, 64, 4, 5, None, P, P, P, P, P) == MOE_EINVAL
    assert lib.moe_forward_biased(P, P, P, P, P, P, P, P, 8, 64, 4, 2, 64, 7, P) == MOE_EFMT


def test_bias_update_validates():
    lib = moe.lib()
    for E in (0, 257, -1):
        assert lib.moe_update_expert_bias(P, E, 1e-3, P) == MOE_EINVAL
    for coeff in (float("inf"), float("nan")):
        assert lib.moe_update_expert_bias(P, 8, coeff, P) == MOE_EINVAL
    assert lib.moe_update_expert_bias(None, 8, 1e-3, P) == MOE_EINVAL
    assert lib.moe_update_expert_bias(P, 8, 1e-3, None) == MOE_EINVAL
    assert lib.moe_update_expert_bias(P, 8, 1e-3, BAD) == MOE_EALIGN
    assert "expert_bias" in lib.moe_last_error().decode()


def test_workspace_bytes():
    wb = moe.lib().moe_workspace_bytes
    assert wb(0, 2880, 32, 4, 2880, 0) == 0
    assert wb(8, 100, 4, 2, 64, 0) == 0        # invalid shape
    b16 = wb(8192, 2880, 32, 4, 2880, 0)
    b4 = wb(8192, 2880, 32, 4, 2880, 1)
    A = 8192 * 4
    # h (bf16) + y (fp32) dominate; at this token count MXFP4 (scaled matrix-core engine)
    # holds h as three fp8 pieces instead, plus two fp8 pieces of x, and one scale dword
    # per 32-element block of each
    assert b16 >= A * 2880 * 2 + A * 2880 * 4
    extra = A * 2880 + 2 * 8192 * 2880 + 8192 * 96 * 4 + A * 96 * 4
    assert extra <= b4 - b16 < extra + 4096
    assert b16 % 256 == 0


def test_set_workspace_rejects_misaligned():
    assert moe.lib().moe_set_workspace(0x1010, 4096) == MOE_EALIGN
    assert moe.lib().moe_set_workspace(None, 0) == MOE_OK


def test_plain_c_program_links_and_calls_the_library(tmp_path):
    """The header is plain C (C99, no C++): a C program includes it, links libmoe.so, and
    gets the host-side validation and zero-token results without a GPU."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no C compiler")
    src = tmp_path / "use.c"
    src.write_text(r'''
#include <stdio.h>
#include "moe.h"
int main(void) {
  int rc = 0;
  if (moe_forward(0, 0, 0, 0, 0, 0, 0, 0, 64, 4, 2, 64, MOE_FMT_MXFP8, 0) != MOE_OK) rc |= 1;
  if (moe_forward(0, 0, 0, 0, 0, 0, 0, 8, 64, 4, 5, 64, MOE_FMT_BF16, 0) != MOE_EINVAL) rc |= 2;
  if (moe_update_expert_bias(0, 300, 1e-3f, 0) != MOE_EINVAL) rc |= 4;
  if (moe_workspace_bytes(0, 64, 4, 2, 64, MOE_FMT_BF16) != 0) rc |= 8;
  printf("%s\n", moe_version());
  return rc;
}
''')
    lib_dir = os.path.dirname(moe.LIB_PATH)
    exe = tmp_path / "use"
    r = subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), str(src),
                        "-L", lib_dir, "-l:libmoe.so", f"-Wl,-rpath,{lib_dir}", "-o", str(exe)],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, (r.returncode, r.stdout, r.stderr)
    assert "gfx950" in r.stdout


def test_product_path_never_touches_the_oracle():
    """The package (binding and kernels) imports nothing from oracle/ and has no CPU fallback:
    its sources never name the oracle package, and importing it leaves oracle unloaded.
    The oracle in turn imports nothing from the package."""
    import subprocess
    import sys
    pkg = os.path.join(ROOT, "mixture_experts_transformer_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "import oracle" not in text and "from oracle" not in text, f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith(".py"):
            assert "mixture_experts_transformer_amd" not in open(os.path.join(ROOT, "oracle", f)).read(), f
    code = ("import sys, mixture_experts_transformer_amd as m; m.lib(); "
            "print('oracle' in sys.modules)")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert r.stdout.strip() == "False"


def test_too_small_caller_workspace_is_enomem():
    """A caller workspace smaller than the call needs fails with MOE_ENOMEM before any HIP call
    (the addresses are fake: nothing is launched), naming both sizes."""
    lib = moe.lib()
    MOE_ENOMEM = -4
    T, D, E, k, F = 256, 2880, 32, 4, 2880
    need = lib.moe_workspace_bytes(T, D, E, k, F, 0)
    assert need > 4096
    assert lib.moe_set_workspace(0x100000, 4096) == MOE_OK
    try:
        assert fwd(T=T, D=D, E=E, k=k, F=F) == MOE_ENOMEM
        msg = lib.moe_last_error().decode()
        assert "4096" in msg and str(need) in msg
        assert lib.moe_route(P, P, P, T, D, E, k, None, P, P, P, P, P) == MOE_ENOMEM
        assert lib.moe_experts(P, P, P, P, P, P, P, P, T, D, E, k, F, 1, P) == MOE_ENOMEM
        assert lib.moe_forward_biased(P, P, P, P, P, P, P, P, T, D, E, k, F, 2, P) == MOE_ENOMEM
    finally:
        assert lib.moe_set_workspace(None, 0) == MOE_OK


def test_caller_workspace_is_per_thread():
    """moe_set_workspace binds the calling thread only: two threads with buffers of different
    sizes each see their own size in the MOE_ENOMEM message."""
    import threading
    lib = moe.lib()
    MOE_ENOMEM = -4
    seen = {}

    def worker(size):
        assert lib.moe_set_workspace(0x200000, size) == MOE_OK
        try:
            rc = fwd(T=256, D=2880, E=32, k=4, F=2880)
            seen[size] = (rc, lib.moe_last_error().decode())
        finally:
            lib.moe_set_workspace(None, 0)

    for size in (4096, 8192):
        th = threading.Thread(target=worker, args=(size,))
        th.start()
        th.join()
    assert lib.moe_set_workspace(0x300000, 1 << 20) == MOE_OK
    try:
        ths = [threading.Thread(target=worker, args=(s,)) for s in (12288, 16384)]
        for th in ths:
            th.start()
        for th in ths:
            th.join()
        rc = fwd(T=256, D=2880, E=32, k=4, F=2880)       # this thread keeps its own 1 MiB
        assert rc == MOE_ENOMEM and f"holds {1 << 20} bytes" in lib.moe_last_error().decode()
    finally:
        lib.moe_set_workspace(None, 0)
    for size in (4096, 8192, 12288, 16384):
        rc, msg = seen[size]
        assert rc == MOE_ENOMEM and f"holds {size} bytes" in msg, (size, msg)


def test_backward_validates():
    """moe_backward: bf16 weights only (MOE_EFMT otherwise), shape and pointer checks first,
    and no workspace size for formats it does not take."""
    lib = moe.lib()
    bw = lambda fmt=0, T=8, ptrs=None: lib.moe_backward(*(ptrs or [P] * 11), T, 64, 4, 2, 64, fmt,
                                                       *([P] * 7))
    assert bw(fmt=1) == MOE_EFMT and "bf16" in lib.moe_last_error().decode()
    assert bw(fmt=2) == MOE_EFMT
    assert bw(fmt=9) == MOE_EFMT
    assert lib.moe_backward(*([P] * 11), 8, 96, 4, 2, 64, 0, *([P] * 7)) == MOE_EINVAL
    # within the forward's limits and T*k*2*max(D, F) < 2^30, but the weight gradients' padded
    # activations (T*k + 64 E columns of max(D, 2F) rows) pass 2^31 bytes
    assert lib.moe_backward(*([P] * 11), 8191, 64, 256, 4, 16384, 0, *([P] * 7)) == MOE_EINVAL
    assert "64*E" in lib.moe_last_error().decode()
    for which in range(11):
        ptrs = [P] * 11
        ptrs[which] = None
        assert bw(ptrs=ptrs) == MOE_EINVAL, which
        ptrs[which] = BAD
        assert bw(ptrs=ptrs) == MOE_EALIGN, which
    assert lib.moe_backward_workspace_bytes(256, 2880, 32, 4, 2880, 1) == 0
    assert lib.moe_backward_workspace_bytes(0, 2880, 32, 4, 2880, 0) == 0
    need = lib.moe_backward_workspace_bytes(256, 2880, 32, 4, 2880, 0)
    # per routed row at least u (fp32, 2F) and dx contributions (fp32, max(D, F)); the weights
    # are read as stored, so nothing of the size of an expert matrix set is held
    A = 256 * 4
    assert need > A * (2 * 2880 + 2880) * 4
    assert need < 32 * 2880 * 2880 * 2
    assert lib.moe_set_workspace(0x100000, 4096) == MOE_OK
    try:
        assert lib.moe_backward(*([P] * 11), 256, 2880, 32, 4, 2880, 0, *([P] * 7)) == -4
    finally:
        lib.moe_set_workspace(None, 0)
