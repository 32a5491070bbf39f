"""The allocation-free entry point (moe_forward_noalloc) against moe_forward, through the C
ABI: two calls in a row, the second with fewer tokens, each bitwise equal to moe_forward on
the same inputs (the same kernels in the same order), and within the parity bar of the
oracle; a shape past the fixed scratch is refused before any launch."""
import numpy as np
import pytest
import torch

import mixture_experts_transformer_amd as moe
import oracle
from synth import get_config, make_inputs
from _gpu import assert_close, note, upload

pytestmark = pytest.mark.gpu

MOE_ENOMEM = -4


def call_noalloc(d, cfg, out):
    lib = moe.lib()
    rc = lib.moe_forward_noalloc(d["x"].data_ptr(), d["router_w"].data_ptr(), d["router_b"].data_ptr(),
                                 d["w1"].data_ptr(), d["b1"].data_ptr(), d["w2"].data_ptr(), d["b2"].data_ptr(),
                                 cfg.T, cfg.D, cfg.E, cfg.k, cfg.F, moe.FMT[cfg.fmt], out.data_ptr())
    return rc


@pytest.mark.parametrize("base", ["C2", "X1", "Y1"])
def test_noalloc_matches_forward_twice(base):
    torch.cuda.set_device(0)
    moe.lib().moe_set_stream(torch.cuda.current_stream().cuda_stream)
    for T, seed in ((384, 7101), (96, 7102)):             # the second call is smaller
        cfg = get_config(base, name=f"noalloc{T}", T=T, seed=seed)
        inp = make_inputs(cfg)
        d = upload(inp)
        note(f"noalloc {base} T={T} fmt={cfg.fmt}")
        out = torch.full((T, cfg.D), float("nan"), dtype=torch.float32, device="cuda")
        rc = call_noalloc(d, cfg, out)
        assert rc == 0, moe.lib().moe_last_error().decode()
        ref = moe.forward(d["x"], d["router_w"], d["router_b"], d["w1"], d["b1"], d["w2"], d["b2"], cfg.k,
                          cfg.fmt)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), f"{base} T={T}: moe_forward_noalloc differs from moe_forward"
        want = oracle.moe_forward(inp.x, inp.wr, inp.br, inp.w1, inp.b1, inp.w2, inp.b2, k=cfg.k, F=cfg.F,
                                  fmt=cfg.fmt)
        assert_close(out.cpu().numpy(), want, f"noalloc {base} T={T} vs oracle")


def test_noalloc_refuses_shapes_past_the_scratch():
    cap = (64 << 20)
    T = 1024
    assert moe.workspace_bytes(T, 2880, 32, 4, 2880, "bf16") > cap
    cfg = get_config("C2", name="noalloc-big", T=T, seed=7103)
    d = upload(make_inputs(cfg))
    out = torch.zeros((T, cfg.D), dtype=torch.float32, device="cuda")
    note("noalloc refusal T=1024")
    assert call_noalloc(d, cfg, out) == MOE_ENOMEM
    assert "scratch" in moe.lib().moe_last_error().decode()
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0              # nothing was launched
