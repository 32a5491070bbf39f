"""The forward captured into a HIP graph (torch.cuda.graph) and replayed.

Once its workspace is sized by an eager call, a forward launches only kernels on the
caller's stream (no allocation, no memset), so it can be captured.  Every replay, with
eager forwards of other inputs between the replays, must equal the eager output bit for
bit."""
import numpy as np
import pytest
import torch

import mixture_experts_transformer_amd as moe
from synth import get_config, make_expert_bias, make_inputs
from _gpu import DEV, note, upload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("base,T,E,biased", [
    ("C2", 256, 8, False),      # bf16, streaming tiles
    ("C2", 2048, 8, True),      # bf16, matrix-core tiles, load-balancing bias
    ("C4", 2048, 8, False),     # MXFP4 on the scaled engine (split kernel + fp8 pieces)
    ("X1", 128, 8, False),      # MXFP4 streaming decode
    ("Y1", 1024, 8, True),      # MXFP8, matrix-core tiles, bias
])
def test_forward_graph_replays_match_eager(base, T, E, biased):
    cfg = get_config(base, name=f"graph{T}", T=T, E=E, D=512, F=512, seed=4000 + T)
    inp = make_inputs(cfg)
    other = make_inputs(get_config(base, name=f"graphb{T}", T=T, E=E, D=512, F=512, seed=5000 + T))
    d, d2 = upload(inp), upload(other)
    eb = torch.from_numpy(make_expert_bias(E, T)).to(DEV) if biased else None
    note(f"graph capture {base} T={T} E={E} fmt={cfg.fmt} biased={biased}")

    def fwd(dd, out):
        return moe.forward(dd["x"], dd["router_w"], dd["router_b"], dd["w1"], dd["b1"], dd["w2"], dd["b2"],
                           cfg.k, cfg.fmt, out=out, expert_bias=eb)

    ref = fwd(d, None)
    ref2 = fwd(d2, None)
    torch.cuda.synchronize()
    out_g = torch.empty_like(ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fwd(d, out_g)                            # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fwd(d, out_g)
    torch.cuda.synchronize()
    for rep in range(3):
        out_g.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref), f"replay {rep} differs from the eager forward"
        mid = fwd(d2, None)                      # eager work on the same workspace in between
        torch.cuda.synchronize()
        assert torch.equal(mid, ref2)
    del g


def test_graph_survives_a_larger_eager_call():
    """A graph captured while the library-owned workspace was small keeps replaying correctly
    after an eager call of a larger shape grew the workspace: the captured buffer is retired,
    not freed, until moe_release."""
    base = "C2"
    small = get_config(base, name="graph-small", T=64, E=8, D=512, F=512, seed=6101)
    large = get_config(base, name="graph-large", T=4096, E=8, D=512, F=512, seed=6102)
    ds, dl = upload(make_inputs(small)), upload(make_inputs(large))
    note("graph capture, then a larger eager call, then replay")

    def fwd(dd, cfg, out=None):
        return moe.forward(dd["x"], dd["router_w"], dd["router_b"], dd["w1"], dd["b1"], dd["w2"], dd["b2"],
                           cfg.k, cfg.fmt, out=out)

    torch.cuda.synchronize()
    moe.release()                                # start from an empty library-owned workspace
    ref = fwd(ds, small)
    torch.cuda.synchronize()
    assert moe.workspace_bytes(64, 512, 8, 4, 512) < moe.workspace_bytes(4096, 512, 8, 4, 512)
    out_g = torch.empty_like(ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fwd(ds, small, out_g)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        fwd(ds, small, out_g)
    torch.cuda.synchronize()
    big = fwd(dl, large)                         # grows the workspace (the old one is kept)
    torch.cuda.synchronize()
    big_ref = big.clone()
    for rep in range(3):
        out_g.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out_g, ref), f"replay {rep} after the larger call differs"
        again = fwd(dl, large)
        torch.cuda.synchronize()
        assert torch.equal(again, big_ref)
    del g
    torch.cuda.synchronize()
    moe.release()


@pytest.mark.parametrize("T", [64, 512])       # few rows per expert (streaming tiles) and many
def test_backward_graph_replays_match_eager(T):
    """moe_backward captured into a graph after an eager call of the same shape: every replay,
    with eager backward calls of other inputs between the replays, equals the eager gradients
    bit for bit (the backward clears what it accumulates with kernels, not memsets)."""
    cfg = get_config("C2", name=f"gbwd{T}", T=T, E=4, D=256, F=256, seed=7000 + T)
    other = get_config("C2", name=f"gbwdb{T}", T=T, E=4, D=256, F=256, seed=7100 + T)
    d, d2 = upload(make_inputs(cfg)), upload(make_inputs(other))
    note(f"backward graph capture T={T} E=4 D=F=256")
    gen = torch.Generator().manual_seed(7200 + T)
    dout = torch.randn(T, 256, generator=gen).to(DEV)
    dout2 = torch.randn(T, 256, generator=gen).to(DEV)
    r = moe.route(d["x"], d["router_w"], d["router_b"], cfg.k, want_logits=False)
    r2 = moe.route(d2["x"], d2["router_w"], d2["router_b"], cfg.k, want_logits=False)

    def bwd(dd, rr, g, out=None):
        return moe.backward(dd["x"], dd["router_w"], dd["w1"], dd["b1"], dd["w2"], dd["b2"], rr, g, cfg.k, out=out)

    ref = {n: t.clone() for n, t in bwd(d, r, dout).items()}
    ref2 = {n: t.clone() for n, t in bwd(d2, r2, dout2).items()}
    torch.cuda.synchronize()
    out = {n: torch.empty_like(t) for n, t in ref.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        bwd(d, r, dout, out)                     # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        bwd(d, r, dout, out)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in out.values():
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for n in ref:
            assert torch.equal(out[n], ref[n]), f"replay {rep}: {n} differs from the eager backward"
        mid = bwd(d2, r2, dout2)                 # eager work on the same workspace in between
        torch.cuda.synchronize()
        for n in ref2:
            assert torch.equal(mid[n], ref2[n]), n
    del g
