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
