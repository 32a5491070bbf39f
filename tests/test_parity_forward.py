"""GPU moe_forward end to end vs the oracle, at every workload's full size.

Every workload is compared on every output (the large ones in test_forward_large_full).
At the large ones the integer routing is also compared in full (through moe_route, same
kernels as moe_forward) and the fp32 output on a sample of tokens the oracle evaluates on
its own: a token's output depends only on its
own row, so the oracle runs the block on the sampled rows alone.  The C5 sample takes, for
every live expert, the first token routed to it, plus random tokens, so every expert's tiles
(the Zipf head, the middle and the tail, on the scaled matrix-core engine) are compared."""
import numpy as np
import pytest
import torch

import mixture_experts_transformer_amd as moe
import oracle
from synth import get_config, make_expert_bias, make_inputs
from _gpu import DEV, assert_close, note, upload

pytestmark = pytest.mark.gpu


def forward(inp, d=None):
    cfg = inp.cfg
    d = d or upload(inp)
    out = moe.forward(d["x"], d["router_w"], d["router_b"], d["w1"], d["b1"], d["w2"], d["b2"], cfg.k, cfg.fmt)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("name", ["C1", "C2", "X1", "Y1"])
def test_forward_full(name):
    inp = make_inputs(name)
    cfg = inp.cfg
    note(f"forward {name} full: T={cfg.T} E={cfg.E} fmt={cfg.fmt}")
    out = forward(inp).cpu().numpy()
    ref = oracle.moe_forward(inp.x, inp.wr, inp.br, inp.w1, inp.b1, inp.w2, inp.b2, k=cfg.k, F=cfg.F, fmt=cfg.fmt)
    assert_close(out, ref, f"forward {name}")


def pick_sample(name, idx, E, n):
    g = np.random.default_rng(123)
    T = idx.shape[0]
    if name != "C5":
        return np.sort(g.choice(T, size=n, replace=False))
    counts = np.bincount(idx.reshape(-1), minlength=E)
    live = np.flatnonzero(counts)
    first = [int(np.flatnonzero((idx == e).any(axis=1))[0]) for e in live]
    sample = np.unique(np.concatenate([np.array(first), g.choice(T, size=n, replace=False)]))
    assert np.array_equal(np.unique(idx[sample]), live)      # every live expert is compared
    return sample


@pytest.mark.parametrize("name,n", [("C3", 256), ("C4", 256), ("X2", 256), ("C5", 64), ("Y2", 256)])
def test_forward_large_sampled(name, n):
    inp = make_inputs(name)
    cfg = inp.cfg
    d = upload(inp)
    note(f"forward {name}: T={cfg.T} E={cfg.E} fmt={cfg.fmt}")
    out = forward(inp, d)
    r = moe.route(d["x"], d["router_w"], d["router_b"], cfg.k, want_logits=False)
    torch.cuda.synchronize()
    idx_ref = oracle.select_experts(oracle.router_logits(inp.x, inp.wr, inp.br), cfg.k)
    assert np.array_equal(r["idx"].cpu().numpy(), idx_ref), f"{name}: top-k indices differ"
    counts_ref, offsets_ref, perm_ref, _ = oracle.route_assignments(idx_ref, cfg.E)
    assert np.array_equal(r["offsets"].cpu().numpy(), offsets_ref)
    assert np.array_equal(r["perm"].cpu().numpy(), perm_ref)
    sample = pick_sample(name, idx_ref, cfg.E, n)
    ref = oracle.moe_forward(inp.x[sample], inp.wr, inp.br, inp.w1, inp.b1, inp.w2, inp.b2,
                             k=cfg.k, F=cfg.F, fmt=cfg.fmt)
    got = out.cpu().numpy()
    assert np.all(np.isfinite(got))
    assert_close(got[sample], ref, f"forward {name} ({sample.size} sampled tokens)")


@pytest.mark.parametrize("name", ["C3", "C4", "X2", "C5", "Y2"])
def test_forward_large_full(name):
    """The large workloads on every output: the oracle runs the whole layer (float64, one
    expert at a time), so every row tile of every expert, the Zipf head and tail, the padding
    of each group's last tile and every column tile's edge are compared."""
    inp = make_inputs(name)
    cfg = inp.cfg
    note(f"forward {name} full: T={cfg.T} E={cfg.E} fmt={cfg.fmt}")
    out = forward(inp).cpu().numpy()
    ref = oracle.moe_forward(inp.x, inp.wr, inp.br, inp.w1, inp.b1, inp.w2, inp.b2, k=cfg.k, F=cfg.F, fmt=cfg.fmt)
    assert_close(out, ref, f"forward {name} (all {cfg.T} tokens)")


def test_forward_split_stream_follows_the_calling_stream():
    """On the scaled engine the forward forks the split of x into fp8 pieces onto a second
    stream beside the routing and joins it before mlp1.  Against the oracle on every output;
    then on a non-default stream whose x is written by that stream just before the call (the
    fork must wait for it), and again after moe_release has destroyed the second stream, it
    gives the default stream's output bit for bit."""
    cfg = get_config("C4", name="fwd-stream", T=700, D=256, F=256, E=8, k=4, seed=8109)
    assert cfg.fmt == "mxfp4" and cfg.T * cfg.k >= 128 * cfg.E   # the scaled engine's regime
    inp = make_inputs(cfg)
    d = upload(inp)
    note("forward with the split on the second stream: default stream, caller stream, after release")
    ref = forward(inp, d).clone()
    want = oracle.moe_forward(inp.x, inp.wr, inp.br, inp.w1, inp.b1, inp.w2, inp.b2, k=cfg.k, F=cfg.F, fmt=cfg.fmt)
    assert_close(ref.cpu().numpy(), want, "forward, split on the second stream")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for _ in range(3):
            x2 = torch.zeros_like(d["x"])
            x2.copy_(d["x"])                         # written on the calling stream just before
            out = moe.forward(x2, d["router_w"], d["router_b"], d["w1"], d["b1"], d["w2"], d["b2"],
                              cfg.k, cfg.fmt)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    moe.release()
    again = forward(inp, d)
    assert torch.equal(again, ref)


@pytest.mark.parametrize("name", ["C2", "C3", "C4", "C5", "X1", "X2", "Y2"])
def test_forward_is_bitwise_deterministic(name):
    inp = make_inputs(name)
    d = upload(inp)
    note(f"determinism {name}")
    a = forward(inp, d)
    b = forward(inp, d)
    assert torch.equal(a, b)


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4", "mxfp8"])
def test_forward_power_of_two_scaling_is_exact(fmt):
    """W2, b2 doubled (bf16: exponent + 1; MXFP4/MXFP8: every W2 scale byte + 1, b2 doubled)
    doubles the output bit for bit: scaling by 2 commutes with every rounding on the path."""
    base = {"bf16": "C2", "mxfp4": "C4", "mxfp8": "Y1"}[fmt]
    cfg = get_config(base, name="scale", T=1024, E=8, seed=31)
    inp = make_inputs(cfg)
    d = upload(inp)
    note(f"power-of-two scaling {fmt}")
    out = forward(inp, d)
    nz = (inp.b2 & 0x7FFF) != 0
    b2s = np.where(nz, inp.b2 + np.uint16(1 << 7), inp.b2).astype(np.uint16)
    if fmt == "bf16":
        nzw = (inp.w2 & 0x7FFF) != 0
        w2s = np.where(nzw, inp.w2 + np.uint16(1 << 7), inp.w2).astype(np.uint16)
    else:
        w2s = inp.w2.copy()
        w2s[cfg.E * cfg.D * (cfg.F // 2 if fmt == "mxfp4" else cfg.F):] += 1
    from _gpu import u16, weights
    d2 = dict(d, w2=weights(w2s, fmt), b2=u16(b2s))
    out2 = forward(inp, d2)
    assert torch.equal(out2, 2 * out)


@pytest.mark.parametrize("name", ["C1", "C2", "X1", "Y1"])
def test_forward_with_expert_bias(name):
    """The biased entry point over the whole block: the bias moves the selection (most tokens
    at this size) and the gates stay on the unbiased logits."""
    inp = make_inputs(name)
    cfg = inp.cfg
    eb = make_expert_bias(cfg.E, cfg.T)
    note(f"forward {name} biased: T={cfg.T} E={cfg.E} fmt={cfg.fmt}")
    d = upload(inp)
    out = moe.forward(d["x"], d["router_w"], d["router_b"], d["w1"], d["b1"], d["w2"], d["b2"], cfg.k, cfg.fmt,
                      expert_bias=torch.from_numpy(eb).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.moe_forward(inp.x, inp.wr, inp.br, inp.w1, inp.b1, inp.w2, inp.b2, k=cfg.k, F=cfg.F,
                             fmt=cfg.fmt, expert_bias=eb)
    assert_close(out.cpu().numpy(), ref, f"forward {name} biased")

