"""GPU backward (moe_backward, bf16 expert weights) against the float64 oracle's gradients.

Every gradient (dx, d_router_w, d_router_b, dw1, db1, dw2, db2) is compared element by
element with the oracle on the routing the GPU's moe_route returns (itself checked bit for
bit against the oracle's): whole tensors on small layers, and on a layer of the 20B shape
(256 tokens, D = F = 2880, 32 experts, top-4) the whole dx and router gradients plus the
expert gradients of three experts (the most and least loaded and a middle one).

Tolerance (derived: the stated bars are for the forward's output).  The gradient products
take some operands rounded once to bf16 (dz = g dout, du and h: unit roundoff 2^-9), so every
gradient carries a relative error of the order of 2^-9 whatever its size, while its entries
grow with the rows an expert sums (to ~10^3 on these layers).  Per tensor: relative L2 error
<= 1e-2 (the forward's bar), and max abs error <= max(3e-2, 1e-2 * max|ref|): the forward's
absolute bar where gradients are of order one, and beyond that the same 1e-2 measured against
the tensor's largest entry.  Measured: at most 5e-3 of max|ref| (and 1e-7 relative for db2,
which takes no rounded operand)."""
import numpy as np
import pytest
import torch

import mixture_experts_transformer_amd as moe
import oracle
from synth import f32_to_bf16_bits, get_config, make_dout, make_inputs
from _gpu import DEV, MAX_ABS, REL_L2, errors, note, upload

pytestmark = pytest.mark.gpu


class Report:
    """Collects every tensor's errors before asserting, so one run shows them all."""

    def __init__(self):
        self.bad = []

    def check(self, got, ref, what):
        rel, mx = errors(got, ref)
        scale = float(np.max(np.abs(ref))) if ref.size else 0.0
        note(f"{what}: rel_l2={rel:.3e} max_abs={mx:.3e} max|ref|={scale:.3g} "
             f"rms(ref)={float(np.sqrt(np.mean(np.square(ref)))) if ref.size else 0:.3g}")
        if not (rel <= REL_L2 and mx <= max(MAX_ABS, 1e-2 * scale)):
            self.bad.append(f"{what}: rel_l2={rel:.3e} max_abs={mx:.3e}")

    def done(self):
        assert not self.bad, "; ".join(self.bad)

NAMES = ("dx", "dwr", "dbr", "dw1", "db1", "dw2", "db2")


def gpu_backward(cfg, inp, dout_np):
    d = upload(inp)
    r = moe.route(d["x"], d["router_w"], d["router_b"], cfg.k, want_logits=False)
    dout = torch.from_numpy(dout_np).to(DEV)
    g = moe.backward(d["x"], d["router_w"], d["w1"], d["b1"], d["w2"], d["b2"], r, dout, cfg.k)
    torch.cuda.synchronize()
    return d, r, dout, g


def with_empty_expert(inp, e):
    """The same layer with router bias -64 (exact in bf16) on expert e, so it gets no token."""
    inp.br = inp.br.copy()
    inp.br[e] = f32_to_bf16_bits(np.array([-64.0], dtype=np.float32))[0]
    return inp


CASES = {
    # the tiny workload: every gradient whole
    "C1": dict(base="C1"),
    # several row tiles per expert, ragged sizes (1000 tokens, D = 256, F = 384) and an empty expert
    "ragged": dict(base="C2", name="bwd-ragged", T=1000, D=256, F=384, E=8, k=4, seed=8101, empty=5),
    # weights large enough that the SwiGLU clamps engage on both halves
    "clamped": dict(base="C2", name="bwd-clamp", T=300, D=128, F=192, E=6, k=2, seed=8102, weight_std=0.45),
    # every expert selected by every token (k = E), a single token
    "k_equals_E_one_token": dict(base="C2", name="bwd-kE", T=1, D=64, F=64, E=4, k=4, seed=8105),
    # the largest expert count: most of the 256 experts get no row
    "256_experts": dict(base="C2", name="bwd-e256", T=64, D=64, F=128, E=256, k=2, seed=8106),
}


@pytest.mark.parametrize("case", list(CASES))
def test_backward_full(case):
    spec = dict(CASES[case])
    base = spec.pop("base")
    empty = spec.pop("empty", None)
    cfg = get_config(base, **spec) if spec else get_config(base)
    inp = make_inputs(cfg)
    if empty is not None:
        inp = with_empty_expert(inp, empty)
    dout = make_dout(cfg.T, cfg.D, seed=cfg.seed)
    note(f"backward {case}: T={cfg.T} D={cfg.D} E={cfg.E} k={cfg.k} F={cfg.F}")
    _, r, _, g = gpu_backward(cfg, inp, dout)
    idx = oracle.select_experts(oracle.router_logits(inp.x, inp.wr, inp.br), cfg.k)
    assert np.array_equal(r["idx"].cpu().numpy(), idx)
    if empty is not None:
        assert not (idx == empty).any()
    if case == "clamped":
        u = np.einsum("td,egd->teg", oracle.bf16_to_f64(inp.x),
                      np.stack([oracle.expert_weight(inp.w1, "bf16", cfg.E, 2 * cfg.F, cfg.D, e) for e in range(cfg.E)]))
        routed = u[np.arange(cfg.T)[:, None], idx]
        assert (routed[..., :cfg.F] > 7).any() and (np.abs(routed[..., cfg.F:]) > 7).any()
    ref = oracle.moe_backward_grouped(inp.x, inp.wr, inp.br, inp.w1, inp.b1, inp.w2, inp.b2, idx, dout,
                                      cfg.k, cfg.F, "bf16")
    rep = Report()
    for n in NAMES:
        got = g[n].cpu().numpy()
        want = ref[n] if n in ("dx", "dwr", "dbr") else np.stack([ref[n][e] for e in range(cfg.E)])
        assert got.shape == want.shape, n
        rep.check(got, want, f"backward {case} {n}")
    rep.done()
    if empty is not None:
        for n in ("dw1", "db1", "dw2", "db2"):
            assert not g[n][empty].any(), n
        assert g["dbr"][empty].item() == 0.0 and not g["dwr"][empty].any()


def test_backward_20b_shape_every_expert():
    """The backward at the 20B shape with 256 tokens (the streaming tiles, few rows per
    expert): every gradient whole, every expert's weight and bias gradients included."""
    cfg = get_config("C2")
    inp = make_inputs("C2")
    dout = make_dout(cfg.T, cfg.D, seed=8103)
    note("backward 20B shape (C2), 256 tokens")
    _, r, _, g = gpu_backward(cfg, inp, dout)
    idx = oracle.select_experts(oracle.router_logits(inp.x, inp.wr, inp.br), cfg.k)
    assert np.array_equal(r["idx"].cpu().numpy(), idx)
    counts = np.bincount(idx.reshape(-1), minlength=cfg.E)
    pick = [int(e) for e in np.flatnonzero(counts)]
    ref = oracle.moe_backward_grouped(inp.x, inp.wr, inp.br, inp.w1, inp.b1, inp.w2, inp.b2, idx, dout,
                                      cfg.k, cfg.F, "bf16", weight_experts=pick)
    rep = Report()
    for n in ("dx", "dwr", "dbr"):
        rep.check(g[n].cpu().numpy(), ref[n], f"backward C2 {n}")
    for e in pick:
        for n in ("dw1", "db1", "dw2", "db2"):
            rep.check(g[n][e].cpu().numpy(), ref[n][e], f"backward C2 {n}[{e}] ({counts[e]} rows)")
    rep.done()


def test_backward_t8192_zipf_layer():
    """The backward at the layer bench.py times at T = 8192 (20B shape, Zipf-skewed routing:
    the matrix-core tiles, the weight-gradient mode over long and short expert K ranges):
    every gradient whole, the weight and bias gradients of every live expert included (the
    oracle runs the whole layer, one expert at a time)."""
    cfg = get_config("C3")
    inp = make_inputs("C3")
    dout = make_dout(cfg.T, cfg.D, seed=8107)
    note("backward 20B shape (C3), 8192 tokens, Zipf routing")
    _, r, _, g = gpu_backward(cfg, inp, dout)
    idx = oracle.select_experts(oracle.router_logits(inp.x, inp.wr, inp.br), cfg.k)
    assert np.array_equal(r["idx"].cpu().numpy(), idx)
    counts = np.bincount(idx.reshape(-1), minlength=cfg.E)
    pick = [int(e) for e in np.flatnonzero(counts)]
    ref = oracle.moe_backward_grouped(inp.x, inp.wr, inp.br, inp.w1, inp.b1, inp.w2, inp.b2, idx, dout,
                                      cfg.k, cfg.F, "bf16", weight_experts=pick)
    rep = Report()
    for n in ("dx", "dwr", "dbr"):
        rep.check(g[n].cpu().numpy(), ref[n], f"backward C3 {n}")
    for e in pick:
        for n in ("dw1", "db1", "dw2", "db2"):
            rep.check(g[n][e].cpu().numpy(), ref[n][e], f"backward C3 {n}[{e}] ({counts[e]} rows)")
    rep.done()


def test_backward_is_deterministic():
    cfg = get_config("C2", name="bwd-det", T=700, D=256, F=256, E=8, k=4, seed=8104)
    inp = make_inputs(cfg)
    dout = make_dout(cfg.T, cfg.D, seed=8104)
    note("backward determinism")
    d, r, dt, g1 = gpu_backward(cfg, inp, dout)
    g2 = moe.backward(d["x"], d["router_w"], d["w1"], d["b1"], d["w2"], d["b2"], r, dt, cfg.k)
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(g1[n], g2[n]), n


def test_backward_side_stream_follows_the_calling_stream():
    """At many rows per expert the backward forks its memory-bound work onto a side stream and
    joins it back: called on a non-default stream, and again after moe_release has destroyed
    the side stream, it gives the default stream's gradients bit for bit."""
    cfg = get_config("C2", name="bwd-stream", T=700, D=256, F=256, E=8, k=4, seed=8108)
    assert cfg.T * cfg.k >= 128 * cfg.E             # the matrix-core regime, where the side stream runs
    inp = make_inputs(cfg)
    dout = make_dout(cfg.T, cfg.D, seed=8108)
    note("backward on a caller stream and after release")
    d, r, dt, ref = gpu_backward(cfg, inp, dout)
    ref = {n: t.clone() for n, t in ref.items()}
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = {n: torch.empty_like(t) for n, t in ref.items()}
        moe.backward(d["x"], d["router_w"], d["w1"], d["b1"], d["w2"], d["b2"], r, dt, cfg.k, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(out[n], ref[n]), n
    moe.release()
    again = moe.backward(d["x"], d["router_w"], d["w1"], d["b1"], d["w2"], d["b2"], r, dt, cfg.k)
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(again[n], ref[n]), n


def test_backward_zero_tokens_zeroes_parameter_gradients():
    cfg = get_config("C1")
    inp = make_inputs("C1")
    d = upload(inp)
    note("backward T=0")
    x0 = d["x"][:0]
    empty_i = torch.empty(0, dtype=torch.int32, device=DEV)
    r = {"idx": empty_i.view(0, cfg.k), "gates": torch.empty((0, cfg.k), dtype=torch.float32, device=DEV),
         "offsets": torch.zeros(cfg.E + 1, dtype=torch.int32, device=DEV), "perm": empty_i}
    dout = torch.empty((0, cfg.D), dtype=torch.float32, device=DEV)
    g = moe.backward(x0, d["router_w"], d["w1"], d["b1"], d["w2"], d["b2"], r, dout, cfg.k)
    torch.cuda.synchronize()
    assert g["dx"].numel() == 0
    for n in NAMES[1:]:
        assert g[n].numel() > 0 and not g[n].any(), n
