"""GPU routing stage vs the oracle: logits, top-k indices, counts, offsets and the
permutation must match bit for bit; gates to 1e-6 absolute.  Every case runs both ways: with
logits requested and without, as the forward calls it."""
import numpy as np
import pytest
import torch

import mixture_experts_transformer_amd as moe
import oracle
from synth import f32_to_bf16_bits, get_config, make_expert_bias, make_routing_inputs
from _gpu import DEV, GATE_ABS, note, u16

pytestmark = pytest.mark.gpu


def run_and_compare(x, wr, br, k, label, ebias=None):
    """ebias: the load-balancing expert bias (fp32 [E]) for the biased entry point, or None."""
    T, E = x.shape[0], wr.shape[0]
    note(f"route {label}: T={T} D={x.shape[1]} E={E} k={k}{' biased' if ebias is not None else ''}")
    eb = None if ebias is None else torch.from_numpy(np.ascontiguousarray(ebias, dtype=np.float32)).to(DEV)
    r = moe.route(u16(x), u16(wr), u16(br), k, expert_bias=eb)
    rf = moe.route(u16(x), u16(wr), u16(br), k, want_logits=False, expert_bias=eb)   # as the forward calls it
    torch.cuda.synchronize()
    l_ref = oracle.router_logits(x, wr, br)
    idx_ref = oracle.select_experts(l_ref, k, ebias)
    g_ref = oracle.gate_weights(l_ref, idx_ref)
    counts_ref, offsets_ref, perm_ref, _ = oracle.route_assignments(idx_ref, E)
    logits = r["logits"].cpu().numpy()
    nbad = int(np.sum(logits.view(np.uint32) != l_ref.view(np.uint32)))
    assert nbad == 0, f"{label}: {nbad} logits differ from the oracle's fp32 rounding"
    gerr = 0.0
    for path, rr in (("with logits", r), ("without logits", rf)):
        assert np.array_equal(rr["idx"].cpu().numpy(), idx_ref), f"{label} ({path}): top-k indices differ"
        assert np.array_equal(rr["counts"].cpu().numpy(), counts_ref), f"{label} ({path}): counts differ"
        assert np.array_equal(rr["offsets"].cpu().numpy(), offsets_ref), f"{label} ({path}): offsets differ"
        assert np.array_equal(rr["perm"].cpu().numpy(), perm_ref), f"{label} ({path}): permutation differs"
        ge = np.max(np.abs(rr["gates"].cpu().numpy().astype(np.float64) - g_ref)) if T else 0.0
        assert ge <= GATE_ABS, f"{label} ({path}): gate error {ge:.3e}"
        gerr = max(gerr, ge)
    # smallest margin between the k-th and (k+1)-th logit: how close the case came to a tie
    if k < E and T:
        key = l_ref if ebias is None else l_ref + np.asarray(ebias, np.float32)[None, :]
        srt = -np.sort(-key.astype(np.float64), axis=1)
        note(f"  min top-k margin {np.min(srt[:, k - 1] - srt[:, k]):.3e}, max gate err {gerr:.2e}")
    return r


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "C5", "X1", "X2"])
def test_route_workloads(name):
    cfg = get_config(name)
    x, wr, br = make_routing_inputs(cfg)
    r = run_and_compare(x, wr, br, cfg.k, name)
    if name == "C5":
        counts = r["counts"].cpu().numpy()
        assert counts[0] == 0 and counts[cfg.E - 1] == 0 and (counts == 0).sum() == 13


def rand_layer(seed, T, D, E, bias_std=0.5):
    g = np.random.default_rng(seed)
    x = f32_to_bf16_bits(g.standard_normal((T, D)).astype(np.float32))
    wr = f32_to_bf16_bits(g.standard_normal((E, D)).astype(np.float32) * np.float32(0.05))
    br = f32_to_bf16_bits(g.standard_normal(E).astype(np.float32) * np.float32(bias_std))
    return x, wr, br


@pytest.mark.parametrize("T,D,E,k", [
    (1, 64, 4, 2), (15, 64, 5, 1), (17, 128, 16, 16), (63, 64, 33, 4), (65, 192, 100, 8),
    (1000, 64, 256, 4), (300, 2880, 1, 1), (129, 256, 7, 7), (2049, 64, 64, 2),
    # one expert per lane in the top-k (E <= 64): at 64 experts, k = E, 4096 assignments
    (2048, 64, 64, 2), (1024, 128, 64, 4), (16, 64, 64, 64), (33, 2880, 64, 3),
])
def test_route_ragged_shapes(T, D, E, k):
    run_and_compare(*rand_layer(T * 7 + E, T, D, E), k, f"ragged T={T} D={D} E={E} k={k}")


@pytest.mark.parametrize("T", [70, 2048])
def test_route_exact_ties_go_to_lower_index(T):
    D, E, k = 64, 40, 5
    x = np.zeros((T, D), dtype=np.uint16)
    _, wr, _ = rand_layer(1, T, D, E)
    br = np.full(E, f32_to_bf16_bits(np.float32([0.5]))[0], dtype=np.uint16)
    r = run_and_compare(x, wr, br, k, "all-equal logits")
    assert (r["idx"].cpu().numpy() == np.arange(k)).all()
    assert np.allclose(r["gates"].cpu().numpy(), 1.0 / k, atol=1e-7)


@pytest.mark.parametrize("T", [200, 8192])
def test_route_duplicated_router_rows(T):
    D, E, k = 128, 12, 4
    x, wr, br = rand_layer(2, T, D, E, bias_std=0.0)
    for a, b in [(0, 1), (3, 9), (10, 11)]:
        wr[b] = wr[a]
        br[b] = br[a]
    run_and_compare(x, wr, br, k, "duplicated rows")


@pytest.mark.parametrize("T", [512, 4096])
def test_route_near_ties_resolved_exactly(T):
    """Router rows that differ from another expert's in one element by one bf16 ulp: logits
    a few fp32 ulps apart, whose order the fp64 router must still get right."""
    D, E, k = 2880, 32, 4
    x, wr, br = rand_layer(5, T, D, E, bias_std=0.0)
    g = np.random.default_rng(6)
    for a, b in [(0, 1), (4, 5), (8, 9), (12, 13), (20, 21), (30, 31)]:
        wr[b] = wr[a]
        d = int(g.integers(0, D))
        wr[b, d] = wr[a, d] + np.uint16(1)         # one ulp in one element
        br[b] = br[a]
    run_and_compare(x, wr, br, k, "near ties (one-ulp router rows)")


def test_route_empty_experts_at_edges():
    T, D, E, k = 500, 64, 32, 4
    x, wr, br = rand_layer(3, T, D, E)
    neg = f32_to_bf16_bits(np.float32([-64.0]))[0]
    for e in (0, 1, 2, 15, 30, 31):      # first, consecutive, middle and last experts empty
        br[e] = neg
    r = run_and_compare(x, wr, br, k, "empty experts")
    c = r["counts"].cpu().numpy()
    assert all(c[e] == 0 for e in (0, 1, 2, 15, 30, 31))


def test_route_is_deterministic():
    x, wr, br = rand_layer(4, 4096, 2880, 32)
    a = moe.route(u16(x), u16(wr), u16(br), 4)
    b = moe.route(u16(x), u16(wr), u16(br), 4)
    for key in ("logits", "idx", "gates", "counts", "offsets", "perm"):
        assert torch.equal(a[key], b[key]), key


def test_route_reused_and_garbage_workspace():
    """A caller's workspace full of random bytes, or left by earlier calls of other shapes,
    must not change any result."""
    shapes = [(256, 2880, 32, 4), (100, 64, 8, 2), (256, 2880, 32, 4), (1024, 128, 64, 4), (17, 64, 5, 5)]
    nbytes = max(moe.workspace_bytes(T, D, E, k, 64) for T, D, E, k in shapes)
    g = torch.Generator().manual_seed(7)
    ws = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, generator=g).cuda()
    moe.set_workspace(ws)
    try:
        for i, (T, D, E, k) in enumerate(shapes):
            run_and_compare(*rand_layer(100 + i, T, D, E), k, f"garbage/reused workspace #{i} T={T} E={E}")
        # every arrival word set to what a launch leaves behind, except for the tag
        ws.fill_(0xFF)
        run_and_compare(*rand_layer(200, 256, 2880, 32), 4, "workspace of 0xFF bytes")
    finally:
        moe.set_workspace(None)


# ----------------------------------------------------------- load-balancing expert bias
@pytest.mark.parametrize("T,D,E,k", [
    # one expert per lane (E <= 64) and the wave-argmax path (E > 64)
    (257, 64, 32, 4), (100, 128, 64, 8), (40, 64, 5, 5), (2049, 2880, 32, 4),
    (129, 192, 100, 6), (64, 64, 256, 16), (1000, 128, 128, 4),
])
def test_route_expert_bias(T, D, E, k):
    x, wr, br = rand_layer(T * 3 + E, T, D, E)
    eb = make_expert_bias(E, T + E)
    r = run_and_compare(x, wr, br, k, f"bias T={T} D={D} E={E} k={k}", ebias=eb)
    if k < E:
        # the bias moved the selection of some tokens
        r0 = moe.route(u16(x), u16(wr), u16(br), k)
        torch.cuda.synchronize()
        moved = (np.sort(r["idx"].cpu().numpy(), 1) != np.sort(r0["idx"].cpu().numpy(), 1)).any(1).sum()
        note(f"  {moved} of {T} tokens change experts under the bias")
        assert moved > 0


@pytest.mark.parametrize("E", [40, 80])
def test_route_expert_bias_ties_and_reordering(E):
    """Equal logits with a repeating bias: the best bias class wins, lower indices first,
    gates 1/k; then far-apart logits that the bias puts in increasing order, so the first
    slot's logit is the smallest and the gate softmax must shift by the largest."""
    T, D, k = 70, 64, 5
    x = np.zeros((T, D), dtype=np.uint16)
    _, wr, _ = rand_layer(3, T, D, E)
    br = np.full(E, f32_to_bf16_bits(np.float32([0.5]))[0], dtype=np.uint16)
    eb = (np.arange(E) % 3).astype(np.float32) * np.float32(0.25)
    r = run_and_compare(x, wr, br, k, f"biased ties E={E}", ebias=eb)
    assert (r["idx"].cpu().numpy() == np.arange(2, 2 + 3 * k, 3)).all()
    assert np.allclose(r["gates"].cpu().numpy(), 1.0 / k, atol=1e-7)
    vals = np.full(E, -1024.0, np.float32)
    vals[[3, 7, 11]] = [-512.0, 512.0, 0.0]
    br2 = f32_to_bf16_bits(vals)
    eb2 = np.zeros(E, np.float32)
    eb2[[3, 7, 11]] = [8192.0, 1024.0, 4096.0]
    r2 = run_and_compare(x, wr, br2, 3, f"biased reorder E={E}", ebias=eb2)
    assert (r2["idx"].cpu().numpy() == np.array([3, 11, 7])).all()
    g = r2["gates"].cpu().numpy()
    assert np.isfinite(g).all() and (g[:, 2] == 1.0).all()


def test_route_zero_expert_bias_is_bitwise_unbiased():
    T, D, E, k = 3000, 128, 48, 4
    x, wr, br = rand_layer(9, T, D, E)
    note(f"route zero bias: T={T} E={E}")
    a = moe.route(u16(x), u16(wr), u16(br), k)
    b = moe.route(u16(x), u16(wr), u16(br), k, expert_bias=torch.zeros(E, dtype=torch.float32, device=DEV))
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key


@pytest.mark.parametrize("T,D,E,k", [(512, 256, 32, 4), (300, 128, 100, 6), (64, 64, 256, 8), (40, 64, 1, 1)])
def test_expert_bias_balancing_loop(T, D, E, k):
    """Biased routing and the load-balancing update in turn, six steps from a zero bias, on
    the GPU and in the oracle: every step's routing bit for bit, the bias bit for bit.  The
    step (0.05, not the training default 1e-3) is large enough to move tokens every step."""
    x, wr, br = rand_layer(T + 5 * E, T, D, E)
    note(f"balancing loop T={T} D={D} E={E} k={k}")
    eb = torch.zeros(E, dtype=torch.float32, device=DEV)
    eb_ref = np.zeros(E, np.float32)
    l_ref = oracle.router_logits(x, wr, br)
    spread = []
    for step in range(6):
        r = moe.route(u16(x), u16(wr), u16(br), k, want_logits=False, expert_bias=eb)
        moe.update_expert_bias(eb, r["counts"], 0.05)
        torch.cuda.synchronize()
        idx_ref = oracle.select_experts(l_ref, k, eb_ref)
        counts_ref = oracle.route_assignments(idx_ref, E)[0]
        assert np.array_equal(r["idx"].cpu().numpy(), idx_ref), f"step {step}: top-k differs"
        assert np.array_equal(r["counts"].cpu().numpy(), counts_ref), f"step {step}: counts differ"
        eb_ref = oracle.update_expert_bias(eb_ref, counts_ref, 0.05)
        assert eb.cpu().numpy().tobytes() == eb_ref.tobytes(), f"step {step}: bias differs"
        spread.append(int(counts_ref.max() - counts_ref.min()))
    note(f"  load spread per step: {spread}")
    if E > k:
        assert spread[-1] < spread[0]


@pytest.mark.parametrize("E", [1, 7, 64, 200, 256])
def test_expert_bias_update_direct(E):
    """Counts with some experts exactly at the mean, a bias with -0 entries and a large
    coefficient: the new bias bit for bit."""
    g = np.random.default_rng(E)
    counts = g.integers(0, 9, E).astype(np.int32)
    counts[: E // 2] = 4
    counts[E // 2:] = np.where(np.arange(E - E // 2) % 2 == 0, 2, 6)[: E - E // 2]
    if (E - E // 2) % 2:
        counts[-1] = 4                                  # keep the mean at exactly 4
    bias = (g.standard_normal(E) * 0.1).astype(np.float32)
    bias[::5] = -0.0
    for coeff in (1e-3, 0.375, 3e-8):
        note(f"bias update E={E} coeff={coeff}")
        eb = torch.from_numpy(bias.copy()).to(DEV)
        moe.update_expert_bias(eb, torch.from_numpy(counts).to(DEV), coeff)
        torch.cuda.synchronize()
        ref = oracle.update_expert_bias(bias, counts, coeff)
        assert eb.cpu().numpy().tobytes() == ref.tobytes()

