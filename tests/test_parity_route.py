"""GPU routing stage vs the oracle: logits, top-k indices, counts, offsets and the
permutation must match bit for bit; gates to 1e-6 absolute."""
import numpy as np
import pytest
import torch

import mixture_experts_transformer_amd as moe
import oracle
from synth import f32_to_bf16_bits, get_config, make_routing_inputs
from _gpu import GATE_ABS, note, u16

pytestmark = pytest.mark.gpu


def run_and_compare(x, wr, br, k, label):
    T, E = x.shape[0], wr.shape[0]
    note(f"route {label}: T={T} D={x.shape[1]} E={E} k={k}")
    r = moe.route(u16(x), u16(wr), u16(br), k)
    torch.cuda.synchronize()
    l_ref = oracle.router_logits(x, wr, br)
    idx_ref = oracle.select_experts(l_ref, k)
    g_ref = oracle.gate_weights(l_ref, idx_ref)
    counts_ref, offsets_ref, perm_ref, _ = oracle.route_assignments(idx_ref, E)
    logits = r["logits"].cpu().numpy()
    nbad = int(np.sum(logits.view(np.uint32) != l_ref.view(np.uint32)))
    assert nbad == 0, f"{label}: {nbad} logits differ from the oracle's fp32 rounding"
    assert np.array_equal(r["idx"].cpu().numpy(), idx_ref), f"{label}: top-k indices differ"
    assert np.array_equal(r["counts"].cpu().numpy(), counts_ref), f"{label}: counts differ"
    assert np.array_equal(r["offsets"].cpu().numpy(), offsets_ref), f"{label}: offsets differ"
    assert np.array_equal(r["perm"].cpu().numpy(), perm_ref), f"{label}: permutation differs"
    gerr = np.max(np.abs(r["gates"].cpu().numpy().astype(np.float64) - g_ref)) if T else 0.0
    assert gerr <= GATE_ABS, f"{label}: gate error {gerr:.3e}"
    # smallest margin between the k-th and (k+1)-th logit: how close the case came to a tie
    if k < E and T:
        srt = -np.sort(-l_ref.astype(np.float64), axis=1)
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


def test_route_exact_ties_go_to_lower_index():
    T, D, E, k = 70, 64, 40, 5
    x = np.zeros((T, D), dtype=np.uint16)
    _, wr, _ = rand_layer(1, T, D, E)
    br = np.full(E, f32_to_bf16_bits(np.float32([0.5]))[0], dtype=np.uint16)
    r = run_and_compare(x, wr, br, k, "all-equal logits")
    assert (r["idx"].cpu().numpy() == np.arange(k)).all()
    assert np.allclose(r["gates"].cpu().numpy(), 1.0 / k, atol=1e-7)


def test_route_duplicated_router_rows():
    T, D, E, k = 200, 128, 12, 4
    x, wr, br = rand_layer(2, T, D, E, bias_std=0.0)
    for a, b in [(0, 1), (3, 9), (10, 11)]:
        wr[b] = wr[a]
        br[b] = br[a]
    run_and_compare(x, wr, br, k, "duplicated rows")


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
