"""Seeded input generator: determinism, encodings, shapes, and the realised Zipf loads."""
import numpy as np
import pytest

from synth import CONFIGS, f32_to_bf16_bits, get_config, make_inputs, make_router_inputs, zipf_plan


def test_bf16_rounding_is_nearest_even():
    # 1 + 2^-8 is exactly half an ulp above 1.0 in bf16: ties go to the even mantissa (1.0);
    # 1 + 3*2^-8 is half an ulp above 1 + 2^-7: ties go to 1 + 2^-6... i.e. the even neighbour
    vals = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-20, -2.5, 3.0e38], dtype=np.float32)
    got = f32_to_bf16_bits(vals)
    assert got.tolist() == [0x3F80, 0x3F80, 0x3F82, 0x3F81, 0xC020, 0x7F62]


def test_generator_is_deterministic():
    a = make_inputs(get_config("C1"))
    b = make_inputs(get_config("C1"))
    for f in ("x", "wr", "br", "w1", "b1", "w2", "b2"):
        assert np.array_equal(getattr(a, f), getattr(b, f))
    # a different seed changes the draws
    c = make_inputs(get_config("C1", seed=99))
    assert not np.array_equal(a.x, c.x)


def test_generator_shapes_and_encodings():
    cfg = get_config("C4", T=64, D=64, F=64, E=4)
    inp = make_inputs(cfg)
    E, D, F = 4, 64, 64
    assert inp.x.shape == (64, D) and inp.x.dtype == np.uint16
    assert inp.w1.dtype == np.uint8 and inp.w1.size == E * 2 * F * (D // 2 + D // 32)
    assert inp.w2.size == E * D * (F // 2 + F // 32)
    scales1 = inp.w1[E * 2 * F * D // 2:]
    assert scales1.min() >= 127 - 8 and scales1.max() <= 127 - 4
    codes = inp.w1[:E * 2 * F * D // 2]
    nib = np.concatenate([codes & 15, codes >> 4])
    counts = np.bincount(nib, minlength=16)
    assert counts.min() > 0.8 * nib.size / 16           # uniform over the 16 codes
    # RMSNorm'd activations: per-row mean square ~ 1
    xf = (inp.x.astype(np.uint32) << 16).view(np.float32)
    assert np.allclose(np.mean(xf.astype(np.float64) ** 2, axis=1), 1.0, atol=0.02)


def test_bf16_weight_distribution():
    inp = make_inputs(get_config("C2", E=2, T=8))
    w = (inp.w1.astype(np.uint32) << 16).view(np.float32)
    assert abs(w.std() - 0.02) < 2e-4 and abs(w.mean()) < 1e-4
    b = (inp.b1.astype(np.uint32) << 16).view(np.float32)
    assert abs(b.std() - 0.01) < 1e-3


def test_mxfp8_weight_buffer():
    """Codes uniform over the 254 finite E4M3 codes (no NaN code), scale bytes in the
    configured range, buffer = codes then scales."""
    cfg = get_config("Y1", E=2, T=8, D=256, F=256)
    inp = make_inputs(cfg)
    n = 2 * (2 * 256) * 256
    codes, scales = inp.w1[:n], inp.w1[n:]
    assert inp.w1.size == n + n // 32
    assert not np.isin(codes, [0x7F, 0xFF]).any()
    hist = np.bincount(codes, minlength=256)
    assert hist.max() < 2.0 * n / 254 and (hist > 0).sum() == 254
    lo, hi = cfg.scale_exp
    assert scales.min() == 127 + lo and scales.max() == 127 + hi


def test_zipf_plan_targets():
    for name in ("C3", "C5"):
        cfg = CONFIGS[name]
        p = zipf_plan(cfg)
        assert abs(p["target"].sum() - cfg.T * cfg.k) < 1e-6 * cfg.T * cfg.k
        assert p["target"].max() <= cfg.T + 1e-9
        assert p["empty"].sum() == cfg.n_empty
        if cfg.n_empty:
            assert p["empty"][0] and p["empty"][cfg.E - 1]
            assert np.all(p["target"][p["empty"]] == 0)


@pytest.mark.parametrize("name", ["C3", "C5"])
def test_stored_router_bias_reproduces_recorded_loads(name):
    """The stored bias, through the oracle's router and top-k, gives exactly the recorded counts
    (and the Zipf shape: head expert near T, empty experts empty)."""
    import oracle
    from synth.generate import _read_router_bias, router_bias_path
    cfg = CONFIGS[name]
    br = _read_router_bias(cfg)
    rec = np.array([int(l.split()[3]) for l in open(router_bias_path(cfg)) if not l.startswith("#")])
    x, wr = make_router_inputs(cfg)
    idx = oracle.select_experts(oracle.router_logits(x, wr, br), cfg.k)
    counts = np.bincount(idx.reshape(-1), minlength=cfg.E)
    assert np.array_equal(counts, rec)
    plan = zipf_plan(cfg)
    assert np.all(counts[plan["empty"]] == 0)
    assert counts.max() > 0.95 * cfg.T
    live = ~plan["empty"]
    rel = counts[live] / plan["target"][live]
    big = plan["target"][live] >= 200
    assert np.all(np.abs(rel[big] - 1) < 0.15)
