"""Pins for the float64 oracle, written independently of it.

Each check compares the oracle with something fixed outside it: closed forms
evaluated another way, exact rational arithmetic, brute-force enumeration, the
printed E2M1 table, algebraic invariants of the block, and special cases that
reduce to a plain dense MLP.  A mistake anywhere in the oracle -- a dropped bias,
a swapped nibble, a sign, a clamp on the wrong side, a transposed weight, an
unstable sort, softmax over the wrong set -- fails at least one of them (the
comment on each test says which mistakes it catches).

Pages: torchtitan GPT-OSS guide (grouped GEMM section: counts/offsets, mlp1/mlp2,
SwiGLU variant); "gptoss" re-implementation page (top-4 of 32, weighted
combination); GPT-OSS-in-Transformers blog (MXFP4 = E2M1 + 32-element block scale).
"""
import itertools
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import (SWIGLU_ALPHA, SWIGLU_LIMIT, bf16_to_f64, e2m1_value, e4m3_value, expert_weight,
                    gate_weights, moe_forward, mxfp4_decode, mxfp8_decode, route_assignments,
                    router_logits, select_experts, swiglu, update_expert_bias)
from synth import f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- helpers (test-side, independent)
def bf16_closed_form(bits: int) -> float:
    s, e, m = bits >> 15, (bits >> 7) & 0xFF, bits & 0x7F
    if e == 0:
        v = math.ldexp(m / 128.0, -126)
    else:
        v = math.ldexp(1.0 + m / 128.0, e - 127)
    return -v if s else v


def e2m1_closed_form(code: int) -> float:
    s, e, m = code >> 3, (code >> 1) & 3, code & 1
    v = 0.5 * m if e == 0 else math.ldexp(1.0 + 0.5 * m, e - 1)
    return -v if s else v


def e4m3_closed_form(code: int) -> float:
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    if e == 15 and m == 7:
        return math.nan
    v = math.ldexp(m / 8.0, -6) if e == 0 else math.ldexp(1.0 + m / 8.0, e - 7)
    return -v if s else v


def mxfp8_elementwise(buf: np.ndarray, E: int, rows: int, K: int, e: int) -> np.ndarray:
    """Decode MXFP8 expert e element by element from byte addresses."""
    out = np.empty((rows, K))
    scale_base = E * rows * K + e * rows * (K // 32)
    for r in range(rows):
        for i in range(K):
            code = int(buf[e * rows * K + r * K + i])
            s = int(buf[scale_base + r * (K // 32) + i // 32])
            out[r, i] = e4m3_closed_form(code) * math.ldexp(1.0, s - 127)
    return out


def mxfp4_elementwise(buf: np.ndarray, E: int, rows: int, K: int, e: int) -> np.ndarray:
    """Decode expert e element by element from byte addresses (layout stated in the library header)."""
    out = np.empty((rows, K))
    code_base = e * rows * (K // 2)
    scale_base = E * rows * (K // 2) + e * rows * (K // 32)
    for r in range(rows):
        for i in range(K):
            byte = int(buf[code_base + r * (K // 2) + i // 2])
            code = (byte >> 4) if (i & 1) else (byte & 15)
            s = int(buf[scale_base + r * (K // 32) + i // 32])
            out[r, i] = e2m1_closed_form(code) * math.ldexp(1.0, s - 127)
    return out


def to_f32(v: float) -> float:
    return struct.unpack("<f", struct.pack("<f", v))[0]


def biased_key(l, b):
    """fp32 logit + fp32 bias rounded once to fp32, one element at a time through Python floats:
    the float64 sum of two fp32 values rounded again to fp32 equals the correctly rounded fp32
    sum (53 >= 2*24 + 2 makes the double rounding innocuous for addition)."""
    l = np.asarray(l, dtype=np.float32)
    b = np.asarray(b, dtype=np.float32)
    return np.array([[to_f32(float(l[t, e]) + float(b[e])) for e in range(l.shape[1])]
                     for t in range(l.shape[0])])


def sigmoid_tanh(z):
    """Logistic function through tanh: another route than the oracle's 1/(1+exp(-z))."""
    return 0.5 * (1.0 + np.tanh(0.5 * np.asarray(z, dtype=np.float64)))


def dense_reference(x, wr, br, w1, b1, w2, b2, k, F, fmt, ebias=None):
    """Every expert on every token, then a masked softmax mixture: no permutation, no grouping.
    With ``ebias`` the mask follows the fp32 key logit + bias; the softmax stays on the logits.

    Catches: a transposed weight, a dropped bias, gate and linear halves swapped,
    the gate weight applied outside mlp2's bias, a wrong token<->row mapping in the
    permuted formulation.
    """
    T, D = x.shape
    E = wr.shape[0]
    xf = bf16_to_f64(x)
    W1 = np.stack([expert_weight(w1, fmt, E, 2 * F, D, e) for e in range(E)])  # [E, 2F, D]
    W2 = np.stack([expert_weight(w2, fmt, E, D, F, e) for e in range(E)])      # [E, D, F]
    B1 = bf16_to_f64(b1).reshape(E, 2 * F)
    B2 = bf16_to_f64(b2).reshape(E, D)
    u = np.einsum("td,egd->teg", xf, W1) + B1[None]
    gate = np.where(u[..., :F] > SWIGLU_LIMIT, SWIGLU_LIMIT, u[..., :F])
    lin = np.where(u[..., F:] > SWIGLU_LIMIT, SWIGLU_LIMIT,
                   np.where(u[..., F:] < -SWIGLU_LIMIT, -SWIGLU_LIMIT, u[..., F:]))
    h = gate * sigmoid_tanh(SWIGLU_ALPHA * gate) * (1.0 + lin)
    Y = np.einsum("tef,edf->ted", h, W2) + B2[None]                          # [T, E, D]
    # exact logits via rationals, rounded once to fp32
    l = np.array([[to_f32(float(sum(Fraction(bf16_closed_form(int(a))) * Fraction(bf16_closed_form(int(b)))
                                     for a, b in zip(x[t], wr[e])) + Fraction(bf16_closed_form(int(br[e])))))
                   for e in range(E)] for t in range(T)])
    sel = l if ebias is None else biased_key(l, ebias)
    mask = np.zeros((T, E), dtype=bool)
    for t in range(T):
        # k largest, ties to the lower index: repeatedly take the first maximum
        avail = list(range(E))
        for _ in range(k):
            best = max(avail, key=lambda e: (sel[t, e], -e))
            mask[t, best] = True
            avail.remove(best)
    masked = np.where(mask, l, -np.inf)
    z = np.exp(masked - masked.max(axis=1, keepdims=True))
    gh = z / z.sum(axis=1, keepdims=True)
    return np.einsum("te,ted->td", gh, Y), l, mask


def tiny_layer(seed, T, D, E, k, F, fmt, wstd=0.3, bstd=0.2, br_std=0.5, mx8_scales=(115, 119)):
    """Small random layer (bits).  With MXFP4 weights the SwiGLU clamps engage; bf16 and MXFP8
    layers engage them when wstd or mx8_scales (E8M0 bytes drawn in [lo, hi)) are raised."""
    g = np.random.default_rng(seed)
    bf = lambda *s, std=1.0: f32_to_bf16_bits(g.standard_normal(s).astype(np.float32) * np.float32(std))
    x = bf(T, D)
    wr = bf(E, D, std=0.3)
    br = bf(E, std=br_std)
    if fmt == "bf16":
        w1 = bf(E, 2 * F, D, std=wstd)
        w2 = bf(E, D, F, std=wstd)
    elif fmt == "mxfp8":
        def mx8(rows, K):
            codes = g.integers(0, 256, E * rows * K, dtype=np.uint8)
            codes[(codes & 0x7F) == 0x7F] -= 1               # no NaN codes
            scales = g.integers(mx8_scales[0], mx8_scales[1], E * rows * K // 32, dtype=np.uint8)
            return np.concatenate([codes, scales])
        w1, w2 = mx8(2 * F, D), mx8(D, F)
    else:
        def mx(rows, K):
            codes = g.integers(0, 256, E * rows * K // 2, dtype=np.uint8)
            scales = g.integers(123, 128, E * rows * K // 32, dtype=np.uint8)
            return np.concatenate([codes, scales])
        w1, w2 = mx(2 * F, D), mx(D, F)
    b1 = bf(E, 2 * F, std=bstd)
    b2 = bf(E, D, std=bstd)
    return x, wr, br, w1, b1, w2, b2


# ------------------------------------------------------------------------------- encodings
def test_bf16_decode_all_finite_patterns():
    """Every finite bf16 pattern against (-1)^s 2^(e-127)(1+m/128) (subnormals 2^-126 m/128)."""
    bits = np.arange(65536, dtype=np.uint32)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    bits = bits[finite].astype(np.uint16)
    got = bf16_to_f64(bits)
    want = np.array([bf16_closed_form(int(b)) for b in bits])
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))


def test_e2m1_table_matches_golden():
    """E2M1 values against the printed table (catches a wrong exponent bias or sign bit)."""
    rows = [l.split() for l in open(os.path.join(GOLDEN, "e2m1_values.txt")) if not l.startswith("#")]
    assert len(rows) == 16
    for code_hex, sign, ebits, mbit, val in rows:
        c = int(code_hex, 16)
        assert int(sign) == c >> 3 and int(ebits, 2) == (c >> 1) & 3 and int(mbit) == c & 1
        v = float(e2m1_value(c))
        assert v == float(val) and math.copysign(1, v) == math.copysign(1, float(val))
        assert v == e2m1_closed_form(c)


def test_mxfp4_decode_exhaustive_codes_and_scales():
    """All 16 codes x all 255 finite E8M0 bytes against the closed form, with nibble order:
    even element = low nibble; element i uses scale byte i // 32."""
    K = 32
    for s in range(255):
        codes = np.array([[lo | (hi << 4) for hi in range(16) for lo in (hi,)]], dtype=np.uint8)
        # row of 16 bytes = 32 elements: element 2i and 2i+1 both code i, then a second pass
        # with distinct nibbles below
        got = mxfp4_decode(codes, np.array([[s]], dtype=np.uint8))
        want = [e2m1_closed_form(i // 2) * math.ldexp(1.0, s - 127) for i in range(K)]
        assert np.array_equal(got[0], np.array(want)), s
    # distinct nibbles: byte i = lo (i) | hi (15 - i)
    codes = np.array([[(i % 16) | ((15 - i % 16) << 4) for i in range(16)]], dtype=np.uint8)
    got = mxfp4_decode(codes, np.array([[127]], dtype=np.uint8))[0]
    for i in range(16):
        assert got[2 * i] == e2m1_closed_form(i % 16)
        assert got[2 * i + 1] == e2m1_closed_form(15 - i % 16)
    assert np.isnan(mxfp4_decode(codes, np.array([[255]], dtype=np.uint8))).all()


def test_mxfp4_expert_buffer_layout():
    """Experts, rows and 32-element blocks are addressed exactly as the byte layout says."""
    g = np.random.default_rng(7)
    E, rows, K = 3, 5, 64
    buf = np.concatenate([g.integers(0, 256, E * rows * K // 2, dtype=np.uint8),
                          g.integers(100, 150, E * rows * K // 32, dtype=np.uint8)])
    for e in range(E):
        assert np.array_equal(expert_weight(buf, "mxfp4", E, rows, K, e),
                              mxfp4_elementwise(buf, E, rows, K, e))
    with pytest.raises(ValueError):
        expert_weight(buf[:-1], "mxfp4", E, rows, K, 0)


def test_e4m3_all_codes_match_library_and_closed_form():
    """All 256 E4M3 codes against torch's float8_e4m3fn conversion (a library routine) and
    the bit-field closed form: bias 7, subnormals (m/8) 2^-6, 0x7F/0xFF NaN, 448 the
    largest finite (catches a wrong bias, a missing subnormal case, an infinity)."""
    import torch
    codes = np.arange(256)
    got = e4m3_value(codes)
    lib = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(got), np.isnan(lib))
    fin = ~np.isnan(lib)
    assert np.array_equal(got[fin], lib[fin]) and np.array_equal(np.signbit(got[fin]), np.signbit(lib[fin]))
    for c in range(256):
        cf = e4m3_closed_form(c)
        assert (math.isnan(cf) and math.isnan(got[c])) or cf == got[c]
    assert np.nanmax(got) == 448.0 and got[1] == 2.0 ** -9 and got[8] == 2.0 ** -6
    assert np.isnan(got[[0x7F, 0xFF]]).all() and np.isfinite(got[[0x7E, 0xFE]]).all()


def test_mxfp8_decode_codes_scales_and_layout():
    """Every code under every finite E8M0 byte, element i using scale byte i // 32; expert,
    row and block addressing element by element; 255 = NaN; a short buffer is refused."""
    codes = np.arange(256, dtype=np.uint8).reshape(1, 256)
    vals = np.array([e4m3_closed_form(c) for c in range(256)])
    for s in range(0, 255, 7):
        sc = np.array([[s, s + 1, s, s + 1, s, s + 1, s, s + 1]], dtype=np.uint8) if s < 254 else \
            np.full((1, 8), s, dtype=np.uint8)
        got = mxfp8_decode(codes, sc)[0]
        want = vals * np.array([math.ldexp(1.0, int(sc[0, i // 32]) - 127) for i in range(256)])
        assert np.array_equal(np.isnan(got), np.isnan(want))
        assert np.array_equal(got[~np.isnan(want)], want[~np.isnan(want)]), s
    assert np.isnan(mxfp8_decode(codes, np.full((1, 8), 255, dtype=np.uint8))).all()
    g = np.random.default_rng(8)
    E, rows, K = 3, 5, 64
    buf = np.concatenate([g.integers(0, 256, E * rows * K, dtype=np.uint8),
                          g.integers(100, 150, E * rows * K // 32, dtype=np.uint8)])
    for e in range(E):
        a = expert_weight(buf, "mxfp8", E, rows, K, e)
        b = mxfp8_elementwise(buf, E, rows, K, e)
        assert np.array_equal(np.isnan(a), np.isnan(b)) and np.array_equal(a[~np.isnan(a)], b[~np.isnan(b)])
    with pytest.raises(ValueError):
        expert_weight(buf[:-1], "mxfp8", E, rows, K, 0)


# ------------------------------------------------------------------------------- router and top-k
def test_router_logits_exact_rational():
    """Logits = exact rational dot product + bias, rounded once to fp32 (catches a dropped bias,
    a transposed router weight, fp32 accumulation)."""
    x, wr, br, *_ = tiny_layer(1, T=6, D=40, E=5, k=2, F=32, fmt="bf16")
    got = router_logits(x, wr, br)
    assert got.dtype == np.float32 and got.shape == (6, 5)
    for t in range(6):
        for e in range(5):
            exact = sum(Fraction(bf16_closed_form(int(a))) * Fraction(bf16_closed_form(int(b)))
                        for a, b in zip(x[t], wr[e])) + Fraction(bf16_closed_form(int(br[e])))
            assert got[t, e] == np.float32(to_f32(float(exact)))


@pytest.mark.parametrize("E,k", [(4, 1), (4, 2), (6, 3), (8, 4), (5, 5)])
def test_topk_brute_force(E, k):
    """Enumerate every k-subset: the chosen set has the largest logits (ties to lower index),
    slots are in descending logit order (catches ascending order, a wrong tie-break)."""
    g = np.random.default_rng(E * 10 + k)
    T = 64
    # coarse values force many exact ties
    logits = (g.integers(-3, 4, (T, E)) * 0.5).astype(np.float32)
    idx = select_experts(logits, k)
    for t in range(T):
        key = lambda e: (float(logits[t, e]), -e)
        best = max(itertools.combinations(range(E), k), key=lambda S: sorted(key(e) for e in S))
        assert sorted(idx[t].tolist()) == sorted(best)
        assert [key(e) for e in idx[t]] == sorted([key(e) for e in idx[t]], reverse=True)


def test_topk_constructed_ties_and_duplicate_rows():
    """x = 0 with equal biases -> experts 0..k-1 with gates 1/k; duplicated router rows ->
    the lower index comes first."""
    E, D, k = 8, 32, 3
    x = np.zeros((4, D), dtype=np.uint16)
    wr = f32_to_bf16_bits(np.random.default_rng(0).standard_normal((E, D)).astype(np.float32))
    br = np.full(E, f32_to_bf16_bits(np.float32([0.25]))[0], dtype=np.uint16)
    l = router_logits(x, wr, br)
    idx = select_experts(l, k)
    assert (idx == np.arange(k)).all()
    assert np.allclose(gate_weights(l, idx), 1.0 / k, rtol=0, atol=1e-15)
    xr = f32_to_bf16_bits(np.random.default_rng(1).standard_normal((16, D)).astype(np.float32))
    wr2 = wr.copy()
    wr2[5] = wr2[2]                       # experts 2 and 5 now always tie
    br0 = np.zeros(E, dtype=np.uint16)
    l2 = router_logits(xr, wr2, br0)
    idx2 = select_experts(l2, E)
    assert np.array_equal(l2[:, 2], l2[:, 5])
    for t in range(16):
        order = idx2[t].tolist()
        assert order.index(2) < order.index(5)


@pytest.mark.parametrize("E,k", [(4, 2), (6, 3), (8, 4), (5, 5)])
def test_topk_expert_bias_brute_force(E, k):
    """Load-balancing bias: every k-subset enumerated against the fp32 key logit + bias (ties
    to the lower index), slots descending by that key, gates the softmax of the unbiased
    logits over the chosen set (catches the bias left out of the selection, the bias
    leaking into the gates, a key summed in float64)."""
    g = np.random.default_rng(100 + E * 10 + k)
    T = 64
    logits = (g.integers(-3, 4, (T, E)) * 0.5).astype(np.float32)
    bias = (g.integers(-2, 3, E) * 0.25).astype(np.float32)     # coarse: many exact key ties
    idx = select_experts(logits, k, bias)
    key = biased_key(logits, bias)
    for t in range(T):
        kf = lambda e: (float(key[t, e]), -e)
        best = max(itertools.combinations(range(E), k), key=lambda S: sorted(kf(e) for e in S))
        assert sorted(idx[t].tolist()) == sorted(best)
        assert [kf(e) for e in idx[t]] == sorted([kf(e) for e in idx[t]], reverse=True)
    w = gate_weights(logits, idx)
    for t in range(T):
        z = [math.exp(float(logits[t, e])) for e in idx[t]]
        assert np.allclose(w[t], [v / sum(z) for v in z], rtol=1e-12, atol=0)


def test_topk_expert_bias_special_cases():
    """A zero bias is no bias; a bias that dominates forces its experts in key order while the
    gates still come from the logits; the key is rounded to fp32 once, so a bias below half
    an ulp of the logit leaves a tie that the lower index wins."""
    g = np.random.default_rng(7)
    l = g.standard_normal((50, 16)).astype(np.float32) * 2
    for k in (1, 4, 16):
        assert np.array_equal(select_experts(l, k, np.zeros(16, np.float32)), select_experts(l, k))
    forced = np.zeros(16, np.float32)
    forced[[11, 3, 7]] = [3e30, 2e30, 1e30]
    idx = select_experts(l, 3, forced)
    assert (idx == np.array([11, 3, 7])).all()
    w = gate_weights(l, idx)
    ex = np.exp(l[:, [11, 3, 7]].astype(np.float64))
    assert np.allclose(w, ex / ex.sum(axis=1, keepdims=True), rtol=1e-12, atol=0)
    one = np.ones((1, 2), np.float32)
    half_ulp = np.float32(2.0 ** -24)                       # 1 + 2^-24 rounds (to even) to 1
    assert select_experts(one, 1, np.array([0, half_ulp], np.float32))[0, 0] == 0
    assert select_experts(one, 1, np.array([0, 2 * half_ulp], np.float32))[0, 0] == 1
    assert select_experts(one, 1, np.array([half_ulp, 0], np.float32))[0, 0] == 0
    # a bias that puts the smaller of two far-apart logits first: the gates stay finite
    far = np.array([[-512.0, 512.0, -1024.0]], np.float32)
    idx = select_experts(far, 2, np.array([4096, 1024, 0], np.float32))
    assert idx.tolist() == [[0, 1]]
    assert gate_weights(far, idx).tolist() == [[0.0, 1.0]]


def test_expert_bias_update():
    """A hand-worked step, the balanced case, and a brute-force sign against exact rationals
    (catches a flipped sign, the mean taken over tokens instead of assignments per expert,
    a step at the mean)."""
    c = np.float32(1e-3)
    got = update_expert_bias(np.zeros(4, np.float32), np.array([5, 1, 0, 2]), 1e-3)
    assert got.tolist() == [float(-c), float(c), float(c), 0.0]          # mean 2
    b = np.array([0.5, -0.25, 0.0], np.float32)
    assert np.array_equal(update_expert_bias(b, np.array([7, 7, 7]), 1e-3), b)
    assert update_expert_bias(np.array([-0.0], np.float32), np.array([3]), 1e-3).tobytes() == \
        np.array([-0.0], np.float32).tobytes()                              # at the mean: untouched
    g = np.random.default_rng(21)
    for E in (2, 5, 32, 256):
        cnt = g.integers(0, 50, E)
        b0 = (g.standard_normal(E) * 0.3).astype(np.float32)
        new = update_expert_bias(b0, cnt, 1e-3)
        for e in range(E):
            d = Fraction(int(cnt.sum()), E) - int(cnt[e])
            want = b0[e] if d == 0 else np.float32(to_f32(float(b0[e]) + (1 if d > 0 else -1) * float(c)))
            assert new[e].tobytes() == np.float32(want).tobytes()


def test_gate_weights_properties():
    """Sum to 1, descending, k=1 gives 1, and equal to softmax-over-all renormalised on the
    chosen set (catches softmax over all experts without renormalisation, a wrong sign)."""
    g = np.random.default_rng(3)
    l = g.standard_normal((200, 12)).astype(np.float32) * 3
    for k in (1, 2, 4, 12):
        idx = select_experts(l, k)
        w = gate_weights(l, idx)
        assert np.all(np.abs(w.sum(axis=1) - 1) <= 1e-12)
        assert np.all(np.diff(w, axis=1) <= 0)
        full = np.exp(l.astype(np.float64))
        full /= full.sum(axis=1, keepdims=True)
        sel = np.take_along_axis(full, idx.astype(np.int64), axis=1)
        assert np.allclose(w, sel / sel.sum(axis=1, keepdims=True), rtol=1e-12, atol=0)
        if k == 1:
            assert np.all(w == 1.0)


def test_route_assignments_invariants():
    """Counts, offsets and the stable permutation (catches an unstable sort, an inclusive/
    exclusive scan mix-up, empty-group handling)."""
    g = np.random.default_rng(4)
    for E, T, k in [(4, 64, 2), (32, 257, 4), (128, 300, 4), (7, 1, 7)]:
        l = g.standard_normal((T, E)).astype(np.float32)
        l[:, 0] -= 100        # expert 0 and E-1 empty
        l[:, E - 1] -= 100
        if k == E:
            l[:, 0] += 100
            l[:, E - 1] += 100
        idx = select_experts(l, k)
        counts, offsets, perm, rowpos = route_assignments(idx, E)
        flat = idx.reshape(-1)
        assert counts.sum() == T * k and offsets[0] == 0 and offsets[E] == T * k
        assert np.all(np.diff(offsets) == counts) and np.all(counts >= 0)
        assert np.array_equal(np.sort(perm), np.arange(T * k))
        assert np.array_equal(rowpos[perm], np.arange(T * k))
        for e in range(E):
            grp = perm[offsets[e]:offsets[e + 1]]
            assert np.all(flat[grp] == e)
            assert np.all(np.diff(grp) > 0)
        if k < E:
            assert counts[0] == 0 and counts[E - 1] == 0


# ------------------------------------------------------------------------------- SwiGLU
def test_swiglu_closed_form_points():
    """Spot values from properties, not the formula: gate 0 -> 0; linear -1 -> 0; the gate is
    clamped only from above (gate 10 == gate 7, gate -10 keeps -10 sigma(-17.02)); the linear
    half is clamped on both sides; sigma through tanh."""
    F = 1
    def h(gv, lv):
        return float(swiglu(np.array([[gv, lv]], dtype=np.float64), F)[0, 0])
    for lv in (-10, -7, 0, 7, 10):
        assert h(0.0, lv) == 0.0
    for gv in (-10, -1, 0, 1, 6.99, 7, 10):
        assert abs(h(gv, -1.0)) == 0.0
    assert h(10.0, 0.5) == h(7.0, 0.5)
    assert h(7.0, 0.5) != h(6.99, 0.5)
    s = sigmoid_tanh(-1.702 * 10.0)
    assert math.isclose(h(-10.0, 0.0), -10.0 * s, rel_tol=1e-9)   # 1 + tanh(-8.5) cancels ~1e-11
    assert h(-10.0, 0.0) != h(-7.0, 0.0)
    assert h(1.0, 10.0) == h(1.0, 7.0) and math.isclose(h(1.0, 7.0), 8 * sigmoid_tanh(1.702), rel_tol=1e-13)
    assert h(1.0, -10.0) == h(1.0, -7.0) and math.isclose(h(1.0, -7.0), -6 * sigmoid_tanh(1.702), rel_tol=1e-13)
    assert math.isclose(h(10.0, -10.0), -42 * sigmoid_tanh(1.702 * 7), rel_tol=1e-13)


def test_swiglu_gate_is_gelu_like():
    """x sigmoid(1.702 x) is the published sigmoid approximation of GELU (Hendrycks & Gimpel):
    within 0.021 of x Phi(x) on [-6, 6] -- pins alpha's value, not only its role."""
    xs = np.linspace(-6, 6, 2001)
    u = np.concatenate([xs[:, None], np.zeros((xs.size, 1))], axis=1)
    got = swiglu(u, 1)[:, 0]
    gelu = 0.5 * xs * (1 + np.array([math.erf(v / math.sqrt(2)) for v in xs]))
    assert np.max(np.abs(got - gelu)) < 0.021


# ------------------------------------------------------------------------------- whole block
@pytest.mark.parametrize("fmt", ["bf16", "mxfp4", "mxfp8"])
@pytest.mark.parametrize("T,D,E,k,F,seed", [(12, 32, 4, 2, 32, 0), (9, 64, 6, 3, 64, 1), (5, 32, 3, 3, 32, 2)])
def test_block_equals_dense_masked_mixture(fmt, T, D, E, k, F, seed):
    """Permuted/grouped oracle == every-expert-on-every-token masked softmax mixture (1e-12), on
    layers whose weights put some SwiGLU inputs past the clamps."""
    layer = tiny_layer(seed, T, D, E, k, F, fmt, wstd=5.0 / np.sqrt(D), mx8_scales=(119, 123))
    out, r = moe_forward(*layer, k=k, F=F, fmt=fmt, return_routing=True)
    ref, l, mask = dense_reference(*layer, k=k, F=F, fmt=fmt)
    assert np.array_equal(r["logits"], l.astype(np.float32))
    assert np.array_equal(np.sort(r["idx"], axis=1), np.array([np.flatnonzero(m) for m in mask]))
    scale = np.max(np.abs(ref))
    assert np.max(np.abs(out - ref)) <= 1e-12 * scale
    # the SwiGLU clamps were exercised on the routed pairs: some gate input above the limit,
    # some linear input past it on each side
    xf = bf16_to_f64(layer[0])
    W1 = np.stack([expert_weight(layer[3], fmt, E, 2 * F, D, e) for e in range(E)])
    u = np.einsum("td,egd->teg", xf, W1) + bf16_to_f64(layer[4]).reshape(E, 2 * F)[None]
    routed = u[mask]                                   # [T*k, 2F]
    assert (routed[:, :F] > SWIGLU_LIMIT).any()
    assert (routed[:, F:] > SWIGLU_LIMIT).any() and (routed[:, F:] < -SWIGLU_LIMIT).any()


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4"])
def test_block_with_expert_bias_equals_dense_masked_mixture(fmt):
    """The biased block == the dense mixture masked by the biased key, softmax on the logits;
    the bias is large enough to change the selection of most tokens."""
    T, D, E, k, F = 10, 32, 6, 2, 32
    layer = tiny_layer(11, T, D, E, k, F, fmt)
    bias = np.random.default_rng(12).standard_normal(E).astype(np.float32) * 2
    out, r = moe_forward(*layer, k=k, F=F, fmt=fmt, return_routing=True, expert_bias=bias)
    ref, l, mask = dense_reference(*layer, k=k, F=F, fmt=fmt, ebias=bias)
    _, _, mask0 = dense_reference(*layer, k=k, F=F, fmt=fmt)
    assert (mask != mask0).any(axis=1).sum() >= T // 2
    assert np.array_equal(np.sort(r["idx"], axis=1), np.array([np.flatnonzero(m) for m in mask]))
    assert np.max(np.abs(out - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_block_single_expert_is_dense_swiglu_mlp():
    """E = 1, k = 1: out = W2 swiglu(W1 x + b1) + b2 with gate weight 1."""
    T, D, F = 10, 64, 64
    x, wr, br, w1, b1, w2, b2 = tiny_layer(5, T, D, 1, 1, F, "bf16")
    out = moe_forward(x, wr, br, w1, b1, w2, b2, k=1, F=F, fmt="bf16")
    X = bf16_to_f64(x)
    W1 = bf16_to_f64(w1).reshape(2 * F, D)
    W2 = bf16_to_f64(w2).reshape(D, F)
    B1 = bf16_to_f64(b1).reshape(2 * F)
    B2 = bf16_to_f64(b2).reshape(D)
    ref = np.zeros((T, D))
    for t in range(T):
        u = [sum(W1[i, d] * X[t, d] for d in range(D)) + B1[i] for i in range(2 * F)]
        hv = []
        for f in range(F):
            gc = min(u[f], 7.0)
            lc = max(min(u[F + f], 7.0), -7.0)
            hv.append(gc / (1.0 + math.exp(-1.702 * gc)) * (lc + 1.0))
        for o in range(D):
            ref[t, o] = sum(W2[o, f] * hv[f] for f in range(F)) + B2[o]
    assert np.max(np.abs(out - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_block_zero_weights_reduce_to_biases():
    """W1 = 0 -> every row sees swiglu(b1); W2 = 0 -> out = sum_j g_j b2[e_j] (the gate scales
    mlp2's bias; catches the bias added outside the gate scaling)."""
    T, D, E, k, F = 16, 32, 5, 3, 32
    x, wr, br, w1, b1, w2, b2 = tiny_layer(6, T, D, E, k, F, "bf16")
    out, r = moe_forward(x, wr, br, w1, b1, np.zeros_like(w2), b2, k=k, F=F, fmt="bf16", return_routing=True)
    B2 = bf16_to_f64(b2).reshape(E, D)
    ref = np.einsum("tj,tjd->td", r["gates"], B2[r["idx"]])
    assert np.max(np.abs(out - ref)) <= 1e-14
    out0 = moe_forward(x, wr, br, np.zeros_like(w1), b1, w2, b2, k=k, F=F, fmt="bf16")
    B1 = bf16_to_f64(b1).reshape(E, 2 * F)
    W2 = bf16_to_f64(w2).reshape(E, D, F)
    hb = np.minimum(B1[:, :F], 7) * sigmoid_tanh(1.702 * np.minimum(B1[:, :F], 7)) * (np.clip(B1[:, F:], -7, 7) + 1)
    ye = np.einsum("edf,ef->ed", W2, hb) + B2
    ref0 = np.einsum("tj,tjd->td", r["gates"], ye[r["idx"]])
    assert np.max(np.abs(out0 - ref0)) <= 1e-12 * np.max(np.abs(ref0))


def test_block_k_equals_E_is_full_softmax_mixture():
    T, D, E, F = 8, 32, 4, 32
    layer = tiny_layer(8, T, D, E, E, F, "bf16")
    out = moe_forward(*layer, k=E, F=F, fmt="bf16")
    ref, _, mask = dense_reference(*layer, k=E, F=F, fmt="bf16")
    assert mask.all()
    assert np.max(np.abs(out - ref)) <= 1e-12 * np.max(np.abs(ref))


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4", "mxfp8"])
def test_block_power_of_two_scaling_is_exact(fmt):
    """W2, b2 scaled by 2 (bf16: exponent field + 1; mxfp4/mxfp8: every W2 scale byte + 1,
    b2 x 2) scales out by exactly 2."""
    T, D, E, k, F = 16, 64, 4, 2, 64
    x, wr, br, w1, b1, w2, b2 = tiny_layer(9, T, D, E, k, F, fmt)
    out = moe_forward(x, wr, br, w1, b1, w2, b2, k=k, F=F, fmt=fmt)
    b2s = np.where((b2 & 0x7FFF) != 0, b2 + np.uint16(1 << 7), b2).astype(np.uint16)
    if fmt == "bf16":
        w2s = np.where((w2 & 0x7FFF) != 0, w2 + np.uint16(1 << 7), w2).astype(np.uint16)
    else:
        w2s = w2.copy()
        n = E * D * (F // 2 if fmt == "mxfp4" else F)
        w2s[n:] += 1
    out2 = moe_forward(x, wr, br, w1, b1, w2s, b2s, k=k, F=F, fmt=fmt)
    assert np.array_equal(out2, 2 * out)


def test_block_expert_relabelling_invariance():
    T, D, E, k, F = 20, 32, 6, 2, 32
    x, wr, br, w1, b1, w2, b2 = tiny_layer(10, T, D, E, k, F, "bf16")
    out = moe_forward(x, wr, br, w1, b1, w2, b2, k=k, F=F, fmt="bf16")
    p = np.random.default_rng(0).permutation(E)
    l = router_logits(x, wr, br)
    srt = np.sort(l, axis=1)
    assert np.all(np.diff(srt, axis=1) != 0)      # no ties, so the relabelled routing is unique
    out_p = moe_forward(x, wr[p], br[p], w1[p], b1[p], w2[p], b2[p], k=k, F=F, fmt="bf16")
    assert np.max(np.abs(out - out_p)) <= 1e-13 * np.max(np.abs(out))


def test_block_matches_triple_loop_on_tiny_workload():
    """The C1-shaped workload (T=64, D=64, E=4, k=2, F=128) through per-token, per-expert
    Python loops for the two expert matmuls (library matmul replaced by explicit sums)."""
    from synth import make_inputs
    inp = make_inputs("C1")
    out, r = moe_forward(inp.x, inp.wr, inp.br, inp.w1, inp.b1, inp.w2, inp.b2, k=2, F=128, fmt="bf16",
                         return_routing=True)
    E, D, F = 4, 64, 128
    X = bf16_to_f64(inp.x)
    W1 = bf16_to_f64(inp.w1).reshape(E, 2 * F, D)
    W2 = bf16_to_f64(inp.w2).reshape(E, D, F)
    B1 = bf16_to_f64(inp.b1).reshape(E, 2 * F)
    B2 = bf16_to_f64(inp.b2).reshape(E, D)
    for t in (0, 17, 63):
        acc = np.zeros(D)
        for j in range(2):
            e = int(r["idx"][t, j])
            u = np.array([math.fsum(W1[e, i, d] * X[t, d] for d in range(D)) for i in range(2 * F)]) + B1[e]
            gc = np.minimum(u[:F], 7)
            hv = gc * sigmoid_tanh(1.702 * gc) * (np.clip(u[F:], -7, 7) + 1)
            y = np.array([math.fsum(W2[e, o, f] * hv[f] for f in range(F)) for o in range(D)]) + B2[e]
            acc += r["gates"][t, j] * y
        assert np.max(np.abs(out[t] - acc)) <= 1e-12 * max(1.0, np.max(np.abs(acc)))
