"""Pins of the oracle's backward (CPU): finite differences, an independent autograd
formulation of the same block, and exact properties."""
import numpy as np
import pytest
import torch

from oracle import (SWIGLU_ALPHA, SWIGLU_LIMIT, forward_fixed_routing, moe_backward, select_experts,
                    swiglu_backward)


def layer(seed, T, D, E, F, wscale=0.4):
    g = np.random.default_rng(seed)
    x = g.standard_normal((T, D))
    wr = g.standard_normal((E, D)) * 0.3
    br = g.standard_normal(E) * 0.5
    w1 = g.standard_normal((E, 2 * F, D)) * wscale
    b1 = g.standard_normal((E, 2 * F)) * 0.2
    w2 = g.standard_normal((E, D, F)) * 0.2
    b2 = g.standard_normal((E, D)) * 0.2
    return x, wr, br, w1, b1, w2, b2


def routing(x, wr, br, k):
    return select_experts((x @ wr.T + br[None, :]).astype(np.float32), k).astype(np.int64)


NAMES = ["x", "wr", "br", "w1", "b1", "w2", "b2"]


@pytest.mark.parametrize("T,D,E,k,F", [(5, 16, 4, 2, 16), (4, 8, 3, 3, 8), (3, 8, 1, 1, 8)])
def test_backward_matches_central_differences(T, D, E, k, F):
    """Every gradient entry of a tiny layer against a central difference of the fixed-routing
    forward (step 1e-6, float64).  The weights are large enough that some SwiGLU inputs lie
    past the clamps, where the gradient must vanish."""
    p = list(layer(T * 31 + E + 1, T, D, E, F, wscale=4.8 / np.sqrt(D)))
    idx = routing(p[0], p[1], p[2], k)
    dout = np.random.default_rng(9).standard_normal((T, D))
    u = np.einsum("egd,td->teg", p[3], p[0]) + p[4][None]
    assert (u[..., :F] > SWIGLU_LIMIT).any() and (np.abs(u[..., F:]) > SWIGLU_LIMIT).any()
    grads = moe_backward(*p, idx, dout, F)
    f = lambda q: float(np.sum(forward_fixed_routing(*q, idx, F) * dout))
    eps = 1e-6
    for i, name in enumerate(NAMES):
        a = p[i]
        num = np.zeros_like(a)
        for pos in np.ndindex(a.shape):
            old = a[pos]
            a[pos] = old + eps
            fp = f(p)
            a[pos] = old - eps
            fm = f(p)
            a[pos] = old
            num[pos] = (fp - fm) / (2 * eps)
        got = grads["d" + name]
        assert got.shape == a.shape
        scale = max(1.0, np.abs(num).max())
        assert np.max(np.abs(got - num)) <= 2e-6 * scale, name


def torch_reference(p, idx, dout, F):
    """The block written again with torch float64 ops over all experts and a selection mask,
    differentiated by autograd."""
    t = [torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in p]
    x, wr, br, w1, b1, w2, b2 = t
    T, E = x.shape[0], wr.shape[0]
    mask = torch.zeros((T, E), dtype=torch.bool)
    mask[torch.arange(T)[:, None], torch.tensor(idx)] = True
    logits = x @ wr.T + br
    gsm = torch.softmax(torch.where(mask, logits, torch.full_like(logits, -torch.inf)), dim=1)
    u = torch.einsum("td,egd->teg", x, w1) + b1[None]
    gate = torch.clamp(u[..., :F], max=SWIGLU_LIMIT)
    lin = torch.clamp(u[..., F:], min=-SWIGLU_LIMIT, max=SWIGLU_LIMIT)
    h = gate * torch.sigmoid(SWIGLU_ALPHA * gate) * (lin + 1.0)
    y = torch.einsum("tef,edf->ted", h, w2) + b2[None]
    out = torch.einsum("te,ted->td", gsm, y)
    (out * torch.tensor(dout)).sum().backward()
    return {"d" + n: v.grad.numpy() for n, v in zip(NAMES, t)}


@pytest.mark.parametrize("T,D,E,k,F,seed", [(12, 32, 6, 2, 32, 0), (9, 16, 4, 4, 24, 1), (7, 32, 8, 3, 16, 2)])
def test_backward_matches_autograd_of_dense_formulation(T, D, E, k, F, seed):
    p = layer(seed, T, D, E, F, wscale=1.0)
    idx = routing(p[0], p[1], p[2], k)
    dout = np.random.default_rng(seed + 50).standard_normal((T, D))
    got = moe_backward(*p, idx, dout, F)
    ref = torch_reference(p, idx, dout, F)
    for n in got:
        assert np.allclose(got[n], ref[n], rtol=1e-11, atol=1e-11 * max(1.0, np.abs(ref[n]).max())), n


def test_backward_exact_properties():
    """Doubling dout doubles every gradient exactly; one expert per token with k = 1 gives the
    router no gradient (a softmax over one logit is constant); the router-bias gradient of
    each token sums to zero over its selected experts, so dbr sums to zero; the SwiGLU
    backward is zero past the clamps."""
    T, D, E, k, F = 6, 16, 4, 2, 16
    p = layer(3, T, D, E, F)
    idx = routing(p[0], p[1], p[2], k)
    dout = np.random.default_rng(4).standard_normal((T, D))
    a = moe_backward(*p, idx, dout, F)
    b = moe_backward(*p, idx, 2 * dout, F)
    for n in a:
        assert np.array_equal(b[n], 2 * a[n]), n
    assert abs(a["dbr"].sum()) <= 1e-12 * np.abs(a["dbr"]).max()
    idx1 = routing(p[0], p[1], p[2], 1)
    c = moe_backward(*p, idx1, dout, F)
    assert not c["dwr"].any() and not c["dbr"].any()
    u = np.array([[8.0, -9.0, 0.5, 3.0]])                 # F = 2: gate (8, -9), lin (0.5, 3)
    du = swiglu_backward(u, np.ones((1, 2)), 2)
    assert du[0, 0] == 0.0                                # gate past the limit
    u2 = np.array([[0.5, 1.0, 9.0, -7.5]])
    du2 = swiglu_backward(u2, np.ones((1, 2)), 2)
    assert du2[0, 2] == 0.0 and du2[0, 3] == 0.0          # both linear inputs past +-limit


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4"])
@pytest.mark.parametrize("T,D,E,k,F,seed", [(10, 32, 5, 2, 32, 0), (8, 64, 5, 4, 32, 1), (12, 32, 6, 3, 64, 2)])
def test_grouped_backward_equals_loop_backward(fmt, T, D, E, k, F, seed):
    """The per-expert batched form from stored bits == the per-assignment loop on the decoded
    arrays (1e-12 relative), including a subset of experts for the weight gradients and an
    expert that receives no token (its weight gradients are zero)."""
    from synth import f32_to_bf16_bits
    from oracle import bf16_to_f64, expert_weight, moe_backward_grouped, router_logits
    g = np.random.default_rng(100 + seed)
    bf = lambda *s, std=1.0: f32_to_bf16_bits(g.standard_normal(s).astype(np.float32) * np.float32(std))
    x = bf(T, D)
    wr = bf(E, D, std=0.3)
    br = bf(E, std=0.5)
    br[E - 1] = f32_to_bf16_bits(np.array([-64.0], dtype=np.float32))[0]     # expert E-1 gets no token
    if fmt == "bf16":
        w1, w2 = bf(E, 2 * F, D, std=4.0 / np.sqrt(D)), bf(E, D, F, std=0.3)
    else:
        def mx(rows, K):
            return np.concatenate([g.integers(0, 256, E * rows * K // 2, dtype=np.uint8),
                                   g.integers(123, 128, E * rows * K // 32, dtype=np.uint8)])
        w1, w2 = mx(2 * F, D), mx(D, F)
    b1, b2 = bf(E, 2 * F, std=0.2), bf(E, D, std=0.2)
    idx = select_experts(router_logits(x, wr, br), k).astype(np.int64)
    assert not (idx == E - 1).any()
    dout = g.standard_normal((T, D))
    dec = [bf16_to_f64(x), bf16_to_f64(wr), bf16_to_f64(br),
           np.stack([expert_weight(w1, fmt, E, 2 * F, D, e) for e in range(E)]), bf16_to_f64(b1).reshape(E, 2 * F),
           np.stack([expert_weight(w2, fmt, E, D, F, e) for e in range(E)]), bf16_to_f64(b2).reshape(E, D)]
    ref = moe_backward(*dec, idx, dout, F)
    sub = [0, E - 1, E // 2]
    got = moe_backward_grouped(x, wr, br, w1, b1, w2, b2, idx, dout, k, F, fmt, weight_experts=sub)
    close = lambda a, b: np.max(np.abs(a - b)) <= 1e-12 * max(1.0, np.abs(b).max())
    for n in ("dx", "dwr", "dbr"):
        assert close(got[n], ref[n]), n
    for n in ("dw1", "db1", "dw2", "db2"):
        assert sorted(got[n]) == sorted(set(sub)), n
        for e in got[n]:
            assert close(got[n][e], ref[n][e]), (n, e)
    assert not got["dw1"][E - 1].any() and not got["db2"][E - 1].any()
