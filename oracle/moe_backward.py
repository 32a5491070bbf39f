"""Float64 gradients of the GPT-OSS MoE feed-forward block -- test infrastructure only.

The backward of the forward in ``moe_oracle`` (torchtitan GPT-OSS guide, grouped GEMM
section: the block is trained, and its SwiGLU variant's formula and gradient are unit
tested against a reference), with the top-k selection held fixed: the selection is
piecewise constant in the inputs, so gradients flow through the gate softmax, the two
expert matrices and the router, never through the choice of experts (and so never to the
load-balancing bias, which only moves the choice).

Readings (listed with their reasons in the design notes): the clamps pass the gradient
where the input lies inside the closed interval (gate <= limit; -limit <= lin <= limit),
as a clamp's derivative is usually taken; the logits are treated as exact reals (the
forward's fp32 rounding of the logits is a rounding, not part of the function); expert
weights are differentiated as the float64 values they decode to.

Parity unpinned against the pages (they print no gradient values); pinned in tests by
finite differences and by an independent autograd formulation.
"""
from __future__ import annotations

import numpy as np

from .moe_oracle import SWIGLU_ALPHA, SWIGLU_LIMIT


def _sigmoid(z):
    return 1.0 / (1.0 + np.exp(-z))


def forward_fixed_routing(x, wr, br, w1, b1, w2, b2, idx, F: int):
    """The block in float64 on decoded arrays with a given selection idx [T, k]:
    x [T,D], wr [E,D], br [E], w1 [E,2F,D], b1 [E,2F], w2 [E,D,F], b2 [E,D].
    Logits are not rounded.  Returns out [T, D]."""
    T, k = idx.shape
    logits = x @ wr.T + br[None, :]
    sel = np.take_along_axis(logits, idx, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    g = z / z.sum(axis=1, keepdims=True)
    out = np.zeros((T, x.shape[1]))
    for j in range(k):
        for t in range(T):
            e = idx[t, j]
            u = w1[e] @ x[t] + b1[e]
            gate = np.minimum(u[:F], SWIGLU_LIMIT)
            lin = np.clip(u[F:], -SWIGLU_LIMIT, SWIGLU_LIMIT)
            h = gate * _sigmoid(SWIGLU_ALPHA * gate) * (lin + 1.0)
            out[t] += g[t, j] * (w2[e] @ h + b2[e])
    return out


def swiglu_backward(u: np.ndarray, dh: np.ndarray, F: int,
                    alpha: float = SWIGLU_ALPHA, limit: float = SWIGLU_LIMIT) -> np.ndarray:
    """du [..., 2F] from dh [..., F] for h = min(gate, limit) sigma(alpha min(gate, limit))
    (clip(lin, -limit, limit) + 1) with gate = u[..., :F], lin = u[..., F:]."""
    gate, lin = u[..., :F], u[..., F:]
    gc = np.minimum(gate, limit)
    lc = np.clip(lin, -limit, limit)
    s = _sigmoid(alpha * gc)
    d_gc = s + alpha * gc * s * (1.0 - s)                 # d/dgc of gc sigma(alpha gc)
    du_gate = dh * d_gc * (lc + 1.0) * (gate <= limit)
    du_lin = dh * gc * s * ((lin >= -limit) & (lin <= limit))
    return np.concatenate([du_gate, du_lin], axis=-1)


def moe_backward(x, wr, br, w1, b1, w2, b2, idx, dout, F: int) -> dict:
    """Gradients of sum(out * dout) for the block with the selection idx held fixed.

    Arrays as in ``forward_fixed_routing``; dout [T, D].  Returns float64 dx, dwr, dbr, dw1,
    db1, dw2, db2 (each the shape of its input).

    Per assignment a = (t, j) with expert e and gate g: z = h W2[e]^T + b2[e],
    dz = g dout[t] gives dW2[e] += dz^T h, db2[e] += dz, dh = dz W2[e]; the SwiGLU backward
    gives du, then dW1[e] += du^T x[t], db1[e] += du, dx[t] += du W1[e]; dg = <dout[t], z>.
    The gates are a softmax over the selected logits: dl = g (dg - sum_j g_j dg_j) on the
    selected experts, zero elsewhere; then dWr += dl^T x, dbr += dl, dx += dl Wr.
    """
    T, k = idx.shape
    E, D = wr.shape
    logits = x @ wr.T + br[None, :]
    sel = np.take_along_axis(logits, idx, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    g = z / z.sum(axis=1, keepdims=True)
    dx = np.zeros_like(x)
    dw1, db1 = np.zeros_like(w1), np.zeros_like(b1)
    dw2, db2 = np.zeros_like(w2), np.zeros_like(b2)
    dg = np.zeros((T, k))
    for t in range(T):
        for j in range(k):
            e = idx[t, j]
            u = w1[e] @ x[t] + b1[e]
            gate = np.minimum(u[:F], SWIGLU_LIMIT)
            lin = np.clip(u[F:], -SWIGLU_LIMIT, SWIGLU_LIMIT)
            h = gate * _sigmoid(SWIGLU_ALPHA * gate) * (lin + 1.0)
            zt = w2[e] @ h + b2[e]
            dg[t, j] = dout[t] @ zt
            dz = g[t, j] * dout[t]
            dw2[e] += np.outer(dz, h)
            db2[e] += dz
            du = swiglu_backward(u, dz @ w2[e], F)
            dw1[e] += np.outer(du, x[t])
            db1[e] += du
            dx[t] += du @ w1[e]
    dsel = g * (dg - (g * dg).sum(axis=1, keepdims=True))
    dl = np.zeros((T, E))
    np.put_along_axis(dl, idx, dsel, axis=1)
    dwr = dl.T @ x
    dbr = dl.sum(axis=0)
    dx += dl @ wr
    return dict(dx=dx, dwr=dwr, dbr=dbr, dw1=dw1, db1=db1, dw2=dw2, db2=db2)


def moe_backward_grouped(x, wr, br, w1, b1, w2, b2, idx, dout, k: int, F: int, fmt: str,
                         weight_experts=None) -> dict:
    """The gradients of ``moe_backward`` from the stored bits (as ``moe_forward`` takes them:
    x [T,D], wr [E,D], br [E], b1, b2 as bf16 bits; w1/w2 in ``fmt``), computed one expert
    at a time over the tokens routed to it (torchtitan guide, grouped GEMM section: each
    expert's rows form one group), so layers of the 20B shape fit in host memory.

    Same readings as ``moe_backward`` (selection idx [T, k] fixed, clamps pass the gradient
    on the closed interval, logits exact reals).  dx, dwr, dbr are returned whole; dw1, db1,
    dw2, db2 only for the experts in ``weight_experts`` (all when None), as dicts
    {e: array}.  Per expert e with routed rows R (tokens t_r, slots j_r, gates g_r):
    U = X_R W1[e]^T + b1[e], H = swiglu(U), Z = H W2[e]^T + b2[e]; dg_r = <dout[t_r], Z_r>;
    dZ = g dout[t_R]; dW2 = dZ^T H, db2 = sum dZ; dU = swiglu_backward(U, dZ W2[e]);
    dW1 = dU^T X_R, db1 = sum dU, dx[t_r] += dU_r W1[e]; then the softmax backward over
    the selected logits and the router's products, as in ``moe_backward``.
    """
    from .moe_oracle import bf16_to_f64, expert_weight, swiglu

    x64 = bf16_to_f64(np.asarray(x))
    T, D = x64.shape
    wr64 = bf16_to_f64(np.asarray(wr))
    E = wr64.shape[0]
    br64 = bf16_to_f64(np.asarray(br))
    b1_64 = bf16_to_f64(np.asarray(b1)).reshape(E, 2 * F)
    b2_64 = bf16_to_f64(np.asarray(b2)).reshape(E, D)
    idx = np.asarray(idx, dtype=np.int64)
    dout = np.asarray(dout, dtype=np.float64)
    logits = x64 @ wr64.T + br64[None, :]
    sel = np.take_along_axis(logits, idx, axis=1)
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    g = z / z.sum(axis=1, keepdims=True)
    want = set(range(E)) if weight_experts is None else set(int(e) for e in weight_experts)
    dx = np.zeros_like(x64)
    dg = np.zeros((T, k))
    dw1, db1, dw2, db2 = {}, {}, {}, {}
    flat = idx.reshape(-1)
    for e in range(E):
        a = np.flatnonzero(flat == e)                     # assignments t*k + j routed to e
        if e in want:
            dw1[e] = np.zeros((2 * F, D))
            db1[e] = np.zeros(2 * F)
            dw2[e] = np.zeros((D, F))
            db2[e] = np.zeros(D)
        if a.size == 0:
            continue
        t, j = a // k, a % k
        w1e = expert_weight(w1, fmt, E, 2 * F, D, e)
        w2e = expert_weight(w2, fmt, E, D, F, e)
        xr = x64[t]
        U = xr @ w1e.T + b1_64[e][None, :]
        H = swiglu(U, F)
        Z = H @ w2e.T + b2_64[e][None, :]
        dg[t, j] = np.einsum("rd,rd->r", dout[t], Z)
        dZ = g[t, j][:, None] * dout[t]
        dU = swiglu_backward(U, dZ @ w2e, F)
        np.add.at(dx, t, dU @ w1e)
        if e in want:
            dw2[e] = dZ.T @ H
            db2[e] = dZ.sum(axis=0)
            dw1[e] = dU.T @ xr
            db1[e] = dU.sum(axis=0)
    dsel = g * (dg - (g * dg).sum(axis=1, keepdims=True))
    dl = np.zeros((T, E))
    np.put_along_axis(dl, idx, dsel, axis=1)
    dwr = dl.T @ x64
    dbr = dl.sum(axis=0)
    dx += dl @ wr64
    return dict(dx=dx, dwr=dwr, dbr=dbr, dw1=dw1, db1=db1, dw2=dw2, db2=db2)
