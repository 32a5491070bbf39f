"""Float64 reference of the GPT-OSS MoE feed-forward block -- test infrastructure only.

Pages this follows (cited by title and section):

* torchtitan GPT-OSS model guide (discosf.com mirror), section "Grouped matrix
  multiplication: the core of efficient MoE compute": per-expert token counts,
  int32 cumulative offsets, the two grouped GEMMs mlp1/mlp2 over expert weights
  stored (experts, out, in), and the GPT-OSS SwiGLU variant (gate clamped from
  above then multiplied by sigmoid(alpha*gate); linear clamped to [-limit, limit]
  plus one).
* same guide, section "StateDict adapter": the router is a Linear with a bias;
  mlp1 is the fused gate/up projection.
* "gptoss" pure-Python re-implementation page (kexuegongju.com), sections
  "basic parameters" (32 experts, top-4) and "model run flow" (routing top-4,
  expert compute, weighted combination).
* GPT-OSS in Transformers blog (qian.cx), MXFP4 paragraph: E2M1 values (1 sign,
  2 exponent, 1 mantissa bit) with one scale per 32-element block.
* torchtitan guide, section "StateDict adapter": the load-balancing expert bias
  (one value per expert, zero when a checkpoint is loaded).
* torchtitan guide, grouped GEMM section: the grouped product is an overridable seam
  through which MXFP8 converters inject a scaled grouped GEMM (MXFP8 expert weights:
  E4M3 elements with one E8M0 scale per 32, as in the OCP Microscaling spec v1.0).

Readings where the pages are silent (each listed with its reason in the design
notes): softmax over the k selected logits; slots ordered by descending logit
with ties to the lower expert index; logits are the exact dot product plus bias
rounded once to fp32; SwiGLU alpha = 1.702 and limit = 7.0; mlp1's output is
[gate half | linear half]; the gate weight scales mlp2's output including its
bias; E2M1 exponent bias 1 with the even element in the low nibble and E8M0
scale 2**(s-127); within an expert, assignments keep ascending order; the
load-balancing expert bias, when given, is added (fp32) to the logits for the
selection only, and the gates use the unbiased logits.

No intermediate is rounded: h, y and out are exact up to float64 rounding.
"""
from __future__ import annotations

import numpy as np

SWIGLU_ALPHA = 1.702
SWIGLU_LIMIT = 7.0

# E2M1 magnitudes for code bits (e1 e0 m): OCP Microscaling v1.0 FP4 table, bias 1.
_E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64, exactly (the bits are the top half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def e2m1_value(code) -> np.ndarray:
    """Value of a 4-bit E2M1 code: bit 3 is the sign, bits 2..0 index the magnitude table."""
    c = np.asarray(code, dtype=np.int64)
    mag = _E2M1_MAG[c & 7]
    return np.where(c & 8, -mag, mag)


def mxfp4_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 block -> float64 (Transformers blog, MXFP4 paragraph).

    codes  uint8 [rows, K/2]: element 2i in the low nibble of byte i, 2i+1 in the high nibble.
    scales uint8 [rows, K/32]: E8M0, the block of 32 consecutive K elements is multiplied
    by 2**(s - 127); s = 255 encodes NaN.
    """
    codes = np.asarray(codes, dtype=np.uint8)
    rows, half = codes.shape
    # value pair of every byte: (low-nibble element, high-nibble element)
    b = np.arange(256)
    pair = np.stack([e2m1_value(b & 15), e2m1_value(b >> 4)], axis=1)
    q = pair[codes].reshape(rows, (2 * half) // 32, 32)
    s = np.asarray(scales, dtype=np.int64)
    factor = np.where(s == 255, np.nan, np.ldexp(1.0, s - 127))
    return (q * factor[:, :, None]).reshape(rows, 2 * half)


def e4m3_value(code) -> np.ndarray:
    """Value of an 8-bit E4M3 code (OCP Microscaling v1.0 FP8 E4M3: bit 7 sign, 4 exponent
    bits with bias 7, 3 mantissa bits; exponent 0 is subnormal, (m / 8) 2^-6; exponent 15
    with mantissa 7 is NaN and there is no infinity)."""
    c = np.asarray(code, dtype=np.int64)
    ex = (c >> 3) & 15
    m = (c & 7).astype(np.float64)
    mag = np.where(ex == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(ex - 7.0))
    mag = np.where((ex == 15) & ((c & 7) == 7), np.nan, mag)
    return np.where(c & 128, -mag, mag)


def mxfp8_decode(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP8 block -> float64: codes uint8 [rows, K] (E4M3, one per element), scales uint8
    [rows, K/32] (E8M0: 2**(s - 127), 255 = NaN) over 32 consecutive K elements each."""
    codes = np.asarray(codes, dtype=np.uint8)
    rows, K = codes.shape
    q = e4m3_value(codes).reshape(rows, K // 32, 32)
    s = np.asarray(scales, dtype=np.int64)
    factor = np.where(s == 255, np.nan, np.ldexp(1.0, s - 127))
    return (q * factor[:, :, None]).reshape(rows, K)


def expert_weight(w: np.ndarray, fmt: str, E: int, rows: int, K: int, e: int) -> np.ndarray:
    """Expert e's weight [rows, K] in float64 from the stored tensor.

    bf16: ``w`` is uint16 [E, rows, K].  mxfp4: ``w`` is one uint8 buffer holding the codes
    [E][rows][K/2] followed by the scales [E][rows][K/32].  mxfp8: one uint8 buffer holding
    the codes [E][rows][K] followed by the scales [E][rows][K/32].
    """
    if fmt == "bf16":
        return bf16_to_f64(np.asarray(w).reshape(E, rows, K)[e])
    if fmt == "mxfp8":
        flat = np.asarray(w, dtype=np.uint8).reshape(-1)
        ncode = rows * K
        nscale = rows * (K // 32)
        if flat.size != E * (ncode + nscale):
            raise ValueError("mxfp8 buffer has the wrong size")
        codes = flat[e * ncode:(e + 1) * ncode].reshape(rows, K)
        base = E * ncode
        scales = flat[base + e * nscale: base + (e + 1) * nscale].reshape(rows, K // 32)
        return mxfp8_decode(codes, scales)
    if fmt == "mxfp4":
        flat = np.asarray(w, dtype=np.uint8).reshape(-1)
        ncode = rows * (K // 2)
        nscale = rows * (K // 32)
        if flat.size != E * (ncode + nscale):
            raise ValueError("mxfp4 buffer has the wrong size")
        codes = flat[e * ncode:(e + 1) * ncode].reshape(rows, K // 2)
        base = E * ncode
        scales = flat[base + e * nscale: base + (e + 1) * nscale].reshape(rows, K // 32)
        return mxfp4_decode(codes, scales)
    raise ValueError(fmt)


def router_logits(x: np.ndarray, wr: np.ndarray, br: np.ndarray) -> np.ndarray:
    """Router Linear with bias (torchtitan guide, StateDict adapter: router.gate weight/bias).

    l[t,e] = sum_d x[t,d] * Wr[e,d] + br[e], summed in float64 and rounded once to fp32.
    All inputs are bf16 bits.
    """
    l64 = bf16_to_f64(x) @ bf16_to_f64(wr).T + bf16_to_f64(br)[None, :]
    return l64.astype(np.float32)


def select_experts(logits: np.ndarray, k: int, expert_bias: np.ndarray | None = None) -> np.ndarray:
    """Top-k routing ("gptoss" page, basic parameters: top-4 of 32 experts).

    Slot j of token t holds the expert with the j-th largest fp32 logit; equal logits go to
    the lower expert index first.  With a load-balancing expert bias (torchtitan guide,
    "StateDict adapter": ``expert_bias_E``, one value per expert) the selection key is
    the fp32 sum logit + bias (one rounding, nearest even) instead.  Returns int32 [T, k].
    """
    key = np.asarray(logits, dtype=np.float32)
    if expert_bias is not None:
        key = key + np.asarray(expert_bias, dtype=np.float32)[None, :]
    order = np.argsort(-key.astype(np.float64), axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def gate_weights(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Softmax over the k selected fp32 logits of each token, in float64 ("gptoss" page lists
    Softmax among the block's functions; the weighted combination uses these weights)."""
    sel = np.take_along_axis(logits.astype(np.float64), idx.astype(np.int64), axis=1)
    # shifted by the largest selected logit (softmax is shift-invariant); with a selection
    # bias the first slot need not hold it
    z = np.exp(sel - sel.max(axis=1, keepdims=True))
    return z / z.sum(axis=1, keepdims=True)


def update_expert_bias(expert_bias: np.ndarray, counts: np.ndarray, coeff: float) -> np.ndarray:
    """One load-balancing step of the expert bias (torchtitan guide, "StateDict adapter": a
    hook registered after the optimizer with load_balance_coeff = 1e-3; the rule is the
    auxiliary-loss-free balancing of the DeepSeek-V3 report): an expert that received more
    assignments than the mean lowers its bias by coeff, one that received fewer raises it
    by coeff, one exactly at the mean keeps it.  fp32 in and out; the step is one fp32
    rounding of bias + coeff.  Returns the new bias (the input is not modified)."""
    b = np.asarray(expert_bias, dtype=np.float32)
    c = np.asarray(counts, dtype=np.int64)
    mean = c.sum() / c.size                    # exact sign below: |mean - c| >= 1/E when nonzero
    step = np.sign(mean - c) * float(np.float32(coeff))
    new = (b.astype(np.float64) + step).astype(np.float32)
    return np.where(step == 0, b, new)


def route_assignments(idx: np.ndarray, E: int):
    """Per-expert counts, int32 offsets and the token permutation (torchtitan guide, grouped GEMM:
    num_tokens_per_expert and its int32 cumulative sum delimit each expert's rows).

    Assignment a = t*k + j.  counts[e] = #{a : idx[a] = e}; offsets[0] = 0 and
    offsets[e+1] = offsets[e] + counts[e]; perm lists the assignments grouped by expert,
    ascending a inside a group (stable counting sort); rowpos is its inverse.
    """
    flat = idx.reshape(-1).astype(np.int64)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts, dtype=np.int64).astype(np.int32)
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    rowpos = np.empty_like(perm)
    rowpos[perm] = np.arange(perm.size, dtype=np.int32)
    return counts, offsets, perm, rowpos


def swiglu(u: np.ndarray, F: int, alpha: float = SWIGLU_ALPHA, limit: float = SWIGLU_LIMIT) -> np.ndarray:
    """GPT-OSS SwiGLU variant (torchtitan guide, grouped GEMM section).

    u [..., 2F] is mlp1's output: gate = u[..., :F], linear = u[..., F:].
    The gate is clamped from above at ``limit`` and then multiplied by sigmoid(alpha * gate);
    the linear half is clamped to [-limit, limit] and shifted by +1.
    """
    gate = np.minimum(u[..., :F], limit)
    lin = np.clip(u[..., F:], -limit, limit)
    return gate * (1.0 / (1.0 + np.exp(-alpha * gate))) * (lin + 1.0)


def expert_forward(xr: np.ndarray, w1e: np.ndarray, b1e: np.ndarray,
                   w2e: np.ndarray, b2e: np.ndarray, F: int) -> np.ndarray:
    """One expert on float64 rows: mlp1 (weight [2F, D] as (out, in)) + bias, SwiGLU,
    mlp2 (weight [D, F]) + bias (torchtitan guide, grouped GEMM section)."""
    u = xr @ w1e.T + b1e[None, :]
    h = swiglu(u, F)
    return h @ w2e.T + b2e[None, :]


def moe_forward(x, wr, br, w1, b1, w2, b2, k: int, F: int, fmt: str, return_routing: bool = False,
                expert_bias: np.ndarray | None = None):
    """The whole block ("gptoss" page, model run flow: route top-k, expert compute,
    weighted combination), in float64 with fp32 logits.

    Shapes (storage bits): x [T,D] u16, wr [E,D] u16, br [E] u16, b1 [E,2F] u16, b2 [E,D] u16;
    w1/w2 as in ``expert_weight`` with (rows, K) = (2F, D) and (D, F).
    ``expert_bias`` (fp32 [E] or None) biases the selection only (``select_experts``).
    Returns out [T,D] float64 (and the routing when ``return_routing``).
    Experts are visited one at a time so the largest layer never holds more than one
    expert's float64 weights.
    """
    x = np.asarray(x)
    T, D = x.shape
    E = np.asarray(wr).shape[0]
    logits = router_logits(x, wr, br)
    idx = select_experts(logits, k, expert_bias)
    g = gate_weights(logits, idx)
    counts, offsets, perm, rowpos = route_assignments(idx, E)
    x64 = bf16_to_f64(x)
    b1_64 = bf16_to_f64(np.asarray(b1).reshape(E, 2 * F))
    b2_64 = bf16_to_f64(np.asarray(b2).reshape(E, D))
    g_flat = g.reshape(-1)
    y = np.zeros((T * k, D), dtype=np.float64)
    for e in range(E):
        a = perm[offsets[e]:offsets[e + 1]].astype(np.int64)
        if a.size == 0:
            continue
        w1e = expert_weight(w1, fmt, E, 2 * F, D, e)
        w2e = expert_weight(w2, fmt, E, D, F, e)
        ye = expert_forward(x64[a // k], w1e, b1_64[e], w2e, b2_64[e], F)
        y[a] = g_flat[a][:, None] * ye
    out = y.reshape(T, k, D).sum(axis=1)
    if not return_routing:
        return out
    return out, {"logits": logits, "idx": idx, "gates": g, "counts": counts,
                 "offsets": offsets, "perm": perm, "rowpos": rowpos}
