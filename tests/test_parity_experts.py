"""GPU expert stage (mlp1 + SwiGLU, mlp2 + bias + gate, combine) on the oracle's routing.

Isolating the grouped GEMMs from the router follows the stage-by-stage verification of
the "gptoss" re-implementation page (section on testing: each layer is fed the reference
output of the previous one)."""
import numpy as np
import pytest
import torch

import mixture_experts_transformer_amd as moe
import oracle
from synth import f32_to_bf16_bits, get_config, make_inputs
from _gpu import assert_close, note, upload

pytestmark = pytest.mark.gpu


def experts_vs_oracle(inp, label, weight_offset=0):
    cfg = inp.cfg
    note(f"experts {label}: T={cfg.T} D={cfg.D} E={cfg.E} k={cfg.k} F={cfg.F} fmt={cfg.fmt}")
    ref, r = oracle.moe_forward(inp.x, inp.wr, inp.br, inp.w1, inp.b1, inp.w2, inp.b2,
                                k=cfg.k, F=cfg.F, fmt=cfg.fmt, return_routing=True)
    d = upload(inp, weight_offset)
    gates = torch.from_numpy(r["gates"].astype(np.float32)).cuda()
    offsets = torch.from_numpy(r["offsets"]).cuda()
    perm = torch.from_numpy(r["perm"]).cuda()
    out = moe.experts(d["x"], d["w1"], d["b1"], d["w2"], d["b2"], gates, offsets, perm, cfg.k, cfg.fmt)
    torch.cuda.synchronize()
    assert_close(out.cpu().numpy(), ref, label)
    return r


@pytest.mark.parametrize("name", ["C1", "C2", "X1", "Y1"])
def test_experts_workloads(name):
    experts_vs_oracle(make_inputs(name), name)


BASE = {"bf16": "C2", "mxfp4": "C4", "mxfp8": "Y1"}   # workload whose weight recipe a case takes


# shapes chosen to cover both tile configurations (streaming 64x128 when T*k < 128*E, else
# 256x256), row tails inside a tile, column tails of mlp1 (F not a multiple of the tile's
# pair count: 64 or 128) and of mlp2 (D not a multiple of the tile width: 128 or 256),
# single-K-step and multi-step reductions, and the degenerate layers
@pytest.mark.parametrize("fmt", ["bf16", "mxfp4", "mxfp8"])
@pytest.mark.parametrize("T,D,E,k,F", [
    (37, 128, 5, 2, 192),       # streaming tiles, ragged groups, mlp1 pair tail (192 = 128 + 64)
    (300, 64, 3, 3, 64),        # k = E, one K step
    (1000, 192, 4, 2, 320),     # large tiles: mlp1 pair tail (320 = 2*128 + 64)
    (700, 320, 2, 1, 128),      # large tiles: mlp2 column tail (320 = 256 + 64), k = 1
    (2500, 384, 8, 4, 448),     # large tiles, many row tiles per expert
    (1, 64, 4, 2, 64),          # a single token
    (513, 320, 1, 1, 192),      # E = k = 1 (a dense SwiGLU MLP): row tail 513 = 2*256 + 1
    (200, 128, 256, 8, 128),    # 256 experts, most of them empty
])
def test_experts_ragged_shapes(fmt, T, D, E, k, F):
    base = BASE[fmt]
    cfg = get_config(base, name=f"rag{T}", T=T, D=D, E=E, k=k, F=F, seed=1000 + T)
    experts_vs_oracle(make_inputs(cfg), f"ragged {fmt} T={T} D={D} E={E} k={k} F={F}")


@pytest.mark.parametrize("fmt", ["bf16", "mxfp4", "mxfp8"])
def test_experts_with_empty_experts(fmt):
    base = BASE[fmt]
    cfg = get_config(base, name="empty", T=600, D=128, E=16, k=2, F=128, seed=77)
    inp = make_inputs(cfg)
    neg = f32_to_bf16_bits(np.float32([-64.0]))[0]
    br = inp.br.copy()
    br[[0, 1, 7, 15]] = neg
    inp2 = make_inputs(cfg, router_bias=br)
    r = experts_vs_oracle(inp2, f"empty experts {fmt}")
    assert all(r["counts"][e] == 0 for e in (0, 1, 7, 15))


def test_experts_with_clamped_swiglu():
    """Large mlp1 weights push its outputs far past the SwiGLU limit on both sides; W2 is
    scaled by 2^-6 (exponent field - 6, exact) so the output keeps a moderate size."""
    cfg = get_config("C2", name="clamp", T=200, D=256, E=4, k=2, F=128, seed=5, weight_std=0.5)
    inp = make_inputs(cfg)
    u = oracle.bf16_to_f64(inp.x) @ oracle.expert_weight(inp.w1, "bf16", 4, 256, 256, 0).T
    assert (u[:, :128] > 7).mean() > 0.1 and (u[:, 128:] < -7).mean() > 0.1
    nz = (inp.w2 & 0x7FFF) != 0
    inp.w2 = np.where(nz, inp.w2 - np.uint16(6 << 7), inp.w2).astype(np.uint16)
    experts_vs_oracle(inp, "clamped SwiGLU")


@pytest.mark.parametrize("fmt,T", [("mxfp4", 200), ("mxfp4", 2000), ("mxfp8", 200), ("mxfp8", 2000)])
def test_experts_with_clamped_swiglu_mx(fmt, T):
    """The same for MX weights, on the streaming tiles (200 tokens) and the matrix-core tiles
    (2000 tokens: the scaled fp8 x fp4 engine for MXFP4): block scales raised until mlp1's
    outputs pass the limit on both sides; every W2 scale byte lowered by 4 (exact: a power of
    two) so the output keeps a moderate size."""
    E, D, F = 4, 256, 128
    scale = (-3, -1) if fmt == "mxfp4" else (-8, -6)
    cfg = get_config(BASE[fmt], name=f"clamp{fmt}{T}", T=T, D=D, E=E, k=2, F=F, seed=9 + T, scale_exp=scale)
    inp = make_inputs(cfg)
    u = oracle.bf16_to_f64(inp.x) @ oracle.expert_weight(inp.w1, fmt, E, 2 * F, D, 0).T
    assert (u[:, :F] > 7).mean() > 0.1 and (u[:, F:] < -7).mean() > 0.1 and (u[:, F:] > 7).mean() > 0.1
    w2 = inp.w2.copy()
    codes = E * D * (F // 2 if fmt == "mxfp4" else F)
    w2[codes:] -= 4
    inp.w2 = w2
    experts_vs_oracle(inp, f"clamped SwiGLU {fmt} T={T}")


# Weight buffers 16 or 48 bytes past a line boundary: the streaming tiles then copy code
# windows from each row's own start (no line alignment) and bf16 rows without the
# non-temporal hint, and the matrix-core tiles read unaligned windows too.
@pytest.mark.parametrize("offset", [16, 48])
@pytest.mark.parametrize("fmt,T,D,E,k,F", [
    ("bf16", 64, 448, 8, 2, 320),      # streaming tiles
    ("mxfp4", 64, 448, 8, 2, 320),     # streaming tiles, decode path
    ("mxfp4", 700, 320, 2, 1, 448),    # matrix-core tiles, scaled engine
    ("mxfp8", 64, 448, 8, 2, 320),     # MXFP8 decode path
])
def test_experts_unaligned_weight_buffers(offset, fmt, T, D, E, k, F):
    base = BASE[fmt]
    cfg = get_config(base, name=f"off{T}", T=T, D=D, E=E, k=k, F=F, seed=3000 + T + offset)
    experts_vs_oracle(make_inputs(cfg), f"weights +{offset} B {fmt} T={T} D={D} E={E} k={k} F={F}", offset)
