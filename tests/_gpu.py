"""Helpers for the GPU parity tests: upload generated inputs, compare with the oracle."""
import sys

import numpy as np
import torch

import mixture_experts_transformer_amd as moe

DEV = "cuda"

# the parity bar on the fp32 output against the float64 oracle
REL_L2 = 1e-2
MAX_ABS = 3e-2
GATE_ABS = 1e-6   # gates are <= 1: absolute 1e-6 is tighter than 1e-5 relative for all but tiny gates


def note(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a failing run says what it was doing."""
    print(f"[gpu] {msg}", flush=True)
    sys.stdout.flush()


def u16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def weights(a: np.ndarray, fmt: str) -> torch.Tensor:
    if fmt == "bf16":
        return u16(a)
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def at_offset(t: torch.Tensor, offset: int) -> torch.Tensor:
    """The same bytes in a fresh buffer, starting `offset` bytes past an aligned allocation."""
    raw = t.contiguous().view(torch.uint8).reshape(-1)
    buf = torch.zeros(raw.numel() + 256, dtype=torch.uint8, device=t.device)
    base = (256 - buf.data_ptr() % 256) % 256
    view = buf[base + offset: base + offset + raw.numel()]
    view.copy_(raw)
    return view.view(t.dtype).reshape(t.shape)


def upload(inp, weight_offset: int = 0) -> dict:
    """Inputs on the GPU; weight_offset > 0 places w1 and w2 that many bytes past a 256-byte
    boundary (still 16-byte aligned, as the ABI requires)."""
    fmt = inp.cfg.fmt
    w1, w2 = weights(inp.w1, fmt), weights(inp.w2, fmt)
    if weight_offset:
        w1, w2 = at_offset(w1, weight_offset), at_offset(w2, weight_offset)
    return dict(x=u16(inp.x), router_w=u16(inp.wr), router_b=u16(inp.br), w1=w1,
                b1=u16(inp.b1), w2=w2, b2=u16(inp.b2))


def errors(got: np.ndarray, ref: np.ndarray):
    d = got.astype(np.float64) - ref
    rel = np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-300)
    return float(rel), float(np.max(np.abs(d))) if d.size else 0.0


def assert_close(got: np.ndarray, ref: np.ndarray, what: str):
    rel, mx = errors(got, ref)
    note(f"{what}: rel_l2={rel:.3e} max_abs={mx:.3e} (ref max {np.max(np.abs(ref)):.3g})")
    assert rel <= REL_L2, f"{what}: relative L2 error {rel:.3e} > {REL_L2}"
    assert mx <= MAX_ABS, f"{what}: max abs error {mx:.3e} > {MAX_ABS}"
