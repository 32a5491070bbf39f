"""Python binding of the C ABI in ``include/moe.h`` (ctypes; argument marshalling only).

PyTorch supplies device memory and the current stream; every step of the block runs
in the HIP kernels of ``libmoe.so``.  There is no fallback: if the library is missing
or a call fails, a ``MoEError`` is raised.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe.so")

FMT = {"bf16": 0, "mxfp4": 1, "mxfp8": 2}
STAGES = ("router", "topk", "permute", "mlp1", "mlp2", "combine", "split", "backward")

_c_void_p = ctypes.c_void_p
_i64 = ctypes.c_int64

# name -> (restype, argtypes); mirrors include/moe.h
_SIGNATURES = {
    "moe_forward": (ctypes.c_int, [_c_void_p] * 7 + [_i64] * 5 + [ctypes.c_int, _c_void_p]),
    "moe_route": (ctypes.c_int, [_c_void_p] * 3 + [_i64] * 4 + [_c_void_p] * 6),
    "moe_forward_noalloc": (ctypes.c_int, [_c_void_p] * 7 + [_i64] * 5 + [ctypes.c_int, _c_void_p]),
    "moe_forward_biased": (ctypes.c_int, [_c_void_p] * 8 + [_i64] * 5 + [ctypes.c_int, _c_void_p]),
    "moe_route_biased": (ctypes.c_int, [_c_void_p] * 4 + [_i64] * 4 + [_c_void_p] * 6),
    "moe_update_expert_bias": (ctypes.c_int, [_c_void_p, _i64, ctypes.c_float, _c_void_p]),
    "moe_experts": (ctypes.c_int, [_c_void_p] * 8 + [_i64] * 5 + [ctypes.c_int, _c_void_p]),
    "moe_backward": (ctypes.c_int, [_c_void_p] * 11 + [_i64] * 5 + [ctypes.c_int] + [_c_void_p] * 7),
    "moe_backward_workspace_bytes": (ctypes.c_size_t, [_i64] * 5 + [ctypes.c_int]),
    "moe_set_stream": (ctypes.c_int, [_c_void_p]),
    "moe_workspace_bytes": (ctypes.c_size_t, [_i64] * 5 + [ctypes.c_int]),
    "moe_set_workspace": (ctypes.c_int, [_c_void_p, ctypes.c_size_t]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_release": (None, []),
    "moe_profile_enable": (ctypes.c_int, [ctypes.c_int]),
    "moe_profile_read": (ctypes.c_int, [_c_void_p, _c_void_p]),
    "moe_version": (ctypes.c_char_p, []),
}

_lib = None


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where} failed with status {status}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load ``libmoe.so`` (built by ``python -m mixture_experts_transformer_amd.build``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise MoEError(-1, "load", f"{LIB_PATH} is missing; build it with "
                                       "`python -m mixture_experts_transformer_amd.build`")
        l = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(l, name)
            f.restype = res
            f.argtypes = args
        _lib = l
    return _lib


def _check(status: int, where: str) -> None:
    if status != 0:
        msg = lib().moe_last_error()
        raise MoEError(status, where, msg.decode() if msg else "")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _dev(t: torch.Tensor, name: str, itemsize: Optional[int] = None) -> torch.Tensor:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if itemsize is not None and t.element_size() != itemsize:
        raise ValueError(f"{name} must have {itemsize}-byte elements, got {t.dtype}")
    return t


def _bind_stream(device: torch.device) -> None:
    _check(lib().moe_set_stream(torch.cuda.current_stream(device).cuda_stream), "moe_set_stream")


def mxfp8_bytes(E: int, rows: int, K: int) -> int:
    """Bytes of an MXFP8 weight buffer: codes [E][rows][K] then scales [E][rows][K/32]."""
    return E * rows * (K + K // 32)


def mxfp4_bytes(E: int, rows: int, K: int) -> int:
    """Bytes of an MXFP4 weight buffer: codes [E][rows][K/2] then scales [E][rows][K/32]."""
    return E * rows * (K // 2 + K // 32)


def _check_weights(w1, w2, E, D, F, fmt):
    if fmt == "bf16":
        if tuple(w1.shape) != (E, 2 * F, D) or tuple(w2.shape) != (E, D, F):
            raise ValueError(f"bf16 weights must be w1 [{E},{2*F},{D}] and w2 [{E},{D},{F}]")
        _dev(w1, "w1", 2), _dev(w2, "w2", 2)
    elif fmt == "mxfp4":
        if w1.dtype != torch.uint8 or w2.dtype != torch.uint8:
            raise ValueError("mxfp4 weights are uint8 buffers")
        if w1.numel() != mxfp4_bytes(E, 2 * F, D) or w2.numel() != mxfp4_bytes(E, D, F):
            raise ValueError("mxfp4 weight buffers have the wrong size")
        _dev(w1, "w1"), _dev(w2, "w2")
    elif fmt == "mxfp8":
        if w1.dtype != torch.uint8 or w2.dtype != torch.uint8:
            raise ValueError("mxfp8 weights are uint8 buffers")
        if w1.numel() != mxfp8_bytes(E, 2 * F, D) or w2.numel() != mxfp8_bytes(E, D, F):
            raise ValueError("mxfp8 weight buffers have the wrong size")
        _dev(w1, "w1"), _dev(w2, "w2")
    else:
        raise ValueError(f"unknown format {fmt!r}")


def _check_bias(expert_bias, E):
    if expert_bias is not None:
        if expert_bias.dtype != torch.float32 or tuple(expert_bias.shape) != (E,):
            raise ValueError(f"expert_bias must be float32 [{E}]")
        _dev(expert_bias, "expert_bias", 4)


def forward(x, router_w, router_b, w1, b1, w2, b2, k: int, fmt: str = "bf16",
            out: Optional[torch.Tensor] = None, expert_bias: Optional[torch.Tensor] = None) -> torch.Tensor:
    """The whole block: returns out fp32 [T, D].  bf16 tensors may be torch.bfloat16 or
    2-byte integer views of the bits.  ``expert_bias`` (fp32 [E]) is the load-balancing
    bias: it moves the top-k selection, not the gates."""
    T, D = x.shape
    E = router_w.shape[0]
    F = b1.shape[-1] // 2
    _dev(x, "x", 2), _dev(router_w, "router_w", 2), _dev(router_b, "router_b", 2)
    _dev(b1, "b1", 2), _dev(b2, "b2", 2)
    _check_weights(w1, w2, E, D, F, fmt)
    _check_bias(expert_bias, E)
    if out is None:
        out = torch.empty((T, D), dtype=torch.float32, device=x.device)
    _dev(out, "out", 4)
    _bind_stream(x.device)
    if expert_bias is None:
        _check(lib().moe_forward(_ptr(x), _ptr(router_w), _ptr(router_b), _ptr(w1), _ptr(b1), _ptr(w2),
                                 _ptr(b2), T, D, E, k, F, FMT[fmt], _ptr(out)), "moe_forward")
    else:
        _check(lib().moe_forward_biased(_ptr(x), _ptr(router_w), _ptr(router_b), _ptr(expert_bias), _ptr(w1),
                                        _ptr(b1), _ptr(w2), _ptr(b2), T, D, E, k, F, FMT[fmt], _ptr(out)),
               "moe_forward_biased")
    return out


def forward_noalloc(x, router_w, router_b, w1, b1, w2, b2, k: int, fmt: str = "bf16",
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """``forward`` through ``moe_forward_noalloc``: the library allocates nothing (its
    intermediates live in a fixed per-GPU scratch array; shapes that do not fit raise
    ``MoEError`` with MOE_ENOMEM).  Pass ``out`` to allocate nothing here either."""
    T, D = x.shape
    E = router_w.shape[0]
    F = b1.shape[-1] // 2
    _dev(x, "x", 2), _dev(router_w, "router_w", 2), _dev(router_b, "router_b", 2)
    _dev(b1, "b1", 2), _dev(b2, "b2", 2)
    _check_weights(w1, w2, E, D, F, fmt)
    if out is None:
        out = torch.empty((T, D), dtype=torch.float32, device=x.device)
    _dev(out, "out", 4)
    _bind_stream(x.device)
    _check(lib().moe_forward_noalloc(_ptr(x), _ptr(router_w), _ptr(router_b), _ptr(w1), _ptr(b1), _ptr(w2),
                                     _ptr(b2), T, D, E, k, F, FMT[fmt], _ptr(out)), "moe_forward_noalloc")
    return out


def route(x, router_w, router_b, k: int, want_logits: bool = True,
          expert_bias: Optional[torch.Tensor] = None) -> dict:
    """Routing stage: logits (optional), top-k indices, gates, counts, offsets, permutation.
    ``expert_bias`` as in ``forward``."""
    T, D = x.shape
    E = router_w.shape[0]
    _dev(x, "x", 2), _dev(router_w, "router_w", 2), _dev(router_b, "router_b", 2)
    _check_bias(expert_bias, E)
    dev = x.device
    r = {
        "logits": torch.empty((T, E), dtype=torch.float32, device=dev) if want_logits else None,
        "idx": torch.empty((T, k), dtype=torch.int32, device=dev),
        "gates": torch.empty((T, k), dtype=torch.float32, device=dev),
        "counts": torch.empty((E,), dtype=torch.int32, device=dev),
        "offsets": torch.empty((E + 1,), dtype=torch.int32, device=dev),
        "perm": torch.empty((T * k,), dtype=torch.int32, device=dev),
    }
    outs = (_ptr(r["logits"]), _ptr(r["idx"]), _ptr(r["gates"]), _ptr(r["counts"]), _ptr(r["offsets"]),
            _ptr(r["perm"]))
    _bind_stream(dev)
    if expert_bias is None:
        _check(lib().moe_route(_ptr(x), _ptr(router_w), _ptr(router_b), T, D, E, k, *outs), "moe_route")
    else:
        _check(lib().moe_route_biased(_ptr(x), _ptr(router_w), _ptr(router_b), _ptr(expert_bias), T, D, E, k,
                                      *outs), "moe_route_biased")
    return r


def update_expert_bias(expert_bias: torch.Tensor, counts: torch.Tensor, coeff: float = 1e-3) -> torch.Tensor:
    """One load-balancing step of ``expert_bias`` (fp32 [E], updated in place and returned) from
    the per-expert assignment counts (int32 [E], e.g. ``route(...)["counts"]``)."""
    E = expert_bias.numel()
    _check_bias(expert_bias, E)
    if tuple(counts.shape) != (E,) or counts.dtype != torch.int32:
        raise ValueError(f"counts must be int32 [{E}]")
    _dev(counts, "counts", 4)
    _bind_stream(expert_bias.device)
    _check(lib().moe_update_expert_bias(_ptr(counts), E, coeff, _ptr(expert_bias)), "moe_update_expert_bias")
    return expert_bias


def experts(x, w1, b1, w2, b2, gates, offsets, perm, k: int, fmt: str = "bf16",
            out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Expert stage on a given routing (gates fp32 [T,k], offsets int32 [E+1], perm int32 [T*k])."""
    T, D = x.shape
    E = offsets.numel() - 1
    F = b1.shape[-1] // 2
    _dev(x, "x", 2), _dev(b1, "b1", 2), _dev(b2, "b2", 2)
    _check_weights(w1, w2, E, D, F, fmt)
    for t, n in ((gates, "gates"), (offsets, "offsets"), (perm, "perm")):
        _dev(t, n, 4)
    if out is None:
        out = torch.empty((T, D), dtype=torch.float32, device=x.device)
    _dev(out, "out", 4)
    _bind_stream(x.device)
    _check(lib().moe_experts(_ptr(x), _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2), _ptr(gates), _ptr(offsets),
                             _ptr(perm), T, D, E, k, F, FMT[fmt], _ptr(out)), "moe_experts")
    return out


def backward(x, router_w, w1, b1, w2, b2, routing: dict, dout, k: int, fmt: str = "bf16",
             out: Optional[dict] = None) -> dict:
    """Gradients of the block (``moe_backward``) for the routing of a forward (``route``'s dict:
    idx, gates, offsets, perm) and the output gradient ``dout`` (fp32 [T, D]).  Returns fp32
    dx, dwr, dbr, dw1, db1, dw2, db2 (each the shape of its input), written into ``out``'s
    tensors when given (e.g. for a captured graph)."""
    T, D = x.shape
    E = router_w.shape[0]
    F = b1.shape[-1] // 2
    _dev(x, "x", 2), _dev(router_w, "router_w", 2), _dev(b1, "b1", 2), _dev(b2, "b2", 2)
    _check_weights(w1, w2, E, D, F, fmt)
    _dev(dout, "dout", 4)
    if tuple(dout.shape) != (T, D):
        raise ValueError(f"dout must be [{T}, {D}]")
    for n in ("idx", "gates", "offsets", "perm"):
        _dev(routing[n], n, 4)
    dev = x.device
    f32 = lambda *s: torch.empty(s, dtype=torch.float32, device=dev)
    shapes = {"dx": (T, D), "dwr": (E, D), "dbr": (E,), "dw1": (E, 2 * F, D), "db1": (E, 2 * F),
              "dw2": (E, D, F), "db2": (E, D)}
    if out is None:
        g = {n: f32(*sh) for n, sh in shapes.items()}
    else:
        g = out
        for n, sh in shapes.items():
            _dev(g[n], n, 4)
            if tuple(g[n].shape) != sh:
                raise ValueError(f"out[{n!r}] must be {list(sh)}")
    _bind_stream(dev)
    _check(lib().moe_backward(_ptr(x), _ptr(router_w), _ptr(w1), _ptr(b1), _ptr(w2), _ptr(b2),
                              _ptr(routing["idx"]), _ptr(routing["gates"]), _ptr(routing["offsets"]),
                              _ptr(routing["perm"]), _ptr(dout), T, D, E, k, F, FMT[fmt],
                              _ptr(g["dx"]), _ptr(g["dwr"]), _ptr(g["dbr"]), _ptr(g["dw1"]), _ptr(g["db1"]),
                              _ptr(g["dw2"]), _ptr(g["db2"])), "moe_backward")
    return g


def backward_workspace_bytes(T: int, D: int, E: int, k: int, F: int, fmt: str = "bf16") -> int:
    return int(lib().moe_backward_workspace_bytes(T, D, E, k, F, FMT[fmt]))


def workspace_bytes(T: int, D: int, E: int, k: int, F: int, fmt: str = "bf16") -> int:
    return int(lib().moe_workspace_bytes(T, D, E, k, F, FMT[fmt]))


def set_workspace(buf: Optional[torch.Tensor]) -> None:
    """Use ``buf`` (a uint8 GPU tensor, kept alive by the caller) as the workspace; None to return
    to the library-owned one."""
    if buf is None:
        _check(lib().moe_set_workspace(None, 0), "moe_set_workspace")
    else:
        _check(lib().moe_set_workspace(_ptr(_dev(buf, "workspace")), buf.numel() * buf.element_size()),
               "moe_set_workspace")


def release() -> None:
    lib().moe_release()


def profile_enable(on: bool = True) -> None:
    _check(lib().moe_profile_enable(1 if on else 0), "moe_profile_enable")


def profile_read() -> dict:
    """{stage: (total_ms, launches)} since the last read (synchronises on the recorded events)."""
    ms = (ctypes.c_double * len(STAGES))()
    n = (ctypes.c_int64 * len(STAGES))()
    _check(lib().moe_profile_read(ctypes.addressof(ms), ctypes.addressof(n)), "moe_profile_read")
    return {s: (ms[i], n[i]) for i, s in enumerate(STAGES)}


def version() -> str:
    return lib().moe_version().decode()
