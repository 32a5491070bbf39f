"""Seeded input synthesis for the MoE block (shared by the oracle and the GPU path).

Every array is drawn from ``numpy.random.default_rng`` children of
``SeedSequence(cfg.seed).spawn(9)``, taken in the fixed order
x, router weight, router bias, w1, b1, w2, b2, routing-rank permutation,
empty-expert set.  Large weight tensors draw one child stream per expert so the
draw can run on a thread pool and still give the same bytes on every machine.

Encodings (these are the storage formats the library reads):

* bf16: the upper 16 bits of the fp32 value after round-to-nearest-even.
* MXFP8: one uint8 buffer holding the E4M3 codes ``[E][rows][K]`` followed by the
  E8M0 scale bytes ``[E][rows][K/32]`` (OCP Microscaling spec v1.0).
* MXFP4 (GPT-OSS-in-Transformers blog, section on MXFP4: 4-bit E2M1 values
  sharing one scale per 32-element block; OCP Microscaling spec v1.0 for the
  E8M0 scale byte): one uint8 buffer holding the codes ``[E][rows][K/2]``
  (two codes per byte, the even-indexed element in the low nibble) followed by
  the scale bytes ``[E][rows][K/32]``; blocks run along K, the reduction dim.

Nothing here evaluates the MoE block itself; the Zipf router bias that needs
the router's own arithmetic is calibrated by ``oracle/calibrate_router_bias.py``
and read back from ``synth/router_bias/<config>.txt``.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from functools import lru_cache
from typing import Dict, Optional

import numpy as np

from .configs import Config, get_config

_HERE = os.path.dirname(os.path.abspath(__file__))
_STREAMS = ("x", "wr", "br", "w1", "b1", "w2", "b2", "rank", "empty")
_POOL_THREADS = max(1, min(16, os.cpu_count() or 1))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round to nearest, ties to even. Inputs are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def _streams(cfg: Config) -> Dict[str, np.random.SeedSequence]:
    return dict(zip(_STREAMS, np.random.SeedSequence(cfg.seed).spawn(len(_STREAMS))))


def _normal_bf16_rows(ss: np.random.SeedSequence, n_outer: int, inner_shape, std: float) -> np.ndarray:
    """[n_outer, *inner_shape] of N(0, std) rounded to bf16; one child stream per outer index."""
    children = ss.spawn(n_outer)
    out = np.empty((n_outer,) + tuple(inner_shape), dtype=np.uint16)

    def fill(i):
        g = np.random.default_rng(children[i])
        v = g.standard_normal(inner_shape, dtype=np.float32)
        v *= np.float32(std)
        out[i] = f32_to_bf16_bits(v)

    with ThreadPoolExecutor(_POOL_THREADS) as ex:
        list(ex.map(fill, range(n_outer)))
    return out


def _mxfp4_buffer(ss: np.random.SeedSequence, E: int, rows: int, K: int, exp_lo: int, exp_hi: int) -> np.ndarray:
    """MXFP4 weights [E][rows][K]: codes uniform over the 16 E2M1 codes, E8M0 byte 127+U{exp_lo..exp_hi}."""
    assert K % 32 == 0
    children = ss.spawn(E)
    ncode = rows * (K // 2)
    nscale = rows * (K // 32)
    buf = np.empty(E * (ncode + nscale), dtype=np.uint8)
    codes = buf[: E * ncode].reshape(E, ncode)
    scales = buf[E * ncode:].reshape(E, nscale)

    def fill(e):
        g = np.random.default_rng(children[e])
        codes[e] = g.integers(0, 256, ncode, dtype=np.uint8)          # two independent uniform nibbles
        scales[e] = g.integers(127 + exp_lo, 127 + exp_hi + 1, nscale, dtype=np.uint8)

    with ThreadPoolExecutor(_POOL_THREADS) as ex:
        list(ex.map(fill, range(E)))
    return buf


def _mxfp8_buffer(ss: np.random.SeedSequence, E: int, rows: int, K: int, exp_lo: int, exp_hi: int) -> np.ndarray:
    """MXFP8 weights [E][rows][K]: codes [E][rows][K] uniform over the 254 finite E4M3 codes
    (0x7F and 0xFF, the NaN codes, are skipped), then E8M0 bytes 127+U{exp_lo..exp_hi}."""
    assert K % 32 == 0
    children = ss.spawn(E)
    ncode = rows * K
    nscale = rows * (K // 32)
    buf = np.empty(E * (ncode + nscale), dtype=np.uint8)
    codes = buf[: E * ncode].reshape(E, ncode)
    scales = buf[E * ncode:].reshape(E, nscale)

    def fill(e):
        g = np.random.default_rng(children[e])
        u = g.integers(0, 254, ncode, dtype=np.uint8)                   # index into the finite codes
        codes[e] = u + (u >= 0x7F)
        scales[e] = g.integers(127 + exp_lo, 127 + exp_hi + 1, nscale, dtype=np.uint8)

    with ThreadPoolExecutor(_POOL_THREADS) as ex:
        list(ex.map(fill, range(E)))
    return buf


def _activations(cfg: Config, ss: np.random.SeedSequence) -> np.ndarray:
    g = np.random.default_rng(ss)
    v = g.standard_normal((cfg.T, cfg.D), dtype=np.float32)
    if cfg.x_dist == "rmsnorm":
        # gain 1, eps 1e-5, in fp32: only shapes the activations like a pre-MoE norm would
        ms = np.mean(v.astype(np.float64) ** 2, axis=1, keepdims=True).astype(np.float32)
        v = v / np.sqrt(ms + np.float32(1e-5))
    elif cfg.x_dist != "normal":
        raise ValueError(cfg.x_dist)
    return f32_to_bf16_bits(v)


def zipf_plan(cfg: Config) -> dict:
    """Load-shape targets for a Zipf-routed config (pure input structure, no MoE arithmetic).

    Returns ``empty`` (experts that must get no token), ``rank`` (rank 1..n of each live
    expert, -1 for empty ones) and ``target`` (desired token count per expert): the Zipf
    share r**-s of T*k, capped at T because one token picks an expert at most once,
    with the excess spread over the uncapped experts in proportion to their share.
    """
    st = _streams(cfg)
    E, T, k = cfg.E, cfg.T, cfg.k
    empty = np.zeros(E, dtype=bool)
    if cfg.n_empty:
        assert cfg.n_empty >= 2
        g = np.random.default_rng(st["empty"])
        empty[0] = empty[E - 1] = True
        empty[1 + g.choice(E - 2, size=cfg.n_empty - 2, replace=False)] = True
    live = np.flatnonzero(~empty)
    g = np.random.default_rng(st["rank"])
    order = live[g.permutation(live.size)]           # order[0] is rank 1
    rank = np.full(E, -1, dtype=np.int64)
    rank[order] = np.arange(1, live.size + 1)
    share = np.zeros(E)
    share[live] = rank[live].astype(np.float64) ** (-cfg.zipf_s)
    share /= share.sum()
    target = share * (T * k)
    capped = np.zeros(E, dtype=bool)
    for _ in range(E):
        over = target > T
        if not over.any():
            break
        capped |= over
        excess = (target[over] - T).sum()
        target[over] = T
        free = (~capped) & (~empty)
        target[free] += excess * share[free] / share[free].sum()
    return {"empty": empty, "rank": rank, "target": target}


def router_bias_path(cfg: Config) -> str:
    return os.path.join(_HERE, "router_bias", f"{cfg.name}.txt")


def _read_router_bias(cfg: Config) -> np.ndarray:
    path = router_bias_path(cfg)
    if not os.path.exists(path):
        raise FileNotFoundError(
            f"{path} is missing: run `python -m oracle.calibrate_router_bias {cfg.name}` to write it")
    vals = [int(line.split()[1], 16) for line in open(path)
            if line.strip() and not line.startswith("#")]
    if len(vals) != cfg.E:
        raise ValueError(f"{path}: expected {cfg.E} entries, found {len(vals)}")
    return np.array(vals, dtype=np.uint16)


def make_router_inputs(cfg) -> tuple:
    """(x [T,D], router weight [E,D]) as bf16 bits, identical to ``make_inputs``'s draws."""
    if isinstance(cfg, str):
        cfg = get_config(cfg)
    st = _streams(cfg)
    x = _activations(cfg, st["x"])
    wr = f32_to_bf16_bits(np.random.default_rng(st["wr"]).standard_normal((cfg.E, cfg.D), dtype=np.float32)
                          * np.float32(cfg.weight_std))
    return x, wr


def make_routing_inputs(cfg) -> tuple:
    """(x, router weight, router bias) as bf16 bits, identical to ``make_inputs``'s draws."""
    if isinstance(cfg, str):
        cfg = get_config(cfg)
    x, wr = make_router_inputs(cfg)
    return x, wr, _router_bias(cfg, _streams(cfg))


def _router_bias(cfg: Config, st) -> np.ndarray:
    if cfg.router_bias == "zero":
        return np.zeros(cfg.E, dtype=np.uint16)
    if cfg.router_bias == "normal":
        return f32_to_bf16_bits(np.random.default_rng(st["br"]).standard_normal(cfg.E, dtype=np.float32)
                                * np.float32(cfg.bias_std))
    if cfg.router_bias == "zipf":
        return _read_router_bias(cfg)
    raise ValueError(cfg.router_bias)


@dataclass
class MoEInputs:
    """Host copies of one layer's inputs, as raw storage bits.

    x [T,D] u16 (bf16); wr [E,D] u16; br [E] u16; w1: bf16 -> [E,2F,D] u16, mxfp4 -> flat u8
    (codes [E][2F][D/2] then scales [E][2F][D/32]); b1 [E,2F] u16; w2: bf16 -> [E,D,F] u16,
    mxfp4 -> flat u8 (codes [E][D][F/2] then scales [E][D][F/32]); b2 [E,D] u16.
    """
    cfg: Config
    x: np.ndarray
    wr: np.ndarray
    br: np.ndarray
    w1: np.ndarray
    b1: np.ndarray
    w2: np.ndarray
    b2: np.ndarray


def _build(cfg: Config, router_bias: Optional[np.ndarray]) -> MoEInputs:
    st = _streams(cfg)
    T, D, E, F = cfg.T, cfg.D, cfg.E, cfg.F
    x, wr = make_router_inputs(cfg)
    br = np.asarray(router_bias, dtype=np.uint16) if router_bias is not None else _router_bias(cfg, st)
    if cfg.fmt == "bf16":
        w1 = _normal_bf16_rows(st["w1"], E, (2 * F, D), cfg.weight_std)
        w2 = _normal_bf16_rows(st["w2"], E, (D, F), cfg.weight_std)
    elif cfg.fmt == "mxfp4":
        lo, hi = cfg.scale_exp
        w1 = _mxfp4_buffer(st["w1"], E, 2 * F, D, lo, hi)
        w2 = _mxfp4_buffer(st["w2"], E, D, F, lo, hi)
    elif cfg.fmt == "mxfp8":
        lo, hi = cfg.scale_exp
        w1 = _mxfp8_buffer(st["w1"], E, 2 * F, D, lo, hi)
        w2 = _mxfp8_buffer(st["w2"], E, D, F, lo, hi)
    else:
        raise ValueError(cfg.fmt)
    b1 = f32_to_bf16_bits(np.random.default_rng(st["b1"]).standard_normal((E, 2 * F), dtype=np.float32)
                          * np.float32(cfg.bias_std))
    b2 = f32_to_bf16_bits(np.random.default_rng(st["b2"]).standard_normal((E, D), dtype=np.float32)
                          * np.float32(cfg.bias_std))
    return MoEInputs(cfg, x, wr, br, w1, b1, w2, b2)


@lru_cache(maxsize=2)
def _cached(name: str, overrides: tuple) -> MoEInputs:
    return _build(get_config(name, **dict(overrides)), None)


def make_inputs(cfg, router_bias: Optional[np.ndarray] = None, **overrides) -> MoEInputs:
    """Inputs for a named config (``"C3"``) or a ``Config``; results for names are cached.

    ``router_bias`` (bf16 bits) replaces the config's router-bias rule; it is how the
    calibration script tries candidate biases without a stored file.
    """
    if isinstance(cfg, str) and router_bias is None:
        return _cached(cfg, tuple(sorted(overrides.items())))
    if isinstance(cfg, str):
        cfg = get_config(cfg, **overrides)
    elif overrides:
        raise TypeError("overrides need a config name")
    return _build(cfg, router_bias)


def make_expert_bias(E: int, seed: int, steps_std: float = 300.0, step: float = 1e-3) -> np.ndarray:
    """A load-balancing expert bias, fp32 [E]: whole numbers of update steps of size ``step``
    (the torchtitan guide gives load_balance_coeff = 1e-3), the step counts drawn from
    round(N(0, steps_std)), so the values are k * fp32(step) with many near zero and exact
    repeats between experts."""
    n = np.rint(np.random.default_rng(seed).normal(0.0, steps_std, E))
    return (n.astype(np.float32) * np.float32(step)).astype(np.float32)



def make_dout(T: int, D: int, seed: int, std: float = 1.0) -> np.ndarray:
    """A seeded output gradient for the backward, fp32 [T, D] drawn from N(0, std^2)."""
    return (np.random.default_rng(np.random.SeedSequence([seed, 0x6D6F65]))
            .standard_normal((T, D), dtype=np.float32) * np.float32(std))
