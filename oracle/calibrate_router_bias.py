"""Calibrate the router bias of the Zipf-routed workloads -- test infrastructure.

The workload table asks for a router bias "drawn so that expert load is
Zipf-skewed".  Reading taken: the *realised* per-expert token counts should follow
the Zipf targets of ``synth.zipf_plan`` (empty experts get none).  Realised counts
depend on the router's own arithmetic, so they are computed here with the oracle
(``router_logits`` + ``select_experts``), never with the GPU library.

Procedure: start from b_e = s_L * ln(target_e / (T k)) with s_L = 0.02 sqrt(D) (the
spread of the router's dot products), then repeat 40 times
b_e += 0.5 s_L (ln target_e - ln max(count_e, 0.5)) with the bias held in bf16; empty
experts get b = -64.  The iterate with the smallest worst-case |count/target - 1| over
the live experts is written to ``synth/router_bias/<config>.txt`` as bf16 bits.

    python -m oracle.calibrate_router_bias C3 C5
"""
from __future__ import annotations

import os
import sys

import numpy as np

from synth import get_config, zipf_plan, router_bias_path, f32_to_bf16_bits, make_router_inputs
from .moe_oracle import bf16_to_f64, router_logits, select_experts

ITERS = 40


def realised_counts(x, wr, br_bits, k, E):
    idx = select_experts(router_logits(x, wr, br_bits), k)
    return np.bincount(idx.reshape(-1), minlength=E)


def calibrate(name: str, verbose: bool = True):
    cfg = get_config(name)
    assert cfg.router_bias == "zipf"
    plan = zipf_plan(cfg)
    empty, target = plan["empty"], plan["target"]
    live = ~empty
    x, wr = make_router_inputs(cfg)
    sL = 0.02 * np.sqrt(cfg.D)
    b = np.full(cfg.E, -64.0)
    b[live] = sL * np.log(target[live] / (cfg.T * cfg.k))
    best = None
    for it in range(ITERS + 1):
        bits = f32_to_bf16_bits(b.astype(np.float32))
        bits[empty] = f32_to_bf16_bits(np.float32([-64.0]))[0]
        c = realised_counts(x, wr, bits, cfg.k, cfg.E)
        err = np.max(np.abs(c[live] / target[live] - 1.0))
        if c[empty].any():
            err = np.inf
        if best is None or err < best[0]:
            best = (err, bits.copy(), c.copy(), it)
        if verbose:
            print(f"{name} iter {it:2d}: worst |count/target-1| = {err:.4f}", flush=True)
        b = bf16_to_f64(bits)
        b[live] += 0.5 * sL * (np.log(target[live]) - np.log(np.maximum(c[live], 0.5)))
    err, bits, c, it = best
    path = router_bias_path(cfg)
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w") as f:
        f.write(f"# router bias (bf16 bits) for workload {name}: T={cfg.T} D={cfg.D} E={cfg.E} "
                f"k={cfg.k} seed={cfg.seed} zipf_s={cfg.zipf_s} empty={int(empty.sum())}\n")
        f.write("# written by oracle/calibrate_router_bias.py (oracle router + top-k only)\n")
        f.write(f"# iterate {it}, worst |count/target-1| over live experts = {err:.4f}\n")
        f.write("# columns: expert bias_bits target_count realised_count\n")
        for e in range(cfg.E):
            f.write(f"{e} {int(bits[e]):04x} {target[e]:.1f} {int(c[e])}\n")
    if verbose:
        print(f"wrote {path} (iterate {it}, worst rel err {err:.4f})")
    return bits, c


if __name__ == "__main__":
    for n in (sys.argv[1:] or ["C3", "C5"]):
        calibrate(n)
