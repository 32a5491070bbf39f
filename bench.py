"""Throughput of the GPT-OSS MoE block on one MI355X.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload C2] [--all]

One step = one moe_forward over one batch of synthetic tokens (router, top-k, grouping,
mlp1 + SwiGLU, mlp2 + gate, combine).  Inputs are resident in device memory before the
timed region.  The expert weights are rotated over several device copies so no step finds
the previous step's weights in the 256 MB Infinity Cache, as consecutive MoE layers of a
model would not.  Prints one JSON line (per workload with --all).

The dominant kernel's roofline comes from the library's own per-launch HIP events on the
stream the kernels run on; its HBM traffic from the rocprofv3 counter summary in
profiles/ when that summary was taken on the current kernel source.  The CPU baseline is
the float64 oracle timed on the host on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE-layer tokens/sec + TFLOP/s (frac. of peak) at GPT-OSS-20B shape, bf16 & MXFP4"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 matrix peak
FP8_PEAK_TFLOPS = 5000.0       # MI355X dense fp8 matrix peak: the rate of the scaled fp8 x fp4 instruction
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense FP4 matrix peak (reported for MXFP4 weights only)
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
GEMM_SRC = os.path.join(ROOT, "mixture_experts_transformer_amd", "csrc", "gemm.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def mx_engine(cfg):
    """True where the library runs the expert GEMMs on the scaled fp8 x fp4 instruction: MXFP4
    weights with at least 128 routed rows per expert on average (its matrix-core tiles)."""
    return cfg.fmt == "mxfp4" and cfg.T * cfg.k >= 128 * cfg.E


def algorithmic(cfg, counts):
    """Algorithmic flops and bytes of one forward, and per-kernel bytes for mlp1/mlp2.

    Bytes count each input once and the output once: touched experts' weights and biases,
    the router, x (bf16) and out (fp32).  Per kernel, mlp1 reads x (bf16; on the scaled
    engine its two fp8 pieces, the same two bytes per element) and writes h, mlp2 reads h
    and writes y (fp32); h is bf16 (bf16 weights), a bf16 pair (MXFP4, few rows) or three
    fp8 pieces and one scale dword per 32 elements (scaled engine); MXFP8 weights are one
    byte per element plus one scale byte per 32 and carry h as a bf16 pair.
    """
    T, D, E, k, F = cfg.T, cfg.D, cfg.E, cfg.k, cfg.F
    A = T * k
    touched = int(np.count_nonzero(counts))
    if cfg.fmt == "bf16":
        w1_e, w2_e = 2 * F * D * 2, D * F * 2
    elif cfg.fmt == "mxfp8":
        w1_e, w2_e = 2 * F * (D + D // 32), D * (F + F // 32)
    else:
        w1_e, w2_e = 2 * F * (D // 2 + D // 32), D * (F // 2 + F // 32)
    b1_e, b2_e = 2 * F * 2, D * 2
    if mx_engine(cfg):
        hbytes = A * (3 * F + ((F // 32 + 7) // 8 * 8) * 4)
    else:
        hbytes = A * F * 2 * (1 if cfg.fmt == "bf16" else 2)
    flops = T * (2 * D * E + 6 * k * D * F)
    step_bytes = touched * (w1_e + b1_e + w2_e + b2_e) + E * D * 2 + E * 2 + T * D * 2 + T * D * 4
    mlp1_bytes = touched * (w1_e + b1_e) + T * D * 2 + hbytes
    mlp2_bytes = touched * (w2_e + b2_e) + hbytes + A * D * 4
    return dict(flops=flops, bytes=step_bytes, touched=touched,
                mlp1=dict(flops=4 * A * D * F, bytes=mlp1_bytes, unit_bytes=w1_e + b1_e),
                mlp2=dict(flops=2 * A * F * D, bytes=mlp2_bytes, unit_bytes=w2_e + b2_e))


def cpu_baseline(inp, n_tokens, min_seconds=10.0):
    """Time the oracle on the first n_tokens of the workload (float64 NumPy on host cores),
    repeating the forward until at least min_seconds have elapsed."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    cfg = inp.cfg
    x = inp.x[:n_tokens]
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.moe_forward(x, inp.wr, inp.br, inp.w1, inp.b1, inp.w2, inp.b2, k=cfg.k, F=cfg.F, fmt=cfg.fmt)
        reps += 1
        dt = time.perf_counter() - t0
        if dt >= min_seconds:
            break
    return {"value": round(reps * n_tokens / dt, 3), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n_tokens} of the {cfg.T} tokens of workload {cfg.name}, float64 forward "
                      f"repeated {reps} times ({dt:.1f} s)"}


def source_key():
    """Hash of the grouped-GEMM kernel source with comments and blank lines removed, so the
    stored counters stay valid across comment-only edits and go stale on any code change."""
    import re
    text = open(GEMM_SRC).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    lines = [re.sub(r"//.*$", "", l).rstrip() for l in text.splitlines()]
    code = "\n".join(l for l in lines if l.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def stored_traffic(workload, kernel):
    if not os.path.exists(TRAFFIC_FILE):
        return None
    try:
        rec = json.load(open(TRAFFIC_FILE)).get(f"{workload}/{kernel}")
    except Exception:
        return None
    if not rec:
        return None
    if rec.get("source_sha") != source_key():
        return None       # counters were taken on another version of the kernel
    return rec.get("bytes_per_launch")


def bench_workload(name, steps, warmup, with_cpu):
    import torch
    import mixture_experts_transformer_amd as moe
    from synth import get_config, make_inputs

    cfg = get_config(name)
    log(f"[bench] {name}: generating inputs")
    inp = make_inputs(name)
    dev = torch.device("cuda:0")
    t16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    tw = t16 if cfg.fmt == "bf16" else (lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev))
    x, wr, br, b1, b2 = t16(inp.x), t16(inp.wr), t16(inp.br), t16(inp.b1), t16(inp.b2)
    w1_0, w2_0 = tw(inp.w1), tw(inp.w2)
    per_copy = w1_0.numel() * w1_0.element_size() + w2_0.numel() * w2_0.element_size()
    copies = int(min(8, max(2, math.ceil(2.0e9 / per_copy))))
    w1s, w2s = [w1_0], [w2_0]
    for _ in range(copies - 1):
        w1s.append(w1_0.clone())
        w2s.append(w2_0.clone())
    out = torch.empty((cfg.T, cfg.D), dtype=torch.float32, device=dev)
    r = moe.route(x, wr, br, cfg.k, want_logits=False)
    counts = r["counts"].cpu().numpy()
    alg = algorithmic(cfg, counts)

    def step(i):
        moe.forward(x, wr, br, w1s[i % copies], b1, w2s[i % copies], b2, cfg.k, cfg.fmt, out=out)

    log(f"[bench] {name}: warmup {warmup} steps ({copies} weight copies of {per_copy / 1e6:.0f} MB)")
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # timed region: K steps, nothing else on the stream
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / steps
    # second pass of K steps with the library's per-launch HIP events (on the stream the
    # kernels run on) for the per-kernel durations; the events add small gaps, which is
    # why the throughput comes from the pass above
    moe.profile_read()                       # discard
    moe.profile_enable(True)
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    moe.profile_enable(False)
    stages = moe.profile_read()
    log(f"[bench] {name}: {ms * 1e3:.1f} us/step; per-kernel average: " +
        ", ".join(f"{s} {tms / max(n, 1) * 1e3:.1f} us" for s, (tms, n) in stages.items()))

    # dominant kernel: largest share of the step
    dom = max(("mlp1", "mlp2"), key=lambda s: stages[s][0])
    tms, n = stages[dom]
    avg_s = tms / n / 1e3
    # the matrix instruction the kernel issues: bf16 (bf16 weights, or MXFP4 decoded to bf16
    # at few rows per expert), or the scaled fp8 x fp4 one, which runs at the fp8 rate and
    # issues each flop once per activation piece (x: 2, h: 3)
    mx = mx_engine(cfg)
    peak_t = FP8_PEAK_TFLOPS if mx else BF16_PEAK_TFLOPS
    pieces = (2 if dom == "mlp1" else 3) if mx else (2 if (cfg.fmt != "bf16" and dom == "mlp2") else 1)
    hbm_bound = alg[dom]["flops"] * pieces / alg[dom]["bytes"] < peak_t * 1e12 / (HBM_PEAK_GBS * 1e9)
    if hbm_bound:
        achieved = alg[dom]["bytes"] / avg_s / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = alg[dom]["flops"] / avg_s / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": peak_t, "unit": "TFLOP/s",
                "frac": round(achieved / peak_t, 4)}
    roof["kernel"] = dom
    roof["instruction"] = ("v_mfma_scale_f32_32x32x64_f8f6f4 (fp8 E4M3 activation pieces x MXFP4)" if mx
                           else "v_mfma_f32_32x32x16_bf16")
    roof["issued_flop_per_algorithmic_flop"] = pieces
    roof["issued_frac"] = round(alg[dom]["flops"] * pieces / avg_s / 1e12 / peak_t, 4)
    roof["avg_launch_us"] = round(avg_s * 1e6, 2)
    roof["traffic"] = stored_traffic(name, dom)

    step_s = ms / 1e3
    res = {
        "metric": METRIC,
        "value": round(cfg.T / step_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8xfp4" if mx else "bf16",
        "data": "synthetic",
        "config": {"workload": f"{name}: T={cfg.T} D={cfg.D} E={cfg.E} k={cfg.k} F={cfg.F} "
                               f"{cfg.fmt} expert weights ({cfg.note})",
                   "tokens": cfg.T, "experts": cfg.E, "top_k": cfg.k, "hidden": cfg.D, "intermediate": cfg.F,
                   "weights": cfg.fmt, "weight_copies_rotated": copies, "touched_experts": alg["touched"]},
        "step_tflops": round(alg["flops"] / step_s / 1e12, 2),
        "step_mfma_frac": round(alg["flops"] / step_s / 1e12 / BF16_PEAK_TFLOPS, 4),
        # for MXFP4 weights the fractions of the fp8 and FP4 peaks are reported beside the
        # bf16 one so nothing is hidden
        "step_fp8_peak_frac": (round(alg["flops"] / step_s / 1e12 / FP8_PEAK_TFLOPS, 4)
                               if cfg.fmt == "mxfp4" else None),
        "step_fp4_peak_frac": (round(alg["flops"] / step_s / 1e12 / FP4_PEAK_TFLOPS, 4)
                               if cfg.fmt == "mxfp4" else None),
        "step_hbm_gbs": round(alg["bytes"] / step_s / 1e9, 1),
        "step_hbm_frac": round(alg["bytes"] / step_s / 1e9 / HBM_PEAK_GBS, 4),
        "kernel_us": {s: round(tms / max(n, 1) * 1e3, 2) for s, (tms, n) in stages.items()},
        "roofline": roof,
    }
    if with_cpu:
        n_cpu = min(cfg.T, 256 if cfg.E <= 32 else 64)
        log(f"[bench] {name}: timing the CPU oracle on {n_cpu} tokens")
        res["cpu_baseline"] = cpu_baseline(inp, n_cpu)
    del w1s, w2s
    torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="C2", help="C2 (default), C3, C4, C5, X1, X2, Y1, Y2")
    ap.add_argument("--all", action="store_true", help="one line per target workload: C2 C3 X1 X2")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 3 plain device copies of MIB MiB (reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the MoE block is built and timed on a single MI355X; "
              "run it with --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "copies": 3}), flush=True)
        return
    names = ["C2", "C3", "X1", "X2"] if args.all else [args.workload]
    for i, name in enumerate(names):
        res = bench_workload(name, args.steps, args.warmup, with_cpu=(not args.no_cpu) and i == 0)
        print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
