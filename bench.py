"""Throughput of the GPT-OSS MoE block on one MI355X.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--workload C2] [--all] [--no-targets]

One step = one moe_forward over one batch of synthetic tokens (router, top-k, grouping,
mlp1 + SwiGLU, mlp2 + gate, combine).  The default line is the 256-token bf16 layer (C2);
it also carries, under "targets", the same measurement of the other target layers: bf16 at
8192 tokens with a Zipf load (C3) and MXFP4 weights at 256 and 8192 tokens (X1, X2).  Inputs are resident in device memory before the
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
FP4_PEAK_TFLOPS = 10100.0      # MI355X dense FP4/FP6 matrix peak: the rate of the scaled fp6 x fp4 instruction
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
GEMM_SRC = os.path.join(ROOT, "mixture_experts_transformer_amd", "csrc", "gemm.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def mx_engine(cfg):
    """True where the library runs the expert GEMMs on the scaled matrix instruction (fp8 pieces
    of x times MXFP4 in mlp1, fp6 pieces of h times MXFP4 in mlp2): MXFP4 weights with at least
    128 routed rows per expert on average (its matrix-core tiles)."""
    return cfg.fmt == "mxfp4" and cfg.T * cfg.k >= 128 * cfg.E


def algorithmic(cfg, counts):
    """Algorithmic flops and bytes of one forward, and per-kernel bytes for mlp1/mlp2.

    Bytes count each input once and the output once: touched experts' weights and biases,
    the router, x (bf16) and out (fp32).  Per kernel, mlp1 reads x (bf16; on the scaled
    engine its two fp8 pieces, the same two bytes per element) and writes h, mlp2 reads h
    and writes y (fp32); h is bf16 (bf16 weights), a bf16 pair (MXFP4, few rows) or three
    fp6 pieces (six bits each) and one scale dword per 32 elements (scaled engine); MXFP8
    weights are one
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
        hbytes = A * (3 * F * 6 // 8 + ((F // 32 + 7) // 8 * 8) * 4)
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
    blas = "unknown"
    try:
        from threadpoolctl import threadpool_info
        pools = [p for p in threadpool_info() if p.get("user_api") == "blas"]
        threads = max([p.get("num_threads", 1) for p in pools] or [os.cpu_count() or 1])
        if pools:
            p = pools[0]
            blas = f"{p.get('internal_api', '?')} {p.get('version', '?')} ({p.get('architecture', '?')})"
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
            "cpu_model": cpu_model(), "host_cpus": os.cpu_count(), "blas": blas,
            "sample": f"first {n_tokens} of the {cfg.T} tokens of workload {cfg.name}, float64 forward "
                      f"repeated {reps} times ({dt:.1f} s)"}


def cpu_model():
    """The host CPU's model name (/proc/cpuinfo), or the platform string."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or platform.machine()


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


def bench_workload(name, steps, warmup, with_cpu, library=False):
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
    # at few rows per expert), or the scaled one, which issues each flop once per activation
    # piece (x: 2 fp8 pieces in mlp1, at the fp8 rate; h: 3 fp6 pieces in mlp2, at the FP6/FP4
    # rate)
    mx = mx_engine(cfg)
    peak_t = (FP8_PEAK_TFLOPS if dom == "mlp1" else FP4_PEAK_TFLOPS) if mx else BF16_PEAK_TFLOPS
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
    roof["instruction"] = ((f"v_mfma_scale_f32_32x32x64_f8f6f4 ({'fp8 E4M3' if dom == 'mlp1' else 'fp6 E2M3'} "
                            "activation pieces x MXFP4)") if mx else "v_mfma_f32_32x32x16_bf16")
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
        "dtype": ("fp8xfp4" if dom == "mlp1" else "fp6xfp4") if mx else "bf16",
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
    if library and cfg.fmt == "bf16":
        log(f"[bench] {name}: timing the library grouped GEMM on the same products")
        res["library_comparison"] = library_comparison(cfg, x, w1_0, w2_0, r)
    if with_cpu:
        n_cpu = min(cfg.T, 256 if cfg.E <= 32 else 64)
        log(f"[bench] {name}: timing the CPU oracle on {n_cpu} tokens")
        res["cpu_baseline"] = cpu_baseline(inp, n_cpu)
    del w1s, w2s
    torch.cuda.empty_cache()
    return res


def library_comparison(cfg, x, w1, w2, r, reps=20):
    """The two expert products of one forward run by the library grouped GEMM that torchtitan's
    GPT-OSS MoE calls (torch._grouped_mm, here PyTorch's ROCm build) on this GPU, timed for
    context beside mlp1 and mlp2.  A = x's routed rows (mlp1) and N(0, 1) rows standing in for
    h (mlp2); B = the layer's expert weights transposed to [E][K][N]; each expert's rows padded
    to a multiple of 16, as torchtitan pads them.  The products alone: no gather, SwiGLU, bias,
    gate or combine, which the library leaves to other launches.  Beside them one dense
    torch.mm (hipBLASLt) over the same padded row count with one expert's weights: the vendor
    GEMM's own rate at this shape.  bf16 weights only; rates are algorithmic flops (unpadded
    rows) per second, the dense one over its padded rows."""
    import torch
    E, D, F, k = cfg.E, cfg.D, cfg.F, cfg.k
    dev = x.device
    counts = r["counts"].cpu().numpy().astype(np.int64)
    padded = (counts + 15) // 16 * 16
    M = int(padded.sum())
    ends = np.cumsum(padded)
    offs = torch.tensor(ends, dtype=torch.int32, device=dev)
    # routed rows in the library's padded layout: expert e's rows at [ends[e] - padded[e], ...)
    perm = r["perm"].long()
    dst = torch.cat([torch.arange(int(e0), int(e0) + int(c), device=dev)
                     for e0, c in zip(ends - padded, counts)]) if counts.sum() else torch.empty(0, device=dev)
    a1 = torch.zeros((M, D), dtype=torch.bfloat16, device=dev)
    a1[dst.long()] = x.view(torch.bfloat16)[perm // k]
    a2 = torch.randn((M, F), dtype=torch.bfloat16, device=dev, generator=torch.Generator(device=dev).manual_seed(3))
    b1 = w1.view(torch.bfloat16).view(E, 2 * F, D).transpose(1, 2).contiguous()
    b2 = w2.view(torch.bfloat16).view(E, D, F).transpose(1, 2).contiguous()
    rows = int(counts.sum())
    alg = {"mlp1": 2.0 * rows * D * 2 * F, "mlp2": 2.0 * rows * F * D}
    dense = {"mlp1": 2.0 * M * D * 2 * F, "mlp2": 2.0 * M * F * D}

    def timed(fn):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps / 1e3

    out = {"library": f"torch {torch.__version__} torch._grouped_mm and torch.mm (bf16, fp32 accumulate)",
           "padded_rows": M, "rows": rows}
    try:
        t = {"mlp1": timed(lambda: torch._grouped_mm(a1, b1, offs=offs)),
             "mlp2": timed(lambda: torch._grouped_mm(a2, b2, offs=offs))}
        out["grouped_mm_us"] = {s: round(v * 1e6, 1) for s, v in t.items()}
        out["grouped_mm_tflops"] = {s: round(alg[s] / v / 1e12, 1) for s, v in t.items()}
    except Exception as ex:  # an unsupported library path is reported, not fatal
        out["grouped_mm_error"] = repr(ex)[:200]
    t = {"mlp1": timed(lambda: torch.mm(a1, b1[0])), "mlp2": timed(lambda: torch.mm(a2, b2[0]))}
    out["dense_mm_us"] = {s: round(v * 1e6, 1) for s, v in t.items()}
    out["dense_mm_tflops"] = {s: round(dense[s] / v / 1e12, 1) for s, v in t.items()}
    del a1, a2, b1, b2
    torch.cuda.empty_cache()
    return out


def bench_backward(name, steps, warmup):
    """Time moe_backward (bf16 expert weights) on a workload's layer and routing: the gradient
    of every input and parameter for a seeded output gradient, the routing held fixed.

    Algorithmic work per token (the gradient math, not the recomputation of mlp1's output
    that the backward does instead of keeping it): flops 12 k D F + 4 D E (each forward
    product twice: input and weight gradients); bytes: the touched experts' weights read
    once and their fp32 gradients written once, plus x, dout and dx."""
    import torch
    import mixture_experts_transformer_amd as moe
    from synth import get_config, make_dout, make_inputs

    cfg = get_config(name)
    if cfg.fmt != "bf16":
        raise ValueError("the backward takes bf16 expert weights")
    inp = make_inputs(name)
    dev = torch.device("cuda:0")
    t16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)
    x, wr, br, b1, b2 = t16(inp.x), t16(inp.wr), t16(inp.br), t16(inp.b1), t16(inp.b2)
    w1, w2 = t16(inp.w1), t16(inp.w2)
    dout = torch.from_numpy(make_dout(cfg.T, cfg.D, seed=cfg.seed)).to(dev)
    r = moe.route(x, wr, br, cfg.k, want_logits=False)
    touched = int(np.count_nonzero(r["counts"].cpu().numpy()))
    T, D, E, k, F = cfg.T, cfg.D, cfg.E, cfg.k, cfg.F
    flops = T * (12 * k * D * F + 4 * D * E)
    issued = T * (18 * k * D * F + 4 * D * E)      # + mlp1 recomputed, dout as a bf16 pair
    byts = touched * (3 * D * F * (2 + 4) + 2 * F * (2 + 4) + D * (2 + 4)) + E * D * (2 + 4) + T * D * (2 + 4 + 4)

    def step():
        moe.backward(x, wr, w1, b1, w2, b2, r, dout, k)

    log(f"[bench] {name} backward: warmup {warmup} steps")
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    s = ms / 1e3
    log(f"[bench] {name} backward: {ms * 1e3:.1f} us/step")
    res = {"workload": f"{name}: T={T} D={D} E={E} k={k} F={F} bf16, gradients of x, router, w1, b1, w2, b2",
           "ms_per_step": round(ms, 4), "tokens_per_s": round(T / s, 1),
           "tflops": round(flops / s / 1e12, 2), "mfma_frac": round(flops / s / 1e12 / BF16_PEAK_TFLOPS, 4),
           "issued_mfma_frac": round(issued / s / 1e12 / BF16_PEAK_TFLOPS, 4),
           "hbm_gbs": round(byts / s / 1e9, 1), "hbm_frac": round(byts / s / 1e9 / HBM_PEAK_GBS, 4)}
    del w1, w2
    torch.cuda.empty_cache()
    return res


TARGETS = ("C3", "X1", "X2")     # the other target workloads: bf16 at 8192 tokens, MXFP4 at 256 and 8192


def target_summary(res):
    """The fields of a target workload's measurement that go into the headline line."""
    keep = ("value", "unit", "ms_per_step", "steps", "warmup", "dtype", "step_tflops", "step_mfma_frac",
            "step_fp8_peak_frac", "step_fp4_peak_frac", "step_hbm_gbs", "step_hbm_frac", "kernel_us", "roofline",
            "library_comparison")
    out = {k: res[k] for k in keep if k in res}
    out["workload"] = res["config"]["workload"]
    return out


def mfma_calibration(iters=20000):
    """Sustained v_mfma_f32_32x32x16_bf16 rate of this GPU on operands held in registers (the
    calibration kernel of mixture_experts_transformer_amd/calib): random bf16 operands N(0, 1)
    and constant ones (all 1.0), at one and two waves per SIMD on every CU.  Returns one dict
    per case: TFLOP/s over the launch and its fraction of the 2.5 PF bf16 peak (the clock the
    chip holds under each load, and the matrix cores' busy fraction, come from rocprofv3's
    GRBM_GUI_ACTIVE and SQ_VALU_MFMA_BUSY_CYCLES on the same command)."""
    import ctypes
    import torch
    from mixture_experts_transformer_amd import build as _b
    lib = ctypes.CDLL(_b.CALIB_LIB)
    lib.moe_calib_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p,
                                   ctypes.c_void_p]
    per_iter = lib.moe_calib_products_per_iteration()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    out = []
    for operands in ("random", "constant"):
        for wps in (1, 2):
            blocks = cus * wps
            waves = 4 * blocks
            n = waves * 6 * 64 * 8
            if operands == "random":
                src = torch.randn(n, generator=torch.Generator().manual_seed(5)).to(torch.bfloat16).cuda()
            else:
                src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
            sink = torch.empty(waves * 64, dtype=torch.float32, device="cuda")
            cyc = torch.empty(waves, dtype=torch.int64, device="cuda")
            st = torch.cuda.current_stream().cuda_stream
            run = lambda: lib.moe_calib_mfma(src.data_ptr(), blocks, iters, sink.data_ptr(), cyc.data_ptr(), st)
            if run() != 0:
                raise RuntimeError("calibration kernel launch failed")
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(3):
                run()
            e1.record()
            torch.cuda.synchronize()
            sec = e0.elapsed_time(e1) / 3 / 1e3
            flops = waves * iters * per_iter * 2 * 32 * 32 * 16
            out.append({"calibration": "mfma_bf16_32x32x16", "operands": operands, "waves_per_simd": wps,
                        "tflops": round(flops / sec / 1e12, 1), "frac_of_peak": round(flops / sec / 2.5e15, 4),
                        "ms": round(sec * 1e3, 3)})
    return out


def hbm_calibration(gib=2):
    """Sustained HBM read rate of this GPU: a plain stream of 16-byte loads over a buffer of
    `gib` GiB (the calibration kernel of mixture_experts_transformer_amd/calib), at one to eight
    workgroups of 256 lanes per CU; returns the best rate in GB/s and the sweep."""
    import ctypes
    import torch
    from mixture_experts_transformer_amd import build as _b
    lib = ctypes.CDLL(_b.CALIB_LIB)
    lib.moe_calib_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    n = gib << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    st = torch.cuda.current_stream().cuda_stream
    sweep = {}
    for per_cu in (1, 2, 4, 8):
        blocks = cus * per_cu
        sink = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
        run = lambda: lib.moe_calib_stream(src.data_ptr(), n, blocks, sink.data_ptr(), st)
        if run() != 0:
            raise RuntimeError("stream calibration launch failed")
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            run()
        e1.record()
        torch.cuda.synchronize()
        sweep[per_cu] = round(n * 5 / (e0.elapsed_time(e1) / 1e3) / 1e9, 1)
    return {"read_gbs": max(sweep.values()), "by_workgroups_per_cu": sweep}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="C2", help="C2 (default), C3, C4, C5, X1, X2, Y1, Y2")
    ap.add_argument("--all", action="store_true", help="one line per target workload: C2 C3 X1 X2")
    ap.add_argument("--no-targets", action="store_true",
                    help="time only --workload (by default the C2 line also carries C3, X1 and X2 under 'targets')")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--backward", action="store_true", help="time only moe_backward on --workload (bf16)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 3 plain device copies of MIB MiB (reference for the HBM byte counters)")
    ap.add_argument("--mfma-calibration", action="store_true",
                    help="only measure the sustained bf16 matrix-core rate (random and constant operands)")
    ap.add_argument("--hbm-calibration", action="store_true",
                    help="only measure the sustained HBM read rate (plain 16-byte load stream)")
    ap.add_argument("--library-comparison", action="store_true",
                    help="with a bf16 --workload: also time the same expert products on torch._grouped_mm "
                         "and a dense torch.mm (the default line does this for C2 and C3)")
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
    if args.mfma_calibration:
        for line in mfma_calibration():
            print(json.dumps(line), flush=True)
        return
    if args.hbm_calibration:
        print(json.dumps({"calibration": "hbm_read", **hbm_calibration()}), flush=True)
        return
    if args.backward:
        print(json.dumps(bench_backward(args.workload, args.steps, args.warmup)), flush=True)
        return
    if args.all:
        for i, name in enumerate(["C2", *TARGETS]):
            res = bench_workload(name, args.steps, args.warmup, with_cpu=(not args.no_cpu) and i == 0)
            print(json.dumps(res), flush=True)
        return
    headline = args.workload == "C2" and not args.no_targets
    res = bench_workload(args.workload, args.steps, args.warmup, with_cpu=not args.no_cpu,
                         library=args.library_comparison or headline)
    if headline:
        # the headline workload's line also carries the other target workloads, each timed the
        # same way (own warm-up, K timed steps between synchronisations, then an event pass)
        res["targets"] = {}
        for name in TARGETS:
            res["targets"][name] = target_summary(bench_workload(name, args.steps, args.warmup, with_cpu=False,
                                                                 library=True))
        res["backward"] = {name: bench_backward(name, args.steps, args.warmup) for name in ("C2", "C3")}
        # what the matrix cores sustain on this GPU, the reference for the T = 8192 targets'
        # matrix-core fractions (random operands: the clock drops under load)
        res["mfma_calibration"] = {f"{c['operands']}_{c['waves_per_simd']}wps_tflops": c["tflops"]
                                   for c in mfma_calibration()}
        # and what HBM sustains for a plain read stream: the headline roofline also as a
        # fraction of that measured rate
        hbm = hbm_calibration()
        res["hbm_calibration"] = hbm
        res["roofline"]["frac_of_measured_peak"] = round(res["roofline"]["achieved"] / hbm["read_gbs"], 4)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
