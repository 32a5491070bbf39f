"""Workload table for the GPT-OSS MoE block.

Shapes follow the GPT-OSS-20B MoE layer: hidden size 2880, 32 experts, top-4
routing (kexuegongju.com "gptoss" re-implementation page, section "basic
parameters").  The intermediate size F = 2880 and the wider 128-expert layer
are the synthetic layer sizes of this benchmark, not numbers the pages print.

Symbols: T tokens, D hidden, E experts, k experts per token, F intermediate
(mlp1 produces G = 2F values: the gate half then the linear half).
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Config:
    name: str
    T: int
    D: int
    E: int
    k: int
    F: int
    fmt: str                      # "bf16", "mxfp4" or "mxfp8" (expert weights)
    seed: int
    x_dist: str                   # "normal" (fp32 N(0,1)) or "rmsnorm" (N(0,1) then RMSNorm)
    router_bias: str              # "zero", "normal" (N(0,0.01)) or "zipf" (calibrated to a Zipf load)
    zipf_s: float = 0.0
    n_empty: int = 0              # experts forced to receive no token (zipf configs only)
    weight_std: float = 0.02      # bf16 weights N(0, weight_std)
    bias_std: float = 0.01        # expert biases N(0, bias_std)
    scale_exp: Tuple[int, int] = (-8, -4)  # MXFP4/MXFP8: E8M0 exponent drawn uniformly in this closed range
    note: str = ""

    @property
    def A(self) -> int:
        return self.T * self.k

    @property
    def G(self) -> int:
        return 2 * self.F

    def flops(self) -> float:
        """Algorithmic flops of one forward: router 2TDE + mlp1 4AD F + mlp2 2AFD."""
        return float(self.T) * (2 * self.D * self.E + 6 * self.k * self.D * self.F)


CONFIGS = {
    "C1": Config("C1", T=64, D=64, E=4, k=2, F=128, fmt="bf16", seed=1,
                 x_dist="normal", router_bias="zero",
                 note="tiny layer the oracle finishes in milliseconds"),
    "C2": Config("C2", T=256, D=2880, E=32, k=4, F=2880, fmt="bf16", seed=2,
                 x_dist="rmsnorm", router_bias="normal",
                 note="20B shape, decode-like batch, uniform-ish routing"),
    "C3": Config("C3", T=8192, D=2880, E=32, k=4, F=2880, fmt="bf16", seed=3,
                 x_dist="rmsnorm", router_bias="zipf", zipf_s=1.1,
                 note="20B shape, prefill size, Zipf(1.1) expert load"),
    "C4": Config("C4", T=4096, D=2880, E=32, k=4, F=2880, fmt="mxfp4", seed=4,
                 x_dist="rmsnorm", router_bias="normal",
                 note="20B shape, MXFP4 expert weights"),
    "C5": Config("C5", T=16384, D=2880, E=128, k=4, F=2880, fmt="mxfp4", seed=5,
                 x_dist="rmsnorm", router_bias="zipf", zipf_s=1.2, n_empty=13,
                 note="128 experts, MXFP4, Zipf(1.2) load, 13 empty experts"),
    "X1": Config("X1", T=256, D=2880, E=32, k=4, F=2880, fmt="mxfp4", seed=6,
                 x_dist="rmsnorm", router_bias="normal",
                 note="MXFP4 at the decode-like batch"),
    "X2": Config("X2", T=8192, D=2880, E=32, k=4, F=2880, fmt="mxfp4", seed=7,
                 x_dist="rmsnorm", router_bias="normal",
                 note="MXFP4 at prefill size"),
    # MXFP8 expert weights (E4M3 codes uniform over the 254 finite ones, RMS ~100, so the
    # scales sit lower: RMS 0.012 .. 0.1 per block, like the MXFP4 workloads' weights)
    "Y1": Config("Y1", T=256, D=2880, E=32, k=4, F=2880, fmt="mxfp8", seed=8,
                 x_dist="rmsnorm", router_bias="normal", scale_exp=(-13, -10),
                 note="MXFP8 at the decode-like batch"),
    "Y2": Config("Y2", T=8192, D=2880, E=32, k=4, F=2880, fmt="mxfp8", seed=9,
                 x_dist="rmsnorm", router_bias="normal", scale_exp=(-13, -10),
                 note="MXFP8 at prefill size"),
}


def get_config(base_name: str, **overrides) -> Config:
    """Look up a named workload; keyword overrides give a variant (e.g. T=..., name=...)."""
    base = CONFIGS[base_name]
    if not overrides:
        return base
    d = dict(base.__dict__)
    d.update(overrides)
    return Config(**d)
