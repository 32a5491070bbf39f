"""Seeded synthetic inputs for the GPT-OSS MoE feed-forward block.

This package is shared by the CPU oracle (``oracle/``) and by the GPU path's
tests and benchmark.  It holds only input synthesis -- random draws, the bf16
and MXFP4 *encodings* of those draws, and the routing-load targets -- and none
of the block's own arithmetic (no router product, no top-k, no expert MLP).
"""
from .configs import CONFIGS, Config, get_config  # noqa: F401
from .generate import (  # noqa: F401
    MoEInputs,
    make_dout,
    f32_to_bf16_bits,
    make_expert_bias,
    make_inputs,
    make_router_inputs,
    make_routing_inputs,
    zipf_plan,
    router_bias_path,
)
