"""CPU oracle for the GPT-OSS MoE feed-forward block -- TEST INFRASTRUCTURE.

A plain, slow, float64 NumPy statement of what the block computes, used only to
check the GPU library.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the library and its Python
binding never do, and this package imports nothing from them.

Every function here is pinned by ``tests/test_oracle.py`` against brute force,
closed forms, invariants and exact special cases (see that file's docstrings).
"""
from .moe_oracle import (  # noqa: F401
    SWIGLU_ALPHA,
    SWIGLU_LIMIT,
    bf16_to_f64,
    e2m1_value,
    e4m3_value,
    expert_forward,
    expert_weight,
    gate_weights,
    moe_forward,
    mxfp4_decode,
    mxfp8_decode,
    route_assignments,
    router_logits,
    select_experts,
    swiglu,
    update_expert_bias,
)
from .moe_backward import (forward_fixed_routing, moe_backward, moe_backward_grouped,  # noqa: F401,E402
                           swiglu_backward)
