"""GPT-OSS mixture-of-experts feed-forward block on AMD Instinct MI355X (gfx950).

The compute lives in ``libmoe.so`` (hand-written HIP kernels behind the C ABI of
``include/moe.h``); ``moe`` is its ctypes binding.
"""
from .moe import (  # noqa: F401
    FMT,
    LIB_PATH,
    STAGES,
    MoEError,
    backward,
    backward_workspace_bytes,
    experts,
    forward,
    forward_noalloc,
    lib,
    mxfp4_bytes,
    mxfp8_bytes,
    profile_enable,
    profile_read,
    release,
    route,
    set_workspace,
    update_expert_bias,
    version,
    workspace_bytes,
)
