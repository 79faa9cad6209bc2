"""libmoe: the routed mixture-of-experts block forward on AMD Instinct MI355X.

The compute lives in ``libmoe.so`` (hand-written HIP for gfx950, C ABI in
``include/moe.h``); ``binding`` is its ctypes binding."""
from .binding import (  # noqa: F401
    ACT_SILU, ACT_SITU, CALL_BLOCK, CALL_COMBINE, CALL_DOWN, CALL_GATE_UP, CALL_LATENT,
    CALL_PERMUTE, CALL_ROUTE, CALL_SHARED, DTYPE_BF16, DTYPE_F32, MoeError, Weights, make_config,
    moe_block_forward, moe_combine, moe_expert_down, moe_expert_down_scatter, moe_expert_gate_up,
    moe_expert_gate_up_gather, moe_latent_project, moe_permute, moe_permute_static, moe_route, moe_shared_expert,
    moe_validate_config, moe_workspace_size, status_str, workspace)
