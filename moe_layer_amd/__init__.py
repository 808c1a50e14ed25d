"""MI355X-native (gfx950) MoE-layer forward pass on one GPU's share.

The computation lives in the HIP library ``libmoe_layer_amd.so`` (C ABI in
``include/moe.h``); this package is its thin torch binding.  Importing it
does not load the library; the first call does, and fails loudly if the
library has not been built.
"""
from ._lib import (  # noqa: F401
    EXPORTED, MOE_DTYPE_BF16, MOE_DTYPE_F32, MOE_OP_EXPERT_DOWN, MOE_OP_EXPERT_UP,
    MOE_OP_GROUPED_GEMM, MoeError, abi_version, expert_workspace, lib,
    moe_combine, moe_dispatch, moe_expert_down, moe_expert_up, moe_grouped_gemm, moe_permute,
    moe_repack_ep_to_tp, moe_repack_tp_to_ep, moe_route, moe_route_permute, moe_route_permute_noalloc, moe_route_workspace_bytes,
    moe_workspace_bytes, route_workspace, SwitchPolicy, switch_crossover, MODE_TP, MODE_EP,
    SWITCH_STAY, SWITCH_TO_EP, SWITCH_TO_TP, SWITCH_VETOED, moe_schedule_requests, schedule_workspace,
)
from .layer import MoeLayerBuffers, moe_layer_forward  # noqa: F401
