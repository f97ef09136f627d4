"""MI355X-native sparse Mixture-of-Experts layer forward with token-choice
top-k routing: HIP kernels behind the C ABI in include/moe.h, and a thin ctypes
binding (top_routing_dispatch_amd.binding) with the same function names."""
from .binding import (  # noqa: F401
    MoEError, lib, make_config, workspace,
    moe_capacity, moe_workspace_size, moe_route, moe_permute, moe_expert_ffn,
    moe_combine, moe_load_stats, moe_layer_forward, moe_layer_forward_timed, moe_layer_forward_static,
    moe_ep_send_layout, MOE_STATIC_SCRATCH_BYTES, moe_reload_tuning, moe_layer_stages, moe_check_dispatch,
    moe_ep_recv_layout, moe_layer_backward, moe_expert_choice_capacity, moe_expert_choice_forward, STAGES, EXPORTED,
    MOE_OK, MOE_ERR_INVALID_ARGUMENT, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE_TOO_SMALL, MOE_ERR_HIP,
    MOE_ERR_DEBUG_CHECK,
    MOE_F32, MOE_BF16, MOE_SOFTMAX_TOPK, MOE_TOPK_SOFTMAX, MOE_SIGMOID_BIAS, MOE_SWIGLU, MOE_GELU,
    MOE_OP_ROUTE, MOE_OP_PERMUTE, MOE_OP_EXPERT_FFN, MOE_OP_SHARED_FFN, MOE_OP_LOAD_STATS, MOE_OP_LAYER,
    MOE_OP_EXPERT_CHOICE, MOE_OP_LAYER_BACKWARD,
)
