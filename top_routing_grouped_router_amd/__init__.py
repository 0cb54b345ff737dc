"""MI355X (gfx950) hot path of one Mixture-of-Experts layer.

The computation lives in libmoe.so (hand-written HIP kernels behind the C ABI
of include/moe.h); this package holds its sources (csrc/), the build step
(build.py), a ctypes binding with the same names as the C entry points
(_lib.py) and the layer's call sequence (layer.py).
"""
from ._lib import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    MOE_BF16,
    MOE_F32,
    MoEError,
    alloc_workspace,
    lib,
    make_dims,
    moe_capacity,
    moe_check_placement,
    moe_combine,
    moe_combine_bwd,
    moe_coselect,
    moe_coselect_cross,
    moe_dispatch_expand,
    moe_dispatch_pack,
    moe_dispatch_plan,
    moe_expert_dgrad_down,
    moe_expert_dgrad_up,
    moe_expert_capacity,
    moe_expert_down,
    moe_expert_up,
    moe_expert_up_gather,
    moe_expert_wgrad,
    moe_expert_wgrad_gather,
    moe_grouped_swiglu_bwd,
    moe_grouped_swiglu_bwd_gather,
    moe_grouped_swiglu_fwd,
    moe_grouped_swiglu_fwd_gather,
    moe_permute,
    moe_placement_greedy,
    moe_route,
    moe_route_bwd,
    moe_route_bwd_dense,
    moe_route_flips,
    moe_router_zloss,
    moe_shuffle_plan,
    workspace_bytes,
)
from .layer import MoELayer  # noqa: F401
