"""MI355X (gfx950) Mixture-of-Experts forward path.

The computation -- router scores (optional), router top-k, reorder onto
experts, fused gate/up SwiGLU grouped GEMM, down grouped GEMM, weighted
combination -- runs in the HIP kernels of ``libmoe.so`` behind the C ABI of include/moe.h.  This package is
a thin ctypes binding over it plus the seeded synthetic-input generators
(``expert_dispatch_router_amd.synth``).
"""
from ._lib import (  # noqa: F401
    LIB_PATH,
    MOE_SCORE_SIGMOID,
    MOE_SCORE_SOFTMAX,
    MOE_STATIC_WORKSPACE_BYTES,
    SIGNATURES,
    MoeError,
    MoeOptions,
    Timer,
    lib,
    moe_abi_version,
    moe_forward,
    moe_forward_router,
    moe_forward_static,
    moe_plan,
    moe_plan_ex,
    moe_route,
    moe_route_workspace_size,
    moe_router_logits,
    moe_router_workspace_size,
    moe_workspace_size,
    status_string,
)

forward = moe_forward
route = moe_route
