"""Routed Mixture-of-Experts SwiGLU FFN layer (forward + backward) for MI355X.

The computation lives in libmoe.so (hand-written HIP kernels for gfx950 behind
the C ABI of include/moe.h).  This package is its thin binding: ``_lib`` maps
the C calls one to one; ``layer.MoELayer`` owns the buffers of one step.
"""

from ._lib import (  # noqa: F401
    Plan,
    MoeError,
    lib,
    moe_route,
    moe_route_balanced,
    moe_route_sinkhorn,
    moe_route_expert_choice,
    moe_balance_update,
    moe_permute,
    moe_expert_ffn,
    moe_combine,
    moe_backward,
    moe_aux_stats,
    moe_aux_stats_masked,
    decode_aux,
    probe_enable,
    probe_read,
    kernel_names,
    mx_quantize_rows,
    workspace_region,
    keep_intermediates,
    LIB_PATH,
)
from .layer import MoELayer  # noqa: F401
