"""fp64 CPU oracle for the routed MoE SwiGLU feed-forward layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with
the HIP library (no kernels, headers, helpers, tables or pre/post-processing);
both sides receive the same seeded inputs and nothing else.

Every floating-point step here is computed in float64 with numpy, from the
device-rounded inputs upcast exactly to float64.  By default nothing in
between is rounded (the exact layer); ``layer_forward`` / ``layer_backward``
take an optional ``store`` rounding that is applied only to the values the
layer keeps in its storage dtype (the bf16 / f16 layer of the pages).
The per-expert steps the layer passes are made of (``expert_*_step``,
``router_backward``) are exposed too, so a test can run one step of the
oracle on the inputs a GPU step received.
"""

from .moe_oracle import (  # noqa: F401
    router_logits,
    softmax_rows,
    topk_select,
    gate_weights,
    balanced_selection_scores,
    sinkhorn_column_scales,
    sinkhorn_selection_scores,
    relu_gates,
    relu_select,
    relu_gate_weights,
    expert_choice_select,
    balance_bias_update,
    near_tie_tokens,
    expert_permutation,
    silu,
    swiglu_rows,
    shared_experts_forward,
    combine,
    expert_gate_up_step,
    expert_down_step,
    expert_down_backward_step,
    expert_gate_up_backward_step,
    router_backward,
    aux_statistics,
    real_token_counts,
    layer_forward,
    layer_backward,
    layer_loss,
)
from .mx import mx_fake_quant, e4m3_round, mx_block_scale  # noqa: F401
from .rounding import round_to_format  # noqa: F401
