"""CPU oracle (float64, materialised scores) for fused shifted-window attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, by __graft_entry__.smoke() and by the
CPU-baseline leg of bench.py, never by the HIP library or its binding.
"""

from .wattn_oracle import (  # noqa: F401
    local_coords,
    window_token_coords,
    region_label,
    shift_mask,
    rope_angles,
    rope_rotate,
    window_logits,
    softmax_rows,
    window_weights,
    window_head_output,
    window_attention,
    unmasked_pairs,
    window_attention_lse,
    window_attention_backward,
)
from .hsmla_oracle import (  # noqa: F401
    select_blocks,
    block_origin,
    relu_linear_attention,
    softmax_attention,
    local_residual_window,
    window_tokens,
    local_residual,
    gated_local_path,
    global_linear_attention,
)
from .cla_oracle import (  # noqa: F401
    sigmoid,
    depthwise3x3,
    pointwise,
    cla_gate_logits,
    gated_window_attention,
    gated_window_attention_backward,
    cyclic_schedule,
)
from .model_oracle import (  # noqa: F401
    layernorm,
    linear,
    gelu,
    stem_conv,
    patch_merge,
    swin_block,
    stage_window,
    flashswin_forward,
)
