"""Seeded synthetic inputs shared by the oracle-side tests, the GPU tests and the benchmark.

This package draws random tensors and builds the learned-parameter inputs (the RoPE
frequency table and the low-rank bias factors) that the attention operator receives.
It holds none of the attention arithmetic itself: no rotation, no scores, no softmax.
"""

from .generate import (  # noqa: F401
    CONFIGS,
    WorkloadConfig,
    round_bf16,
    qkv,
    omega_schedule,
    theta_table,
    rib_factors,
    make_inputs,
    GatedConfig,
    GATED_CONFIGS,
    block_gate,
    make_gated_inputs,
    cla_params,
    StackConfig,
    STACK_CONFIGS,
    make_stack_layer,
    ModelConfig,
    MODEL_CONFIGS,
    block_params,
    model_params,
    images,
)
