"""Seeded synthetic inputs for the vertical-slash attention path.

This package is the only code shared by the oracle and the HIP path. It draws
random tensors and applies rotary position embedding (the model's own input
transform); it contains none of the sparse-attention method's arithmetic.
"""
from .inputs import (  # noqa: F401
    WorkloadConfig, CONFIGS, config_by_name, generate, layout_permutation,
    bf16_bits_from_f32, f32_from_bf16_bits, round_to_dtype,
)
