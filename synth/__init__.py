"""Seeded synthetic inputs for the block-sparse mixed-precision attention path.

This package only makes test and benchmark inputs: bf16 tensors, outlier channel
indices and per-head (hi, keep) boundary draws. It holds none of the attention
method's arithmetic, and it is the one module that both the CPU oracle's callers
and the GPU path's callers use.
"""
from .gen import (  # noqa: F401
    CONFIGS,
    Config,
    bf16_bits_to_float32,
    float32_to_bf16_bits,
    normal_bf16,
    outlier_channels,
    policy_draws,
    uniform_u64,
    make_prefill_inputs,
    make_decode_inputs,
    make_skip_decode_inputs,
    apply_block_structure,
)
