"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This package holds no arithmetic of the attention method: it only draws
random numbers, rounds them to the storage dtype and lays them out.
"""
from .inputs import (  # noqa: F401
    CONFIGS,
    GATE_MODES,
    config_prefill_inputs,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    round_to_bf16,
    prefill_inputs,
    decode_initial,
    decode_step_inputs,
    grad_output,
)
