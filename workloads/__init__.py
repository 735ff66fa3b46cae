"""Seeded synthetic inputs for the modal-SSM Hyena operator.

This package is shared by the oracle's tests, the GPU tests and the benchmark.
It only draws and rounds random numbers: it holds none of the operator's
arithmetic (no powers of poles, no products of activations, no scans).
"""

from .configs import CONFIGS, Config, get_config
from .generate import (
    ModalParams,
    bf16_bits_to_f32,
    decode_inputs,
    dense_weights,
    modal_params,
    prompt_inputs,
    round_to_bf16_bits,
    stack_prompt,
)

__all__ = [
    "CONFIGS",
    "Config",
    "get_config",
    "ModalParams",
    "bf16_bits_to_f32",
    "decode_inputs",
    "dense_weights",
    "modal_params",
    "prompt_inputs",
    "round_to_bf16_bits",
    "stack_prompt",
]
