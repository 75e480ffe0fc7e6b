"""Seeded synthetic inputs shared by the oracle-side tests and the GPU side.

This package holds random-number generation and storage-format conversion
only; none of the attention method's arithmetic lives here.
"""
from .inputs import (  # noqa: F401
    CONFIGS,
    BridgeInputs,
    audio_tokens_for,
    make_bridge_inputs,
    ConfigInputs,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    iid_normal,
    make_inputs,
    make_upstream_grad,
)
