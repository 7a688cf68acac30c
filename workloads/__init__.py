"""Seeded synthetic inputs for the attention workloads.

This module only draws and lays out inputs: it holds none of the attention
arithmetic, and both the HIP library's tests/bench and the oracle consume what
it returns.  See ``generators`` for the recipes.
"""

from .generators import (  # noqa: F401
    WORKLOADS,
    PrefillWorkload,
    DecodeWorkload,
    ChunkedPrefillWorkload,
    chunked_prefill_inputs,
    f32_to_bf16_bits,
    f32_to_e4m3_bits,
    quantize_e4m3,
    bf16_bits_to_f32,
    prefill_inputs,
    decode_inputs,
    decode_inputs_fp8,
    BF16_NAN,
)
