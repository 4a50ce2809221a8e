"""Seeded synthetic inputs for the layer-end KV-eviction compressor.

This package only draws random tensors and rounds them to bf16. It holds none
of the compressor's arithmetic (no logits, softmax, pooling, selection or
gather), so both the CPU oracle and the HIP path can consume its output
without sharing any of the method's code.
"""
from .configs import LayerConfig, CONFIGS, get_config
from .gen import (
    LayerInputs,
    layer_inputs,
    layer_seed,
    f32_to_bf16_bits,
    bf16_bits_to_f32,
    chunk_windows,
    SynthLayerWeights,
    model_weights,
    prompt_hidden,
)

__all__ = [
    "LayerConfig",
    "CONFIGS",
    "get_config",
    "LayerInputs",
    "layer_inputs",
    "layer_seed",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "chunk_windows",
    "SynthLayerWeights",
    "model_weights",
    "prompt_hidden",
]
