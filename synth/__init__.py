"""Seeded synthetic inputs for the routed MoE layer over block-quantized experts.

This module draws the inputs only: router logits (or the router matrix and
bias), activations and the packed expert planes. It holds none of the layer's
arithmetic (no router product, no routing, no dequantisation, no FFN), so both
the CPU oracle and the HIP path can consume its output without sharing any of
the method's code.
"""
from .configs import CONFIGS, LayerConfig, get_config
from .gen import (
    make_layer, make_logits, make_router, make_x, make_expert_planes, plane_sizes,
    zipf_bias, f32_to_bf16_bits, bf16_bits_to_f32,
)

__all__ = [
    "CONFIGS", "LayerConfig", "get_config", "make_layer", "make_logits", "make_router",
    "make_x", "make_expert_planes", "plane_sizes", "zipf_bias",
    "f32_to_bf16_bits", "bf16_bits_to_f32",
]
