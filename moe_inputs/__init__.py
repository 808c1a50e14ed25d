"""Seeded synthetic inputs for one MoE layer's forward pass.

This package is the only code that the CPU oracle and the GPU path share.  It
draws random numbers and lays them out as host arrays; it holds none of the
layer's arithmetic (no gate product, softmax, top-k, permutation, expert FFN,
combine or repack).
"""
from .configs import CONFIGS, LayerConfig, get_config
from .gen import (
    bf16_bits_from_f32,
    ep_rank_for,
    make_layer_inputs,
    make_repack_inputs,
    make_full_model,
)

__all__ = [
    "CONFIGS",
    "LayerConfig",
    "get_config",
    "bf16_bits_from_f32",
    "ep_rank_for",
    "make_layer_inputs",
    "make_repack_inputs",
    "make_full_model",
]
