"""Seeded synthetic workloads for the MoE expert-layer forward pass.

This package holds only shapes and random inputs: it computes none of the
layer's arithmetic, so both the CPU oracle and the HIP path can take their
inputs from it without sharing any of the method.
"""
from .configs import CONFIGS, LayerConfig, get_config, valid_mask, midpoint_split, boundary_split
from .gen import make_inputs, LayerInputs

__all__ = [
    "CONFIGS", "LayerConfig", "get_config", "valid_mask", "midpoint_split",
    "boundary_split", "make_inputs", "LayerInputs",
]
