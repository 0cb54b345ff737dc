"""Seeded synthetic inputs for the MoE-layer hot path.

This package is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It holds the workload shapes and the random-number recipes only:
no step of the MoE layer's arithmetic lives here.
"""
from .configs import CONFIGS, Config, get_config
from .generate import (
    bf16_round,
    bf16_bits,
    bf16_from_bits,
    make_layer_inputs,
    make_routing,
    stream,
)

__all__ = [
    "CONFIGS",
    "Config",
    "get_config",
    "bf16_round",
    "bf16_bits",
    "bf16_from_bits",
    "make_layer_inputs",
    "make_routing",
    "stream",
]
