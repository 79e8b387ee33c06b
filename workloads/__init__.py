"""Seeded synthetic workloads for the MoE-LoRA expert layer.

This package holds the layer shapes and the seeded input generators. It holds
none of the layer's arithmetic: it only draws tensors (and the router logits,
which are an input to the layer) and hands them to whichever side asks, the
CPU oracle or the HIP library.
"""
from .configs import LayerConfig, CONFIGS, PARITY_CONFIGS, BENCH_CONFIG, get_config
from .synth import make_inputs, make_block_inputs, seed_for, expert_histogram

__all__ = [
    "LayerConfig", "CONFIGS", "PARITY_CONFIGS", "BENCH_CONFIG", "get_config",
    "make_inputs", "make_block_inputs", "seed_for", "expert_histogram",
]
