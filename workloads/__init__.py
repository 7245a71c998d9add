"""Seeded synthetic inputs for the W4 g128 MoE layer.

This package draws random inputs only: activations, router weights and
biases, fp16 master weights, and (for full-size runs) packed int4 codes with
fp16 scales drawn directly.  It holds none of the layer's arithmetic, so both
the HIP library's tests/benchmark and the CPU oracle can take their inputs
from it.
"""
from .configs import CONFIGS, MoEConfig, get_config  # noqa: F401
