"""Seeded synthetic inputs for the routed MoE-LoRA layer.

This package only draws random numbers and rounds them to bf16 bit patterns.
It holds none of the layer's arithmetic (no routing, no GEMMs, no SwiGLU), so
both the fp64 oracle tests and the HIP path can consume the same inputs.
"""

from .workloads import (  # noqa: F401
    LayerConfig,
    SlotSpec,
    Workload,
    NAMED_CONFIGS,
    f32_to_bf16_bits,
    make_config,
)
