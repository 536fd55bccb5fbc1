"""fp64 CPU oracle for the routed MoE-LoRA expert layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.
The product path (the HIP library and its Python binding) never imports it, and
this package imports nothing from the product path.
"""

from .moe_lora_ref import (  # noqa: F401
    Adapter,
    bf16_bits_to_f64,
    e4m3_to_f64,
    expert_sort,
    finalize,
    forward_permuted,
    fp8_block_weights,
    layer,
    layer_sampled,
    permute_rows,
    route,
    route_deepseek_v3,
    route_renormalize,
    shared_outer_adapter,
    silu,
)
