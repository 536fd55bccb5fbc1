"""MI355X-native (gfx950) routed MoE-LoRA expert layer.

The compute lives in libmoe_lora.so (hand-written HIP kernels behind the C ABI of
include/moe_lora.h); this package only builds that library and marshals torch
tensors into its calls.
"""

from ._lib import (  # noqa: F401
    ERR_HIP,
    ERR_INVALID_ARGUMENT,
    ERR_UNSUPPORTED,
    ERR_WORKSPACE_TOO_SMALL,
    EXPORTED,
    LIB_PATH,
    MAX_RANK,
    MAX_SLOTS,
    OK,
    ROUTING_DEEPSEEK_V3,
    ROUTING_RENORMALIZE,
    Adapters,
    Dims,
    Grouped,
    MoELoRAError,
    Options,
    load,
)
