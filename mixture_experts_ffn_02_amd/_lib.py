"""ctypes view of libmoe_lora.so (the C ABI declared in include/moe_lora.h).

Loading fails loudly when the HIP library has not been built: there is no other
implementation of the layer behind this binding.
"""

from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_float, c_int, c_int32, c_size_t, c_void_p

MAX_SLOTS = 8
MAX_RANK = 64
MAX_EXPERTS = 512
MAX_TOPK = 32

OK = 0
ERR_INVALID_ARGUMENT = 1
ERR_UNSUPPORTED = 2
ERR_WORKSPACE_TOO_SMALL = 3
ERR_HIP = 4
ERR_SCRATCH_TOO_SMALL = 5
NOALLOC_SCRATCH_BYTES = 64 << 20

ROUTING_RENORMALIZE = 0
ROUTING_DEEPSEEK_V3 = 1

LIB_NAME = "libmoe_lora.so"
LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), LIB_NAME)

# every symbol include/moe_lora.h declares
EXPORTED = (
    "moe_lora_status_string",
    "moe_lora_version",
    "moe_lora_route_workspace_size",
    "moe_lora_route",
    "moe_lora_permute",
    "moe_lora_forward_workspace_size",
    "moe_lora_forward",
    "moe_lora_forward_noalloc",
    "moe_lora_forward_fp8",
    "moe_lora_pack_weights",
    "moe_lora_pack_weights_fp8",
    "moe_lora_finalize",
)


class Dims(ctypes.Structure):
    _fields_ = [("num_tokens", c_int32), ("hidden", c_int32), ("inter", c_int32),
                ("num_experts", c_int32), ("top_k", c_int32)]


class Grouped(ctypes.Structure):
    _fields_ = [("n_group", c_int32), ("topk_group", c_int32),
                ("routed_scaling_factor", c_float), ("correction_bias", c_void_p)]


class Adapters(ctypes.Structure):
    _fields_ = [("num_slots", c_int32), ("token_slot", c_void_p),
                ("rank", c_int32 * MAX_SLOTS), ("scaling", c_float * MAX_SLOTS),
                ("a_gate_up", c_void_p * MAX_SLOTS), ("b_gate_up", c_void_p * MAX_SLOTS),
                ("a_down", c_void_p * MAX_SLOTS), ("b_down", c_void_p * MAX_SLOTS),
                ("shared_outer", c_int32)]


class Options(ctypes.Structure):
    _fields_ = [("two_stream_max_tokens", c_int32), ("force_path", c_int32),
                ("gate_up_event_begin", c_void_p), ("gate_up_event_end", c_void_p),
                ("packed_weights", c_int32), ("fp8_pow2_scales", c_int32),
                ("reserved", c_int32 * 2)]


class MoELoRAError(RuntimeError):
    def __init__(self, call: str, status: int, text: str):
        super().__init__(f"{call} failed: {text} (status {status})")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library once; raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    # torch first: its bundled HIP runtime then also serves this library (same SONAME),
    # so one runtime owns the streams and allocations both sides use
    import torch  # noqa: F401
    if not os.path.exists(path):
        raise ImportError(
            f"{LIB_NAME} is not built ({path} missing); build it with "
            "`python -c 'import __graft_entry__ as g; g.build()'` -- there is no fallback path")
    lib = ctypes.CDLL(path)
    lib.moe_lora_status_string.restype = ctypes.c_char_p
    lib.moe_lora_status_string.argtypes = [c_int]
    lib.moe_lora_version.restype = c_int
    lib.moe_lora_version.argtypes = []
    lib.moe_lora_route_workspace_size.restype = c_size_t
    lib.moe_lora_route_workspace_size.argtypes = [POINTER(Dims)]
    lib.moe_lora_route.restype = c_int
    lib.moe_lora_route.argtypes = [POINTER(Dims), c_int, POINTER(Grouped), c_void_p, c_void_p,
                                   c_void_p, c_void_p, c_void_p, c_void_p, c_void_p, c_size_t,
                                   c_void_p]
    lib.moe_lora_permute.restype = c_int
    lib.moe_lora_permute.argtypes = [POINTER(Dims), c_void_p, c_void_p, c_void_p, c_void_p]
    lib.moe_lora_forward_workspace_size.restype = c_size_t
    lib.moe_lora_forward_workspace_size.argtypes = [POINTER(Dims), POINTER(Adapters)]
    lib.moe_lora_forward.restype = c_int
    lib.moe_lora_forward.argtypes = [POINTER(Dims), c_void_p, c_void_p, c_void_p, c_void_p,
                                     c_void_p, c_void_p, POINTER(Adapters), c_void_p, c_void_p,
                                     c_size_t, c_void_p, c_void_p, POINTER(Options)]
    lib.moe_lora_forward_noalloc.restype = c_int
    lib.moe_lora_forward_noalloc.argtypes = [POINTER(Dims), c_void_p, c_void_p, c_void_p, c_void_p,
                                             c_void_p, c_void_p, POINTER(Adapters), c_void_p, c_void_p,
                                             POINTER(Options)]
    lib.moe_lora_forward_fp8.restype = c_int
    lib.moe_lora_forward_fp8.argtypes = [POINTER(Dims), c_void_p, c_void_p, c_void_p, c_void_p,
                                         c_void_p, c_void_p, c_void_p, c_void_p, POINTER(Adapters),
                                         c_void_p, c_void_p, c_size_t, c_void_p, c_void_p,
                                         POINTER(Options)]
    lib.moe_lora_pack_weights.restype = c_int
    lib.moe_lora_pack_weights.argtypes = [POINTER(Dims), c_void_p, c_void_p, c_void_p, c_void_p,
                                          c_void_p]
    lib.moe_lora_pack_weights_fp8.restype = c_int
    lib.moe_lora_pack_weights_fp8.argtypes = [POINTER(Dims), c_void_p, c_void_p, c_void_p, c_void_p,
                                              c_void_p]
    lib.moe_lora_finalize.restype = c_int
    lib.moe_lora_finalize.argtypes = [POINTER(Dims), c_void_p, c_void_p, c_void_p, c_void_p,
                                      c_void_p]
    _lib = lib
    return lib


def status_string(code: int) -> str:
    return load().moe_lora_status_string(int(code)).decode()


def check(call: str, code: int) -> None:
    if code != OK:
        raise MoELoRAError(call, code, status_string(code))
