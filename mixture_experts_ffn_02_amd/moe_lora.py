"""Thin torch-facing binding of the four C calls (argument marshalling only).

PyTorch provides device memory and streams; every step of the layer runs in the HIP
kernels of libmoe_lora.so.  Tensors are passed by data pointer: bf16 tensors may be
``torch.bfloat16`` or 16-bit integer views of the same bits.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass, field
from typing import Optional, Sequence

import torch

from . import _lib
from ._lib import Adapters, Dims, Grouped, MoELoRAError, Options, check, load  # noqa: F401

ROUTING_RENORMALIZE = _lib.ROUTING_RENORMALIZE
ROUTING_DEEPSEEK_V3 = _lib.ROUTING_DEEPSEEK_V3
# moe_lora_options.packed_weights bits
PACKED_GATE_UP = 1
PACKED_DOWN = 2


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to the MoE-LoRA library must be contiguous")
    return t.data_ptr()


def _stream(s) -> Optional[int]:
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, torch.cuda.Stream):
        return s.cuda_stream
    return int(s)


def dims(num_tokens: int, hidden: int, inter: int, num_experts: int, top_k: int) -> Dims:
    return Dims(num_tokens, hidden, inter, num_experts, top_k)


@dataclass
class LoRASlots:
    """Resident adapter slots (per-slot compact weights, device tensors).

    shared_outer: the shared-outer layout, where a_gate_up[s] is [r, H] and b_down[s] is
    [H, r], one set used by every expert (b_gate_up and a_down stay per expert).
    """

    token_slot: torch.Tensor  # [T] int32
    rank: Sequence[int]
    scaling: Sequence[float]
    a_gate_up: Sequence[torch.Tensor]  # [E, r, H]  (shared-outer: [r, H])
    b_gate_up: Sequence[torch.Tensor]  # [E, 2I, r]
    a_down: Sequence[torch.Tensor]     # [E, r, I]
    b_down: Sequence[torch.Tensor]     # [E, H, r]  (shared-outer: [H, r])
    shared_outer: bool = False

    def to_c(self) -> Adapters:
        n = len(self.rank)
        if n > _lib.MAX_SLOTS:
            raise ValueError("too many adapter slots")
        a = Adapters()
        a.num_slots = n
        a.token_slot = _ptr(self.token_slot)
        a.shared_outer = 1 if self.shared_outer else 0
        for s in range(n):
            a.rank[s] = int(self.rank[s])
            a.scaling[s] = float(self.scaling[s])
            a.a_gate_up[s] = _ptr(self.a_gate_up[s])
            a.b_gate_up[s] = _ptr(self.b_gate_up[s])
            a.a_down[s] = _ptr(self.a_down[s])
            a.b_down[s] = _ptr(self.b_down[s])
        return a


def moe_lora_route_workspace_size(d: Dims) -> int:
    return int(load().moe_lora_route_workspace_size(ctypes.byref(d)))


def moe_lora_forward_workspace_size(d: Dims, lora: Optional[Adapters]) -> int:
    return int(load().moe_lora_forward_workspace_size(ctypes.byref(d),
                                                       ctypes.byref(lora) if lora else None))


def moe_lora_route(d: Dims, logits, topk_ids, topk_weights, expert_offsets, e2p, p2e, ws,
                   routing: int = ROUTING_RENORMALIZE, grouped: Optional[Grouped] = None,
                   stream=None) -> None:
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    check("moe_lora_route", load().moe_lora_route(
        ctypes.byref(d), int(routing), ctypes.byref(grouped) if grouped is not None else None,
        _ptr(logits), _ptr(topk_ids), _ptr(topk_weights), _ptr(expert_offsets), _ptr(e2p),
        _ptr(p2e), _ptr(ws), ws_bytes, _stream(stream)))


def moe_lora_permute(d: Dims, x, p2e, x_perm, stream=None) -> None:
    check("moe_lora_permute", load().moe_lora_permute(
        ctypes.byref(d), _ptr(x), _ptr(p2e), _ptr(x_perm), _stream(stream)))


def moe_lora_forward(d: Dims, x, x_perm, expert_offsets, p2e, w_gate_up, w_down,
                     lora: Optional[Adapters], y_perm, ws, main=None, side=None,
                     opts: Optional[Options] = None) -> None:
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    check("moe_lora_forward", load().moe_lora_forward(
        ctypes.byref(d), _ptr(x), _ptr(x_perm), _ptr(expert_offsets), _ptr(p2e), _ptr(w_gate_up),
        _ptr(w_down), ctypes.byref(lora) if lora is not None else None, _ptr(y_perm), _ptr(ws),
        ws_bytes, _stream(main), None if side is None else _stream(side),
        ctypes.byref(opts) if opts is not None else None))


def moe_lora_forward_noalloc(d: Dims, x, x_perm, expert_offsets, p2e, w_gate_up, w_down,
                             lora: Optional[Adapters], y_perm, main=None,
                             opts: Optional[Options] = None) -> None:
    check("moe_lora_forward_noalloc", load().moe_lora_forward_noalloc(
        ctypes.byref(d), _ptr(x), _ptr(x_perm), _ptr(expert_offsets), _ptr(p2e), _ptr(w_gate_up),
        _ptr(w_down), ctypes.byref(lora) if lora is not None else None, _ptr(y_perm), _stream(main),
        ctypes.byref(opts) if opts is not None else None))


def moe_lora_forward_fp8(d: Dims, x, x_perm, expert_offsets, p2e, w_gate_up, w_gate_up_scale, w_down,
                         w_down_scale, lora: Optional[Adapters], y_perm, ws, main=None, side=None,
                         opts: Optional[Options] = None) -> None:
    ws_bytes = ws.numel() * ws.element_size() if ws is not None else 0
    check("moe_lora_forward_fp8", load().moe_lora_forward_fp8(
        ctypes.byref(d), _ptr(x), _ptr(x_perm), _ptr(expert_offsets), _ptr(p2e), _ptr(w_gate_up),
        _ptr(w_gate_up_scale), _ptr(w_down), _ptr(w_down_scale),
        ctypes.byref(lora) if lora is not None else None, _ptr(y_perm), _ptr(ws), ws_bytes,
        _stream(main), None if side is None else _stream(side),
        ctypes.byref(opts) if opts is not None else None))


def moe_lora_pack_weights(d: Dims, w_gate_up, w_down, w_gate_up_packed, w_down_packed,
                          stream=None) -> None:
    check("moe_lora_pack_weights", load().moe_lora_pack_weights(
        ctypes.byref(d), _ptr(w_gate_up), _ptr(w_down), _ptr(w_gate_up_packed), _ptr(w_down_packed),
        _stream(stream)))


def moe_lora_pack_weights_fp8(d: Dims, w_gate_up, w_down, w_gate_up_packed, w_down_packed,
                              stream=None) -> None:
    check("moe_lora_pack_weights_fp8", load().moe_lora_pack_weights_fp8(
        ctypes.byref(d), _ptr(w_gate_up), _ptr(w_down), _ptr(w_gate_up_packed), _ptr(w_down_packed),
        _stream(stream)))


def moe_lora_finalize(d: Dims, y_perm, topk_weights, e2p, out, stream=None) -> None:
    check("moe_lora_finalize", load().moe_lora_finalize(
        ctypes.byref(d), _ptr(y_perm), _ptr(topk_weights), _ptr(e2p), _ptr(out), _stream(stream)))


@dataclass
class RouteOut:
    topk_ids: torch.Tensor
    topk_weights: torch.Tensor
    expert_offsets: torch.Tensor
    e2p: torch.Tensor
    p2e: torch.Tensor


class MoELoRALayer:
    """The routed MoE-LoRA layer on one GPU: route -> permute -> forward -> finalize.

    Buffers (routing outputs, workspaces, intermediates) are allocated once per token
    count and reused, so repeated calls at one shape allocate nothing.  packed_weights
    (PACKED_GATE_UP | PACKED_DOWN bits; True = both) makes the layer keep tile-packed
    copies of those expert weights (written once by moe_lora_pack_weights) and run the
    GEMMs on them; weights_prepacked gives the bits of the weights that are passed in
    already packed.  With w_gate_up_scale / w_down_scale the expert weights are FP8: uint8
    E4M3 codes [E, 2I, H] / [E, H, I] with fp32 scales per 128 x 128 block, run through
    moe_lora_forward_fp8 (packed_weights / weights_prepacked then refer to the FP8
    tile-packed layout of moe_lora_pack_weights_fp8).
    """

    def __init__(self, hidden: int, inter: int, num_experts: int, top_k: int,
                 w_gate_up: torch.Tensor, w_down: torch.Tensor,
                 routing: int = ROUTING_RENORMALIZE, n_group: int = 1, topk_group: int = 1,
                 routed_scaling_factor: float = 1.0, correction_bias: Optional[torch.Tensor] = None,
                 gather_on_load: bool = True, packed_weights=0, weights_prepacked=0,
                 w_gate_up_scale: Optional[torch.Tensor] = None, w_down_scale: Optional[torch.Tensor] = None,
                 fp8_pow2_scales: bool = False):
        load()
        self.w_scales = None
        if (w_gate_up_scale is None) != (w_down_scale is None):
            raise ValueError("FP8 weights need both block-scale tensors")
        if w_gate_up_scale is not None:
            self.w_scales = (w_gate_up_scale, w_down_scale)
        self.fp8_pow2_scales = bool(fp8_pow2_scales) and self.w_scales is not None
        self.H, self.I, self.E, self.k = hidden, inter, num_experts, top_k
        both = PACKED_GATE_UP | PACKED_DOWN
        to_pack = both if packed_weights is True else int(packed_weights)
        pre = both if weights_prepacked is True else int(weights_prepacked)
        if (to_pack | pre) & ~both:
            raise ValueError("packed_weights / weights_prepacked take PACKED_GATE_UP | PACKED_DOWN bits")
        to_pack &= ~pre
        if to_pack:
            w1p = torch.empty_like(w_gate_up) if to_pack & PACKED_GATE_UP else None
            w2p = torch.empty_like(w_down) if to_pack & PACKED_DOWN else None
            pack = moe_lora_pack_weights_fp8 if self.w_scales is not None else moe_lora_pack_weights
            pack(self.dims(0), w_gate_up if w1p is not None else None, w_down if w2p is not None else None,
                 w1p, w2p)
            w_gate_up = w1p if w1p is not None else w_gate_up
            w_down = w2p if w2p is not None else w_down
        self.packed_weights = to_pack | pre
        self.w_gate_up, self.w_down = w_gate_up, w_down
        self.routing = routing
        self.correction_bias = correction_bias
        self.grouped = None
        if routing == ROUTING_DEEPSEEK_V3:
            self.grouped = Grouped(n_group, topk_group, routed_scaling_factor,
                                   _ptr(correction_bias) if correction_bias is not None else None)
        self.gather_on_load = gather_on_load
        self._bufs = {}

    def dims(self, T: int) -> Dims:
        return Dims(T, self.H, self.I, self.E, self.k)

    def _buffers(self, T: int, lora: Optional[Adapters], device) -> dict:
        key = (T, None if lora is None else tuple(lora.rank[: lora.num_slots]))
        b = self._bufs.get(key)
        if b is None:
            d = self.dims(T)
            R = T * self.k
            i32 = dict(dtype=torch.int32, device=device)
            b = {
                "ids": torch.empty((T, self.k), **i32),
                "w": torch.empty((T, self.k), dtype=torch.float32, device=device),
                "off": torch.empty((self.E + 1,), **i32),
                "e2p": torch.empty((R,), **i32),
                "p2e": torch.empty((R,), **i32),
                # per-workgroup expert histograms of the two-launch routing (written before read)
                "rws": torch.empty((max(1, moe_lora_route_workspace_size(d)),), dtype=torch.uint8,
                                   device=device),
                "fws": torch.empty((max(1, moe_lora_forward_workspace_size(d, lora)),),
                                   dtype=torch.uint8, device=device),
                "x_perm": None if self.gather_on_load else torch.empty((R, self.H), dtype=torch.bfloat16,
                                                                       device=device),
                "y": torch.empty((R, self.H), dtype=torch.bfloat16, device=device),
                "out": torch.empty((T, self.H), dtype=torch.bfloat16, device=device),
            }
            self._bufs[key] = b
        return b

    def __call__(self, x: torch.Tensor, logits: torch.Tensor, lora: Optional[LoRASlots] = None,
                 side_stream=None, opts: Optional[Options] = None, stream=None) -> torch.Tensor:
        T = x.shape[0]
        c_lora = lora.to_c() if lora is not None else None
        b = self._buffers(T, c_lora, x.device)
        d = self.dims(T)
        moe_lora_route(d, logits, b["ids"], b["w"], b["off"], b["e2p"], b["p2e"], b["rws"],
                       self.routing, self.grouped, stream)
        if not self.gather_on_load:
            moe_lora_permute(d, x, b["p2e"], b["x_perm"], stream)
        if self.packed_weights or self.fp8_pow2_scales:
            o = Options()
            if opts is not None:
                ctypes.memmove(ctypes.byref(o), ctypes.byref(opts), ctypes.sizeof(Options))
            o.packed_weights = self.packed_weights
            o.fp8_pow2_scales = int(self.fp8_pow2_scales)
            opts = o
        if self.w_scales is not None:
            moe_lora_forward_fp8(d, x, b["x_perm"], b["off"], b["p2e"], self.w_gate_up, self.w_scales[0],
                                 self.w_down, self.w_scales[1], c_lora, b["y"], b["fws"], stream,
                                 side_stream, opts)
        else:
            moe_lora_forward(d, x, b["x_perm"], b["off"], b["p2e"], self.w_gate_up, self.w_down,
                             c_lora, b["y"], b["fws"], stream, side_stream, opts)
        moe_lora_finalize(d, b["y"], b["w"], b["e2p"], b["out"], stream)
        return b["out"]

    def last_route(self, T: int, lora: Optional[LoRASlots] = None) -> RouteOut:
        b = self._buffers(T, lora.to_c() if lora is not None else None, None)
        return RouteOut(b["ids"], b["w"], b["off"], b["e2p"], b["p2e"])
