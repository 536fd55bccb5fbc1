"""Helpers for the GPU tests: move a synthetic Workload to the device and run the
layer through the C ABI (via the thin torch binding)."""

from __future__ import annotations

import functools
import sys
from typing import Optional

import numpy as np
import torch

import oracle
from mixture_experts_ffn_02_amd import moe_lora as ml
from synth import Workload

REL_L2_TOL = 1e-2
MAX_ABS_TOL = 3e-2


def dev():
    return torch.device("cuda:0")


def t16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev())


def bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return t.cpu().numpy().view(np.uint16)


def f64(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_bits_to_f64(bits(t))


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def layer_errors(got: np.ndarray, ref: np.ndarray):
    rel = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.abs(got - ref).max()) if got.size else 0.0
    return rel, mx


def assert_layer_close(got: np.ndarray, ref: np.ndarray, what: str = ""):
    rel, mx = layer_errors(got, ref)
    say(f"  {what} rel_l2={rel:.3e} max_abs={mx:.3e}")
    assert np.isfinite(got).all(), what
    assert rel <= REL_L2_TOL and mx <= MAX_ABS_TOL, (what, rel, mx)


def _stream_stack(wl: Workload, fn: str, shape, chunk: int = 8, keep: Optional[dict] = None) -> torch.Tensor:
    """Device tensor [E, *shape] filled expert-chunk by expert-chunk (bounded host memory
    unless keep is given: then keep[e] holds expert e's host bits for the oracle)."""
    cfg = wl.cfg
    out = torch.empty((cfg.E,) + tuple(shape), dtype=torch.int16, device=dev())
    for e0, block in wl.expert_chunks(fn, chunk):
        out[e0:e0 + block.shape[0]].copy_(torch.from_numpy(block.view(np.int16)))
        if keep is not None:
            for i in range(block.shape[0]):
                keep[e0 + i] = block[i]
    return out


class GpuLayer:
    """A Workload's tensors on the GPU plus the oracle's view of the same bits."""

    def __init__(self, wl: Workload, stream_weights: bool = False, keep_host: bool = False):
        self.wl = wl
        cfg = self.cfg = wl.cfg
        self.x_np, self.logits_np = wl.x(), wl.logits()
        self.bias_np = wl.correction_bias()
        self.slots_np = wl.token_slot()
        self.x, self.logits = t16(self.x_np), t16(self.logits_np)
        self.bias = torch.from_numpy(self.bias_np).to(dev()) if self.bias_np is not None else None
        if stream_weights:
            # keep_host: the generated bits stay on the host for the oracle (22.5 GB at the
            # DeepSeek-V3 share), instead of being regenerated per expert on demand
            self._w1c, self._w2c = {}, {}
            self.w1 = _stream_stack(wl, "w_gate_up", (2 * cfg.I, cfg.H), keep=self._w1c if keep_host else None)
            self.w2 = _stream_stack(wl, "w_down", (cfg.H, cfg.I), keep=self._w2c if keep_host else None)
            self.w1_np = self.w2_np = None
        else:
            self.w1_np, self.w2_np = wl.w_gate_up_all(), wl.w_down_all()
            self.w1, self.w2 = t16(self.w1_np), t16(self.w2_np)
        self.lora_np = [wl.lora_all(a) for a in range(cfg.num_slots)]
        self.lora_t = [{k: t16(v) for k, v in d.items()} for d in self.lora_np]
        self.routing = ml.ROUTING_DEEPSEEK_V3 if cfg.routing == "deepseek_v3" else ml.ROUTING_RENORMALIZE

    # -- oracle getters (bf16 bits)
    def w_gate_up(self, e):
        return self.w1_np[e] if self.w1_np is not None else self._w1_cached(e)

    def w_down(self, e):
        return self.w2_np[e] if self.w2_np is not None else self._w2_cached(e)

    def _w1_cached(self, e):
        c = self._w1c
        if e not in c:
            c[e] = self.wl.w_gate_up(e)
        return c[e]

    def _w2_cached(self, e):
        c = self._w2c
        if e not in c:
            c[e] = self.wl.w_down(e)
        return c[e]

    def packed_layer(self, mask: int) -> ml.MoELoRALayer:
        """The same layer on tile-packed copies of the weights named by mask."""
        c = self.cfg
        return ml.MoELoRALayer(c.H, c.I, c.E, c.top_k, self.w1, self.w2, self.routing, c.n_group,
                               c.topk_group, c.routed_scaling_factor, self.bias, packed_weights=mask)

    def oracle_layer(self, x_np=None, logits_np=None):
        """Every token's output (and the routing) from the oracle, on the same bits."""
        c = self.cfg
        return oracle.layer(self.x_np if x_np is None else x_np,
                            self.logits_np if logits_np is None else logits_np, c.top_k, c.I,
                            self.w_gate_up, self.w_down, self.oracle_adapters(), self.slots_np, c.routing,
                            self.bias_np, c.n_group, c.topk_group, c.routed_scaling_factor,
                            num_experts=c.E)

    def oracle_adapters(self, shared_outer: bool = False):
        ads = []
        for a, sp in enumerate(self.cfg.slots):
            if shared_outer:
                d = self.lora_np[a]
                ads.append(oracle.shared_outer_adapter(
                    sp.rank, sp.scaling, self.wl.lora_a_gate_up_shared(a), lambda e, d=d: d["b_gate_up"][e],
                    lambda e, d=d: d["a_down"][e], self.wl.lora_b_down_shared(a)))
                continue
            d = self.lora_np[a]
            ads.append(oracle.Adapter(sp.rank, sp.scaling,
                                      lambda e, d=d: d["a_gate_up"][e], lambda e, d=d: d["b_gate_up"][e],
                                      lambda e, d=d: d["a_down"][e], lambda e, d=d: d["b_down"][e]))
        return ads

    def oracle_route(self):
        c = self.cfg
        return oracle.route(self.logits_np, c.top_k, c.routing, self.bias_np, c.n_group, c.topk_group,
                            c.routed_scaling_factor)

    # -- GPU side
    def layer(self, gather_on_load: bool = True) -> ml.MoELoRALayer:
        c = self.cfg
        return ml.MoELoRALayer(c.H, c.I, c.E, c.top_k, self.w1, self.w2, self.routing, c.n_group,
                               c.topk_group, c.routed_scaling_factor, self.bias, gather_on_load)

    def lora_slots(self, token_slot: Optional[np.ndarray] = None, zero_b: bool = False,
                   shared_outer: bool = False, replicate_shared: bool = False):
        """Device adapter slots.  shared_outer: the shared-outer layout (one gate_up A and
        one down B per slot); replicate_shared: the same weights in the routed layout, the
        shared matrices copied for every expert."""
        c = self.cfg
        if c.num_slots == 0:
            return None
        ts = self.slots_np if token_slot is None else token_slot
        L = self.lora_t
        bg = [torch.zeros_like(d["b_gate_up"]) if zero_b else d["b_gate_up"] for d in L]
        bd = [torch.zeros_like(d["b_down"]) if zero_b else d["b_down"] for d in L]
        ag = [d["a_gate_up"] for d in L]
        if shared_outer or replicate_shared:
            ag = [t16(self.wl.lora_a_gate_up_shared(a)) for a in range(c.num_slots)]
            bd = [t16(self.wl.lora_b_down_shared(a)) for a in range(c.num_slots)]
            if replicate_shared:
                ag = [t.unsqueeze(0).expand(c.E, *t.shape).contiguous() for t in ag]
                bd = [t.unsqueeze(0).expand(c.E, *t.shape).contiguous() for t in bd]
        return ml.LoRASlots(torch.from_numpy(np.ascontiguousarray(ts, dtype=np.int32)).to(dev()),
                            [s.rank for s in c.slots], [s.scaling for s in c.slots],
                            ag, bg, [d["a_down"] for d in L], bd, shared_outer=shared_outer)
