"""Shared helpers for the tests: build oracle inputs from a synthetic Workload."""

import functools

import numpy as np

import oracle


def oracle_adapters(wl, shared_outer=False):
    cfg = wl.cfg
    ads = []
    for a, sp in enumerate(cfg.slots):
        if shared_outer:
            ads.append(oracle.shared_outer_adapter(
                sp.rank, sp.scaling, wl.lora_a_gate_up_shared(a),
                functools.lru_cache(None)(lambda e, a=a: wl.lora_b_gate_up(a, e)),
                functools.lru_cache(None)(lambda e, a=a: wl.lora_a_down(a, e)),
                wl.lora_b_down_shared(a)))
            continue
        ads.append(oracle.Adapter(
            rank=sp.rank, scaling=sp.scaling,
            a_gate_up=functools.lru_cache(None)(lambda e, a=a: wl.lora_a_gate_up(a, e)),
            b_gate_up=functools.lru_cache(None)(lambda e, a=a: wl.lora_b_gate_up(a, e)),
            a_down=functools.lru_cache(None)(lambda e, a=a: wl.lora_a_down(a, e)),
            b_down=functools.lru_cache(None)(lambda e, a=a: wl.lora_b_down(a, e)),
        ))
    return ads


def oracle_layer(wl, with_lora=True, token_slot=None, w_gate_up=None, w_down=None, adapters=None):
    cfg = wl.cfg
    ads = (oracle_adapters(wl) if adapters is None else adapters) if with_lora else []
    return oracle.layer(
        wl.x(), wl.logits(), cfg.top_k, cfg.I,
        w_gate_up or functools.lru_cache(None)(wl.w_gate_up),
        w_down or functools.lru_cache(None)(wl.w_down),
        ads, wl.token_slot() if token_slot is None else token_slot,
        cfg.routing, wl.correction_bias(), cfg.n_group, cfg.topk_group, cfg.routed_scaling_factor,
        num_experts=cfg.E)


def rel_l2(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))
