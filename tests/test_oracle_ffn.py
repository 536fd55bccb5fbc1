"""Pins for the oracle's expert FFN with LoRA and the whole layer (CPU only).

Each pin compares the oracle with a different formula for the same quantity:
merged weights W + s B A, a dense SwiGLU MLP, a per-slice LoRA, a hand-derived
closed form, zero-padded ranks, token permutations, and single-slot batches.
"""

import dataclasses
import functools
import math

import numpy as np
import pytest

import oracle
from helpers import oracle_adapters, oracle_layer, rel_l2
from synth import NAMED_CONFIGS, Workload, f32_to_bf16_bits, make_config

SMALL = make_config(name="small_multislot", cfg_id=101, T=40, H=64, I=32, E=6, top_k=2,
                    slots=((4, 2.0), (8, 0.5), (2, 1.0)), slot_assignment="uniform",
                    lora_a_std=0.2, lora_b_std=0.2, w_std=0.1)


def _f(bits):
    return oracle.bf16_bits_to_f64(bits)


def _merged_reference(wl, token_slot=None):
    """Base MoE on merged weights W1' = W1 + s B1 A1, W2' = W2 + s B2 A2, written
    directly with numpy per routed (token, j) pair."""
    cfg = wl.cfg
    x = _f(wl.x())
    ids, w = oracle.route(wl.logits(), cfg.top_k, cfg.routing, wl.correction_bias(), cfg.n_group,
                          cfg.topk_group, cfg.routed_scaling_factor)
    slots = wl.token_slot() if token_slot is None else token_slot
    out = np.zeros((cfg.T, cfg.H))
    cache = {}
    for t in range(cfg.T):
        a = int(slots[t])
        for j in range(cfg.top_k):
            e = int(ids[t, j])
            key = (e, a if 0 <= a < cfg.num_slots else -1)
            if key not in cache:
                W1 = _f(wl.w_gate_up(e))
                W2 = _f(wl.w_down(e))
                if key[1] >= 0:
                    s = cfg.slots[a].scaling
                    W1 = W1 + s * _f(wl.lora_b_gate_up(a, e)) @ _f(wl.lora_a_gate_up(a, e))
                    W2 = W2 + s * _f(wl.lora_b_down(a, e)) @ _f(wl.lora_a_down(a, e))
                cache[key] = (W1, W2)
            W1, W2 = cache[key]
            g = W1 @ x[t]
            h = g[: cfg.I] / (1.0 + np.exp(-g[: cfg.I])) * g[cfg.I:]
            out[t] += w[t, j] * (W2 @ h)
    return out


@pytest.mark.parametrize("cfg", [SMALL, NAMED_CONFIGS[1],
                                 dataclasses.replace(NAMED_CONFIGS[4], T=12, H=256, I=128, E=16)])
def test_lora_equals_merged_weights(cfg):
    wl = Workload(cfg)
    got = oracle_layer(wl)["out"]
    want = _merged_reference(wl)
    assert rel_l2(got, want) < 1e-12
    np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-12)


def test_dense_swiglu_mlp_when_one_expert_top1():
    """E = 1, k = 1: the layer is a dense SwiGLU MLP with merged weights (textbook form)."""
    cfg = make_config(cfg_id=102, T=9, H=32, I=16, E=1, top_k=1, slots=((4, 2.0),),
                      lora_a_std=0.3, lora_b_std=0.3)
    wl = Workload(cfg)
    out = oracle_layer(wl)["out"]
    x = _f(wl.x())
    W1 = _f(wl.w_gate_up(0)) + 2.0 * _f(wl.lora_b_gate_up(0, 0)) @ _f(wl.lora_a_gate_up(0, 0))
    W2 = _f(wl.w_down(0)) + 2.0 * _f(wl.lora_b_down(0, 0)) @ _f(wl.lora_a_down(0, 0))
    gate, up = x @ W1[:16].T, x @ W1[16:].T
    mlp = (gate * (1.0 / (1.0 + np.exp(-gate))) * up) @ W2.T
    np.testing.assert_allclose(out, mlp, rtol=1e-11, atol=1e-13)


def test_hand_derived_tiny_layer():
    """H = 2, I = 1, E = 2, k = 1, one rank-1 slot with s = 2, worked by hand:
    gate row reads x0, up row reads x1, the LoRA adds 2*x0 to up; the down weight
    is [1, 0.5] and the down LoRA adds 2*h to the second output.
        h = silu(x0) * (x1 + 2 x0),  y = [h, 0.5 h + 2 h]."""
    one, zero, half = 1.0, 0.0, 0.5
    bits = lambda a: f32_to_bf16_bits(np.asarray(a, np.float32))  # noqa: E731
    x = bits([[1.5, -0.5], [-2.0, 0.25], [0.75, 3.0]])
    logits = bits([[0.0, 1.0], [2.0, -1.0], [0.0, 0.0]])  # experts 1, 0, 0 (tie -> 0)
    w1 = bits([[one, zero], [zero, one]])
    w2 = bits([[one], [half]])
    ad = oracle.Adapter(rank=1, scaling=2.0,
                        a_gate_up=lambda e: bits([[one, zero]]), b_gate_up=lambda e: bits([[zero], [one]]),
                        a_down=lambda e: bits([[one]]), b_down=lambda e: bits([[zero], [one]]))
    res = oracle.layer(x, logits, 1, 1, lambda e: w1, lambda e: w2, [ad], np.array([0, -1, 0]))
    assert res["ids"].tolist() == [[1], [0], [0]]
    silu = lambda v: v / (1.0 + math.exp(-v))  # noqa: E731
    h0 = silu(1.5) * (-0.5 + 3.0)
    h1 = silu(-2.0) * 0.25  # slot -1: no LoRA
    h2 = silu(0.75) * (3.0 + 1.5)
    want = [[h0, 0.5 * h0 + 2 * h0], [h1, 0.5 * h1], [h2, 0.5 * h2 + 2 * h2]]
    np.testing.assert_allclose(res["out"], want, rtol=1e-15, atol=0)


def test_zero_lora_is_exactly_base():
    wl = Workload(SMALL)
    base = oracle_layer(wl, with_lora=False)["out"]
    # all slots -1
    none = oracle_layer(wl, token_slot=np.full(SMALL.T, -1, np.int32))["out"]
    np.testing.assert_array_equal(none, base)
    # out-of-range slots are treated as no adapter
    bad = oracle_layer(wl, token_slot=np.full(SMALL.T, 7, np.int32))["out"]
    np.testing.assert_array_equal(bad, base)
    # B = 0 for every slot
    ads = oracle_adapters(wl)
    for ad in ads:
        ad.b_gate_up = lambda e, r=ad.rank: np.zeros((2 * SMALL.I, r), np.uint16)
        ad.b_down = lambda e, r=ad.rank: np.zeros((SMALL.H, r), np.uint16)
    zb = oracle_layer(wl, adapters=ads)["out"]
    np.testing.assert_array_equal(zb, base)


def test_token_permutation_equivariance():
    wl = Workload(SMALL)
    res = oracle_layer(wl)
    perm = np.random.default_rng(3).permutation(SMALL.T)
    ads = oracle_adapters(wl)
    res_p = oracle.layer(wl.x()[perm], wl.logits()[perm], SMALL.top_k, SMALL.I,
                         wl.w_gate_up, wl.w_down, ads, wl.token_slot()[perm], num_experts=SMALL.E)
    np.testing.assert_allclose(res_p["out"], res["out"][perm], rtol=1e-13, atol=1e-15)


def test_mixed_slots_equal_union_of_single_slot_runs():
    wl = Workload(SMALL)
    slots = wl.token_slot()
    mixed = oracle_layer(wl)["out"]
    for a in range(SMALL.num_slots):
        single = oracle_layer(wl, token_slot=np.full(SMALL.T, a, np.int32))["out"]
        rows = slots == a
        assert rows.any()
        np.testing.assert_allclose(mixed[rows], single[rows], rtol=1e-13, atol=1e-15)


def test_zero_padded_rank_leaves_output_unchanged():
    wl = Workload(SMALL)
    want = oracle_layer(wl)["out"]
    ads = oracle_adapters(wl)
    pad = 5
    padded = []
    for ad in ads:
        r = ad.rank

        def pa(f):
            return lambda e: np.concatenate([f(e), np.zeros((pad, f(e).shape[1]), np.uint16)], 0)

        def pb(f):
            return lambda e: np.concatenate([f(e), np.zeros((f(e).shape[0], pad), np.uint16)], 1)

        padded.append(oracle.Adapter(r + pad, ad.scaling, pa(ad.a_gate_up), pb(ad.b_gate_up),
                                     pa(ad.a_down), pb(ad.b_down)))
    got = oracle_layer(wl, adapters=padded)["out"]
    np.testing.assert_allclose(got, want, rtol=1e-13, atol=1e-15)


def test_per_slice_gate_up_lora_equals_block_diagonal_merged():
    """Separate rank-r LoRAs on the gate and up halves == one rank-2r LoRA with
    A = [A_g; A_u] and block-diagonal B (the slices form listed for w13 LoRA)."""
    cfg = make_config(cfg_id=103, T=20, H=48, I=24, E=4, top_k=2, slots=((6, 2.0),),
                      lora_a_std=0.2, lora_b_std=0.2, w_std=0.1)
    wl = Workload(cfg)
    rng = np.random.default_rng(9)
    r, I, H = 3, cfg.I, cfg.H
    bits = lambda a: f32_to_bf16_bits(np.asarray(a, np.float32))  # noqa: E731
    Ag = {e: bits(rng.standard_normal((r, H)) * 0.2) for e in range(4)}
    Au = {e: bits(rng.standard_normal((r, H)) * 0.2) for e in range(4)}
    Bg = {e: bits(rng.standard_normal((I, r)) * 0.2) for e in range(4)}
    Bu = {e: bits(rng.standard_normal((I, r)) * 0.2) for e in range(4)}
    z = np.zeros((I, r), np.uint16)
    merged = oracle.Adapter(
        2 * r, 2.0,
        a_gate_up=lambda e: np.concatenate([Ag[e], Au[e]], 0),
        b_gate_up=lambda e: np.block([[Bg[e], z], [z, Bu[e]]]),
        a_down=lambda e: np.zeros((2 * r, I), np.uint16),
        b_down=lambda e: np.zeros((H, 2 * r), np.uint16))
    got = oracle_layer(wl, adapters=[merged])["out"]
    # per-slice form, written directly
    x = _f(wl.x())
    ids, w = oracle.route_renormalize(wl.logits(), 2)
    want = np.zeros((cfg.T, H))
    for t in range(cfg.T):
        for j in range(2):
            e = int(ids[t, j])
            g = _f(wl.w_gate_up(e)) @ x[t]
            g[:I] += 2.0 * _f(Bg[e]) @ (_f(Ag[e]) @ x[t])
            g[I:] += 2.0 * _f(Bu[e]) @ (_f(Au[e]) @ x[t])
            h = g[:I] / (1 + np.exp(-g[:I])) * g[I:]
            want[t] += w[t, j] * (_f(wl.w_down(e)) @ h)
    np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-14)


@pytest.mark.parametrize("cfg", [NAMED_CONFIGS[1], dataclasses.replace(NAMED_CONFIGS[2], T=8)])
def test_tolerance_discriminates_plausible_mistakes(cfg):
    """The layer tolerance (rel L2 1e-2) must tell right from wrong: dropping the LoRA,
    doubling its scaling, or swapping the gate/up halves moves the output far more."""
    wl = Workload(cfg)
    ref = oracle_layer(wl)["out"]
    no_lora = oracle_layer(wl, with_lora=False)["out"]
    assert rel_l2(no_lora, ref) > 0.05
    ads = oracle_adapters(wl)
    for ad in ads:
        ad.scaling *= 2
    assert rel_l2(oracle_layer(wl, adapters=ads)["out"], ref) > 0.05
    I = cfg.I
    swap = lambda f: (lambda e: np.concatenate([f(e)[I:], f(e)[:I]], 0))  # noqa: E731
    ads = oracle_adapters(wl)
    for ad in ads:
        ad.b_gate_up = swap(ad.b_gate_up)
    swapped = oracle_layer(wl, w_gate_up=swap(wl.w_gate_up), adapters=ads)["out"]
    assert rel_l2(swapped, ref) > 0.2


def test_sampled_layer_equals_full_layer():
    wl = Workload(SMALL)
    res = oracle_layer(wl)
    toks = [0, 3, 17, 39]
    ads = oracle_adapters(wl)
    got = oracle.layer_sampled(wl.x(), res["ids"], res["weights"], toks, SMALL.I, wl.w_gate_up,
                               wl.w_down, ads, wl.token_slot())
    np.testing.assert_allclose(got, res["out"][toks], rtol=1e-13, atol=1e-15)


def _merged_shared_outer_reference(wl):
    """Base MoE on merged weights for shared-outer slots, W1' = W1[e] + s B1[a][e] A1[a]
    and W2' = W2[e] + s B2[a] A2[a][e], written directly with numpy per routed pair."""
    cfg = wl.cfg
    x = _f(wl.x())
    ids, w = oracle.route(wl.logits(), cfg.top_k, cfg.routing, wl.correction_bias(), cfg.n_group,
                          cfg.topk_group, cfg.routed_scaling_factor)
    slots = wl.token_slot()
    out = np.zeros((cfg.T, cfg.H))
    cache = {}
    for t in range(cfg.T):
        a = int(slots[t])
        for j in range(cfg.top_k):
            e = int(ids[t, j])
            key = (e, a if 0 <= a < cfg.num_slots else -1)
            if key not in cache:
                W1 = _f(wl.w_gate_up(e))
                W2 = _f(wl.w_down(e))
                if key[1] >= 0:
                    s = cfg.slots[a].scaling
                    W1 = W1 + s * _f(wl.lora_b_gate_up(a, e)) @ _f(wl.lora_a_gate_up_shared(a))
                    W2 = W2 + s * _f(wl.lora_b_down_shared(a)) @ _f(wl.lora_a_down(a, e))
                cache[key] = (W1, W2)
            W1, W2 = cache[key]
            g = W1 @ x[t]
            h = g[: cfg.I] / (1.0 + np.exp(-g[: cfg.I])) * g[cfg.I:]
            out[t] += w[t, j] * (W2 @ h)
    return out


@pytest.mark.parametrize("cfg", [SMALL, NAMED_CONFIGS[1],
                                 dataclasses.replace(NAMED_CONFIGS[4], T=12, H=256, I=128, E=16)])
def test_shared_outer_lora_equals_merged_weights(cfg):
    """Shared-outer slots (gate_up A and down B shared by the experts) against the merged
    weights of the same slots."""
    wl = Workload(cfg)
    got = oracle_layer(wl, adapters=oracle_adapters(wl, shared_outer=True))["out"]
    want = _merged_shared_outer_reference(wl)
    assert rel_l2(got, want) < 1e-12
    np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-12)


def test_shared_outer_differs_from_routed_and_from_base():
    """The shared weights are used: the output moves away from both the routed-LoRA and
    the base layer by far more than the layer tolerance."""
    wl = Workload(SMALL)
    shared = oracle_layer(wl, adapters=oracle_adapters(wl, shared_outer=True))["out"]
    assert rel_l2(shared, oracle_layer(wl)["out"]) > 0.05
    assert rel_l2(shared, oracle_layer(wl, with_lora=False)["out"]) > 0.05
