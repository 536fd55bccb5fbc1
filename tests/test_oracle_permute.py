"""Pins for the oracle's expert-sorted pack, permute and finalize (CPU only)."""

import numpy as np
import pytest

import oracle
from synth import NAMED_CONFIGS, Workload, f32_to_bf16_bits


def _brute_sort(ids, E):
    """Stable counting sort written out with Python loops."""
    flat = [int(v) for v in np.asarray(ids).reshape(-1)]
    counts = [0] * E
    for e in flat:
        counts[e] += 1
    offsets = [0]
    for e in range(E):
        offsets.append(offsets[-1] + counts[e])
    fill = list(offsets[:-1])
    e2p = [0] * len(flat)
    for j, e in enumerate(flat):
        e2p[j] = fill[e]
        fill[e] += 1
    p2e = [0] * len(flat)
    for j, p in enumerate(e2p):
        p2e[p] = j
    return counts, offsets, e2p, p2e


@pytest.mark.parametrize("cfg_id", [1, 2, 4, 5])
def test_expert_sort_matches_counting_sort(cfg_id):
    cfg = NAMED_CONFIGS[cfg_id]
    wl = Workload(cfg)
    ids, _ = oracle.route(wl.logits(), cfg.top_k, cfg.routing, wl.correction_bias(), cfg.n_group,
                          cfg.topk_group, cfg.routed_scaling_factor)
    s = oracle.expert_sort(ids, cfg.E)
    counts, offsets, e2p, p2e = _brute_sort(ids, cfg.E)
    assert s["counts"].tolist() == counts
    assert s["offsets"].tolist() == offsets
    assert s["e2p"].tolist() == e2p
    assert s["p2e"].tolist() == p2e


def test_expert_sort_invariants_prefill():
    cfg = NAMED_CONFIGS[3]
    ids, _ = oracle.route_renormalize(Workload(cfg).logits(), cfg.top_k)
    s = oracle.expert_sort(ids, cfg.E)
    R = cfg.R
    assert s["counts"].sum() == R and s["offsets"][-1] == R and s["offsets"][0] == 0
    # inverse bijections
    assert np.array_equal(s["p2e"][s["e2p"]], np.arange(R))
    assert np.array_equal(np.sort(s["p2e"]), np.arange(R))
    flat = ids.reshape(-1)
    row_expert = flat[s["p2e"]]
    assert (np.diff(row_expert) >= 0).all()  # experts non-decreasing along permuted rows
    for e in range(cfg.E):
        seg = s["p2e"][s["offsets"][e]:s["offsets"][e + 1]]
        assert (np.diff(seg) > 0).all()  # stable: expanded index increasing inside an expert
    # the skewed logits give unequal loads (max well above the mean)
    assert s["counts"].max() > 3 * R / cfg.E


def test_round_trip_identity_expert_unit_weights():
    """y_perm = x_perm with all weights 1: finalize(permute(x)) = k * x exactly."""
    for k in (1, 2, 8):
        rng = np.random.default_rng(k)
        T, E, H = 37, 16, 24
        xb = f32_to_bf16_bits(rng.standard_normal((T, H)).astype(np.float32))
        ids = np.stack([rng.permutation(E)[:k] for _ in range(T)]).astype(np.int32)
        s = oracle.expert_sort(ids, E)
        xp = oracle.permute_rows(xb, s["p2e"], k)
        out = oracle.finalize(oracle.bf16_bits_to_f64(xp), np.ones((T, k)), s["e2p"])
        np.testing.assert_array_equal(out, k * oracle.bf16_bits_to_f64(xb))
        if k == 1:
            np.testing.assert_array_equal(out, oracle.bf16_bits_to_f64(xb))


def test_finalize_weighted_sum_by_hand():
    # two tokens, k = 2, rows placed by hand
    y = np.array([[1.0, 2.0], [10.0, 20.0], [100.0, 200.0], [1000.0, 2000.0]])
    w = np.array([[0.25, 0.75], [0.5, 0.5]])
    e2p = np.array([2, 0, 3, 1])
    out = oracle.finalize(y, w, e2p)
    np.testing.assert_array_equal(out, [[0.25 * 100 + 0.75 * 1, 0.25 * 200 + 0.75 * 2],
                                        [0.5 * 1000 + 0.5 * 10, 0.5 * 2000 + 0.5 * 20]])


def test_empty_experts_and_single_expert():
    ids = np.zeros((5, 1), dtype=np.int32) + 3
    s = oracle.expert_sort(ids, 6)
    assert s["counts"].tolist() == [0, 0, 0, 5, 0, 0]
    assert s["offsets"].tolist() == [0, 0, 0, 0, 5, 5, 5]
    assert s["p2e"].tolist() == [0, 1, 2, 3, 4]
