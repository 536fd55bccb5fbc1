"""Pins for the oracle's routing (CPU only).

The oracle is checked here against things other than itself: brute-force Python
sorts on every token, the RenormalizeNaive order of operations, closed forms for
two-expert softmax, special cases of the grouped routing, and brute force over
every group subset.
"""

import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle
from synth import NAMED_CONFIGS, Workload, f32_to_bf16_bits, make_config

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _brute_topk(keys_row, k):
    """Explicit sort of (-key, index) pairs: the tie rule written out."""
    pairs = sorted((-float(v), e) for e, v in enumerate(keys_row))
    return [e for _, e in pairs[:k]]


def _bits(vals):
    return f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


@pytest.mark.parametrize("cfg_id", [1, 2, 3, 4])
def test_renormalize_ids_match_brute_force_sort(cfg_id):
    cfg = NAMED_CONFIGS[cfg_id]
    wl = Workload(cfg)
    lb = wl.logits()
    l = oracle.bf16_bits_to_f64(lb)
    ids, w = oracle.route_renormalize(lb, cfg.top_k)
    T = cfg.T if cfg.T <= 1024 else 1024  # brute force on the first 1024 tokens of the big one
    for t in range(T):
        assert list(ids[t]) == _brute_topk(l[t], cfg.top_k), t


def test_renormalize_ties_lower_index_wins():
    # exact ties at the k / k+1 boundary and inside the selection
    lb = _bits([[1.0, 2.0, 2.0, 0.5, 2.0, -1.0]])
    ids, w = oracle.route_renormalize(lb, 2)
    assert list(ids[0]) == [1, 2]
    ids, w = oracle.route_renormalize(lb, 3)
    assert list(ids[0]) == [1, 2, 4]
    np.testing.assert_allclose(w[0], [1 / 3] * 3, rtol=0, atol=1e-15)


def test_renormalize_equals_renormalize_naive():
    """softmax over all experts -> top-k -> renormalize == top-k -> softmax over the k."""
    wl = Workload(NAMED_CONFIGS[2])
    lb = wl.logits()
    l = oracle.bf16_bits_to_f64(lb)
    ids, w = oracle.route_renormalize(lb, 8)
    p = np.exp(l - l.max(axis=1, keepdims=True))
    p /= p.sum(axis=1, keepdims=True)
    order = np.argsort(-p, axis=1, kind="stable")[:, :8]
    np.testing.assert_array_equal(order, ids)
    sel = np.take_along_axis(p, order, axis=1)
    naive = sel / sel.sum(axis=1, keepdims=True)
    np.testing.assert_allclose(naive, w, rtol=0, atol=1e-15)


def test_renormalize_two_expert_closed_form():
    """k = 2: w0 = 1 / (1 + exp(l1 - l0)) exactly (closed form of a 2-way softmax)."""
    rng = np.random.default_rng(5)
    lb = _bits(rng.standard_normal((64, 6)).astype(np.float32))
    l = oracle.bf16_bits_to_f64(lb)
    ids, w = oracle.route_renormalize(lb, 2)
    for t in range(64):
        a, b = l[t, ids[t, 0]], l[t, ids[t, 1]]
        assert a >= b
        assert abs(w[t, 0] - 1.0 / (1.0 + math.exp(b - a))) < 1e-15
        assert abs(w[t, 1] - 1.0 / (1.0 + math.exp(a - b))) < 1e-15


@pytest.mark.parametrize("cfg_id", [1, 2, 4])
def test_weights_sum_to_one(cfg_id):
    cfg = NAMED_CONFIGS[cfg_id]
    ids, w = oracle.route_renormalize(Workload(cfg).logits(), cfg.top_k)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=0, atol=1e-14)
    assert (w > 0).all()
    assert (np.diff(w, axis=1) <= 1e-15).all()  # descending logits -> non-increasing weights


def _sigmoid(v):
    return 1.0 / (1.0 + math.exp(-v))


def _brute_dsv3(l_row, bias, k, n_group, topk_group, rsf):
    """Grouped routing written out with Python loops and explicit subset enumeration."""
    E = len(l_row)
    per = E // n_group
    s = [_sigmoid(float(v)) for v in l_row]
    key = [s[e] + float(bias[e]) for e in range(E)]
    gscore = []
    for g in range(n_group):
        ks = sorted((key[e] for e in range(g * per, (g + 1) * per)), reverse=True)
        gscore.append(sum(ks[:2]))
    # best subset of topk_group groups: maximal scores, ties by lower group index
    best = None
    for sub in itertools.combinations(range(n_group), topk_group):
        sig = sorted(((-gscore[g], g) for g in sub))
        if best is None or sig < best[0]:
            best = (sig, sub)
    chosen = sorted(best[1])
    cand = [e for g in chosen for e in range(g * per, (g + 1) * per)]
    pairs = sorted((-key[e], e) for e in cand)
    ids = [e for _, e in pairs[:k]]
    tot = sum(s[e] for e in ids)
    return ids, [rsf * s[e] / tot for e in ids], chosen, gscore


def test_deepseek_v3_matches_brute_force_cfg5():
    cfg = NAMED_CONFIGS[5]
    wl = Workload(cfg)
    lb, bias = wl.logits(), wl.correction_bias()
    l = oracle.bf16_bits_to_f64(lb)
    ids, w = oracle.route_deepseek_v3(lb, bias, cfg.top_k, cfg.n_group, cfg.topk_group,
                                      cfg.routed_scaling_factor)
    for t in range(0, cfg.T, 4):  # every 4th token: 256 tokens x 70 subsets
        bi, bw, chosen, gscore = _brute_dsv3(l[t], bias, cfg.top_k, cfg.n_group, cfg.topk_group,
                                             cfg.routed_scaling_factor)
        assert list(ids[t]) == bi, t
        np.testing.assert_allclose(w[t], bw, rtol=1e-14, atol=0)
        # every chosen group's score >= every unchosen group's score
        lo = min(gscore[g] for g in chosen)
        hi = max([gscore[g] for g in range(cfg.n_group) if g not in chosen], default=-np.inf)
        assert lo >= hi
    np.testing.assert_allclose(w.sum(axis=1), cfg.routed_scaling_factor, rtol=1e-14)


def test_deepseek_v3_single_group_is_plain_topk_of_biased_sigmoid():
    rng = np.random.default_rng(11)
    lb = _bits(rng.standard_normal((40, 32)).astype(np.float32))
    bias = (rng.standard_normal(32) * 0.3).astype(np.float32)
    l = oracle.bf16_bits_to_f64(lb)
    ids, w = oracle.route_deepseek_v3(lb, bias, 6, 1, 1, 1.0)
    for t in range(40):
        key = [_sigmoid(l[t, e]) + float(bias[e]) for e in range(32)]
        assert list(ids[t]) == _brute_topk(key, 6)


def test_deepseek_v3_no_bias_one_group_selects_like_renormalize():
    """sigmoid is monotone: with zero bias and one group the ids equal Renormalize's."""
    wl = Workload(NAMED_CONFIGS[2])
    lb = wl.logits()
    ids_r, _ = oracle.route_renormalize(lb, 8)
    ids_d, w_d = oracle.route_deepseek_v3(lb, np.zeros(128, np.float32), 8, 1, 1, 1.0)
    np.testing.assert_array_equal(ids_r, ids_d)
    np.testing.assert_allclose(w_d.sum(axis=1), 1.0, atol=1e-14)


def test_deepseek_v3_group_restriction_matters():
    """Sensitivity: with groups the selection differs from the ungrouped top-k on cfg5."""
    cfg = NAMED_CONFIGS[5]
    wl = Workload(cfg)
    lb, bias = wl.logits(), wl.correction_bias()
    g, _ = oracle.route_deepseek_v3(lb, bias, 8, 8, 4, 2.5)
    u, _ = oracle.route_deepseek_v3(lb, bias, 8, 1, 1, 2.5)
    assert (np.sort(g, axis=1) != np.sort(u, axis=1)).any(axis=1).mean() > 0.2
    per = 256 // 8
    for t in range(cfg.T):
        assert len(set(int(e) // per for e in g[t])) <= 4


def test_golden_routing_fixture():
    """Hand-derived routing cases (see tests/golden/routing_cases.json for the derivation)."""
    with open(os.path.join(GOLDEN, "routing_cases.json")) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        lb = _bits(case["logits"])
        if case["method"] == "renormalize":
            ids, w = oracle.route_renormalize(lb, case["top_k"])
        else:
            ids, w = oracle.route_deepseek_v3(lb, np.asarray(case["bias"], np.float32), case["top_k"],
                                              case["n_group"], case["topk_group"], case["rsf"])
        assert ids.tolist() == case["ids"], case["name"]
        want = [[eval(expr, {"__builtins__": {}, "math": math}) for expr in row] for row in case["weights"]]
        np.testing.assert_allclose(w, want, rtol=1e-13, atol=0, err_msg=case["name"])
