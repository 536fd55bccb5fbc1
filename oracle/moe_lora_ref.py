"""Plain fp64 definition of the routed MoE-LoRA expert layer (the oracle).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py; never by the product path.  It shares no code with
the HIP library.

Sources (the pages, cited by title and section):
  [P1] sglang PR "[LoRA] bf16 MoE-LoRA for trtllm backend with two-stream overlap +
       routing opts": Files-changed table (launcher row: routing -> permute -> gate_up
       GEMM -> activation adding gate_up_lora_delta before SwiGLU -> down GEMM ->
       finalize), section 2(A) steps 1-5 (gate_up LoRA call with mul_routed_weight=False,
       down LoRA call with mul_routed_weight=True on activation_lora_input).
  [P2] sglang PR "[LoRA] Experimental fast LoRA path ... FP8 and NVFP4 models":
       Optimizations (LoRA deltas applied after gate_up / before activation and after
       down / before reduction).
  [P4] sglang PR "[LoRA] Fix experimental fast-path multi-adapter correctness ...":
       Motivation item 2 / Modifications (slot, rank and scaling are per request).
  [P5] vLLM API page "trtllm_lora_moe": TrtLlmBf16LoRAExperts routing methods,
       _TrtLlmLoRAExpertsBase.apply (steps 1-4), _unpermute_activation
       (expanded = token*top_k + k), _finalize_with_w2_lora (weighted top-k sum).

Every array of bf16 data arrives as uint16 bit patterns and is decoded exactly to
fp64 (bf16 is a subset of fp64).  Nothing is rounded afterwards: no bf16
intermediates, no split-K, no fusion.

Readings of points the pages leave open (each is also listed in the design notes):
  * Renormalize: top-k of the raw logits (ties -> lower expert index), then a softmax
    over the k selected logits.  RenormalizeNaive (softmax over all experts, top-k,
    renormalize) gives the same ids and the same weights up to rounding.
  * DeepSeek-V3 grouped routing is named on [P5] but not defined there; the oracle
    follows the published DeepSeek-V3 gate: sigmoid scores, a correction bias used
    for selection only, contiguous expert groups scored by the sum of their two
    largest biased scores, top ``topk_group`` groups, top-k experts inside them,
    weights = routed_scaling_factor * s / sum(s) over the unbiased sigmoid scores.
    PARITY UNPINNED against the pages (they print no formula); self-consistency is
    pinned by special-case reductions and brute force in tests/.
  * Order of the k ids of a token: descending key, ties by ascending expert index.
  * Order of rows inside one expert after the permute: ascending expanded index.
  * gate/up halves: rows [0, I) of the gate_up weight are gate, [I, 2I) are up.
  * the LoRA scaling multiplies the whole low-rank product: s * B (A v).
  * routed_scaling_factor is folded into the routing weights, so base and LoRA
    contributions scale together.
  * a token whose slot is outside [0, num_slots) gets no LoRA (the pages' -1
    sentinel for "no adapter").
  * shared-outer LoRA ([P1] section 2): the gate_up A and the down B are shared by all
    experts, the gate_up B and the down A are per expert; rounding and weighting as in
    the routed layer (the down delta is added to the expert output before finalize).
  * FP8 expert weights ([P2] title and Optimizations: the LoRA deltas are applied around
    an FP8 fused MoE; the pages fix no format): OCP E4M3 codes (sign, 4 exponent bits
    with bias 7, 3 mantissa bits, subnormals, 0x7f / 0xff NaN, no infinities), one fp32
    scale per 128 x 128 block of each expert matrix, weight = value(code) * scale of its
    block.  The layer is then the bf16 layer's definition on those weights; the LoRA
    matrices stay bf16.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Callable, Optional, Sequence

import numpy as np

BitsFn = Callable[[int], np.ndarray]


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact bf16 -> fp64: a bf16 pattern is the upper half of an fp32 pattern."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Value of each OCP E4M3 code (uint8) in fp64, written out from the format's fields."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    exp = (c >> 3) & 0xF
    man = (c & 0x7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + man / 8.0, exp - 7)
    subnormal = sign * np.ldexp(man / 8.0, -6)
    v = np.where(exp == 0, subnormal, normal)
    return np.where((c & 0x7F) == 0x7F, np.nan, v)


def fp8_block_weights(codes: np.ndarray, scales: np.ndarray, block: int = 128) -> np.ndarray:
    """One expert matrix [N, K] from E4M3 codes [N, K] and fp32 block scales
    [ceil(N / block), ceil(K / block)]: w[n, k] = value(codes[n, k]) * scales[n // block, k // block]."""
    v = e4m3_to_f64(codes)
    N, K = v.shape
    s = np.asarray(scales, dtype=np.float64)
    return v * s[np.arange(N)[:, None] // block, np.arange(K)[None, :] // block]


def _weights_f64(w: np.ndarray) -> np.ndarray:
    """Expert matrix as fp64: bf16 bit patterns (uint16/int16) are decoded; fp64 arrays (an
    FP8 matrix already dequantized by fp8_block_weights) are used as they are."""
    return w if np.asarray(w).dtype == np.float64 else bf16_bits_to_f64(w)


def silu(g: np.ndarray) -> np.ndarray:
    """silu(g) = g / (1 + exp(-g)) in fp64 (the SwiGLU gate of [P1] activation)."""
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


# ---------------------------------------------------------------- routing
def route_renormalize(logits_bits: np.ndarray, top_k: int):
    """Renormalize routing ([P5] routing methods; definition: top-k then softmax over the k).

    For each token the list (-logit_e, e) sorted ascending is the definition of the
    order; a stable argsort of -logit reproduces exactly that order.
    Returns ids [T, k] int32 and weights [T, k] fp64.
    """
    l = bf16_bits_to_f64(logits_bits)
    T, E = l.shape
    if not 1 <= top_k <= E:
        raise ValueError("top_k must be in [1, E]")
    order = np.argsort(-l, axis=1, kind="stable")
    ids = order[:, :top_k].astype(np.int32)
    sel = np.take_along_axis(l, ids.astype(np.int64), axis=1)
    m = sel[:, :1]
    ex = np.exp(sel - m)
    w = ex / ex.sum(axis=1, keepdims=True)
    return ids, w


def route_deepseek_v3(logits_bits: np.ndarray, corr_bias: Optional[np.ndarray], top_k: int,
                      n_group: int, topk_group: int, routed_scaling_factor: float):
    """DeepSeek-V3 grouped sigmoid routing ([P5] DeepSeekV3 routing method with its
    n_group / topk_group / routed_scaling_factor arguments).  Parity unpinned (see header).
    Returns ids [T, k] int32 and weights [T, k] fp64."""
    l = bf16_bits_to_f64(logits_bits)
    T, E = l.shape
    if n_group < 1 or E % n_group != 0:
        raise ValueError("E must be a multiple of n_group")
    if not 1 <= topk_group <= n_group:
        raise ValueError("topk_group must be in [1, n_group]")
    per = E // n_group
    if not 1 <= top_k <= topk_group * per:
        raise ValueError("top_k must fit in the chosen groups")
    s = 1.0 / (1.0 + np.exp(-l))
    bias = np.zeros(E) if corr_bias is None else np.asarray(corr_bias, dtype=np.float32).astype(np.float64)
    key = s + bias[None, :]
    # group score = sum of the group's two largest biased scores (one if the group has one expert)
    kg = np.sort(key.reshape(T, n_group, per), axis=2)[:, :, ::-1]
    gscore = kg[:, :, : min(2, per)].sum(axis=2)
    ids = np.empty((T, top_k), dtype=np.int32)
    for t in range(T):
        gorder = np.argsort(-gscore[t], kind="stable")[:topk_group]
        cand = np.sort(np.concatenate([np.arange(g * per, (g + 1) * per) for g in gorder]))
        pick = np.argsort(-key[t, cand], kind="stable")[:top_k]
        ids[t] = cand[pick]
    ss = np.take_along_axis(s, ids.astype(np.int64), axis=1)
    w = routed_scaling_factor * ss / ss.sum(axis=1, keepdims=True)
    return ids, w


def route(logits_bits, top_k, method="renormalize", corr_bias=None, n_group=1, topk_group=1,
          routed_scaling_factor=1.0):
    if method == "renormalize":
        return route_renormalize(logits_bits, top_k)
    if method == "deepseek_v3":
        return route_deepseek_v3(logits_bits, corr_bias, top_k, n_group, topk_group, routed_scaling_factor)
    raise ValueError(f"unknown routing method {method!r}")


# ---------------------------------------------------------------- permute
def expert_sort(ids: np.ndarray, num_experts: int) -> dict:
    """Expert-sorted pack of the routed rows ([P1] "routing -> permute"; [P5]
    expanded index = token*top_k + k and expanded_idx_to_permuted_idx).

    counts[e] = number of expanded rows routed to e; offsets = exclusive prefix sum;
    e2p[j] = offsets[ids_j] + #{j' < j : ids_j' = ids_j}; p2e is its inverse.
    """
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    R = flat.size
    counts = np.bincount(flat, minlength=num_experts).astype(np.int64)
    if counts.size != num_experts:
        raise ValueError("expert id out of range")
    offsets = np.zeros(num_experts + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    # stable sort by expert: equal experts keep ascending expanded index
    p2e = np.argsort(flat, kind="stable")
    e2p = np.empty(R, dtype=np.int64)
    e2p[p2e] = np.arange(R)
    return {
        "counts": counts.astype(np.int32),
        "offsets": offsets.astype(np.int32),
        "e2p": e2p.astype(np.int32),
        "p2e": p2e.astype(np.int32),
    }


def permute_rows(x_bits: np.ndarray, p2e: np.ndarray, top_k: int) -> np.ndarray:
    """x_perm[p] = x[p2e[p] // top_k] (a pure gather of bf16 rows; [P1] permute)."""
    return np.ascontiguousarray(x_bits[np.asarray(p2e) // top_k])


# ---------------------------------------------------------------- expert FFN with LoRA
@dataclass
class Adapter:
    """One resident LoRA slot: rank, scaling and per-expert weight getters (bf16 bits).

    a_gate_up(e) -> [r, H], b_gate_up(e) -> [2I, r], a_down(e) -> [r, I], b_down(e) -> [H, r].
    """

    rank: int
    scaling: float
    a_gate_up: BitsFn
    b_gate_up: BitsFn
    a_down: BitsFn
    b_down: BitsFn


def shared_outer_adapter(rank: int, scaling: float, a_gate_up: np.ndarray, b_gate_up: BitsFn,
                         a_down: BitsFn, b_down: np.ndarray) -> Adapter:
    """A shared-outer LoRA slot ([P1] section 2, "Shared-outer LoRA"): the gate_up A
    ([r, H]) and the down B ([H, r]) are one weight set that every expert uses (selected
    by the adapter alone), while the gate_up B and the down A stay per expert:

        g = W1[e] x + s_a B1[a][e] (A1[a] x)
        y = W2[e] h + s_a B2[a] (A2[a][e] h)

    The layer is otherwise the routed one, so the slot is an Adapter whose A1 and B2
    getters ignore the expert index.
    """
    return Adapter(rank, scaling, lambda e: a_gate_up, b_gate_up, a_down, lambda e: b_down)


def _valid_slot(slot: np.ndarray, num_slots: int) -> np.ndarray:
    s = np.asarray(slot, dtype=np.int64)
    return np.where((s >= 0) & (s < num_slots), s, -1)


def _expert_rows(X: np.ndarray, e: int, I: int, w_gate_up: BitsFn, w_down: BitsFn,
                 adapters: Sequence[Adapter], row_slot: np.ndarray) -> np.ndarray:
    """y for a block of rows routed to expert e ([P1] section 2(A) steps 1-5):

        g = W1[e] x + s_a B1[a][e] (A1[a][e] x)      (LoRA added before SwiGLU, unweighted)
        h = silu(g[:I]) * g[I:]
        y = W2[e] h + s_a B2[a][e] (A2[a][e] h)      (down LoRA on the activation)
    """
    W1 = _weights_f64(w_gate_up(e))
    W2 = _weights_f64(w_down(e))
    G = X @ W1.T
    for a, ad in enumerate(adapters):
        rows = np.nonzero(row_slot == a)[0]
        if rows.size == 0:
            continue
        A1 = bf16_bits_to_f64(ad.a_gate_up(e))
        B1 = bf16_bits_to_f64(ad.b_gate_up(e))
        G[rows] += ad.scaling * ((X[rows] @ A1.T) @ B1.T)
    Hact = silu(G[:, :I]) * G[:, I:]
    Y = Hact @ W2.T
    for a, ad in enumerate(adapters):
        rows = np.nonzero(row_slot == a)[0]
        if rows.size == 0:
            continue
        A2 = bf16_bits_to_f64(ad.a_down(e))
        B2 = bf16_bits_to_f64(ad.b_down(e))
        Y[rows] += ad.scaling * ((Hact[rows] @ A2.T) @ B2.T)
    return Y


def forward_permuted(x_bits: np.ndarray, offsets: np.ndarray, p2e: np.ndarray, top_k: int, I: int,
                     w_gate_up: BitsFn, w_down: BitsFn, adapters: Sequence[Adapter] = (),
                     token_slot: Optional[np.ndarray] = None) -> np.ndarray:
    """y_perm [R, H] fp64, unweighted, rows in expert-sorted order ([P5] return contract
    of the routed op: gemm2_output permuted and unweighted)."""
    x = bf16_bits_to_f64(x_bits)
    offsets = np.asarray(offsets, dtype=np.int64)
    p2e = np.asarray(p2e, dtype=np.int64)
    R = p2e.size
    H = x.shape[1]
    tok = p2e // top_k
    if token_slot is None or len(adapters) == 0:
        rslot = np.full(R, -1, dtype=np.int64)
    else:
        rslot = _valid_slot(token_slot, len(adapters))[tok]
    y = np.zeros((R, H), dtype=np.float64)
    for e in range(offsets.size - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi == lo:
            continue  # an expert with no rows reads no weights
        y[lo:hi] = _expert_rows(x[tok[lo:hi]], e, I, w_gate_up, w_down, adapters, rslot[lo:hi])
    return y


def finalize(y_perm: np.ndarray, weights: np.ndarray, e2p: np.ndarray) -> np.ndarray:
    """out[t] = sum_j w[t, j] * y_perm[e2p[t*k + j]] ([P5] _finalize_with_w2_lora)."""
    w = np.asarray(weights, dtype=np.float64)
    T, k = w.shape
    rows = np.asarray(y_perm, dtype=np.float64)[np.asarray(e2p, dtype=np.int64)].reshape(T, k, -1)
    return np.einsum("tk,tkh->th", w, rows)


# ---------------------------------------------------------------- whole layer
def layer(x_bits, logits_bits, top_k, I, w_gate_up: BitsFn, w_down: BitsFn, adapters=(),
          token_slot=None, method="renormalize", corr_bias=None, n_group=1, topk_group=1,
          routed_scaling_factor=1.0, num_experts=None) -> dict:
    """route -> permute -> expert FFN with LoRA -> finalize, all in fp64."""
    E = logits_bits.shape[1] if num_experts is None else num_experts
    ids, w = route(logits_bits, top_k, method, corr_bias, n_group, topk_group, routed_scaling_factor)
    srt = expert_sort(ids, E)
    y = forward_permuted(x_bits, srt["offsets"], srt["p2e"], top_k, I, w_gate_up, w_down,
                         adapters, token_slot)
    out = finalize(y, w, srt["e2p"])
    return {"ids": ids, "weights": w, **srt, "y_perm": y, "out": out}


def layer_sampled(x_bits, ids, weights, tokens: Sequence[int], I, w_gate_up: BitsFn, w_down: BitsFn,
                  adapters=(), token_slot=None) -> np.ndarray:
    """out rows for a subset of tokens, one token at a time, given its routing.

    This is the same definition as ``layer`` restricted to the listed tokens (the
    FFN of one routed row does not depend on the other rows), so it lets large
    workloads be checked on sampled outputs.
    """
    x = bf16_bits_to_f64(x_bits)
    ids = np.asarray(ids, dtype=np.int64)
    w = np.asarray(weights, dtype=np.float64)
    tokens = np.asarray(tokens, dtype=np.int64)
    k = ids.shape[1]
    slots = (np.full(x.shape[0], -1) if token_slot is None or len(adapters) == 0
             else _valid_slot(token_slot, len(adapters)))
    out = np.zeros((tokens.size, x.shape[1]), dtype=np.float64)
    # group the (token, j) pairs by expert so each expert's weights are decoded once
    pairs = [(int(ids[t, j]), i, j) for i, t in enumerate(tokens) for j in range(k)]
    pairs.sort()
    i0 = 0
    while i0 < len(pairs):
        e = pairs[i0][0]
        i1 = i0
        while i1 < len(pairs) and pairs[i1][0] == e:
            i1 += 1
        rows = [pairs[q][1] for q in range(i0, i1)]
        js = [pairs[q][2] for q in range(i0, i1)]
        X = x[tokens[rows]]
        Y = _expert_rows(X, e, I, w_gate_up, w_down, adapters, slots[tokens[rows]])
        for q, (r, j) in enumerate(zip(rows, js)):
            out[r] += w[tokens[r], j] * Y[q]
        i0 = i1
    return out
