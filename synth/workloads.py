"""Seeded synthetic workloads for the routed MoE-LoRA expert layer.

The layer shapes follow the MoE blocks named on the pages: the bf16
Qwen3-30B-A3B-Instruct-2507 block used for the verification runs of
"[LoRA] bf16 MoE-LoRA for trtllm backend with two-stream overlap + routing opts"
(Verification section: hidden 2048, 128 experts, top-8, expert intermediate
768, dummy rank-16 adapter), and one GPU's share of a DeepSeek-V3 layer (the
DeepSeekV3 routing method listed by the vLLM ``TrtLlmBf16LoRAExperts`` API page,
``_supports_routing_method``).  No dataset or checkpoint is used: every tensor is
drawn here.

Recipe (fixed, so every tensor and every expert can be regenerated alone):
  * RNG = numpy ``Generator(PCG64(SeedSequence([seed, cfg_id, tensor_id, slot, expert])))``
  * draws are float32 ``standard_normal`` scaled by the tensor's std, then rounded
    to bf16 with round-to-nearest-even; the bf16 bit patterns are what both the
    oracle and the GPU consume.
  * the DeepSeek-V3 correction bias stays float32 (it is a routing parameter).
  * for the skewed prefill workload, a per-expert offset ~N(0, 0.5) (float32,
    drawn once) is added to the float32 logits before the bf16 rounding; this is
    part of data generation, not of the routing method.

Nothing in this module computes any part of the layer.
"""

from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Iterator, Optional, Sequence

import numpy as np

# tensor namespaces inside the seed sequence
_T_X = 1
_T_LOGITS = 2
_T_LOGIT_OFFSET = 3
_T_CORR_BIAS = 4
_T_SLOT = 5
_T_W1 = 10
_T_W2 = 11
_T_A1 = 20
_T_B1 = 21
_T_A2 = 22
_T_B2 = 23
_T_A1_SHARED = 24
_T_B2_SHARED = 25
_T_W1_FP8 = 30
_T_W2_FP8 = 31
_T_W1_SCALE = 32
_T_W2_SCALE = 33


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even); return uint16 bit patterns.

    Inputs are finite draws, so NaN handling is not needed here.
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u >> np.uint32(16)) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


@dataclass(frozen=True)
class SlotSpec:
    """One resident LoRA adapter slot: its rank and its scaling (alpha / r)."""

    rank: int
    scaling: float


@dataclass(frozen=True)
class LayerConfig:
    name: str
    cfg_id: int
    T: int
    H: int
    I: int
    E: int
    top_k: int
    routing: str = "renormalize"  # "renormalize" | "deepseek_v3"
    n_group: int = 1
    topk_group: int = 1
    routed_scaling_factor: float = 1.0
    corr_bias_std: float = 0.0  # DeepSeek-V3 correction bias std (float32); 0 = no bias tensor
    logit_offset_std: float = 0.0  # per-expert skew added to logits at generation time
    x_std: float = 1.0
    logit_std: float = 1.0
    w_std: float = 0.02
    lora_a_std: float = 0.02
    lora_b_std: float = 0.02
    slots: Sequence[SlotSpec] = field(default_factory=tuple)
    slot_assignment: str = "all0"  # "all0" | "uniform" | "none"

    @property
    def R(self) -> int:
        return self.T * self.top_k

    @property
    def num_slots(self) -> int:
        return len(self.slots)

    def describe(self) -> dict:
        d = {
            "T": self.T, "hidden": self.H, "inter": self.I, "experts": self.E,
            "top_k": self.top_k, "routing": self.routing,
            "lora_slots": [(s.rank, s.scaling) for s in self.slots],
        }
        if self.routing == "deepseek_v3":
            d.update(n_group=self.n_group, topk_group=self.topk_group,
                     routed_scaling_factor=self.routed_scaling_factor)
        return d


def make_config(**kw) -> LayerConfig:
    kw.setdefault("name", "custom")
    kw.setdefault("cfg_id", 100)
    if "slots" in kw:
        kw["slots"] = tuple(SlotSpec(*s) if not isinstance(s, SlotSpec) else s for s in kw["slots"])
    return LayerConfig(**kw)


_QWEN = dict(H=2048, I=768, E=128, top_k=8)

NAMED_CONFIGS = {
    # tiny layer: every path on a few tiles, parity-only
    1: LayerConfig(name="tiny_T16_H256_I128_E8_k2_r8", cfg_id=1, T=16, H=256, I=128, E=8, top_k=2,
                   w_std=0.02, lora_a_std=0.02, lora_b_std=0.01,
                   slots=(SlotSpec(8, 2.0),)),
    # decode batch of a Qwen3-30B-A3B-like MoE block: weight streaming, HBM-bound
    2: LayerConfig(name="decode_T64_H2048_I768_E128_k8_r16", cfg_id=2, T=64, **_QWEN,
                   slots=(SlotSpec(16, 2.0),)),
    # prefill at the same shapes with skewed expert loads: MFMA-bound
    3: LayerConfig(name="prefill_T8192_H2048_I768_E128_k8_r16", cfg_id=3, T=8192, **_QWEN,
                   logit_offset_std=0.5, slots=(SlotSpec(16, 2.0),)),
    # multi-adapter decode: four slots of different rank, slot per token ~ U{0..3}
    4: LayerConfig(name="multiadapter_T256_H2048_I768_E128_k8_r8-64", cfg_id=4, T=256, **_QWEN,
                   slots=(SlotSpec(8, 1.0), SlotSpec(16, 2.0), SlotSpec(32, 1.0), SlotSpec(64, 0.5)),
                   slot_assignment="uniform"),
    # one GPU's share of a DeepSeek-V3 layer with grouped sigmoid routing
    5: LayerConfig(name="dsv3_T1024_H7168_I2048_E256_k8_r32", cfg_id=5, T=1024, H=7168, I=2048, E=256,
                   top_k=8, routing="deepseek_v3", n_group=8, topk_group=4, routed_scaling_factor=2.5,
                   corr_bias_std=0.1, w_std=0.01, lora_a_std=0.01, lora_b_std=0.01,
                   slots=(SlotSpec(32, 1.0),)),
}


def _workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


class Workload:
    """Deterministic tensors for one LayerConfig and one seed (uint16 = bf16 bits)."""

    def __init__(self, cfg: LayerConfig, seed: int = 0):
        self.cfg = cfg
        self.seed = int(seed)

    # -- raw draws -------------------------------------------------------
    def _rng(self, tensor: int, slot: int = 0, expert: int = 0) -> np.random.Generator:
        ss = np.random.SeedSequence([self.seed, self.cfg.cfg_id, tensor, slot, expert])
        return np.random.Generator(np.random.PCG64(ss))

    def _normal_bf16(self, shape, std: float, tensor: int, slot: int = 0, expert: int = 0) -> np.ndarray:
        a = self._rng(tensor, slot, expert).standard_normal(size=shape, dtype=np.float32)
        if std != 1.0:
            a *= np.float32(std)
        return f32_to_bf16_bits(a)

    # -- activations and routing inputs ------------------------------------
    def x(self) -> np.ndarray:
        c = self.cfg
        return self._normal_bf16((c.T, c.H), c.x_std, _T_X)

    def logits(self) -> np.ndarray:
        c = self.cfg
        a = self._rng(_T_LOGITS).standard_normal(size=(c.T, c.E), dtype=np.float32)
        if c.logit_std != 1.0:
            a *= np.float32(c.logit_std)
        if c.logit_offset_std > 0.0:
            off = self._rng(_T_LOGIT_OFFSET).standard_normal(size=(c.E,), dtype=np.float32)
            off *= np.float32(c.logit_offset_std)
            a += off[None, :]
        return f32_to_bf16_bits(a)

    def correction_bias(self) -> Optional[np.ndarray]:
        c = self.cfg
        if c.routing != "deepseek_v3":
            return None
        if c.corr_bias_std <= 0.0:
            return np.zeros((c.E,), dtype=np.float32)
        b = self._rng(_T_CORR_BIAS).standard_normal(size=(c.E,), dtype=np.float32)
        b *= np.float32(c.corr_bias_std)
        return b

    def token_slot(self) -> np.ndarray:
        c = self.cfg
        if c.num_slots == 0 or c.slot_assignment == "none":
            return np.full((c.T,), -1, dtype=np.int32)
        if c.slot_assignment == "all0":
            return np.zeros((c.T,), dtype=np.int32)
        if c.slot_assignment == "uniform":
            return self._rng(_T_SLOT).integers(0, c.num_slots, size=(c.T,), dtype=np.int32)
        raise ValueError(f"unknown slot assignment {c.slot_assignment!r}")

    # -- expert weights (per expert, so large configs can stream) ------------
    def w_gate_up(self, e: int) -> np.ndarray:
        """[2I, H]: rows [0, I) gate, rows [I, 2I) up."""
        c = self.cfg
        return self._normal_bf16((2 * c.I, c.H), c.w_std, _T_W1, 0, e)

    def w_down(self, e: int) -> np.ndarray:
        """[H, I]."""
        c = self.cfg
        return self._normal_bf16((c.H, c.I), c.w_std, _T_W2, 0, e)

    def lora_a_gate_up(self, a: int, e: int) -> np.ndarray:
        c = self.cfg
        return self._normal_bf16((c.slots[a].rank, c.H), c.lora_a_std, _T_A1, a, e)

    def lora_b_gate_up(self, a: int, e: int) -> np.ndarray:
        c = self.cfg
        return self._normal_bf16((2 * c.I, c.slots[a].rank), c.lora_b_std, _T_B1, a, e)

    def lora_a_down(self, a: int, e: int) -> np.ndarray:
        c = self.cfg
        return self._normal_bf16((c.slots[a].rank, c.I), c.lora_a_std, _T_A2, a, e)

    def lora_b_down(self, a: int, e: int) -> np.ndarray:
        c = self.cfg
        return self._normal_bf16((c.H, c.slots[a].rank), c.lora_b_std, _T_B2, a, e)

    # shared-outer layout: one gate_up A and one down B per slot for all experts
    def lora_a_gate_up_shared(self, a: int) -> np.ndarray:
        c = self.cfg
        return self._normal_bf16((c.slots[a].rank, c.H), c.lora_a_std, _T_A1_SHARED, a)

    def lora_b_down_shared(self, a: int) -> np.ndarray:
        c = self.cfg
        return self._normal_bf16((c.H, c.slots[a].rank), c.lora_b_std, _T_B2_SHARED, a)

    # -- stacked forms ---------------------------------------------------
    # -- FP8 expert weights (E4M3 codes + one fp32 scale per 128 x 128 block) --------
    # root mean square of the E4M3 values when every finite code is equally likely (the
    # largest binade, 256 .. 448, dominates); scales divide it out for full-range codes
    FP8_FULL_RANGE_RMS = 100.0

    def _fp8_codes(self, shape, tensor: int, e: int, full_range: bool = False) -> np.ndarray:
        """Random E4M3 codes.  Default: uniform sign and mantissa, exponent field 4..7
        (magnitudes 0.125 .. 1.875 before scaling).  full_range: every finite code equally
        likely (+-0, the subnormals, up to +-448); the two NaN codes 0x7f / 0xff never."""
        g = self._rng(tensor, 0, e)
        if full_range:
            c = g.integers(0, 254, size=shape, dtype=np.uint16)
            return np.where(c >= 127, c + 1, c).astype(np.uint8)  # skip 0x7f
        sign = g.integers(0, 2, size=shape, dtype=np.uint8) << 7
        exp = g.integers(4, 8, size=shape, dtype=np.uint8) << 3
        man = g.integers(0, 8, size=shape, dtype=np.uint8)
        return sign | exp | man

    def _fp8_scales(self, n: int, k: int, tensor: int, e: int, pow2: bool,
                    full_range: bool = False) -> np.ndarray:
        """fp32 block scales around w_std: uniform in [0.5, 1.5) * w_std, or (pow2) the
        power of two nearest w_std times 2^{-1, 0, 1}.  Full-range codes: around
        w_std / FP8_FULL_RANGE_RMS instead."""
        c = self.cfg
        std = c.w_std / self.FP8_FULL_RANGE_RMS if full_range else c.w_std
        shape = ((n + 127) // 128, (k + 127) // 128)
        g = self._rng(tensor, 0, e)
        if pow2:
            base = np.round(np.log2(std))
            return np.ldexp(np.ones(shape, np.float32), (base + g.integers(-1, 2, size=shape)).astype(np.int32))
        return (g.uniform(0.5, 1.5, size=shape) * std).astype(np.float32)

    def w_gate_up_fp8(self, e: int, pow2: bool = False, full_range: bool = False) -> tuple:
        """Expert e's gate_up weight as (codes uint8 [2I, H], scales fp32 [2I/128, H/128])."""
        c = self.cfg
        return (self._fp8_codes((2 * c.I, c.H), _T_W1_FP8, e, full_range),
                self._fp8_scales(2 * c.I, c.H, _T_W1_SCALE, e, pow2, full_range))

    def w_down_fp8(self, e: int, pow2: bool = False, full_range: bool = False) -> tuple:
        """Expert e's down weight as (codes uint8 [H, I], scales fp32 [H/128, I/128])."""
        c = self.cfg
        return (self._fp8_codes((c.H, c.I), _T_W2_FP8, e, full_range),
                self._fp8_scales(c.H, c.I, _T_W2_SCALE, e, pow2, full_range))

    def _stack(self, fn, count: int, shape, experts: Optional[Sequence[int]] = None) -> np.ndarray:
        experts = list(range(count)) if experts is None else list(experts)
        out = np.empty((len(experts),) + tuple(shape), dtype=np.uint16)

        def fill(i):
            out[i] = fn(experts[i])

        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(len(experts))))
        return out

    def w_gate_up_all(self, experts: Optional[Sequence[int]] = None) -> np.ndarray:
        c = self.cfg
        return self._stack(self.w_gate_up, c.E, (2 * c.I, c.H), experts)

    def w_down_all(self, experts: Optional[Sequence[int]] = None) -> np.ndarray:
        c = self.cfg
        return self._stack(self.w_down, c.E, (c.H, c.I), experts)

    def lora_all(self, a: int, experts: Optional[Sequence[int]] = None) -> dict:
        """Per-slot stacked LoRA weights: dict of a_gate_up [E,r,H], b_gate_up [E,2I,r],
        a_down [E,r,I], b_down [E,H,r]."""
        c = self.cfg
        r = c.slots[a].rank
        return {
            "a_gate_up": self._stack(lambda e: self.lora_a_gate_up(a, e), c.E, (r, c.H), experts),
            "b_gate_up": self._stack(lambda e: self.lora_b_gate_up(a, e), c.E, (2 * c.I, r), experts),
            "a_down": self._stack(lambda e: self.lora_a_down(a, e), c.E, (r, c.I), experts),
            "b_down": self._stack(lambda e: self.lora_b_down(a, e), c.E, (c.H, r), experts),
        }

    def expert_chunks(self, fn_name: str, chunk: int = 8) -> Iterator[tuple[int, np.ndarray]]:
        """Yield (first_expert, stacked block) of ``chunk`` experts at a time, for streaming
        very large weight sets to the device without holding them on the host."""
        c = self.cfg
        fn = getattr(self, fn_name)
        for e0 in range(0, c.E, chunk):
            experts = range(e0, min(c.E, e0 + chunk))
            sample = fn(experts[0])
            block = np.empty((len(experts),) + sample.shape, dtype=np.uint16)
            block[0] = sample

            def fill(i):
                block[i] = fn(experts[i])

            with ThreadPoolExecutor(_workers()) as ex:
                list(ex.map(fill, range(1, len(experts))))
            yield e0, block

    def with_T(self, T: int) -> "Workload":
        return Workload(dataclasses.replace(self.cfg, T=T), self.seed)
