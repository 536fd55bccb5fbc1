"""FP8 expert weights through the C-ABI (moe_lora_forward_fp8) on the GPU.

Parity: the layer on E4M3 codes with 128 x 128 fp32 block scales against the fp64 oracle
on the dequantized weights (tile heights 16, 64 and 128 with LoRA; decode without LoRA).
Bit identity: with power-of-two block scales every dequantized weight is exact in bf16,
so the path that scales each weight in its conversion (opts.fp8_pow2_scales, and the
general path on 128-row tiles) must give the same bits as the bf16 kernels run on those
bf16 weights.  The general path on tiles of up to 64 rows scales the fp32 sum of each
128-wide K block instead (a different rounding order): held to the oracle's bar.
Code range: one case draws every finite E4M3 code (+-0, the subnormals, up to +-448), so
the hardware conversions (the general one and the fused scaled one) meet all of them.
"""

import numpy as np
import pytest
import torch

import oracle
from gpu_util import GpuLayer, assert_layer_close, dev, f64, say, t16
from mixture_experts_ffn_02_amd import moe_lora as ml
from synth import NAMED_CONFIGS, Workload, make_config

pytestmark = pytest.mark.gpu

MID8 = make_config(name="fp8_mid_T512_H512_I256_E32_k8", cfg_id=212, T=512, H=512, I=256, E=32, top_k=8,
                   slots=((32, 1.0), (16, 2.0), (8, 0.5)), slot_assignment="uniform")
TALL8 = make_config(name="fp8_tall_T1024_H256_I256_E8_k2", cfg_id=213, T=1024, H=256, I=256, E=8, top_k=2,
                    slots=((16, 2.0),))
# 16 rows per expert on average: 32-row gate_up and down tiles
SHORT8 = make_config(name="fp8_short_T64_H512_I256_E32_k8", cfg_id=214, T=64, H=512, I=256, E=32, top_k=8,
                     slots=((16, 2.0), (32, 1.0)), slot_assignment="uniform")
# 8 rows per expert on average: 16-row tiles, whose B stages keep the codes in LDS.  Tiles
# with two slots, or one of rank above 32, stage the expand's B rows as bf16 through the
# same buffers: loaded during the last K steps when the ranks are multiples of 8 (DEC8_MS),
# after the K loop otherwise (DEC8_ODD)
DEC8_MS = make_config(name="fp8_dec_T64_H512_I256_E64_k8_r16_64", cfg_id=217, T=64, H=512, I=256, E=64,
                      top_k=8, slots=((16, 2.0), (64, 1.0)), slot_assignment="uniform")
DEC8_ODD = make_config(name="fp8_dec_T64_H512_I256_E64_k8_r13_40", cfg_id=218, T=64, H=512, I=256, E=64,
                       top_k=8, slots=((13, 2.0), (40, 0.5)), slot_assignment="uniform")


def _stack(fn, E):
    codes, scales = zip(*(fn(e) for e in range(E)))
    return np.stack(codes), np.stack(scales)


class Fp8Case:
    def __init__(self, cfg, pow2=False, full_range=False):
        self.g = GpuLayer(Workload(cfg))
        c = self.cfg = cfg
        wl = self.g.wl
        self.c1, self.s1 = _stack(lambda e: wl.w_gate_up_fp8(e, pow2, full_range), c.E)
        self.c2, self.s2 = _stack(lambda e: wl.w_down_fp8(e, pow2, full_range), c.E)
        self.dq1 = {}
        self.dq2 = {}

    def w1(self, e):
        if e not in self.dq1:
            self.dq1[e] = oracle.fp8_block_weights(self.c1[e], self.s1[e])
        return self.dq1[e]

    def w2(self, e):
        if e not in self.dq2:
            self.dq2[e] = oracle.fp8_block_weights(self.c2[e], self.s2[e])
        return self.dq2[e]

    def layer(self, packed=0, pow2_path=False):
        c, g = self.cfg, self.g
        t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev())
        return ml.MoELoRALayer(c.H, c.I, c.E, c.top_k, t(self.c1), t(self.c2), g.routing, c.n_group,
                               c.topk_group, c.routed_scaling_factor, g.bias, packed_weights=packed,
                               w_gate_up_scale=t(self.s1), w_down_scale=t(self.s2),
                               fp8_pow2_scales=pow2_path)

    def run(self, with_lora=True, packed=0, pow2_path=False, side=None):
        g = self.g
        out = self.layer(packed, pow2_path)(g.x, g.logits, g.lora_slots() if with_lora else None,
                                            side_stream=side)
        torch.cuda.synchronize()
        return out.clone()

    def oracle(self, with_lora=True):
        c, g = self.cfg, self.g
        ads = g.oracle_adapters() if with_lora else []
        return oracle.layer(g.x_np, g.logits_np, c.top_k, c.I, self.w1, self.w2, ads, g.slots_np,
                            c.routing, g.bias_np, c.n_group, c.topk_group, c.routed_scaling_factor,
                            num_experts=c.E)


@pytest.mark.parametrize("cfg,with_lora", [(NAMED_CONFIGS[1], True), (NAMED_CONFIGS[2], True),
                                           (NAMED_CONFIGS[2], False), (DEC8_MS, True), (DEC8_ODD, True),
                                           (SHORT8, True), (MID8, True), (TALL8, True)],
                         ids=["tiny", "decode", "decode-base", "16row-two-slots", "16row-odd-ranks",
                              "short-32row", "mid-64row", "tall-128row"])
def test_fp8_layer_parity(cfg, with_lora):
    say(f"[fp8] {cfg.name} lora={with_lora}")
    case = Fp8Case(cfg)
    out = case.run(with_lora)
    ref = case.oracle(with_lora)
    assert_layer_close(f64(out), ref["out"], f"fp8 {cfg.name}")


def _bf16_from_dequant(case, which):
    codes, scales = (case.c1, case.s1) if which == 1 else (case.c2, case.s2)
    w = np.stack([oracle.fp8_block_weights(codes[e], scales[e]) for e in range(codes.shape[0])])
    t = torch.from_numpy(w).to(torch.bfloat16)
    assert torch.equal(t.to(torch.float64), torch.from_numpy(w))  # exact in bf16
    return t.to(dev())


@pytest.mark.parametrize("cfg", [NAMED_CONFIGS[1], NAMED_CONFIGS[2], DEC8_MS, MID8, TALL8],
                         ids=["tiny", "decode", "16row-two-slots", "mid-64row", "tall-128row"])
def test_fp8_pow2_scales_bit_identical_to_bf16_kernels(cfg):
    say(f"[fp8 vs bf16] {cfg.name}")
    case = Fp8Case(cfg, pow2=True)
    out8 = case.run()
    # the fused scaled conversion (opts.fp8_pow2_scales) gives the bf16 kernels' bits
    out_p2 = case.run(pow2_path=True, packed=ml.PACKED_GATE_UP | ml.PACKED_DOWN)
    c, g = case.cfg, case.g
    layer16 = ml.MoELoRALayer(c.H, c.I, c.E, c.top_k, _bf16_from_dequant(case, 1),
                              _bf16_from_dequant(case, 2), g.routing, c.n_group, c.topk_group,
                              c.routed_scaling_factor, g.bias)
    out16 = layer16(g.x, g.logits, g.lora_slots())
    torch.cuda.synchronize()
    assert torch.equal(out_p2, out16)
    # the general path: per-weight scaling on 128-row tiles gives the same bits, block-sum
    # scaling on shorter tiles stays within the oracle's bar
    if cfg is TALL8:
        assert torch.equal(out8, out16)
    assert_layer_close(f64(out8), case.oracle()["out"], f"fp8 general path, pow2 scales {cfg.name}")


@pytest.mark.parametrize("cfg", [NAMED_CONFIGS[1], NAMED_CONFIGS[2], DEC8_MS, DEC8_ODD, SHORT8, MID8, TALL8],
                         ids=["tiny", "decode", "16row-two-slots", "16row-odd-ranks", "short-32row", "mid-64row",
                              "tall-128row"])
def test_fp8_packed_layouts_bit_identical(cfg):
    """The FP8 tile-packed layout (each weight alone and both) only reorders the codes."""
    say(f"[fp8 packed] {cfg.name}")
    case = Fp8Case(cfg)
    ref = case.run()
    for packed in (ml.PACKED_GATE_UP, ml.PACKED_DOWN, ml.PACKED_GATE_UP | ml.PACKED_DOWN):
        assert torch.equal(case.run(packed=packed), ref), packed


@pytest.mark.parametrize("cfg", [NAMED_CONFIGS[2], DEC8_MS], ids=["decode", "16row-two-slots"])
def test_fp8_with_shared_outer_adapters(cfg):
    """FP8 expert weights under the shared-outer LoRA layout (one gate_up A and one down B
    per slot): held to the oracle, and bit-identical to the routed layout fed copies of the
    shared matrices for every expert."""
    say(f"[fp8 shared-outer] {cfg.name}")
    case = Fp8Case(cfg)
    c, g = case.cfg, case.g
    layer = case.layer()
    shared = layer(g.x, g.logits, g.lora_slots(shared_outer=True)).clone()
    copies = layer(g.x, g.logits, g.lora_slots(replicate_shared=True)).clone()
    torch.cuda.synchronize()
    assert torch.equal(shared, copies)
    ref = oracle.layer(g.x_np, g.logits_np, c.top_k, c.I, case.w1, case.w2, g.oracle_adapters(shared_outer=True),
                       g.slots_np, c.routing, g.bias_np, c.n_group, c.topk_group, c.routed_scaling_factor,
                       num_experts=c.E)
    assert_layer_close(f64(shared), ref["out"], f"fp8 shared-outer {cfg.name}")


def test_fp8_graph_replay_matches_oracle_and_eager():
    """The FP8 layer's calls (route, forward, finalize) captured in a HIP graph at the decode
    shape: every replay held to the oracle and equal to the eager result, with eager work
    of the same layer between replays, and after new inputs are written into the captured
    buffers."""
    cfg = NAMED_CONFIGS[2]
    say(f"[fp8 graph] {cfg.name}")
    case = Fp8Case(cfg)
    c, g = case.cfg, case.g
    wl2 = Workload(cfg, 1)
    x2_np, lg2_np = wl2.x(), wl2.logits()
    x2, lg2 = t16(x2_np), t16(lg2_np)
    want1 = case.oracle()["out"]
    want2 = oracle.layer(x2_np, lg2_np, c.top_k, c.I, case.w1, case.w2, g.oracle_adapters(), g.slots_np,
                         c.routing, g.bias_np, c.n_group, c.topk_group, c.routed_scaling_factor,
                         num_experts=c.E)["out"]
    layer, lora = case.layer(), g.lora_slots()
    x_in, lg_in = g.x.clone(), g.logits.clone()  # the captured input buffers

    def eager(x, lg):
        out = layer(x, lg, lora).clone()
        torch.cuda.synchronize()
        return out

    ref1 = eager(x_in, lg_in)  # also the warm-up
    ref2 = eager(x2, lg2)
    assert_layer_close(f64(ref1), want1, "fp8 eager, first inputs")
    assert_layer_close(f64(ref2), want2, "fp8 eager, second inputs")

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = layer(x_in, lg_in, lora)
    torch.cuda.synchronize()
    for i in range(3):
        graph.replay()
        torch.cuda.synchronize()
        assert_layer_close(f64(out), want1, f"fp8 replay {i}")
        assert torch.equal(out, ref1), f"fp8 replay {i} differs from the eager result"
        assert torch.equal(eager(x2, lg2), ref2)
    x_in.copy_(x2)
    lg_in.copy_(lg2)
    for i in range(2):
        graph.replay()
        torch.cuda.synchronize()
        assert_layer_close(f64(out), want2, f"fp8 replay {i} on refilled inputs")
        assert torch.equal(out, ref2), f"fp8 replay {i} on refilled inputs differs"


FINITE_E4M3 = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)


@pytest.mark.parametrize("cfg", [NAMED_CONFIGS[1], MID8], ids=["tiny", "mid-64row"])
def test_fp8_every_finite_code(cfg):
    """Weights whose codes span every finite E4M3 value: the general conversion (arbitrary
    scales) within the bar of the oracle; with power-of-two scales both conversions within
    the bar, and the scaled conversion bit-identical to the bf16 kernels on the exactly
    dequantized weights."""
    say(f"[fp8 full code range] {cfg.name}")
    case = Fp8Case(cfg, full_range=True)
    for codes in (case.c1, case.c2):
        np.testing.assert_array_equal(np.unique(codes), FINITE_E4M3)
    assert_layer_close(f64(case.run()), case.oracle()["out"], f"fp8 all codes {cfg.name}")
    case2 = Fp8Case(cfg, pow2=True, full_range=True)
    ref = case2.oracle()["out"]
    out8 = case2.run()
    assert_layer_close(f64(out8), ref, f"fp8 all codes pow2 scales {cfg.name}")
    out_p2 = case2.run(pow2_path=True, packed=ml.PACKED_GATE_UP | ml.PACKED_DOWN)
    assert_layer_close(f64(out_p2), ref, f"fp8 all codes pow2 path {cfg.name}")
    c, g = case2.cfg, case2.g
    layer16 = ml.MoELoRALayer(c.H, c.I, c.E, c.top_k, _bf16_from_dequant(case2, 1),
                              _bf16_from_dequant(case2, 2), g.routing, c.n_group, c.topk_group,
                              c.routed_scaling_factor, g.bias)
    out16 = layer16(g.x, g.logits, g.lora_slots())
    torch.cuda.synchronize()
    assert torch.equal(out_p2, out16)


def test_fp8_with_side_stream_runs_the_fused_path():
    """A side stream given to the FP8 entry point is left unused: the call runs the fused
    path (the decomposed two-stream path is bf16 only) and gives the same bits."""
    cfg = NAMED_CONFIGS[2]
    say(f"[fp8 side stream] {cfg.name}")
    case = Fp8Case(cfg)
    ref = case.run()
    side = torch.cuda.Stream()
    out = case.run(side=side)
    assert torch.equal(out, ref)
    assert_layer_close(f64(out), case.oracle()["out"], "fp8 decode with a side stream")
    opts = ml.Options()
    opts.force_path = 2
    g = case.g
    with pytest.raises(ml.MoELoRAError) as ei:
        case.layer()(g.x, g.logits, g.lora_slots(), side_stream=side, opts=opts)
    assert ei.value.status == ml._lib.ERR_UNSUPPORTED
