"""Pins for the oracle's FP8 expert weights (CPU only).

The E4M3 decode is checked code by code against torch's float8_e4m3fn (an independent
implementation of the OCP format), the block-scale layout against a Kronecker-product
construction, and the layer on FP8 weights against the already pinned bf16 layer on the
same weight values (power-of-two block scales keep every dequantized weight exactly
representable in bf16, so both definitions must agree exactly).
"""

import numpy as np
import torch

import oracle
from helpers import oracle_adapters
from synth import Workload, make_config

FP8_SMALL = make_config(name="fp8_small", cfg_id=111, T=24, H=256, I=128, E=4, top_k=2,
                        slots=((8, 2.0), (4, 0.5)), slot_assignment="uniform", w_std=0.05)


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))  # -0 for 0x80


def test_e4m3_landmarks():
    v = oracle.e4m3_to_f64(np.array([0x38, 0x7E, 0x01, 0x08, 0xB8, 0x00], dtype=np.uint8))
    assert list(v) == [1.0, 448.0, 2.0 ** -9, 2.0 ** -6, -1.0, 0.0]
    pos = oracle.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)  # finite positive codes are ordered by value


def test_block_scale_layout():
    rng = np.random.default_rng(0)
    codes = np.full((300, 260), 0x38, dtype=np.uint8)  # every value 1.0
    scales = rng.uniform(0.5, 2.0, size=(3, 3)).astype(np.float32)
    w = oracle.fp8_block_weights(codes, scales)
    ref = np.kron(scales.astype(np.float64), np.ones((128, 128)))[:300, :260]
    assert np.array_equal(w, ref)


def _bf16_bits_exact(w64):
    t = torch.from_numpy(w64).to(torch.bfloat16)
    assert np.array_equal(t.to(torch.float64).numpy(), w64)  # exactly representable
    return t.view(torch.int16).numpy().view(np.uint16)


def test_fp8_layer_equals_bf16_layer_on_the_same_values():
    wl = Workload(FP8_SMALL)
    c = wl.cfg
    w1 = {e: oracle.fp8_block_weights(*wl.w_gate_up_fp8(e, pow2=True)) for e in range(c.E)}
    w2 = {e: oracle.fp8_block_weights(*wl.w_down_fp8(e, pow2=True)) for e in range(c.E)}
    b1 = {e: _bf16_bits_exact(w1[e]) for e in range(c.E)}
    b2 = {e: _bf16_bits_exact(w2[e]) for e in range(c.E)}
    args = (wl.x(), wl.logits(), c.top_k, c.I)
    kw = dict(adapters=oracle_adapters(wl), token_slot=wl.token_slot(), num_experts=c.E)
    fp8 = oracle.layer(*args, w1.__getitem__, w2.__getitem__, **kw)
    bf16 = oracle.layer(*args, b1.__getitem__, b2.__getitem__, **kw)
    assert np.array_equal(fp8["out"], bf16["out"])
    assert np.abs(fp8["out"]).max() > 0
