"""The seeded generators: bf16 rounding and determinism (CPU only)."""

import numpy as np
import torch

from synth import NAMED_CONFIGS, Workload, f32_to_bf16_bits


def test_bf16_rounding_is_round_to_nearest_even():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -1.00390625, 0.0, -0.0], np.float32)])
    want = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(f32_to_bf16_bits(a), want)


def test_workload_is_deterministic_and_streams_per_expert():
    wl = Workload(NAMED_CONFIGS[1])
    np.testing.assert_array_equal(wl.x(), Workload(NAMED_CONFIGS[1]).x())
    allw = wl.w_gate_up_all()
    for e in range(NAMED_CONFIGS[1].E):
        np.testing.assert_array_equal(allw[e], wl.w_gate_up(e))
    blocks = dict(wl.expert_chunks("w_down", chunk=3))
    np.testing.assert_array_equal(blocks[3][1], wl.w_down(4))
    assert not np.array_equal(Workload(NAMED_CONFIGS[1], seed=1).x(), wl.x())


def test_named_config_shapes_and_distributions():
    c4 = NAMED_CONFIGS[4]
    wl = Workload(c4)
    s = wl.token_slot()
    assert s.min() == 0 and s.max() == 3 and len(set(s.tolist())) == 4
    assert wl.lora_b_down(3, 0).shape == (2048, 64)
    c5 = NAMED_CONFIGS[5]
    b = Workload(c5).correction_bias()
    assert b.dtype == np.float32 and b.shape == (256,) and 0.05 < b.std() < 0.2
