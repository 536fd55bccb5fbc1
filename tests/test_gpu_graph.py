"""HIP-graph capture of the layer's calls (route, forward, finalize), on the fused
one-stream path and on the two-stream path whose LoRA work forks to a side stream and
joins before the activation.

The library allocates nothing and records only kernels and event waits on the streams it
is given, so the calls can be captured once and replayed.  Every replay is held to the fp64
oracle (a corruption that the eager path shares would pass a replay-equals-eager check)
and must also equal the eager result bit for bit, with eager work and synchronizations of
the program between the replays; a replay must follow new data written into the captured
input buffers, and is held to the oracle of those inputs.
"""

import pytest
import torch

from gpu_util import GpuLayer, assert_layer_close, f64, say, t16
from synth import NAMED_CONFIGS, Workload

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg_id", [2, 4], ids=lambda c: NAMED_CONFIGS[c].name)
@pytest.mark.parametrize("two_stream", [False, True], ids=["one_stream", "two_stream"])
def test_graph_replay_matches_oracle_and_eager(cfg_id, two_stream):
    cfg = NAMED_CONFIGS[cfg_id]
    say(f"[graph] {cfg.name} two_stream={two_stream}")
    g = GpuLayer(Workload(cfg, 0), stream_weights=True, keep_host=True)
    wl2 = Workload(cfg, 1)
    x2_np, lg2_np = wl2.x(), wl2.logits()
    x2, lg2 = t16(x2_np), t16(lg2_np)
    # the oracle of both input sets (same weights, adapters and token slots)
    want1 = g.oracle_layer()["out"]
    want2 = g.oracle_layer(x2_np, lg2_np)["out"]
    layer, lora = g.layer(), g.lora_slots()
    side = torch.cuda.Stream() if two_stream else None
    x_in, lg_in = g.x.clone(), g.logits.clone()  # the captured input buffers

    def eager(x, lg):
        out = layer(x, lg, lora, side_stream=side).clone()
        torch.cuda.synchronize()
        return out

    ref1 = eager(x_in, lg_in)  # also the warm-up: buffers and library events exist now
    ref2 = eager(x2, lg2)
    assert not torch.equal(ref1, ref2)
    assert_layer_close(f64(ref1), want1, "eager, first inputs")
    assert_layer_close(f64(ref2), want2, "eager, second inputs")

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        out = layer(x_in, lg_in, lora, side_stream=side)
    torch.cuda.synchronize()

    for i in range(3):
        graph.replay()
        torch.cuda.synchronize()
        assert_layer_close(f64(out), want1, f"replay {i}")
        assert torch.equal(out, ref1), f"replay {i} differs from the eager result"
        assert torch.equal(eager(x2, lg2), ref2)  # eager work on the same layer in between

    x_in.copy_(x2)
    lg_in.copy_(lg2)
    for i in range(2):
        graph.replay()
        torch.cuda.synchronize()
        assert_layer_close(f64(out), want2, f"replay {i} on refilled inputs")
        assert torch.equal(out, ref2), f"replay {i} on refilled inputs differs"
