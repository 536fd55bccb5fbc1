#!/usr/bin/env python3
"""Throughput of the routed MoE-LoRA layer on one MI355X.

One step = route -> permute (fused into the GEMM loads) -> forward (gate_up GEMM with
the LoRA delta before SwiGLU, down GEMM with the down LoRA) -> finalize, on one batch of
synthetic bf16 inputs already resident in HBM.  Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--config 2] [--configs 1,2,3,4,5]

The headline workload (--config, default 2) is the decode batch of a Qwen3-30B-A3B-like
MoE block (T=64, hidden 2048, inter 768, 128 experts, top-8, one rank-16 adapter on
gate_up and down): K back-to-back steps bracketed by device synchronizations give
`ms_per_step` and `value`.  The `configs` object then measures every named workload
(tiny, decode, prefill, multi-adapter, DeepSeek-V3 share) under the flushed protocol:
per-step HIP-event times with a 1 GiB scratch read between steps (outside the events,
so no weight or adapter bytes stay in L2 or the 256 MB MALL from one step to the next),
reported as median, p10 and p90, LoRA on and off, with the gate_up GEMM's roofline.

`--only LEG` runs one leg of one workload and prints a short JSON line (for kernel traces
and counters under a profiler).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
METRIC = "MoE-LoRA layer tokens/s (bf16, 1 GPU) + % of no-LoRA base-MoE throughput"
LEGS = ("lora-on", "lora-off", "two-stream", "decomposed-one-stream", "explicit-permute", "row-major",
        "shared-outer", "graph", "fp8", "fp8-pow2")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, help="headline workload id (1-5)")
    ap.add_argument("--configs", default="1,2,3,4,5",
                    help="workload ids measured under the flushed protocol ('' = none)")
    ap.add_argument("--reps", type=int, default=50, help="flushed reps for the decode-sized workloads")
    ap.add_argument("--reps-large", type=int, default=20, help="flushed reps for the prefill and "
                    "DeepSeek-V3-sized workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (for HBM counter calibration) and exit")
    ap.add_argument("--only", choices=LEGS, default=None,
                    help="run only this leg of the --config workload (for traces and counters)")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--weights", choices=("packed-gate-up", "packed", "row-major"),
                    default="packed",
                    help="expert weight layout the GEMMs read: the gate_up weights (or both) "
                         "tile-packed once before timing, or both row-major")
    return ap.parse_args()


def kernel_source_hash() -> str:
    p = os.path.join(ROOT, "mixture_experts_ffn_02_amd", "csrc", "moe_gemm.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def committed_traffic(workload: str):
    """HBM traffic of the gate_up GEMM from the committed counter summary, if it was taken
    on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "gate_up_gemm_traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    rec = d.get(workload)
    if not rec or d.get("moe_gemm_sha") != kernel_source_hash():
        return None
    return rec.get("traffic_bytes_per_launch")


def copy_calibration():
    import torch

    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read_per_launch": n, "bytes_written_per_launch": n}))


class Events:
    """Timing events on torch's current stream (the one the layer runs on).  Each is
    recorded once at creation, so its HIP event exists and its raw handle can be handed to
    the library, which records it around the gate_up GEMM launch."""

    def __init__(self, n: int):
        import torch

        self.ev = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in self.ev:
            e.record()

    def handle(self, i: int) -> int:
        return self.ev[i].cuda_event

    def ms(self, i: int, j: int) -> float:
        return self.ev[i].elapsed_time(self.ev[j])


class Workbench:
    """One named workload resident on the device: inputs, weights (tile-packed as asked),
    adapters, and the layer objects of the legs."""

    def __init__(self, cfg_id: int, weights: str, log):
        import numpy as np
        import torch

        from mixture_experts_ffn_02_amd import moe_lora as ml
        from synth import NAMED_CONFIGS, Workload

        self.ml = ml
        cfg = self.cfg = NAMED_CONFIGS[cfg_id]
        wl = self.wl = Workload(cfg, seed=0)
        dev = self.dev = torch.device("cuda:0")
        self.t16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

        def stack_to_device(fn, shape):
            out = torch.empty((cfg.E,) + tuple(shape), dtype=torch.int16, device=dev)
            for e0, blk in wl.expert_chunks(fn, 16):
                out[e0:e0 + blk.shape[0]].copy_(torch.from_numpy(blk.view(np.int16)))
            return out

        log(f"generating {cfg.name}")
        self.x_np, self.logits_np, self.slots_np = wl.x(), wl.logits(), wl.token_slot()
        self.bias_np = wl.correction_bias()
        self.x, self.logits = self.t16(self.x_np), self.t16(self.logits_np)
        self.bias = torch.from_numpy(self.bias_np).to(dev) if self.bias_np is not None else None
        self.w1 = stack_to_device("w_gate_up", (2 * cfg.I, cfg.H))
        self.w2 = stack_to_device("w_down", (cfg.H, cfg.I))
        lora_t = [{k: self.t16(v) for k, v in wl.lora_all(a).items()} for a in range(cfg.num_slots)]
        self.routing = ml.ROUTING_DEEPSEEK_V3 if cfg.routing == "deepseek_v3" else ml.ROUTING_RENORMALIZE
        self.packed = {"packed-gate-up": ml.PACKED_GATE_UP, "packed": ml.PACKED_GATE_UP | ml.PACKED_DOWN,
                       "row-major": 0}[weights]
        self.layer = self.make_layer(self.w1, self.w2, packed_weights=self.packed)
        self.lora = ml.LoRASlots(torch.from_numpy(self.slots_np).to(dev), [s.rank for s in cfg.slots],
                                 [s.scaling for s in cfg.slots], [d["a_gate_up"] for d in lora_t],
                                 [d["b_gate_up"] for d in lora_t], [d["a_down"] for d in lora_t],
                                 [d["b_down"] for d in lora_t]) if cfg.num_slots else None

    def make_layer(self, w1, w2, **kw):
        c = self.cfg
        kw.setdefault("gather_on_load", True)
        return self.ml.MoELoRALayer(c.H, c.I, c.E, c.top_k, w1, w2, self.routing, c.n_group, c.topk_group,
                                    c.routed_scaling_factor, self.bias, **kw)

    def step(self, layer, lora, opts=None, side=None):
        layer(self.x, self.logits, lora, side_stream=side, opts=opts)

    def gate_up_opts(self, evs: Events, i: int):
        o = self.ml.Options()
        o.gate_up_event_begin = evs.handle(2 * i)
        o.gate_up_event_end = evs.handle(2 * i + 1)
        return o

    def back_to_back(self, layer, lora, steps, warmup, gate_up=False, side=None, opts=None):
        """K steps back to back between two device synchronizations (wall clock); with
        gate_up, also the mean gate_up GEMM time from events the library records around its
        launch (those events idle the GPU between kernels, so such steps are not timed for
        the step time)."""
        import torch

        evs = Events(2 * steps) if gate_up else None
        olist = [self.gate_up_opts(evs, i) for i in range(steps)] if gate_up else [opts] * steps
        for _ in range(warmup):
            self.step(layer, lora, opts, side)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(layer, lora, olist[i], side)
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / steps
        gu = sum(evs.ms(2 * i, 2 * i + 1) for i in range(steps)) / steps if gate_up else None
        return dt, gu

    def flushed(self, layer, lora, reps, warmup, flush, side=None, gate_up=False):
        """Per-step HIP-event times with a 1 GiB scratch read before every step (outside the
        events: it evicts L2 and the 256 MB MALL without leaving dirty lines whose write-back
        would fall inside the step); returns the step times in ms, one per rep, or with
        gate_up the gate_up GEMM's times from events the library records around its launch.
        An event recorded between two kernels idles the GPU for ~6 us, so the step times
        come from reps without the gate_up events and the kernel times from reps of their own."""
        import numpy as np
        import torch

        for _ in range(warmup):
            flush.sum()
            self.step(layer, lora, side=side)
        steps = Events(2 * reps)
        gus = Events(2 * reps) if gate_up else None
        for i in range(reps):
            flush.sum()
            steps.ev[2 * i].record()
            self.step(layer, lora, self.gate_up_opts(gus, i) if gate_up else None, side)
            steps.ev[2 * i + 1].record()
        torch.cuda.synchronize()
        if gate_up:
            return np.array([gus.ms(2 * i, 2 * i + 1) for i in range(reps)])
        return np.array([steps.ms(2 * i, 2 * i + 1) for i in range(reps)])

    def counts(self):
        """Algorithmic bytes and flops of one step from the realized routing (weights of
        the experts that received rows, LoRA of the (slot, expert) pairs used, the step's
        inputs and outputs)."""
        import numpy as np
        import torch

        cfg = self.cfg
        self.step(self.layer, self.lora)
        torch.cuda.synchronize()
        rt = self.layer.last_route(cfg.T, self.lora)
        ids = rt.topk_ids.cpu().numpy()
        offsets = rt.expert_offsets.cpu().numpy()
        active = int((np.diff(offsets) > 0).sum())
        H, I, E, T, k = cfg.H, cfg.I, cfg.E, cfg.T, cfg.top_k
        R = T * k
        w_gu = active * 2 * I * H * 2
        w_dn = active * H * I * 2
        lora_gu, lora_all, lora_flops = 0, 0, 0
        for a, sp in enumerate(cfg.slots):
            rows = self.slots_np == a
            used = np.unique(ids[rows].reshape(-1)) if rows.any() else np.array([], dtype=int)
            lora_gu += len(used) * 2 * I * sp.rank * 2
            lora_all += len(used) * sp.rank * (2 * H + 3 * I) * 2
            lora_flops += int(rows.sum()) * k * 2 * sp.rank * (2 * H + 3 * I)
        io = T * H * 2 + T * E * 2 + T * H * 2 + (E * 4 if self.bias is not None else 0)
        c = {
            "active_experts": active,
            "layer_bytes": w_gu + w_dn + lora_all + io,
            "layer_flops": 2 * R * 3 * I * H + lora_flops,
            "layer_bytes_no_lora": w_gu + w_dn + io,
            "layer_flops_no_lora": 2 * R * 3 * I * H,
            "gate_up_bytes": w_gu + lora_gu + T * H * 2 + R * I * 2,
            # FP8 weights: one byte per weight plus one fp32 scale per 128 x 128 block
            "gate_up_bytes_fp8": (active * 2 * I * H + active * (2 * I // 128) * (H // 128) * 4 + lora_gu
                                  + T * H * 2 + R * I * 2),
            "gate_up_flops": 2 * R * 2 * I * H + (lora_flops * 2 * H // (2 * H + 3 * I) if lora_flops else 0),
        }
        ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
        c["bound"] = "hbm" if c["layer_flops"] / c["layer_bytes"] < ridge else "mfma"
        return c

    def roofline(self, c, gate_up_ms):
        t = gate_up_ms * 1e-3
        if c["bound"] == "hbm":
            a = c["gate_up_bytes"] / t / 1e9
            r = {"bound": "hbm", "achieved": round(a, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                 "frac": round(a / HBM_PEAK_GBS, 4)}
        else:
            a = c["gate_up_flops"] / t / 1e12
            r = {"bound": "mfma", "achieved": round(a, 1), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                 "frac": round(a / BF16_PEAK_TFLOPS, 4)}
        r["kernel"] = "moe_gemm_kernel<MODE_GATEUP> (gate_up GEMM + LoRA expand + SwiGLU)"
        r["kernel_avg_us"] = round(gate_up_ms * 1e3, 2)
        r["algorithmic_bytes_per_launch"] = int(c["gate_up_bytes"])
        r["algorithmic_flops_per_launch"] = int(c["gate_up_flops"])
        r["traffic"] = committed_traffic(self.cfg.name)
        return r

    def layer_roofline(self, c, step_s):
        # the LoRA ratio a layer at its bound could reach: no-LoRA over LoRA-on bytes (HBM
        # bound) or flops (MFMA bound) of the same step
        nl, wl = (("layer_bytes_no_lora", "layer_bytes") if c["bound"] == "hbm"
                  else ("layer_flops_no_lora", "layer_flops"))
        return {"algorithmic_bytes": int(c["layer_bytes"]), "algorithmic_flops": int(c["layer_flops"]),
                "active_experts": c["active_experts"],
                "hbm_frac": round(c["layer_bytes"] / step_s / (HBM_PEAK_GBS * 1e9), 4),
                "mfma_frac": round(c["layer_flops"] / step_s / (BF16_PEAK_TFLOPS * 1e12), 4),
                "lora_ratio_at_bound": round(c[nl] / c[wl], 4)}

    def fp8_layers(self):
        """The same workload's expert weights as E4M3 codes with fp32 128 x 128 block scales
        (general scales, and power-of-two scales with the fused scaled conversion)."""
        import numpy as np
        import torch

        cfg, wl = self.cfg, self.wl

        def fp8_stack(fn):
            pairs = [None] * cfg.E

            def fill(e):
                pairs[e] = fn(e)

            with ThreadPoolExecutor(8) as ex:
                list(ex.map(fill, range(cfg.E)))
            codes = torch.from_numpy(np.stack([p[0] for p in pairs])).to(self.dev)
            scales = torch.from_numpy(np.stack([p[1] for p in pairs])).to(self.dev)
            return codes, scales

        c1, s1 = fp8_stack(wl.w_gate_up_fp8)
        c2, s2 = fp8_stack(wl.w_down_fp8)
        l8 = self.make_layer(c1, c2, packed_weights=self.packed, w_gate_up_scale=s1, w_down_scale=s2)
        p1 = fp8_stack(lambda e: wl.w_gate_up_fp8(e, pow2=True))[1]
        p2 = fp8_stack(lambda e: wl.w_down_fp8(e, pow2=True))[1]
        l8p = self.make_layer(l8.w_gate_up, l8.w_down, weights_prepacked=self.packed, w_gate_up_scale=p1,
                              w_down_scale=p2, fp8_pow2_scales=True)
        return l8, l8p

    def fp8_ok(self):
        c = self.cfg
        return c.H % 128 == 0 and c.I % 128 == 0 and c.E * 3 * c.I * c.H <= (1 << 31)

    def shared_outer_lora(self):
        cfg, lora = self.cfg, self.lora
        return self.ml.LoRASlots(lora.token_slot, lora.rank, lora.scaling,
                                 [self.t16(self.wl.lora_a_gate_up_shared(a)) for a in range(cfg.num_slots)],
                                 lora.b_gate_up, lora.a_down,
                                 [self.t16(self.wl.lora_b_down_shared(a)) for a in range(cfg.num_slots)],
                                 shared_outer=True)


def pct(a, q):
    import numpy as np

    return round(float(np.percentile(a, q)), 4)


def measure_flushed(wb: Workbench, reps: int, warmup: int, flush, log) -> dict:
    """The flushed protocol on one workload: LoRA on and off (same kernels, no adapters)."""
    cfg = wb.cfg
    log(f"flushed protocol: {cfg.name}, {reps} reps")
    st_on = wb.flushed(wb.layer, wb.lora, reps, warmup, flush)
    st_off = wb.flushed(wb.layer, None, reps, warmup, flush)
    gu_on = wb.flushed(wb.layer, wb.lora, reps, warmup, flush, gate_up=True)
    gu_off = wb.flushed(wb.layer, None, reps, warmup, flush, gate_up=True)
    import numpy as np

    c = wb.counts()
    med_on, med_off = float(np.median(st_on)), float(np.median(st_off))
    gu_med = float(np.median(gu_on))
    out = {
        "workload": cfg.name, "T": cfg.T, "reps": reps,
        "step_ms": {"median": round(med_on, 4), "p10": pct(st_on, 10), "p90": pct(st_on, 90)},
        "tokens_per_s": round(cfg.T / (med_on * 1e-3), 1),
        "lora_off_step_ms": {"median": round(med_off, 4), "p10": pct(st_off, 10), "p90": pct(st_off, 90)},
        "lora_off_tokens_per_s": round(cfg.T / (med_off * 1e-3), 1),
        "lora_ratio": round(med_off / med_on, 4),
        "gate_up_us": {"median": round(gu_med * 1e3, 2), "p10": round(pct(gu_on, 10) * 1e3, 2),
                       "p90": round(pct(gu_on, 90) * 1e3, 2)},
        "gate_up_lora_off_us_median": round(float(np.median(gu_off)) * 1e3, 2),
        "roofline": wb.roofline(c, gu_med),
        "layer_roofline": wb.layer_roofline(c, med_on * 1e-3),
    }
    if wb.lora is not None and cfg.T <= 256:
        # the two-stream decomposed path (side-stream LoRA shrink and expand, joined before the
        # activation) under the same protocol; its events bracket the step on the main stream,
        # which waits for the side stream inside the step
        import torch

        side = torch.cuda.Stream()
        st_two = wb.flushed(wb.layer, wb.lora, reps, warmup, flush, side=side)
        out["two_stream_step_ms"] = {"median": round(float(np.median(st_two)), 4), "p10": pct(st_two, 10),
                                     "p90": pct(st_two, 90)}
    if cfg.T <= 16:
        out["note"] = "parity-sized workload: launch-latency bound, roofline not meaningful"
    return out


def run_only(wb: Workbench, leg: str, steps: int, warmup: int):
    """One leg alone (for a profiler): K back-to-back steps, one JSON line."""
    import torch

    res = {"workload": wb.cfg.name, "leg": leg}
    if leg in ("lora-on", "lora-off"):
        lr = wb.lora if leg == "lora-on" else None
        t, _ = wb.back_to_back(wb.layer, lr, steps, warmup)
        _, gu = wb.back_to_back(wb.layer, lr, max(2, steps // 4), 1, gate_up=True)
        res["gate_up_us"] = round(gu * 1e3, 2)
    elif leg == "two-stream":
        side = torch.cuda.Stream()
        t, _ = wb.back_to_back(wb.layer, wb.lora, steps, warmup, side=side)
    elif leg == "decomposed-one-stream":
        o = wb.ml.Options()
        o.force_path = 2
        t, _ = wb.back_to_back(wb.layer, wb.lora, steps, warmup, opts=o)
    elif leg == "explicit-permute":
        lp = wb.make_layer(wb.layer.w_gate_up, wb.layer.w_down, gather_on_load=False,
                           weights_prepacked=wb.packed)
        t, _ = wb.back_to_back(lp, wb.lora, steps, warmup)
    elif leg == "row-major":
        t, _ = wb.back_to_back(wb.make_layer(wb.w1, wb.w2), wb.lora, steps, warmup)
    elif leg == "shared-outer":
        t, _ = wb.back_to_back(wb.layer, wb.shared_outer_lora(), steps, warmup)
    elif leg == "graph":
        t = graph_replay(wb, steps, warmup)
    else:
        l8, l8p = wb.fp8_layers()
        lyr = l8 if leg == "fp8" else l8p
        t, _ = wb.back_to_back(lyr, wb.lora, steps, warmup)
        _, gu = wb.back_to_back(lyr, wb.lora, max(2, steps // 4), 1, gate_up=True)
        res["gate_up_us"] = round(gu * 1e3, 2)
    res["ms_per_step"] = round(t * 1e3, 4)
    return res


def graph_replay(wb: Workbench, steps: int, warmup: int) -> float:
    import torch

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        wb.step(wb.layer, wb.lora)
    torch.cuda.synchronize()
    for _ in range(warmup):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        graph.replay()
    torch.cuda.synchronize()
    t = (time.perf_counter() - t0) / steps
    del graph
    return t


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU (got --gpus {args.gpus}); "
              "multi-GPU sharding is not implemented", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.copy_calibration:
        copy_calibration()
        return

    def log(msg):
        if not args.quiet:
            print(f"[bench] {msg}", file=sys.stderr, flush=True)

    wb = Workbench(args.config, args.weights, log)
    cfg = wb.cfg
    if args.only:
        print(json.dumps(run_only(wb, args.only, args.steps, args.warmup)), flush=True)
        teardown()
        return

    # ---- headline: K back-to-back steps between two synchronizations
    log("timing LoRA on (gather-on-load)")
    t_on, _ = wb.back_to_back(wb.layer, wb.lora, args.steps, args.warmup)
    log("timing LoRA off (same kernels, no adapters)")
    t_off, _ = wb.back_to_back(wb.layer, None, args.steps, args.warmup)
    log("timing the gate_up GEMM alone (library-recorded events, separate steps)")
    _, gate_up_ms = wb.back_to_back(wb.layer, wb.lora, args.steps, 2, gate_up=True)
    _, gate_up_off_ms = wb.back_to_back(wb.layer, None, args.steps, 2, gate_up=True)
    half = max(5, args.steps // 2)
    log("timing LoRA on with the explicit permute call")
    t_perm = run_only(wb, "explicit-permute", half, 3)["ms_per_step"] * 1e-3
    t_two = t_dec1 = None
    if wb.lora is not None and cfg.T <= 256:
        log("timing LoRA on, two-stream decomposed path (and the same path on one stream)")
        t_two = run_only(wb, "two-stream", half, args.warmup)["ms_per_step"] * 1e-3
        t_dec1 = run_only(wb, "decomposed-one-stream", half, args.warmup)["ms_per_step"] * 1e-3
    t_rm = None
    if wb.packed:
        log("timing LoRA on with the row-major weight layout")
        t_rm = run_only(wb, "row-major", half, args.warmup)["ms_per_step"] * 1e-3
    t_shared = None
    if wb.lora is not None:
        log("timing LoRA on, shared-outer layout (one gate_up A and one down B per slot)")
        t_shared = run_only(wb, "shared-outer", half, args.warmup)["ms_per_step"] * 1e-3
    t_graph = None
    if cfg.T <= 256:
        log("timing LoRA on, replays of one captured HIP graph of the step")
        t_graph = graph_replay(wb, args.steps, args.warmup)
    fp8 = None
    if wb.fp8_ok():
        log("timing LoRA on with FP8 expert weights (E4M3 codes, fp32 scale per 128x128 block)")
        l8, l8p = wb.fp8_layers()
        t_fp8, _ = wb.back_to_back(l8, wb.lora, args.steps, args.warmup)
        _, fp8_gu = wb.back_to_back(l8, wb.lora, half, 2, gate_up=True)
        t_fp8_p2, _ = wb.back_to_back(l8p, wb.lora, half, args.warmup)
        del l8, l8p
        fp8 = (t_fp8, fp8_gu, t_fp8_p2)

    c = wb.counts()
    T = cfg.T
    roof = wb.roofline(c, gate_up_ms)
    roof["traffic"] = committed_traffic(cfg.name)
    result = {
        "metric": METRIC,
        "value": round(T / t_on, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(t_on * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,sigma) bf16 tensors of the workload's shapes; no checkpoint)",
        "config": {"workload": cfg.name, **cfg.describe(), "parallelism": "single GPU",
                   "permute": "gathered inside the GEMM and shrink loads",
                   "weights": {"packed-gate-up": "gate_up tile-packed once before timing, down row-major",
                               "packed": "tile-packed once before timing",
                               "row-major": "row-major"}[args.weights]},
        "lora_off_value": round(T / t_off, 1),
        "lora_ratio": round(t_off / t_on, 4),
        "ms_per_step_lora_off": round(t_off * 1e3, 4),
        "ms_per_step_explicit_permute": round(t_perm * 1e3, 4),
        "ms_per_step_two_stream": round(t_two * 1e3, 4) if t_two else None,
        "ms_per_step_decomposed_one_stream": round(t_dec1 * 1e3, 4) if t_dec1 else None,
        "ms_per_step_graph_replay": round(t_graph * 1e3, 4) if t_graph else None,
        "ms_per_step_row_major_weights": round(t_rm * 1e3, 4) if t_rm else None,
        "fp8_weights": None if fp8 is None else {
            "ms_per_step": round(fp8[0] * 1e3, 4), "value": round(T / fp8[0], 1), "unit": "tokens/s",
            "weights": "E4M3 codes, fp32 scale per 128x128 block; LoRA bf16; codes "
                       + ("tile-packed" if wb.packed else "row-major"),
            "gate_up_us": round(fp8[1] * 1e3, 2),
            "gate_up_algorithmic_bytes": int(c["gate_up_bytes_fp8"]),
            "gate_up_achieved_gbs": round(c["gate_up_bytes_fp8"] / (fp8[1] * 1e-3) / 1e9, 1),
            "gate_up_hbm_frac": round(c["gate_up_bytes_fp8"] / (fp8[1] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "ms_per_step_pow2_scales": round(fp8[2] * 1e3, 4)},
        "shared_outer": ({"ms_per_step": round(t_shared * 1e3, 4), "value": round(T / t_shared, 1),
                          "lora_ratio": round(t_off / t_shared, 4)} if t_shared else None),
        "layer_roofline": wb.layer_roofline(c, t_on),
        "roofline": roof,
        "gate_up_lora_off_us": round(gate_up_off_ms * 1e3, 2),
    }

    # ---- every named workload under the flushed protocol
    ids = [int(v) for v in args.configs.split(",") if v.strip()]
    if ids:
        flush = torch.ones((1 << 30) // 4, dtype=torch.float32, device=wb.dev)  # 1 GiB, read per step
        per = {}
        for i in ids:
            if i == args.config:
                w = wb
            else:
                w = Workbench(i, args.weights, log)
            reps = args.reps_large if w.cfg.T >= 1024 else args.reps
            per[str(i)] = measure_flushed(w, reps, args.warmup, flush, log)
            if w is not wb:
                del w
                torch.cuda.empty_cache()
        result["configs"] = {"protocol": "per-step HIP events on the layer's stream, 1 GiB scratch "
                                         "read before every step outside the events; "
                                         f"{args.warmup} warm-up steps; median, p10, p90",
                             **per}
        del flush

    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host")
        result["cpu_baseline"] = cpu_baseline(cfg, wb.wl, wb.x_np, wb.logits_np, wb.slots_np, wb.bias_np,
                                              args.cpu_budget_s)
    print(json.dumps(result), flush=True)
    del wb
    teardown()


def teardown():
    """Finish all device work and hand the memory back before the interpreter exits, so no
    HIP object outlives the program's own use of it."""
    import gc

    import torch

    torch.cuda.synchronize()
    gc.collect()
    torch.cuda.empty_cache()
    torch.cuda.synchronize()


def cpu_baseline(cfg, wl, x_np, logits_np, slots_np, bias_np, budget_s):
    """The fp64 oracle as it stands, on the host cores, over whole batches of the same
    workload (cfg 3 and 5: a bounded token sample)."""
    import functools

    import numpy as np

    import oracle

    ads = []
    for a, sp in enumerate(cfg.slots):
        ads.append(oracle.Adapter(sp.rank, sp.scaling,
                                  functools.lru_cache(None)(lambda e, a=a: wl.lora_a_gate_up(a, e)),
                                  functools.lru_cache(None)(lambda e, a=a: wl.lora_b_gate_up(a, e)),
                                  functools.lru_cache(None)(lambda e, a=a: wl.lora_a_down(a, e)),
                                  functools.lru_cache(None)(lambda e, a=a: wl.lora_b_down(a, e))))
    w1 = functools.lru_cache(None)(wl.w_gate_up)
    w2 = functools.lru_cache(None)(wl.w_down)
    ntok = cfg.T if cfg.T <= 1024 else 64
    sample = f"{ntok} of {cfg.T} tokens, full layer (routing, expert FFN with LoRA, finalize)"
    ids, w = oracle.route(logits_np, cfg.top_k, cfg.routing, bias_np, cfg.n_group, cfg.topk_group,
                          cfg.routed_scaling_factor)
    toks = np.arange(ntok)
    # pre-generate the sampled experts' weights so generation is not timed
    for e in np.unique(ids[toks]):
        w1(int(e)), w2(int(e))
        for ad in ads:
            ad.a_gate_up(int(e)), ad.b_gate_up(int(e)), ad.a_down(int(e)), ad.b_down(int(e))
    reps, total = 0, 0.0
    while reps < 50 and (reps == 0 or total < budget_s):
        t0 = time.perf_counter()
        if ntok == cfg.T:
            oracle.layer(x_np, logits_np, cfg.top_k, cfg.I, w1, w2, ads, slots_np, cfg.routing, bias_np,
                         cfg.n_group, cfg.topk_group, cfg.routed_scaling_factor, num_experts=cfg.E)
        else:
            oracle.route(logits_np[:ntok], cfg.top_k, cfg.routing, bias_np, cfg.n_group,
                         cfg.topk_group, cfg.routed_scaling_factor)
            oracle.layer_sampled(x_np, ids, w, toks, cfg.I, w1, w2, ads, slots_np)
        total += time.perf_counter() - t0
        reps += 1
    threads = None
    try:
        from threadpoolctl import threadpool_info

        threads = max((i.get("num_threads", 1) for i in threadpool_info()), default=1)
    except Exception:
        threads = int(os.environ.get("OMP_NUM_THREADS", "1"))
    return {"value": round(ntok * reps / total, 2), "unit": "tokens/s", "cores": threads,
            "kind": "oracle", "sample": sample + f", {reps} rep(s), {total:.2f} s",
            "host_cpu_count": os.cpu_count(),
            "affinity_cores": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


if __name__ == "__main__":
    main()
