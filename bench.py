#!/usr/bin/env python3
"""Throughput of the routed MoE-LoRA layer on one MI355X.

One step = route -> permute (fused into the GEMM loads) -> forward (gate_up GEMM with
the LoRA delta before SwiGLU, down GEMM with the down LoRA) -> finalize, on one batch of
synthetic bf16 inputs already resident in HBM.  Prints ONE JSON line.

    python bench.py [--steps K] [--warmup W] [--config 2]

The default workload is the decode batch of a Qwen3-30B-A3B-like MoE block (T=64,
hidden 2048, inter 768, 128 experts, top-8, one rank-16 adapter on gate_up and down).
"""

from __future__ import annotations

import argparse
import ctypes
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, help="named workload id (1-5)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a 1 GiB device copy (for HBM counter calibration) and exit")
    ap.add_argument("--only-lora-on", action="store_true",
                    help="run only the LoRA-on leg (for counter collection)")
    ap.add_argument("--quiet", action="store_true")
    ap.add_argument("--weights", choices=("packed-gate-up", "packed", "row-major"),
                    default="packed",
                    help="expert weight layout the GEMMs read: the gate_up weights (or both) "
                         "tile-packed once before timing, or both row-major")
    return ap.parse_args()


class HipEvents:
    """Raw hipEvent_t handles through the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            h = ctypes.c_void_p()
            assert self.hip.hipEventCreate(ctypes.byref(h)) == 0
            evs.append(h)
        return evs

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.hip.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, evs):
        for h in evs:
            self.hip.hipEventDestroy(h)


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
    if not rec or rec.get("moe_gemm_sha") != kernel_source_hash():
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


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on exactly one GPU (got --gpus {args.gpus}); "
              "multi-GPU sharding is not implemented", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    if args.copy_calibration:
        copy_calibration()
        return

    from mixture_experts_ffn_02_amd import moe_lora as ml
    from synth import NAMED_CONFIGS, Workload

    cfg = NAMED_CONFIGS[args.config]
    wl = Workload(cfg, seed=0)
    dev = torch.device("cuda:0")

    def log(msg):
        if not args.quiet:
            print(f"[bench] {msg}", file=sys.stderr, flush=True)

    def t16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev)

    def stack_to_device(fn, shape):
        out = torch.empty((cfg.E,) + tuple(shape), dtype=torch.int16, device=dev)
        for e0, blk in wl.expert_chunks(fn, 8):
            out[e0:e0 + blk.shape[0]].copy_(torch.from_numpy(blk.view(np.int16)))
        return out

    log(f"generating {cfg.name}")
    x_np, logits_np, slots_np = wl.x(), wl.logits(), wl.token_slot()
    bias_np = wl.correction_bias()
    x, logits = t16(x_np), t16(logits_np)
    bias = torch.from_numpy(bias_np).to(dev) if bias_np is not None else None
    w1 = stack_to_device("w_gate_up", (2 * cfg.I, cfg.H))
    w2 = stack_to_device("w_down", (cfg.H, cfg.I))
    lora_t = [{k: t16(v) for k, v in wl.lora_all(a).items()} for a in range(cfg.num_slots)]
    routing = ml.ROUTING_DEEPSEEK_V3 if cfg.routing == "deepseek_v3" else ml.ROUTING_RENORMALIZE
    packed = {"packed-gate-up": ml.PACKED_GATE_UP, "packed": ml.PACKED_GATE_UP | ml.PACKED_DOWN,
              "row-major": 0}[args.weights]
    layer = ml.MoELoRALayer(cfg.H, cfg.I, cfg.E, cfg.top_k, w1, w2, routing, cfg.n_group,
                            cfg.topk_group, cfg.routed_scaling_factor, bias, gather_on_load=True,
                            packed_weights=packed)
    # the same weights in the row-major layout, for the bench line's comparison leg
    layer_rm = ml.MoELoRALayer(cfg.H, cfg.I, cfg.E, cfg.top_k, w1, w2, routing, cfg.n_group,
                               cfg.topk_group, cfg.routed_scaling_factor, bias,
                               gather_on_load=True) if packed else None
    layer_p = ml.MoELoRALayer(cfg.H, cfg.I, cfg.E, cfg.top_k, layer.w_gate_up, layer.w_down, routing,
                              cfg.n_group, cfg.topk_group, cfg.routed_scaling_factor, bias,
                              gather_on_load=False, weights_prepacked=packed)
    lora = ml.LoRASlots(torch.from_numpy(slots_np).to(dev), [s.rank for s in cfg.slots],
                        [s.scaling for s in cfg.slots], [d["a_gate_up"] for d in lora_t],
                        [d["b_gate_up"] for d in lora_t], [d["a_down"] for d in lora_t],
                        [d["b_down"] for d in lora_t]) if cfg.num_slots else None

    hip = HipEvents()
    stream = torch.cuda.current_stream()

    def timed(lyr, lr, steps, warmup, gate_up_events=False):
        opts_list = [None] * steps
        evs = []
        if gate_up_events:
            evs = hip.create(2 * steps)
            opts_list = []
            for i in range(steps):
                o = ml.Options()
                o.gate_up_event_begin = evs[2 * i].value
                o.gate_up_event_end = evs[2 * i + 1].value
                opts_list.append(o)
        for _ in range(warmup):
            lyr(x, logits, lr)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            lyr(x, logits, lr, opts=opts_list[i])
        torch.cuda.synchronize()
        dt = time.perf_counter() - t0
        gate_up_ms = None
        if gate_up_events:
            gate_up_ms = sum(hip.elapsed_ms(evs[2 * i], evs[2 * i + 1]) for i in range(steps)) / steps
            hip.destroy(evs)
        return dt / steps, gate_up_ms

    log("timing LoRA on (gather-on-load)")
    t_on, gate_up_ms = timed(layer, lora, args.steps, args.warmup, gate_up_events=True)
    if args.only_lora_on:
        print(json.dumps({"workload": cfg.name, "ms_per_step": round(t_on * 1e3, 4),
                          "gate_up_us": round(gate_up_ms * 1e3, 2)}), flush=True)
        return
    log("timing LoRA off (same kernels, no adapters)")
    t_off, gate_up_off_ms = timed(layer, None, args.steps, args.warmup, gate_up_events=True)
    log("timing LoRA on with the explicit permute call")
    t_perm, _ = timed(layer_p, lora, max(5, args.steps // 2), 3)
    t_two = None
    if lora is not None and cfg.T <= 256:
        log("timing LoRA on, two-stream decomposed path")
        side = torch.cuda.Stream()
        for _ in range(args.warmup):
            layer(x, logits, lora, side_stream=side)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        n2 = max(5, args.steps // 2)
        for _ in range(n2):
            layer(x, logits, lora, side_stream=side)
        torch.cuda.synchronize()
        t_two = (time.perf_counter() - t0) / n2

    t_rm = None
    if layer_rm is not None:
        log("timing LoRA on with the row-major weight layout")
        t_rm, _ = timed(layer_rm, lora, max(5, args.steps // 2), args.warmup)

    t_shared = None
    if lora is not None:
        log("timing LoRA on, shared-outer layout (one gate_up A and one down B per slot)")
        lora_so = ml.LoRASlots(lora.token_slot, lora.rank, lora.scaling,
                               [t16(wl.lora_a_gate_up_shared(a)) for a in range(cfg.num_slots)],
                               lora.b_gate_up, lora.a_down,
                               [t16(wl.lora_b_down_shared(a)) for a in range(cfg.num_slots)],
                               shared_outer=True)
        t_shared, _ = timed(layer, lora_so, max(5, args.steps // 2), args.warmup)

    t_graph = None
    if cfg.T <= 256:
        log("timing LoRA on, replays of one captured HIP graph of the step")
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            layer(x, logits, lora)
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            graph.replay()
        torch.cuda.synchronize()
        t_graph = (time.perf_counter() - t0) / args.steps
        del graph

    t_fp8, fp8_gate_up_ms, t_fp8_p2 = None, None, None
    fp8_ok = cfg.H % 128 == 0 and cfg.I % 128 == 0 and cfg.E * 3 * cfg.I * cfg.H <= (1 << 31)
    if fp8_ok:
        log("timing LoRA on with FP8 expert weights (E4M3 codes, fp32 scale per 128x128 block)")

        def fp8_stack(fn):
            pairs = [None] * cfg.E

            def fill(e):
                pairs[e] = fn(e)

            with ThreadPoolExecutor(8) as ex:
                list(ex.map(fill, range(cfg.E)))
            codes = torch.from_numpy(np.stack([p[0] for p in pairs])).to(dev)
            scales = torch.from_numpy(np.stack([p[1] for p in pairs])).to(dev)
            return codes, scales

        c1, s1 = fp8_stack(wl.w_gate_up_fp8)
        c2, s2 = fp8_stack(wl.w_down_fp8)
        layer_fp8 = ml.MoELoRALayer(cfg.H, cfg.I, cfg.E, cfg.top_k, c1, c2, routing, cfg.n_group,
                                    cfg.topk_group, cfg.routed_scaling_factor, bias, gather_on_load=True,
                                    packed_weights=packed, w_gate_up_scale=s1, w_down_scale=s2)
        t_fp8, fp8_gate_up_ms = timed(layer_fp8, lora, args.steps, args.warmup, gate_up_events=True)
        # power-of-two block scales with the fused scaled conversion (opts.fp8_pow2_scales)
        p1 = fp8_stack(lambda e: wl.w_gate_up_fp8(e, pow2=True))[1]
        p2 = fp8_stack(lambda e: wl.w_down_fp8(e, pow2=True))[1]
        layer_p2 = ml.MoELoRALayer(cfg.H, cfg.I, cfg.E, cfg.top_k, layer_fp8.w_gate_up, layer_fp8.w_down,
                                   routing, cfg.n_group, cfg.topk_group, cfg.routed_scaling_factor, bias,
                                   gather_on_load=True, weights_prepacked=packed, w_gate_up_scale=p1,
                                   w_down_scale=p2, fp8_pow2_scales=True)
        t_fp8_p2, _ = timed(layer_p2, lora, max(5, args.steps // 2), args.warmup)
        del layer_fp8, layer_p2, c1, c2, s1, s2, p1, p2

    # realized routing -> algorithmic bytes and flops
    layer(x, logits, lora)
    torch.cuda.synchronize()
    rt = layer.last_route(cfg.T, lora)
    ids = rt.topk_ids.cpu().numpy()
    offsets = rt.expert_offsets.cpu().numpy()
    counts = np.diff(offsets)
    active = int((counts > 0).sum())
    H, I, E, T, k = cfg.H, cfg.I, cfg.E, cfg.T, cfg.top_k
    R = T * k
    w_bytes_gu = active * 2 * I * H * 2
    w_bytes_dn = active * H * I * 2
    lora_gu, lora_all, lora_flops = 0, 0, 0
    if cfg.num_slots:
        for a, sp in enumerate(cfg.slots):
            rows = slots_np == a
            used = np.unique(ids[rows].reshape(-1)) if rows.any() else np.array([], dtype=int)
            lora_gu += len(used) * 2 * I * sp.rank * 2
            lora_all += len(used) * sp.rank * (2 * H + 3 * I) * 2
            lora_flops += int(rows.sum()) * k * 2 * sp.rank * (2 * H + 3 * I)
    io_bytes = T * H * 2 + T * E * 2 + T * H * 2 + (E * 4 if bias is not None else 0)
    layer_bytes = w_bytes_gu + w_bytes_dn + lora_all + io_bytes
    layer_flops = 2 * R * 3 * I * H + lora_flops
    gate_up_bytes = w_bytes_gu + lora_gu + T * H * 2 + R * I * 2
    # FP8 weights: one byte per weight plus one fp32 scale per 128 x 128 block
    gate_up_bytes_fp8 = (active * 2 * I * H + active * (2 * I // 128) * (H // 128) * 4 + lora_gu
                         + T * H * 2 + R * I * 2)
    gate_up_flops = 2 * R * 2 * I * H + (lora_flops * 2 * H // (2 * H + 3 * I) if lora_flops else 0)

    tok_on = T / t_on
    tok_off = T / t_off
    ridge = BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
    hbm_bound = (layer_flops / layer_bytes) < ridge
    if hbm_bound:
        achieved = gate_up_bytes / (gate_up_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4)}
    else:
        achieved = gate_up_flops / (gate_up_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": BF16_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / BF16_PEAK_TFLOPS, 4)}
    roof["kernel"] = "moe_gemm_kernel<MODE_GATEUP> (gate_up GEMM + LoRA expand + SwiGLU)"
    roof["kernel_avg_us"] = round(gate_up_ms * 1e3, 2)
    roof["algorithmic_bytes_per_launch"] = int(gate_up_bytes)
    roof["algorithmic_flops_per_launch"] = int(gate_up_flops)
    roof["traffic"] = committed_traffic(cfg.name)

    result = {
        "metric": METRIC,
        "value": round(tok_on, 1),
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
        "lora_off_value": round(tok_off, 1),
        "lora_ratio": round(tok_on / tok_off, 4),
        "ms_per_step_lora_off": round(t_off * 1e3, 4),
        "ms_per_step_explicit_permute": round(t_perm * 1e3, 4),
        "ms_per_step_two_stream": round(t_two * 1e3, 4) if t_two else None,
        "ms_per_step_graph_replay": round(t_graph * 1e3, 4) if t_graph else None,
        "ms_per_step_row_major_weights": round(t_rm * 1e3, 4) if t_rm else None,
        "fp8_weights": None if t_fp8 is None else {
            "ms_per_step": round(t_fp8 * 1e3, 4), "value": round(T / t_fp8, 1), "unit": "tokens/s",
            "weights": "E4M3 codes, fp32 scale per 128x128 block; LoRA bf16; codes "
                       + ("tile-packed" if packed else "row-major"),
            "gate_up_us": round(fp8_gate_up_ms * 1e3, 2),
            "gate_up_algorithmic_bytes": int(gate_up_bytes_fp8),
            "gate_up_achieved_gbs": round(gate_up_bytes_fp8 / (fp8_gate_up_ms * 1e-3) / 1e9, 1),
            "gate_up_hbm_frac": round(gate_up_bytes_fp8 / (fp8_gate_up_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
            "ms_per_step_pow2_scales": round(t_fp8_p2 * 1e3, 4)},
        "shared_outer": ({"ms_per_step": round(t_shared * 1e3, 4), "value": round(T / t_shared, 1),
                          "lora_ratio": round(t_off / t_shared, 4)} if t_shared else None),
        "layer_roofline": {
            "algorithmic_bytes": int(layer_bytes), "algorithmic_flops": int(layer_flops),
            "active_experts": active,
            "hbm_frac": round(layer_bytes / t_on / (HBM_PEAK_GBS * 1e9), 4),
            "mfma_frac": round(layer_flops / t_on / (BF16_PEAK_TFLOPS * 1e12), 4),
        },
        "roofline": roof,
        "gate_up_lora_off_us": round(gate_up_off_ms * 1e3, 2),
    }

    if not args.no_cpu_baseline:
        log("timing the fp64 oracle on the host")
        result["cpu_baseline"] = cpu_baseline(cfg, wl, x_np, logits_np, slots_np, bias_np,
                                              args.cpu_budget_s)
    print(json.dumps(result), flush=True)


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
