"""Benchmark of the FP4 weight-only MoE decode layer on one MI355X.

Workload: the NVFP4 MTP-verify decode layer (4 tokens x top-8 = 32 expanded
rows, E=256, hidden 2048, intermediate 768, three hot experts), seeded
synthetic inputs.  A step is one pass of the whole hot path over one layer:
qmoe_route_topk -> qmoe_fp4_gemv_fc1_swiglu -> qmoe_fp4_gemv_fc2 ->
qmoe_finalize.  Steps rotate over LAYERS distinct copies of the layer weights
so every timed weight byte comes from HBM, not from the 256 MB Infinity Cache.
The steps are captured once in a HIP graph and replayed (the launch path of a
serving loop); --eager times plain launches instead.

value = achieved GB/s on weight bytes (packed E2M1 + block scales + global
scales of the experts the routing actually selected) per layer.

roofline: the dominant kernel (FC1 GEMV + SwiGLU), HBM-bound; its average
duration comes from HIP events around graph replays that hold only FC1
launches over the rotated copies, recorded on the stream they run on.

cpu_baseline: the CPU oracle (test infrastructure, float64 numpy, one
thread) timed on the same layer.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 MoE decode GEMV µs/layer + achieved HBM GB/s (% of peak), 4–64 rows"
HBM_PEAK_GBS = 8000.0
LAYERS = 40


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=80)
    ap.add_argument("--eager", action="store_true")
    ap.add_argument("--workload", default="mtp4", choices=["mtp4", "mtp8", "decode", "mx_decode"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import fp4_weight_only_amd as q
    import synth
    from fp4_weight_only_amd.layer import MoELayer

    cfg = {"mtp4": synth.MTP4, "mtp8": synth.MTP8, "decode": synth.DECODE, "mx_decode": synth.MX_DECODE}[args.workload]
    layers = LAYERS if cfg.fmt == synth.NVFP4 else 8
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t0 = time.time()
    L = synth.layer_inputs(cfg)
    print(f"# generated {cfg.name} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    fmt = q.QMOE_FMT_NVFP4 if cfg.fmt == synth.NVFP4 else q.QMOE_FMT_MXFP4
    base = [to_dev(L.w1), to_dev(L.s1), None if L.g1 is None else to_dev(L.g1),
            to_dev(L.w2), to_dev(L.s2), None if L.g2 is None else to_dev(L.g2)]
    copies = []
    for i in range(layers):
        t = [None if b is None else (b if i == 0 else b.clone()) for b in base]
        copies.append((q.FP4Weights(t[0], t[1], t[2], fmt), q.FP4Weights(t[3], t[4], t[5], fmt)))
    logits = to_dev(L.logits)
    x = to_dev(L.x.view(np.int16)).view(torch.bfloat16)
    layer = MoELayer(cfg.T, cfg.E, cfg.k, cfg.H, cfg.I, copies[0][0], copies[0][1], device=dev)
    layer.run(logits, x)
    torch.cuda.synchronize()
    offsets = layer.offsets.cpu().numpy()
    D = int(np.count_nonzero(np.diff(offsets)))
    B = cfg.B
    fc1_w = cfg.H * cfg.I + (cfg.H // B) * 2 * cfg.I + (4 if L.g1 is not None else 0)
    fc2_w = cfg.I * (cfg.H // 2) + (cfg.I // B) * cfg.H + (4 if L.g2 is not None else 0)
    weight_bytes = D * (fc1_w + fc2_w)
    R = cfg.rows
    fc1_bytes = D * fc1_w + R * cfg.H * 2 + R * cfg.I * 2 + (cfg.E + 1 + R) * 4   # weights, x rows, h, maps
    print(f"# rows={R} distinct experts={D} weight bytes/layer={weight_bytes}", file=sys.stderr, flush=True)

    stream = torch.cuda.Stream()

    def step(i):
        w1, w2 = copies[i % layers]
        layer.set_weights(w1, w2)
        layer.run(logits, x)

    def fc1_only(i):
        w1, _ = copies[i % layers]
        layer.w1 = w1
        layer.fc1(x)

    def capture(fn, n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            for i in range(n):      # warm the allocator/launch path outside the capture
                fn(i)
        stream.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                fn(i)
        return g

    K, W = args.steps, args.warmup
    if args.eager:
        with torch.cuda.stream(stream):
            for i in range(W):
                step(i)
            stream.synchronize()
            t_start = torch.cuda.Event(enable_timing=True)
            t_end = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t_start.record(stream)
            for i in range(K):
                step(i)
            t_end.record(stream)
            torch.cuda.synchronize()
        total_ms = t_start.elapsed_time(t_end)
    else:
        graph = capture(step, layers)
        rem = K % layers
        graph_rem = capture(step, rem) if rem else None
        with torch.cuda.stream(stream):
            for _ in range(max(1, W // layers)):
                graph.replay()
            torch.cuda.synchronize()
            t_start = torch.cuda.Event(enable_timing=True)
            t_end = torch.cuda.Event(enable_timing=True)
            t_start.record(stream)
            for _ in range(K // layers):
                graph.replay()
            if graph_rem is not None:
                graph_rem.replay()
            t_end.record(stream)
            torch.cuda.synchronize()
        total_ms = t_start.elapsed_time(t_end)
    ms_per_step = total_ms / K
    value = weight_bytes / (ms_per_step * 1e-3) / 1e9

    # dominant kernel: FC1 GEMV + SwiGLU, replayed alone over the rotated copies
    g1 = capture(fc1_only, layers)
    reps = 10
    with torch.cuda.stream(stream):
        g1.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g1.replay()
        e1.record(stream)
        torch.cuda.synchronize()
    fc1_us = e0.elapsed_time(e1) * 1e3 / (reps * layers)
    fc1_gbs = fc1_bytes / (fc1_us * 1e-6) / 1e9
    layer.set_weights(*copies[0])

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "rows": R, "distinct_experts": D, "layer_copies": layers,
                   "launch": "eager" if args.eager else "hip_graph"},
        "us_per_layer": round(ms_per_step * 1e3, 3),
        "hbm_frac_weight_bytes": round(value / HBM_PEAK_GBS, 4),
        "weight_bytes_per_layer": weight_bytes,
        "roofline": {"bound": "hbm", "kernel": "fp4_gemv_kernel (FC1+SwiGLU)", "achieved": round(fc1_gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(fc1_gbs / HBM_PEAK_GBS, 4),
                     "traffic": None, "avg_us": round(fc1_us, 3), "bytes_per_launch": fc1_bytes},
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(L, weight_bytes, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def cpu_baseline(L, weight_bytes, budget_s):
    """The oracle as it stands, one thread, on the same layer (bounded sample)."""
    from threadpoolctl import threadpool_limits

    from oracle import moe
    with threadpool_limits(limits=1):
        n, t0 = 0, time.perf_counter()
        while True:
            moe.layer(L)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s or n >= 20:
                break
    per_layer = el / n
    return {"value": round(weight_bytes / per_layer / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} full layers of {L.cfg.name} (route, FC1+SwiGLU, FC2, finalize), float64 numpy, "
                      f"{per_layer * 1e3:.1f} ms/layer",
            "host_cores_total": os.cpu_count()}


if __name__ == "__main__":
    main()
