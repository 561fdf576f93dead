"""Benchmark of the FP4 weight-only MoE expert path on one MI355X.

Default workload: the NVFP4 MTP-verify decode layer (4 tokens x top-8 = 32
expanded rows, E=256, hidden 2048, intermediate 768, three hot experts),
seeded synthetic inputs.  A step is one pass of the whole hot path over one
layer: qmoe_route_topk -> qmoe_fp4_gemv_fc1_swiglu -> qmoe_fp4_gemv_fc2_finalize
(FC2 and the weighted un-permute in one call, bit-identical to
qmoe_fp4_gemv_fc2 followed by qmoe_finalize).  Steps rotate over distinct copies of the layer weights so
every timed weight byte comes from HBM, not from the 256 MB Infinity Cache.
The steps are captured once in a HIP graph and replayed (the launch path of
a serving loop); --eager times plain launches instead.

value = achieved GB/s on weight bytes (packed E2M1 + block scales + global
scales of the experts the routing actually selected) per layer.

Other workloads (--workload): decode / mtp8 / mx_decode (same layer path),
prefill (MXFP4 512 tokens, grouped-GEMM path; also reports TFLOP/s and the
fraction of the bf16 MFMA peak), dequant (MXFP4 standalone dequant, GB/s on
read + write bytes), fp8 (the MTP-verify layer with FP8 E4M3 W8A16 weights:
qmoe_fp8_gemv_fc1_swiglu -> qmoe_fp8_gemv_fc2 -> qmoe_finalize), fp8_prefill
(the prefill layer with FP8 weights, grouped MFMA path), fp8_dequant (FP8
standalone dequant at the dequant workload's shape).  --calibrate-copy runs a plain device-to-device copy of
known size, the reference kernel for scaling HBM traffic counters.

roofline: the dominant kernel of the workload (FC1 for the layer workloads,
the dequant kernel for dequant), HBM-bound; its average duration comes from
HIP events around graph replays that hold only that call over the rotated
copies, recorded on the stream they run on.  roofline.traffic is the HBM
byte count per launch measured with FETCH_SIZE + WRITE_SIZE counters and
scaled by the copy calibration, read from profiles/ and reported only while
the kernel source it was taken on is unchanged (else null).

cpu_baseline: the C++ CPU oracle (test infrastructure, float64, single-
threaded) timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "NVFP4 MoE decode GEMV µs/layer + achieved HBM GB/s (% of peak), 4–64 rows"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
CSRC = os.path.join(ROOT, "fp4_weight_only_amd", "csrc")
LAYER_WORKLOADS = ("mtp4", "mtp8", "decode", "mx_decode", "prefill", "fp8", "fp8_prefill")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=80)
    ap.add_argument("--eager", action="store_true")
    ap.add_argument("--path", default="auto", choices=("auto", "gemv", "grouped"),
                    help="FC kernel path of the layer workloads (auto: the library's AUTO rule)")
    ap.add_argument("--workload", default="mtp4", choices=LAYER_WORKLOADS + ("dequant", "fp8_dequant"))
    ap.add_argument("--layer-call", default="auto", choices=("auto", "multi"),
                    help="decode layer: auto = one kernel launch where the shape allows "
                         "(qmoe_fp4_moe_layer_persistent), multi = the multi-launch fused calls")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="time a plain 1 GiB device copy (reference kernel for traffic counters) and exit")
    return ap.parse_args()


def kernel_sources_digest(files) -> str:
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(name: str, sources) -> int | None:
    """HBM bytes per launch from profiles/traffic_<name>.txt if its source digest is current."""
    path = os.path.join(ROOT, "profiles", f"traffic_{name}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if "=" in line and not line.startswith("#"):
                k, v = line.split("=", 1)
                vals[k.strip()] = v.strip()
    if vals.get("source_digest") != kernel_sources_digest(sources):
        return None
    return int(vals["traffic_bytes_per_launch"])


class Timer:
    """Graph capture + HIP-event timing on one stream."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream

    def capture(self, fn, n):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(self.stream):
            for i in range(n):      # warm the allocator/launch path outside the capture
                fn(i)
        self.stream.synchronize()
        with torch.cuda.graph(g, stream=self.stream):
            for i in range(n):
                fn(i)
        return g

    def run(self, fn, period, steps, warmup, eager=False):
        """Average ms per fn call over `steps` calls (fn(i) rotates over `period` inputs)."""
        torch = self.torch
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(self.stream):
            if eager:
                for i in range(warmup):
                    fn(i)
                torch.cuda.synchronize()
                ev0.record(self.stream)
                for i in range(steps):
                    fn(i)
                ev1.record(self.stream)
                torch.cuda.synchronize()
            else:
                g = self.capture(fn, period)
                rem = steps % period
                g_rem = self.capture(fn, rem) if rem else None
                for _ in range(max(1, warmup // period)):
                    g.replay()
                torch.cuda.synchronize()
                ev0.record(self.stream)
                for _ in range(steps // period):
                    g.replay()
                if g_rem is not None:
                    g_rem.replay()
                ev1.record(self.stream)
                torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) / steps


def base_result(metric, value, unit, args, ms, config, dtype="bf16", higher=True):
    return {"metric": metric, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": args.steps,
            "warmup": args.warmup, "ms_per_step": round(ms, 6), "higher_is_better": higher, "scaling": "weak",
            "vs_baseline": None, "dtype": dtype, "data": "synthetic", "config": config}


def bench_layer(args, torch, q, synth, np):
    from fp4_weight_only_amd.layer import MoELayer

    cfg = {"mtp4": synth.MTP4, "mtp8": synth.MTP8, "decode": synth.DECODE, "mx_decode": synth.MX_DECODE,
           "prefill": synth.MX_PREFILL, "fp8": synth.FP8_MTP4, "fp8_prefill": synth.FP8_PREFILL}[args.workload]
    prefill = args.workload in ("prefill", "fp8_prefill")
    fp8 = cfg.fmt == synth.FP8
    # distinct weight copies: > 256 MB Infinity Cache worth of selected experts
    layers = 40 if cfg.fmt == synth.NVFP4 else (2 if prefill else (16 if fp8 else 8))
    dev = torch.device("cuda:0")
    t0 = time.time()
    L = synth.layer_inputs(cfg)
    print(f"# generated {cfg.name} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    def to_dev(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    fmt = q.QMOE_FMT_NVFP4 if cfg.fmt == synth.NVFP4 else q.QMOE_FMT_MXFP4
    base = [to_dev(L.w1), None if L.s1 is None else to_dev(L.s1), None if L.g1 is None else to_dev(L.g1),
            to_dev(L.w2), None if L.s2 is None else to_dev(L.s2), None if L.g2 is None else to_dev(L.g2)]
    copies = []
    for i in range(layers):
        t = [None if b is None else (b if i == 0 else b.clone()) for b in base]
        if fp8:
            copies.append((q.FP8Weights(t[0], t[2]), q.FP8Weights(t[3], t[5])))
        else:
            copies.append((q.FP4Weights(t[0], t[1], t[2], fmt), q.FP4Weights(t[3], t[4], t[5], fmt)))
    logits = to_dev(L.logits)
    x = to_dev(L.x.view(np.int16)).view(torch.bfloat16)
    path = {"auto": q.QMOE_PATH_AUTO, "gemv": q.QMOE_PATH_GEMV, "grouped": q.QMOE_PATH_GROUPED}[args.path]
    layer = MoELayer(cfg.T, cfg.E, cfg.k, cfg.H, cfg.I, copies[0][0], copies[0][1], path=path, device=dev)
    if args.layer_call == "multi":
        layer.layer_persistent = False
    layer.run(logits, x)
    torch.cuda.synchronize()
    offsets = layer.offsets.cpu().numpy()
    D = int(np.count_nonzero(np.diff(offsets)))
    B = cfg.B
    if fp8:   # one byte per weight, no block scales
        fc1_w = cfg.H * 2 * cfg.I + 4
        fc2_w = cfg.I * cfg.H + 4
    else:
        fc1_w = cfg.H * cfg.I + (cfg.H // B) * 2 * cfg.I + (4 if L.g1 is not None else 0)
        fc2_w = cfg.I * (cfg.H // 2) + (cfg.I // B) * cfg.H + (4 if L.g2 is not None else 0)
    weight_bytes = D * (fc1_w + fc2_w)
    R = cfg.rows
    # FC1 algorithmic bytes: selected experts' weights, x rows of the tokens, h, maps
    fc1_bytes = D * fc1_w + cfg.T * cfg.H * 2 + R * cfg.I * 2 + (cfg.E + 1 + R) * 4
    print(f"# rows={R} distinct experts={D} weight bytes/layer={weight_bytes}", file=sys.stderr, flush=True)

    stream = torch.cuda.Stream()
    tm = Timer(torch, stream)

    def step(i):
        w1, w2 = copies[i % layers]
        layer.set_weights(w1, w2)
        layer.run(logits, x, fused=True)

    def fc1_only(i):
        layer.w1 = copies[i % layers][0]
        layer.fc1(x)

    ms = tm.run(step, layers, args.steps, args.warmup, args.eager)
    value = weight_bytes / (ms * 1e-3) / 1e9
    fc1_ms = tm.run(fc1_only, layers, max(layers * 10, 40), layers, args.eager)
    fc1_gbs = fc1_bytes / (fc1_ms * 1e-3) / 1e9
    layer.set_weights(*copies[0])

    if prefill and fp8:
        sources = ("fp8.hip", "device_common.h", "qmoe_internal.h")
        kname, tname = "fp8_grouped_kernel (FC1+SwiGLU)", "fp8_grouped_fc1_prefill"
        metric = "FP8 W8A16 MoE prefill layer µs/layer + achieved HBM GB/s on weight bytes"
    elif prefill:
        sources = ("grouped.hip", "device_common.h", "qmoe_internal.h")
        kname, tname = "grouped_gemm_kernel (FC1+SwiGLU)", "grouped_fc1_prefill"
        metric = "MXFP4 MoE prefill layer µs/layer + achieved HBM GB/s on weight bytes"
    elif fp8:
        sources = ("fp8.hip", "device_common.h", "qmoe_internal.h")
        kname, tname = "fp8_gemv_kernel (FC1+SwiGLU)", "fp8_gemv_fc1_mtp4"
        metric = "FP8 W8A16 MoE decode µs/layer + achieved HBM GB/s on weight bytes"
    elif q.qmoe_fp4_resolve_path(cfg.T, cfg.k, copies[0][0], path) == q.QMOE_PATH_GROUPED:
        sources = ("grouped.hip", "device_common.h", "qmoe_internal.h")
        kname, tname = "grouped_gemm_kernel (FC1+SwiGLU)", f"grouped_fc1_{args.workload}"
        metric = METRIC
    else:
        sources = ("gemv.hip", "device_common.h", "qmoe_internal.h")
        kname, tname = "fp4_gemv_kernel + splitk_epilogue_kernel (FC1+SwiGLU)", f"gemv_fc1_{args.workload}"
        metric = METRIC
    config = {"workload": cfg.name, "rows": R, "distinct_experts": D, "layer_copies": layers,
              "path": args.path, "launch": "eager" if args.eager else "hip_graph",
              "layer_call": "one launch" if layer.layer_persistent else "multi-launch"}
    result = base_result(metric, value, "GB/s", args, ms, config)
    result.update({"us_per_layer": round(ms * 1e3, 3), "hbm_frac_weight_bytes": round(value / HBM_PEAK_GBS, 4),
                   "weight_bytes_per_layer": weight_bytes})
    if prefill:
        flops = 2.0 * R * (cfg.H * 2 * cfg.I + cfg.I * cfg.H)
        tflops = flops / (ms * 1e-3) / 1e12
        fc1_tflops = 2.0 * R * cfg.H * 2 * cfg.I / (fc1_ms * 1e-3) / 1e12
        result.update({"layer_tflops": round(tflops, 2), "mfma_frac_layer": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                       "fc1_tflops": round(fc1_tflops, 2),
                       "fc1_mfma_frac": round(fc1_tflops / MFMA_BF16_PEAK_TFLOPS, 4)})
    traffic = measured_traffic(tname, sources)
    result["roofline"] = {"bound": "hbm", "kernel": kname, "achieved": round(fc1_gbs, 2), "peak": HBM_PEAK_GBS,
                          "unit": "GB/s", "frac": round(fc1_gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                          "avg_us": round(fc1_ms * 1e3, 3), "bytes_per_launch": fc1_bytes}
    if not args.no_cpu_baseline:
        restore = pin_one_core()
        try:
            result["cpu_baseline"] = (cpu_baseline_prefill(L, D, fc1_w + fc2_w, args.cpu_seconds) if prefill
                                      else cpu_baseline_layer(L, weight_bytes, args.cpu_seconds))
        finally:
            restore()
    return result


def bench_dequant(args, torch, q, synth, np):
    cfg = synth.DEQUANT
    dev = torch.device("cuda:0")
    w, s, g = synth.dequant_inputs(cfg)
    fmt = q.QMOE_FMT_MXFP4 if cfg.fmt == synth.MXFP4 else q.QMOE_FMT_NVFP4
    sets = 4   # input/output buffer sets: ~1 GB, beyond the Infinity Cache
    bufs = []
    for _ in range(sets):
        wd = q.FP4Weights(torch.from_numpy(w).to(dev), torch.from_numpy(s).to(dev),
                          None if g is None else torch.from_numpy(g).to(dev), fmt)
        bufs.append((wd, torch.empty((cfg.E, cfg.N, cfg.K), dtype=torch.bfloat16, device=dev)))
    rd = w.nbytes + s.nbytes + (0 if g is None else g.nbytes)
    wr = cfg.E * cfg.N * cfg.K * 2
    stream = torch.cuda.Stream()
    tm = Timer(torch, stream)

    def step(i):
        wd, out = bufs[i % sets]
        q.qmoe_dequant_fp4(wd, out)

    ms = tm.run(step, sets, args.steps, args.warmup, args.eager)
    gbs = (rd + wr) / (ms * 1e-3) / 1e9
    config = {"workload": cfg.name, "read_bytes": rd, "write_bytes": wr, "buffer_sets": sets,
              "launch": "eager" if args.eager else "hip_graph"}
    result = base_result("MXFP4 standalone dequant GB/s (read + write bytes)", gbs, "GB/s", args, ms, config,
                         dtype="u8")
    traffic = measured_traffic("dequant", ("dequant.hip", "device_common.h", "qmoe_internal.h"))
    result["roofline"] = {"bound": "hbm", "kernel": "dequant_lds_kernel<MXFP4>", "achieved": round(gbs, 2),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                          "traffic": traffic, "avg_us": round(ms * 1e3, 3), "bytes_per_launch": rd + wr}
    if not args.no_cpu_baseline:
        restore = pin_one_core()
        try:
            per = w[0].nbytes + s[0].nbytes + cfg.N * cfg.K * 2
            result["cpu_baseline"] = cpu_baseline_dequant(w, s, g, cfg.fmt, cfg.E, per, cfg.name, args.cpu_seconds)
        finally:
            restore()
    return result


def bench_fp8_dequant(args, torch, q, synth, np):
    c = synth.DEQUANT
    cfg = synth.LayerConfig("fp8_dequant_E32_K2048_N1536", synth.FP8, T=1, E=c.E, k=1, H=c.K, I=c.N // 2)
    dev = torch.device("cuda:0")
    w, _, g = synth.fc_weights(cfg, 1)          # [E][N][K] bytes, K = 2048, N = 1536
    sets = 4
    bufs = [(q.FP8Weights(torch.from_numpy(w).to(dev), torch.from_numpy(g).to(dev)),
             torch.empty(w.shape, dtype=torch.bfloat16, device=dev)) for _ in range(sets)]
    rd, wr = w.nbytes + g.nbytes, w.size * 2
    tm = Timer(torch, torch.cuda.Stream())

    def step(i):
        wd, out = bufs[i % sets]
        q.qmoe_dequant_fp8(wd, out)

    ms = tm.run(step, sets, args.steps, args.warmup, args.eager)
    gbs = (rd + wr) / (ms * 1e-3) / 1e9
    config = {"workload": cfg.name, "read_bytes": rd, "write_bytes": wr, "buffer_sets": sets,
              "launch": "eager" if args.eager else "hip_graph"}
    result = base_result("FP8 standalone dequant GB/s (read + write bytes)", gbs, "GB/s", args, ms, config,
                         dtype="u8")
    traffic = measured_traffic("fp8_dequant", ("fp8.hip", "device_common.h", "qmoe_internal.h"))
    result["roofline"] = {"bound": "hbm", "kernel": "fp8_dequant_kernel", "achieved": round(gbs, 2),
                          "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                          "traffic": traffic, "avg_us": round(ms * 1e3, 3), "bytes_per_launch": rd + wr}
    if not args.no_cpu_baseline:
        restore = pin_one_core()
        try:
            result["cpu_baseline"] = cpu_baseline_dequant(w, None, g, "fp8", c.E, w[0].nbytes * 3, cfg.name,
                                                          args.cpu_seconds)
        finally:
            restore()
    return result


def calibrate_copy(args, torch):
    """A plain device copy of 1 GiB (read 1 GiB + write 1 GiB per launch)."""
    n = 1 << 30
    dev = torch.device("cuda:0")
    a = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    stream = torch.cuda.Stream()
    tm = Timer(torch, stream)
    ms = tm.run(lambda i: b.copy_(a), 1, args.steps, args.warmup, eager=True)
    return {"calibration": "device copy", "bytes_read_per_launch": n, "bytes_written_per_launch": n,
            "avg_us": round(ms * 1e3, 3), "gbs": round(2 * n / (ms * 1e-3) / 1e9, 2)}


def pin_one_core():
    """Pins this process to one host core for the CPU baseline (the oracle is
    single-threaded; the pin makes `cores` = 1 a measured fact) and returns a
    function that restores the previous affinity."""
    prev = os.sched_getaffinity(0)
    os.sched_setaffinity(0, {min(prev)})
    return lambda: os.sched_setaffinity(0, prev)


def cpu_cores_used():
    return len(os.sched_getaffinity(0))


def cpu_baseline_layer(L, weight_bytes, budget_s):
    """The C++ oracle as it stands (single-threaded, float64) on whole layers of the same workload."""
    from oracle import cpp
    cpp.lib()
    n, t0 = 0, time.perf_counter()
    while True:
        cpp.layer(L)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 20:
            break
    per_layer = el / n
    return {"value": round(weight_bytes / per_layer / 1e9, 4), "unit": "GB/s", "cores": cpu_cores_used(), "kind": "oracle",
            "sample": f"{n} full layers of {L.cfg.name} (route, FC1+SwiGLU, FC2, finalize), C++ float64 oracle, "
                      f"{per_layer * 1e3:.1f} ms/layer",
            "host_cores_total": os.cpu_count()}


def cpu_baseline_prefill(L, D, expert_bytes, budget_s):
    """The C++ oracle's FC1+SwiGLU and FC2 on the rows of the first routed experts (in expert order), one
    expert per call, until the budget runs out; GB/s on the weight bytes of the experts processed."""
    import numpy as np

    from oracle import cpp
    c = L.cfg
    cpp.lib()
    idx, _ = cpp.route_topk(L.logits, c.k)
    off, p2e, _ = cpp.expert_maps(idx, c.E)
    n, rows, t0 = 0, 0, time.perf_counter()
    for e in range(c.E):
        lo, hi = int(off[e]), int(off[e + 1])
        if lo == hi:
            continue
        # maps of a batch that holds only expert e's rows
        sub = np.where(np.arange(c.E + 1) <= e, 0, hi - lo).astype(np.int32)
        h, _ = cpp.fc1_swiglu(L.x, c.k, L.w1, L.s1, L.g1, c.fmt, sub, p2e[lo:hi], want_u=False)
        cpp.fc2(h, L.w2, L.s2, L.g2, c.fmt, sub)
        n, rows = n + 1, rows + hi - lo
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(n * expert_bytes / el / 1e9, 4), "unit": "GB/s", "cores": cpu_cores_used(), "kind": "oracle",
            "sample": f"FC1+SwiGLU and FC2 of {n} of {D} routed experts ({rows} of {c.rows} rows) of {c.name}, "
                      f"C++ float64 oracle, {el:.1f} s", "host_cores_total": os.cpu_count()}


def cpu_baseline_dequant(w, s, g, fmt, E, per_expert_bytes, name, budget_s):
    """The C++ oracle's dequant, one expert per call, until the budget runs out."""
    from oracle import cpp
    cpp.lib()
    n, t0 = 0, time.perf_counter()
    while n < E:
        cpp.dequant_bf16(w[n:n + 1], None if s is None else s[n:n + 1], None if g is None else g[n:n + 1], fmt)
        n += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    return {"value": round(n * per_expert_bytes / el / 1e9, 4), "unit": "GB/s", "cores": cpu_cores_used(), "kind": "oracle",
            "sample": f"{n} of {E} experts of {name}, C++ float64 oracle, {el:.1f} s",
            "host_cores_total": os.cpu_count()}


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    torch.cuda.set_device(0)
    if args.calibrate_copy:
        print(json.dumps(calibrate_copy(args, torch)), flush=True)
        return
    import fp4_weight_only_amd as q
    import synth
    if args.workload == "dequant":
        result = bench_dequant(args, torch, q, synth, np)
    elif args.workload == "fp8_dequant":
        result = bench_fp8_dequant(args, torch, q, synth, np)
    else:
        result = bench_layer(args, torch, q, synth, np)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
