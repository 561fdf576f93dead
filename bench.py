"""Benchmark of the FP4 weight-only MoE expert path on one MI355X.

Default workload: the NVFP4 MTP-verify decode layer (4 tokens x top-8 = 32
expanded rows, E=256, hidden 2048, intermediate 768, three hot experts),
seeded synthetic inputs.  A step is one pass of the whole hot path over one
layer, the library's default layer call: qmoe_fp4_moe_layer_persistent (routing,
FC1 + SwiGLU, FC2 and the weighted un-permute in one kernel launch) where the
shape allows, else qmoe_route_topk -> qmoe_fp4_gemv_fc1_swiglu ->
qmoe_fp4_gemv_fc2_finalize (--layer-call multi forces the latter).  Steps
rotate over distinct copies of the layer weights so every timed weight byte
comes from HBM, not from the 256 MB Infinity Cache.  The steps are captured
once in a HIP graph and replayed (the launch path of a serving loop);
--eager times plain launches instead.

value = achieved GB/s on weight bytes (packed E2M1 + block scales + global
scales of the experts the routing actually selected) per layer.

The default line also carries, measured in the same process:
  sweep    -- T = 1, 2, 4, 8 (8..64 expanded rows) of the same layer: µs/layer
              and weight GB/s of the default call, µs/layer of plain launches
              (no graph) and of the multi-launch calls, and the FC1 and
              FC2 + finalize calls on their own with their HBM fractions;
  dequant  -- the MXFP4 standalone dequant's GB/s and fraction of 8 TB/s, and
              of the store ceiling (a plain fill kernel writing the dequant's
              output size), which binds a kernel that writes four bytes per
              byte read.

Other workloads (--workload): decode / mtp2 / mtp8 / mx_decode (same layer
path), prefill (MXFP4 512 tokens, grouped-GEMM path; also reports TFLOP/s and
the fraction of the bf16 MFMA peak), dequant (MXFP4 standalone dequant, GB/s
on read + write bytes), fp8 (the MTP-verify layer with FP8 E4M3 W8A16
weights: qmoe_fp8_gemv_fc1_swiglu -> qmoe_fp8_gemv_fc2 -> qmoe_finalize),
fp8_prefill (the prefill layer with FP8 weights, grouped MFMA path),
fp8_dequant (FP8 standalone dequant at the dequant workload's shape).
--calibrate-copy runs a plain device-to-device copy of known size, the
reference kernel for scaling HBM traffic counters.

roofline: the dominant kernel of the workload -- the single-launch layer
kernel when the layer runs as one launch (its launches are the timed steps),
else FC1 (GEMV + split-K epilogue) for the layer workloads, the dequant kernel
for dequant -- HBM-bound; its average duration comes from HIP events around
graph replays that hold only that call over the rotated copies, recorded on
the stream they run on.  roofline.traffic is the HBM byte count per launch
measured with FETCH_SIZE + WRITE_SIZE counters and scaled by the copy
calibration, read from profiles/ and reported only while the kernel source it
was taken on is unchanged (else null).

cpu_baseline: the C++ CPU oracle (test infrastructure, float64, single-
threaded, pinned to one core) timed on a bounded sample of the same workload.
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
LAYER_WORKLOADS = ("mtp4", "mtp8", "mtp2", "decode", "mx_decode", "prefill", "fp8", "fp8_prefill")
# sources of the single-launch layer kernel (a changed source reports traffic null)
LAYER_SOURCES = ("layer.hip", "gemv_device.h", "route_device.h", "device_common.h", "qmoe_internal.h")



def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=80)
    ap.add_argument("--eager", action="store_true")
    ap.add_argument("--path", default="auto", choices=("auto", "gemv", "grouped"),
                    help="FC kernel path of the layer workloads (auto: the library's AUTO rule)")
    ap.add_argument("--workload", default="mtp4", choices=LAYER_WORKLOADS + ("dequant", "fp8_dequant"))
    ap.add_argument("--layer-call", default="auto", choices=("auto", "multi", "one"),
                    help="decode layer: auto = the library's default (one kernel launch, "
                         "qmoe_fp4_moe_layer_persistent, up to four tokens at hidden size <= 2048), multi = the multi-launch calls, "
                         "one = one launch wherever the shape allows")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="mtp4: skip the T = 1, 2, 4, 8 sweep and the dequant figures of the default line")
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


class LayerRig:
    """One decode/prefill layer on the GPU: `layers` distinct weight copies
    (rotated per step so every timed weight byte comes from HBM), the inputs,
    the MoELayer, and the algorithmic byte counts."""

    def __init__(self, cfg, args, torch, q, synth, np, layers, layer_call="auto"):
        from fp4_weight_only_amd.layer import MoELayer
        self.cfg, self.torch, self.q, self.layers = cfg, torch, q, layers
        self.fp8 = cfg.fmt == synth.FP8
        dev = torch.device("cuda:0")
        t0 = time.time()
        self.L = L = synth.layer_inputs(cfg)
        print(f"# generated {cfg.name} in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

        def to_dev(a):
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

        fmt = q.QMOE_FMT_NVFP4 if cfg.fmt == synth.NVFP4 else q.QMOE_FMT_MXFP4
        base = [to_dev(L.w1), None if L.s1 is None else to_dev(L.s1), None if L.g1 is None else to_dev(L.g1),
                to_dev(L.w2), None if L.s2 is None else to_dev(L.s2), None if L.g2 is None else to_dev(L.g2)]
        self.copies = []
        for i in range(layers):
            t = [None if b is None else (b if i == 0 else b.clone()) for b in base]
            if self.fp8:
                self.copies.append((q.FP8Weights(t[0], t[2]), q.FP8Weights(t[3], t[5])))
            else:
                self.copies.append((q.FP4Weights(t[0], t[1], t[2], fmt), q.FP4Weights(t[3], t[4], t[5], fmt)))
        self.logits = to_dev(L.logits)
        self.x = to_dev(L.x.view(np.int16)).view(torch.bfloat16)
        self.path = {"auto": q.QMOE_PATH_AUTO, "gemv": q.QMOE_PATH_GEMV, "grouped": q.QMOE_PATH_GROUPED}[args.path]
        self.layer = layer = MoELayer(cfg.T, cfg.E, cfg.k, cfg.H, cfg.I, self.copies[0][0], self.copies[0][1],
                                      path=self.path, device=dev)
        self.one_launch_ok = layer.layer_persistent     # the one-launch call applies to this shape
        self.one_launch_default = layer.one_launch      # and run(fused=True) takes it
        if layer_call == "multi":
            layer.one_launch = False
        elif layer_call == "one":
            layer.one_launch = layer.layer_persistent
        layer.run(self.logits, self.x)
        torch.cuda.synchronize()
        offsets = layer.offsets.cpu().numpy()
        self.D = D = int(np.count_nonzero(np.diff(offsets)))
        B = cfg.B
        if self.fp8:   # one byte per weight, no block scales
            self.fc1_w = cfg.H * 2 * cfg.I + 4
            self.fc2_w = cfg.I * cfg.H + 4
        else:
            self.fc1_w = cfg.H * cfg.I + (cfg.H // B) * 2 * cfg.I + (4 if L.g1 is not None else 0)
            self.fc2_w = cfg.I * (cfg.H // 2) + (cfg.I // B) * cfg.H + (4 if L.g2 is not None else 0)
        self.weight_bytes = D * (self.fc1_w + self.fc2_w)
        R = cfg.rows
        maps = (cfg.E + 1 + 2 * R) * 4
        # FC1: selected experts' weights, x rows of the tokens, h, maps
        self.fc1_bytes = D * self.fc1_w + cfg.T * cfg.H * 2 + R * cfg.I * 2 + maps
        # FC2 + finalize: weights, h, routing weights, out
        self.fc2_bytes = D * self.fc2_w + R * cfg.I * 2 + R * 4 + cfg.T * cfg.H * 2 + maps
        # the whole layer: weights, logits, x, out, routing outputs
        self.layer_bytes = self.weight_bytes + cfg.T * cfg.E * 4 + 2 * cfg.T * cfg.H * 2 + 2 * R * 4 + maps
        print(f"# rows={R} distinct experts={D} weight bytes/layer={self.weight_bytes}", file=sys.stderr, flush=True)
        self.tm = Timer(torch, torch.cuda.Stream())

    def time_layer(self, steps, warmup, eager):
        lay, copies, n = self.layer, self.copies, self.layers

        def step(i):
            lay.set_weights(*copies[i % n])
            lay.run(self.logits, self.x, fused=True)
        return self.tm.run(step, n, steps, warmup, eager)

    def time_fc1(self, eager):
        lay, copies, n = self.layer, self.copies, self.layers

        def fc1_only(i):
            lay.w1 = copies[i % n][0]
            lay.fc1(self.x)
        ms = self.tm.run(fc1_only, n, max(n * 10, 40), n, eager)
        lay.set_weights(*copies[0])
        return ms

    def time_fc2(self, eager):
        """FC2 + finalize in one call (qmoe_fp4_gemv_fc2_finalize), h from one FC1 call."""
        lay, copies, n = self.layer, self.copies, self.layers
        lay.set_weights(*copies[0])
        lay.route(self.logits)
        lay.fc1(self.x)

        def fc2_only(i):
            lay.w2 = copies[i % n][1]
            lay.fc2_finalize()
        ms = self.tm.run(fc2_only, n, max(n * 10, 40), n, eager)
        lay.set_weights(*copies[0])
        return ms


def sweep_entry(cfg, args, torch, q, synth, np, rig=None):
    """µs/layer and HBM fractions of one decode layer at its row count: the
    library's default layer call (one launch where it applies), the
    multi-launch calls, plain launches (no graph), and the FC1 and FC2 calls
    on their own."""
    own = rig is None
    if own:
        rig = LayerRig(cfg, args, torch, q, synth, np, 40)
    lay = rig.layer
    lay.one_launch = rig.one_launch_default
    ms = rig.time_layer(args.steps, args.warmup, False)
    eager_ms = rig.time_layer(args.steps, args.warmup, True)
    default_call = "one launch" if lay.one_launch else "multi-launch"
    lay.one_launch = False
    multi_ms = rig.time_layer(args.steps, args.warmup, False)
    one_ms = None
    if rig.one_launch_ok:
        lay.one_launch = True
        one_ms = rig.time_layer(args.steps, args.warmup, False)
    lay.one_launch = rig.one_launch_default
    fc1_ms, fc2_ms = rig.time_fc1(False), rig.time_fc2(False)
    gbs = rig.weight_bytes / (ms * 1e-3) / 1e9
    e = {"T": cfg.T, "rows": cfg.rows, "distinct_experts": rig.D, "layer_call": default_call,
         "us_per_layer": round(ms * 1e3, 3), "weight_GBps": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
         "eager_us_per_layer": round(eager_ms * 1e3, 3), "multi_launch_us_per_layer": round(multi_ms * 1e3, 3),
         "one_launch_us_per_layer": None if one_ms is None else round(one_ms * 1e3, 3),
         "fc1_us": round(fc1_ms * 1e3, 3), "fc1_frac": round(rig.fc1_bytes / (fc1_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
         "fc2_finalize_us": round(fc2_ms * 1e3, 3),
         "fc2_frac": round(rig.fc2_bytes / (fc2_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    print(f"# sweep T={cfg.T}: {e}", file=sys.stderr, flush=True)
    if own:
        del rig
        torch.cuda.empty_cache()
    return e


def bench_layer(args, torch, q, synth, np):
    cfg = {"mtp4": synth.MTP4, "mtp8": synth.MTP8, "mtp2": synth.MTP2, "decode": synth.DECODE,
           "mx_decode": synth.MX_DECODE, "prefill": synth.MX_PREFILL, "fp8": synth.FP8_MTP4,
           "fp8_prefill": synth.FP8_PREFILL}[args.workload]
    prefill = args.workload in ("prefill", "fp8_prefill")
    fp8 = cfg.fmt == synth.FP8
    # distinct weight copies: > 256 MB Infinity Cache worth of selected experts
    layers = 40 if cfg.fmt == synth.NVFP4 else (2 if prefill else (16 if fp8 else 8))
    rig = LayerRig(cfg, args, torch, q, synth, np, layers, args.layer_call)
    layer, D, R = rig.layer, rig.D, cfg.rows
    ms = rig.time_layer(args.steps, args.warmup, args.eager)
    value = rig.weight_bytes / (ms * 1e-3) / 1e9
    fc1_ms = rig.time_fc1(args.eager)
    fc1_gbs = rig.fc1_bytes / (fc1_ms * 1e-3) / 1e9
    fc2_ms = None if (prefill or fp8) else rig.time_fc2(args.eager)
    one_launch = layer.one_launch

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
    elif q.qmoe_fp4_resolve_path(cfg.T, cfg.k, rig.copies[0][0], rig.path) == q.QMOE_PATH_GROUPED:
        sources = ("grouped.hip", "device_common.h", "qmoe_internal.h")
        kname, tname = "grouped_gemm_kernel (FC1+SwiGLU)", f"grouped_fc1_{args.workload}"
        metric = METRIC
    elif one_launch:
        sources = LAYER_SOURCES
        kname, tname = "fp4_layer_kernel (the whole layer, one launch)", f"layer_{args.workload}"
        metric = METRIC
    else:
        sources = ("gemv.hip", "gemv_device.h", "device_common.h", "qmoe_internal.h")
        kname, tname = "fp4_gemv_kernel + splitk_epilogue_kernel (FC1+SwiGLU)", f"gemv_fc1_{args.workload}"
        metric = METRIC
    config = {"workload": cfg.name, "rows": R, "distinct_experts": D, "layer_copies": layers,
              "path": args.path, "launch": "eager" if args.eager else "hip_graph",
              "layer_call": "one launch" if one_launch else "multi-launch"}
    result = base_result(metric, value, "GB/s", args, ms, config)
    result.update({"us_per_layer": round(ms * 1e3, 3), "hbm_frac_weight_bytes": round(value / HBM_PEAK_GBS, 4),
                   "weight_bytes_per_layer": rig.weight_bytes})
    if prefill:
        flops = 2.0 * R * (cfg.H * 2 * cfg.I + cfg.I * cfg.H)
        tflops = flops / (ms * 1e-3) / 1e12
        fc1_tflops = 2.0 * R * cfg.H * 2 * cfg.I / (fc1_ms * 1e-3) / 1e12
        result.update({"layer_tflops": round(tflops, 2), "mfma_frac_layer": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                       "fc1_tflops": round(fc1_tflops, 2),
                       "fc1_mfma_frac": round(fc1_tflops / MFMA_BF16_PEAK_TFLOPS, 4)})
    traffic = measured_traffic(tname, sources)
    if one_launch and not prefill and not fp8:
        # the layer's only kernel: its launches are the timed steps
        gbs = rig.layer_bytes / (ms * 1e-3) / 1e9
        result["roofline"] = {"bound": "hbm", "kernel": kname, "achieved": round(gbs, 2), "peak": HBM_PEAK_GBS,
                              "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                              "avg_us": round(ms * 1e3, 3), "bytes_per_launch": rig.layer_bytes}
    else:
        result["roofline"] = {"bound": "hbm", "kernel": kname, "achieved": round(fc1_gbs, 2),
                              "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(fc1_gbs / HBM_PEAK_GBS, 4),
                              "traffic": traffic, "avg_us": round(fc1_ms * 1e3, 3),
                              "bytes_per_launch": rig.fc1_bytes}
    if fc2_ms is not None:   # the FC2 + finalize call on its own (GEMV + finalize launches)
        result["fc2_finalize"] = {"us": round(fc2_ms * 1e3, 3), "bytes_per_call": rig.fc2_bytes,
                                  "frac": round(rig.fc2_bytes / (fc2_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    if args.workload == "mtp4" and not args.no_sweep:
        # the metric's whole row range, T = 1, 2, 4, 8 (8..64 expanded rows)
        sweep = []
        for c in (synth.DECODE, synth.MTP2, synth.MTP4, synth.MTP8):
            sweep.append(sweep_entry(c, args, torch, q, synth, np, rig if c is cfg else None))
        result["sweep"] = sweep
        layer.one_launch = one_launch
    if not args.no_cpu_baseline:
        restore = pin_one_core()
        try:
            result["cpu_baseline"] = (cpu_baseline_prefill(rig.L, D, rig.fc1_w + rig.fc2_w, args.cpu_seconds)
                                      if prefill else cpu_baseline_layer(rig.L, rig.weight_bytes, args.cpu_seconds))
        finally:
            restore()
    if args.workload == "mtp4" and not args.no_sweep:
        del rig
        torch.cuda.empty_cache()
        dq = bench_dequant(args, torch, q, synth, np, cpu=False)
        wc = write_ceiling(args, torch, dq["config"]["write_bytes"])
        result["dequant"] = {"workload": dq["config"]["workload"], "GBps": dq["value"],
                             "frac": dq["roofline"]["frac"], "us": dq["roofline"]["avg_us"],
                             "write_ceiling_GBps": wc, "frac_of_write_ceiling": round(dq["value"] / wc, 4)}
    return result


def bench_dequant(args, torch, q, synth, np, cpu=True):
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
    if cpu and not args.no_cpu_baseline:
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


def write_ceiling(args, torch, nbytes):
    """GB/s of a plain store kernel (torch's fill) writing `nbytes` per launch
    over four rotated buffers: the store path's ceiling at the dequant's
    output size, which bounds a kernel that writes four bytes per byte read."""
    dev = torch.device("cuda:0")
    bufs = [torch.empty(nbytes // 4, dtype=torch.int32, device=dev) for _ in range(4)]
    tm = Timer(torch, torch.cuda.Stream())
    ms = tm.run(lambda i: bufs[i % 4].fill_(i + 1), 4, args.steps, args.warmup, eager=False)  # never a memset
    return round(nbytes / (ms * 1e-3) / 1e9, 1)


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
