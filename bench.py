#!/usr/bin/env python3
"""Throughput of the DCNv4 forward operator on one MI355X.

One step = one forward pass of the operator (the whole hot path: offset and
weight staging, sampling geometry, bilinear gathers, fp32 accumulation,
rounding and store) over one batch of synthetic inputs that are resident in
HBM when the timed region starts.  Several input sets are rotated so that no
step finds its inputs in the 256 MB Infinity Cache or the L2 from the step
before.

The metric is GB/s of ideal traffic (input and output feature maps once,
the offset/weight tensor once, plus group scales: the 2HWC + 27HWG element
model of the DCNv4 digest page, section "GPU效率的理论分析") and its fraction
of the MI355X HBM peak (8 TB/s); output pixels/s and outputs/s are reported
beside it.

Prints ONE JSON line.  --gpus N with N > 1 is refused: the benchmark measures
one GPU (images are independent, so a batch would shard across GPUs by image
with no communication in the forward pass).
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
# fp32 fma per second on the vector ALU without packed fp32: 256 CUs x 64
# lanes (4 SIMD16 per CU) x 2.4 GHz
VALU_PEAK_GOPS = 256 * 64 * 2.4


def kernel_source_digest() -> str:
    h = hashlib.sha256()
    for f in ("dcn4_kernels.hip", "dcn4_tile_part.hip", "dcn4_internal.h", "dcn4_api.cpp"):
        with open(os.path.join(ROOT, "dynamic_sparse_vision_dcn4_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def load_profile_summary(kind: str, workload: str):
    """A committed rocprofv3 counter summary (profiles/<kind>_<workload>.json)
    if it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"{kind}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_digest") != kernel_source_digest():
        return None
    return t


def load_traffic(workload: str):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by a plain
    copy's counters), or None when the counters predate the source."""
    t = load_profile_summary("traffic", workload)
    return None if t is None else t.get("hbm_bytes_per_launch")


def copy_ceiling(torch, mib=512, reps=5):
    """Plain device copies of `mib` MiB on the current stream: bytes read plus
    bytes written per second (the achievable HBM rate of a streaming copy on
    this GPU, the context for the operator's fraction of the 8 TB/s peak)."""
    n = mib << 20
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    b.copy_(a)
    times = []
    for _ in range(reps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3)
    t = statistics.median(times)
    del a, b
    return {"gbs": round(2 * n / t / 1e9, 1), "bytes_moved": 2 * n,
            "pct_hbm_peak": round(100.0 * 2 * n / t / 1e9 / HBM_PEAK_GBS, 2),
            "what": f"median of {reps} device copies of {mib} MiB (read + write)"}


def settle_clocks(torch, ms):
    """Keep the GPU busy for about `ms` milliseconds with a plain elementwise
    kernel (torch.sin over 256 MiB of fp32, unrelated to the operator and its
    inputs) right before the warmup steps, which are enqueued behind it (the
    graph of the timed steps is captured before, so no host work leaves the
    GPU idle in between).  From idle, this GPU raises its clocks
    over the first ~100 ms of sustained work: the operator's launches took
    136-155 us for the first 40 and ~121 us from about the 200th on in a
    fresh process, and the same curve came back after a 1 s idle gap, while
    after 0.3 s of this elementwise kernel they took 122-124 us from the
    start.  A handful of warmup steps alone would therefore time the clock
    ramp, not the kernel.  Returns the busy time in ms."""
    if ms <= 0:
        return 0.0
    a = torch.randn(64 << 20, device="cuda")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while True:
        for _ in range(10):
            a = torch.sin(a)
        if (time.perf_counter() - t0) * 1e3 >= ms:
            break  # the last batch still runs: the caller's launches follow it
        torch.cuda.synchronize()
    busy = (time.perf_counter() - t0) * 1e3
    del a
    return round(busy, 1)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--workload", default=None,
                    help="workload name (default: the latent-diffusion U-Net block)")
    ap.add_argument("--sets", type=int, default=0,
                    help="input sets rotated across steps (default: enough for 1 GiB)")
    ap.add_argument("--channels-per-lane", type=int, default=0)
    ap.add_argument("--option", action="append", default=[], metavar="NAME=VALUE",
                    help="plan option (kernel, tile_margin, tile_groups, tile_pad)")
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="busy the GPU with a plain elementwise kernel for this long "
                         "before the warmup steps, so that the timed steps run at the "
                         "clocks of sustained work (0: off)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-reps", type=int, default=10)
    ap.add_argument("--backward", action="store_true",
                    help="time the backward pass (dcn4_backward) instead of the forward")
    ap.add_argument("--grads", choices=("both", "x", "om"), default="both",
                    help="backward: the gradients asked for")
    ap.add_argument("--scatter", action="store_true",
                    help="backward: grad_x with fp32 atomics instead of the bucket gather")
    ap.add_argument("--linear", action="store_true",
                    help="time the offset/weight linear layer (dcn4_offset_linear) "
                         "that produces the workload's offset/weight tensor")
    ap.add_argument("--dwconv", action="store_true",
                    help="time the depthwise 3x3 convolution (dcn4_dwconv3x3) on the "
                         "workload's input feature map")
    ap.add_argument("--producer", action="store_true",
                    help="time the offset/weight producer (the depthwise 3x3, then the "
                         "linear layer) and the operator after it, alone and in sequence "
                         "(workloads whose output is the size of their input)")
    ap.add_argument("--eager", action="store_true",
                    help="time one launch per Python call instead of replaying the "
                         "captured K steps")
    ap.add_argument("--dcnv3", action="store_true",
                    help="time the DCNv3-style comparison (softmax pass, then the "
                         "one-thread-per-channel aggregation) beside the default "
                         "DCNv4 plan on the same inputs")
    ap.add_argument("--copy-reference", type=int, default=0, metavar="MIB",
                    help="instead of the operator, run plain device copies of MIB "
                         "MiB (the scale reference for the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} refused: the benchmark measures one GPU "
              "only (sharding a batch over GPUs by image is not built)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import workloads
    import dynamic_sparse_vision_dcn4_amd as d4

    if args.copy_reference:
        copy_reference(torch, args.copy_reference, args.steps)
        return
    args.settled_ms = 0.0

    name = args.workload or workloads.HEADLINE
    w = workloads.WORKLOADS[name]
    if args.backward:
        return bench_backward(args, torch, np, workloads, d4, name, w)
    if args.linear:
        return bench_linear(args, torch, np, workloads, d4, name, w)
    if args.dwconv:
        return bench_dwconv(args, torch, np, workloads, d4, name, w)
    if args.dcnv3:
        return bench_dcnv3(args, torch, np, workloads, d4, name, w)
    if args.producer:
        return bench_producer(args, torch, np, workloads, d4, name, w)
    desc = d4.Desc(w.N, w.H, w.W, w.C, w.G, w.kh, w.kw, w.sh, w.sw, w.ph, w.pw,
                   w.dh, w.dw, w.offset_scale, w.multiscale, w.dtype,
                   w.pixel_scales, w.max_scale)
    opts = {k: int(v) for k, v in (o.split("=", 1) for o in args.option)}
    plan = d4.Plan(desc, channels_per_lane=args.channels_per_lane, **opts)
    Ho, Wo = plan.Ho, plan.Wo
    ideal = plan.ideal_bytes
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.dtype]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    def dev_tensor(raw):
        if w.dtype == "f32":
            t = torch.from_numpy(raw)
        else:
            t = torch.from_numpy(raw.view(np.int16)).view(tdt)
        return t.to(dev)

    nsets = args.sets or max(2, math.ceil((1 << 30) / max(ideal, 1)))
    sets = []
    host0 = None
    for r in range(nsets):
        inp = workloads.make_inputs(w, Ho, Wo, seed=w.seed + r)
        if r == 0:
            host0 = inp
        sc = None if inp.scales is None else torch.from_numpy(inp.scales).to(dev)
        ps = None if inp.pscales is None else torch.from_numpy(inp.pscales).to(dev)
        y = torch.empty(plan.out_shape(), dtype=tdt, device=dev)
        sets.append((dev_tensor(inp.x), dev_tensor(inp.om), sc, ps, y))
    torch.cuda.synchronize()

    def step(i, st=None):
        x, om, sc, ps, y = sets[i % nsets]
        plan.forward(x, om, sc, out=y, stream=(st or stream).cuda_stream, pixel_scales=ps)

    # The K steps are captured once in a HIP graph and the timed region
    # replays it: one host call enqueues every launch, so the GPU runs them
    # back to back whatever the host thread is doing (eagerly, the host's
    # enqueue time per step varied between ~8 and ~190 us from run to run
    # on the same box).  --eager times the launches one Python call each.
    # The capture comes first (after the first warmup step, which also loads
    # the kernels), so that the clock settling, the other warmup steps and
    # one untimed replay then run back to back.
    if args.warmup > 0:
        step(0)
        torch.cuda.synchronize()
    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream(dev)
            for i in range(args.steps):
                step(i, cap)
    args.settled_ms = settle_clocks(torch, args.settle_ms)
    for i in range(1, args.warmup):
        step(i)
    if graph is not None:
        graph.replay()  # one untimed replay
    torch.cuda.synchronize()

    # the timed region: exactly `steps` steps between two synchronisations
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(i)
    t1.record(stream)
    host_enqueue = time.perf_counter() - wall0
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t0.elapsed_time(t1) / args.steps

    # kernel duration: a second pass with events around every launch, on the
    # stream the kernel is launched on
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for i in range(args.steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per_launch_ms = [a.elapsed_time(b) for a, b in ev]
    kern_ms = statistics.mean(per_launch_ms)

    value = ideal / (ms_per_step * 1e-3) / 1e9
    # the roofline uses the same time base as `value`: the average duration
    # of one launch over the timed region (HIP events on the launch stream
    # around the K steps; one launch per step, back to back)
    achieved = value
    out_pix = w.N * Ho * Wo
    traffic = load_traffic(name)
    # the arithmetic floor: 4 multiply-adds per point and output element
    # (the pages' 36HWC for 3x3), fp32 fma on the vector ALU; the counters'
    # VALU instructions per output element beside it when a summary of the
    # current source is committed
    fma_per_out = 4 * w.kh * w.kw
    alu_gops = fma_per_out * out_pix * w.C / (ms_per_step * 1e-3) / 1e9
    valu = load_profile_summary("valu", name)

    line = {
        "metric": "DCNv4 fwd GB/s (ideal bytes) and % of HBM peak; output pixels/sec",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup, "clock_settle_ms": args.settled_ms,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded, the workload's shapes and distributions)",
        "config": {"workload": name, "N": w.N, "H": w.H, "W": w.W, "C": w.C,
                   "group": w.G, "kernel": [w.kh, w.kw], "stride": [w.sh, w.sw],
                   "pad": [w.ph, w.pw], "dilation": [w.dh, w.dw],
                   "group_scales": w.multiscale, "pixel_scales": w.pixel_scales,
                   "max_scale": w.max_scale, "Ho": Ho, "Wo": Wo,
                   "ideal_bytes": ideal, "input_sets": nsets,
                   "launch": "eager" if graph is None else "hip_graph",
                   "plan": plan.info()},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "output_pixels_per_s": round(out_pix / (ms_per_step * 1e-3), 1),
        "outputs_per_s": round(out_pix * w.C / (ms_per_step * 1e-3), 1),
        "kernel_us": {"mean": round(kern_ms * 1e3, 3),
                      "median": round(statistics.median(per_launch_ms) * 1e3, 3),
                      "min": round(min(per_launch_ms) * 1e3, 3),
                      "max": round(max(per_launch_ms) * 1e3, 3)},
        "wall_s_timed": round(wall, 4),
        "host_enqueue_us_per_step": round(host_enqueue / args.steps * 1e6, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "time_base": "mean launch duration over the timed region "
                                  "(= ms_per_step: one launch per step)"},
        "roofline_alu": {"bound": "alu", "achieved": round(alu_gops, 1),
                         "peak": round(VALU_PEAK_GOPS, 1), "unit": "Gfma/s",
                         "frac": round(alu_gops / VALU_PEAK_GOPS, 4),
                         "fma_per_output": fma_per_out,
                         "valu_insts_per_output_measured":
                             None if valu is None else valu.get("valu_insts_per_output")},
        "copy_ceiling": copy_ceiling(torch),
        "kernel_source": kernel_source_digest(),
    }

    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, Ho, Wo, host0, args.cpu_reps)
    print(json.dumps(line), flush=True)


def bench_backward(args, torch, np, workloads, d4, name, w):
    """One step = dcn4_backward_ws on one batch: grad_x (gathered through a
    workspace allocated once before the timed region, or with --scatter added
    with fp32 atomics) and grad_offset_mask written; --grads x / om asks for
    one of them.  Ideal bytes: the inputs the asked gradients depend on
    (grad_x: offset/weight tensor and grad_y; grad_offset_mask: also x) read
    once in the I/O dtype, the gradients written once in fp32."""
    desc = d4.Desc(w.N, w.H, w.W, w.C, w.G, w.kh, w.kw, w.sh, w.sw, w.ph, w.pw,
                   w.dh, w.dw, w.offset_scale, w.multiscale, w.dtype,
                   w.pixel_scales, w.max_scale)
    opts = {k: int(v) for k, v in (o.split("=", 1) for o in args.option)}
    plan = d4.Plan(desc, channels_per_lane=args.channels_per_lane, **opts)
    Ho, Wo = plan.Ho, plan.Wo
    es = 4 if w.dtype == "f32" else 2
    nx = w.N * w.H * w.W * w.C
    ny = w.N * Ho * Wo * w.C
    nom = w.N * Ho * Wo * w.G * 3 * w.K
    want_x, want_om = args.grads in ("both", "x"), args.grads in ("both", "om")
    ideal = ((nom + ny + (nx if want_om else 0)) * es +
             ((nx if want_x else 0) + (nom if want_om else 0)) * 4)
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.dtype]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    def dev_tensor(raw):
        t = torch.from_numpy(raw) if w.dtype == "f32" else torch.from_numpy(raw.view(np.int16)).view(tdt)
        return t.to(dev)

    nsets = args.sets or max(2, math.ceil((1 << 30) / max(ideal, 1)))
    sets = []
    for r in range(nsets):
        inp = workloads.make_inputs(w, Ho, Wo, seed=w.seed + r)
        rng = np.random.default_rng(1000 + r)
        gy = workloads.to_raw(rng.standard_normal((w.N, Ho, Wo, w.C), dtype=np.float32), w.dtype)
        sc = None if inp.scales is None else torch.from_numpy(inp.scales).to(dev)
        ps = None if inp.pscales is None else torch.from_numpy(inp.pscales).to(dev)
        gx = (torch.empty((w.N, w.H, w.W, w.C), dtype=torch.float32, device=dev)
              if want_x else None)
        gom = torch.empty(plan.om_shape(), dtype=torch.float32, device=dev) if want_om else None
        sets.append((dev_tensor(inp.x), dev_tensor(inp.om), dev_tensor(gy), sc, ps, gx, gom))
    ws_bytes = plan.backward_workspace_bytes() if want_x and not args.scatter else 0
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev) if ws_bytes else None
    torch.cuda.synchronize()

    def step(i, st):
        x, om, gy, sc, ps, gx, gom = sets[i % nsets]
        plan.backward(x, om, gy, sc, ps, want_x=want_x, want_om=want_om, grad_x=gx,
                      grad_om=gom, stream=st, workspace=ws, scatter=args.scatter)

    ms = timed_steps(torch, dev, stream, step, args)
    value = ideal / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "DCNv4 bwd GB/s (ideal bytes: x, offset/weight, grad_y read; fp32 grads written)",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "clock_settle_ms": args.settled_ms, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded, the workload's shapes and distributions)",
        "config": {"workload": name, "pass": "backward", "grads": args.grads,
                   "grad_x": ("scatter" if args.scatter else "gather") if want_x else None,
                   "workspace_bytes": ws_bytes, "bucket_capacity": plan.info()["bucket_capacity"],
                   "ideal_bytes": ideal, "input_sets": nsets},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "kernel_source": kernel_source_digest()}), flush=True)


def timed_steps(torch, dev, stream, step, args):
    """ms per step of `step(i, hip_stream)` over args.steps steps after
    args.warmup eager ones (preceded by settle_clocks); the steps replayed
    from a captured HIP graph unless args.eager."""
    if args.warmup > 0:
        step(0, stream.cuda_stream)  # also loads the kernels before the capture
        torch.cuda.synchronize()
    graph = None
    if not args.eager:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream(dev).cuda_stream
            for i in range(args.steps):
                step(i, cap)
    args.settled_ms = settle_clocks(torch, args.settle_ms)
    for i in range(1, args.warmup):
        step(i, stream.cuda_stream)
    if graph is not None:
        graph.replay()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for i in range(args.steps):
            step(i, stream.cuda_stream)
    t1.record(stream)
    torch.cuda.synchronize()
    return t0.elapsed_time(t1) / args.steps


def bench_producer(args, torch, np, workloads, d4, name, w):
    """The producer of the operator's offset/weight tensor on the workload
    (depthwise 3x3 of the input feature map, dcn4_dwconv3x3, then the merged
    linear layer, dcn4_offset_linear), the operator, and the three in
    sequence as one step; each leg's launches replayed from a graph on
    rotated inputs.  `value`: the sequence's output pixels per second."""
    if w.dtype == "f32":
        raise SystemExit("bench.py --producer: the layer runs bf16 and fp16 only")
    plan = d4.Plan(d4.Desc(w.N, w.H, w.W, w.C, w.G, w.kh, w.kw, w.sh, w.sw, w.ph, w.pw,
                           w.dh, w.dw, w.offset_scale, w.multiscale, w.dtype,
                           w.pixel_scales, w.max_scale))
    if (plan.Ho, plan.Wo) != (w.H, w.W):
        raise SystemExit("bench.py --producer: needs an output the size of the input")
    M, Cin, Nout = w.N * w.H * w.W, w.C, w.G * 3 * w.K
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[w.dtype]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    nsets = args.sets or max(2, math.ceil((1 << 30) / max(plan.ideal_bytes, 1)))
    sets = []
    for r in range(nsets):
        inp = workloads.make_inputs(w, plan.Ho, plan.Wo, seed=w.seed + r)
        rng = np.random.default_rng(3000 + r)
        t16 = lambda a: torch.from_numpy(workloads.to_raw(a, w.dtype).view(np.int16)).view(tdt).to(dev)
        x = torch.from_numpy(inp.x.view(np.int16)).view(tdt).to(dev)
        dw = t16((rng.standard_normal((3, 3, Cin)) / 3).astype(np.float32))
        db = torch.from_numpy(rng.standard_normal(Cin).astype(np.float32) / 4).to(dev)
        wt = t16((rng.standard_normal((Nout, Cin)) / np.sqrt(Cin)).astype(np.float32))
        b = torch.from_numpy(rng.standard_normal(Nout).astype(np.float32) / 4).to(dev)
        sets.append(dict(x=x, dw=dw, db=db, w=wt, b=b, feat=torch.empty_like(x),
                         om=torch.empty(plan.om_shape(), dtype=tdt, device=dev),
                         y=torch.empty(plan.out_shape(), dtype=tdt, device=dev)))
    torch.cuda.synchronize()

    def two(i, st):
        t = sets[i % nsets]
        d4.dwconv3x3(t["x"], t["dw"], t["db"], out=t["feat"], stream=st)
        d4.offset_linear(t["feat"].view(M, Cin), t["w"], t["b"], out=t["om"].view(M, Nout),
                         stream=st)

    def op(i, st):
        t = sets[i % nsets]
        plan.forward(t["x"], t["om"], out=t["y"], stream=st)

    def pipeline(i, st):
        two(i, st)
        op(i, st)

    us = {}
    for leg, step in (("dwconv_then_linear", two), ("operator", op),
                      ("producer_then_operator", pipeline)):
        us[leg] = timed_steps(torch, dev, stream, step, args) * 1e3
        print(f"# {leg}: {us[leg]:.2f} us per step", file=sys.stderr, flush=True)
    v = us["producer_then_operator"]
    print(json.dumps({
        "metric": "offset/weight producer and DCNv4 forward in sequence: output pixels/s",
        "value": round(M / (v * 1e-6), 1), "unit": "pixels/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "clock_settle_ms": args.settled_ms, "ms_per_step": round(v * 1e-3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded; the workload's input, normal weights)",
        "config": {"workload": name, "M": M, "Cin": Cin, "Nout": Nout,
                   "input_sets": nsets, "launch": "eager" if args.eager else "hip_graph"},
        "us_per_step": {k: round(t, 3) for k, t in us.items()},
        "kernel_source": kernel_source_digest()}), flush=True)


def bench_dcnv3(args, torch, np, workloads, d4, name, w):
    """DCNv4 against DCNv3's design on the same inputs and GPU ([DCNv4
    digest] abstract: DCNv4's forward reported more than three times as fast
    as DCNv3's).  Three timed legs of `steps` launches each, inputs rotated
    as in the forward benchmark: the default DCNv4 plan (dcn4_forward), the
    one-thread-per-channel aggregation (dcn4_dcnv3_forward, the same result
    bit for bit), and the softmax pass (dcn4_dcnv3_softmax).  DCNv3's
    operator is the aggregation; its module also runs the softmax, reported
    as a second ratio.  Ideal bytes as in the forward benchmark (the softmax
    pass: the offset/weight tensor read and written once)."""
    desc = d4.Desc(w.N, w.H, w.W, w.C, w.G, w.kh, w.kw, w.sh, w.sw, w.ph, w.pw,
                   w.dh, w.dw, w.offset_scale, w.multiscale, w.dtype,
                   w.pixel_scales, w.max_scale)
    plan = d4.Plan(desc)
    Ho, Wo = plan.Ho, plan.Wo
    ideal = plan.ideal_bytes
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.dtype]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    def dev_tensor(raw):
        t = torch.from_numpy(raw) if w.dtype == "f32" else torch.from_numpy(raw.view(np.int16)).view(tdt)
        return t.to(dev)

    nsets = args.sets or max(2, math.ceil((1 << 30) / max(ideal, 1)))
    sets = []
    for r in range(nsets):
        inp = workloads.make_inputs(w, Ho, Wo, seed=w.seed + r)
        om = dev_tensor(inp.om)
        sets.append((dev_tensor(inp.x), om, torch.empty_like(om),
                     torch.empty(plan.out_shape(), dtype=tdt, device=dev)))
    torch.cuda.synchronize()
    legs = {
        "dcn4_forward": lambda i, st: plan.forward(
            sets[i % nsets][0], sets[i % nsets][1], out=sets[i % nsets][3], stream=st),
        "dcnv3_aggregation": lambda i, st: plan.dcnv3_forward(
            sets[i % nsets][0], sets[i % nsets][1], out=sets[i % nsets][3], stream=st),
        "dcnv3_softmax": lambda i, st: plan.dcnv3_softmax(
            sets[i % nsets][1], out=sets[i % nsets][2], stream=st),
    }
    us = {}
    for leg, step in legs.items():
        us[leg] = timed_steps(torch, dev, stream, step, args) * 1e3
        print(f"# {leg}: {us[leg]:.2f} us per launch", file=sys.stderr, flush=True)
    om_bytes = w.N * Ho * Wo * w.G * 3 * w.K * (4 if w.dtype == "f32" else 2)
    v4 = us["dcn4_forward"]
    print(json.dumps({
        "metric": "DCNv4 forward against DCNv3's design: time ratio (DCNv3 / DCNv4)",
        "value": round(us["dcnv3_aggregation"] / v4, 3), "unit": "x",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "clock_settle_ms": args.settled_ms,
        "ms_per_step": round(v4 * 1e-3, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded, the workload's shapes and distributions)",
        "config": {"workload": name, "ideal_bytes": ideal, "input_sets": nsets,
                   "launch": "eager" if args.eager else "hip_graph", "plan": plan.info()},
        "us_per_launch": {k: round(v, 3) for k, v in us.items()},
        "ideal_gbs": {"dcn4_forward": round(ideal / v4 * 1e-3, 1),
                      "dcnv3_aggregation": round(ideal / us["dcnv3_aggregation"] * 1e-3, 1),
                      "dcnv3_softmax": round(2 * om_bytes / us["dcnv3_softmax"] * 1e-3, 1)},
        "ratio_with_softmax": round((us["dcnv3_aggregation"] + us["dcnv3_softmax"]) / v4, 3),
        "kernel_source": kernel_source_digest()}), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix peak


def bench_linear(args, torch, np, workloads, d4, name, w):
    """One step = dcn4_offset_linear over the workload's pixels: features
    [N*Ho*Wo, C] times the merged offset/weight matrix [G*3K, C] plus bias,
    written as the offset/weight tensor.  Ideal bytes: features, weight and
    bias read once, the output written once."""
    if w.dtype == "f32":
        raise SystemExit("bench.py --linear: the layer runs bf16 and fp16 only")
    plan = d4.Plan(d4.Desc(w.N, w.H, w.W, w.C, w.G, w.kh, w.kw, w.sh, w.sw, w.ph, w.pw,
                           w.dh, w.dw, w.offset_scale, w.multiscale, w.dtype,
                           w.pixel_scales, w.max_scale))
    M, Cin, Nout = w.N * plan.Ho * plan.Wo, w.C, w.G * 3 * w.K
    ideal = (M * Cin + Nout * Cin + M * Nout) * 2 + Nout * 4
    flops = 2.0 * M * Cin * Nout
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16}[w.dtype]
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    nsets = args.sets or max(2, math.ceil((1 << 30) / max(ideal, 1)))
    sets = []
    for r in range(nsets):
        f, wt, b = workloads.make_linear_inputs(M, Cin, Nout, w.dtype, seed=w.seed + r)
        sets.append((torch.from_numpy(f.view(np.int16)).view(tdt).to(dev),
                     torch.from_numpy(wt.view(np.int16)).view(tdt).to(dev),
                     torch.from_numpy(b).to(dev),
                     torch.empty((M, Nout), dtype=tdt, device=dev)))
    torch.cuda.synchronize()

    def step(i, st):
        f, wt, b, out = sets[i % nsets]
        d4.offset_linear(f, wt, b, out=out, stream=st)

    ms = timed_steps(torch, dev, stream, step, args)
    gbs = ideal / (ms * 1e-3) / 1e9
    tfs = flops / (ms * 1e-3) / 1e12
    print(json.dumps({
        "metric": "offset/weight linear GB/s (ideal bytes: features, weight, bias read; "
                  "offset/weight tensor written)",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "clock_settle_ms": args.settled_ms, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded normal features and weights)",
        "config": {"workload": name, "pass": "offset_linear", "M": M, "Cin": Cin,
                   "Nout": Nout, "ideal_bytes": ideal, "flops": flops, "input_sets": nsets},
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2),
        "tflops": round(tfs, 2),
        "pct_mfma_peak": round(100.0 * tfs / MFMA_BF16_PEAK_TFLOPS, 2)}), flush=True)


def bench_dwconv(args, torch, np, workloads, d4, name, w):
    """One step = dcn4_dwconv3x3 over the workload's input feature map
    [N, H, W, C] with a [3, 3, C] weight and fp32 bias.  Ideal bytes: input,
    weight and bias read once, output written once."""
    tdt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[w.dtype]
    es = 4 if w.dtype == "f32" else 2
    n_el = w.N * w.H * w.W * w.C
    ideal = 2 * n_el * es + 9 * w.C * es + 4 * w.C
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    nsets = args.sets or max(2, math.ceil((1 << 30) / max(ideal, 1)))
    rng = np.random.default_rng(w.seed)
    wt = torch.from_numpy(rng.standard_normal((3, 3, w.C), dtype=np.float32) / 3).to(tdt).to(dev)
    bias = torch.from_numpy(rng.standard_normal(w.C, dtype=np.float32)).to(dev)
    sets = []
    for r in range(nsets):
        x = torch.from_numpy(np.random.default_rng(w.seed + r).standard_normal(
            (w.N, w.H, w.W, w.C), dtype=np.float32)).to(tdt).to(dev)
        sets.append((x, torch.empty_like(x)))
    torch.cuda.synchronize()

    def step(i, st):
        x, out = sets[i % nsets]
        d4.dwconv3x3(x, wt, bias, out=out, stream=st)

    ms = timed_steps(torch, dev, stream, step, args)
    gbs = ideal / (ms * 1e-3) / 1e9
    print(json.dumps({
        "metric": "depthwise 3x3 GB/s (ideal bytes: input, weight, bias read; output written)",
        "value": round(gbs, 2), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "clock_settle_ms": args.settled_ms, "ms_per_step": round(ms, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
        "data": "synthetic (seeded normal inputs and weights)",
        "config": {"workload": name, "pass": "dwconv3x3", "N": w.N, "H": w.H, "W": w.W,
                   "C": w.C, "ideal_bytes": ideal, "input_sets": nsets},
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 2)}), flush=True)


def copy_reference(torch, mib, steps):
    """Plain device-to-device copies of a known size: rocprofv3's FETCH_SIZE
    and WRITE_SIZE of one such copy dispatch scale the operator's counters."""
    n = mib * (1 << 20) // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(steps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_reference_bytes_read": n * 4, "copy_reference_bytes_written": n * 4,
                      "steps": steps}), flush=True)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, Ho, Wo, inp, reps):
    """The CPU oracle as it stands (fp32 evaluation, OpenMP over output
    pixels) on the host cores: the full batch of the first input set on every
    core the process may use, and its first image on one core."""
    import numpy as np
    import oracle
    from oracle import Shape
    o = oracle.get()
    s = Shape(w.N, w.H, w.W, w.C, w.G, w.kh, w.kw, w.sh, w.sw, w.ph, w.pw,
              w.dh, w.dw, w.offset_scale, w.multiscale, w.pixel_scales, w.max_scale)
    threads = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    env_t = os.environ.get("OMP_NUM_THREADS")
    if env_t and env_t.isdigit():
        threads = min(threads, int(env_t))

    def timed(shape, x, om, ps, nthreads):
        times = []
        for _ in range(reps):
            t = time.perf_counter()
            o.forward_f32(shape, w.dtype, x, om, inp.scales, nthreads=nthreads, pscales=ps)
            times.append(time.perf_counter() - t)
        return statistics.median(times)

    med = timed(s, inp.x, inp.om, inp.pscales, threads)
    ideal = o.ideal_bytes(s, w.dtype)
    s1 = dataclasses.replace(s, N=1)
    med1 = timed(s1, np.ascontiguousarray(inp.x[:1]), np.ascontiguousarray(inp.om[:1]),
                 None if inp.pscales is None else np.ascontiguousarray(inp.pscales[:1]), 1)
    ideal1 = o.ideal_bytes(s1, w.dtype)
    return {"value": round(ideal / med / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the full batch ({w.N} images) on {threads} threads, median of "
                      f"{reps} runs of {med:.2f} s; one image on 1 thread, median of "
                      f"{reps} runs of {med1:.2f} s; fp32 evaluation",
            "output_pixels_per_s": round(w.N * Ho * Wo / med, 1),
            "outputs_per_s": round(w.N * Ho * Wo * w.C / med, 1),
            "single_thread": {"value": round(ideal1 / med1 / 1e9, 4), "unit": "GB/s",
                              "output_pixels_per_s": round(Ho * Wo / med1, 1)},
            "nproc": os.cpu_count(), "cpu_model": cpu_model()}


if __name__ == "__main__":
    main()
