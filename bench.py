"""Benchmark: forward convolution through the HIP library on one MI355X.

A step is one pass of the whole path over the workload's batch: for every
layer, the filter pack, the input lowering (im2win strips by default) and the
MFMA contraction with its fused bias epilogue; chained layers feed each
other's outputs.  Inputs are resident in device memory before timing starts.

Default workload (N=1): the MSCRED-style encoder stack -- 1280 images of three
30x30 symmetric signature matrices, fp32 NCHW, four convolutions 3x3 3->32 s1
p1, 3x3 32->64 s2, 2x2 64->128 s2, 2x2 128->256 s2 ("GPU-Accelerating MSCRED
with CUDA, im2col, GEMM, and a Custom PyTorch Extension", sections
"Experimental Setup" and "Where the Performance Bottleneck Appeared").  The
other workloads (c1, c3, c4, c5) can be timed with --workload.

Prints one JSON line: TFLOP/s of the whole step (2*N*K*P*Q*C*R*S summed over
layers / step time), the roofline position of the dominant kernel measured
with HIP events on its own stream over the timed region, and the fp64
reference convolution timed on the host cores on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "conv2d fwd TFLOPS and % of MFMA peak; workspace bytes vs im2col"
# MI355X published peaks: dense MFMA per storage type, HBM3E bandwidth
PEAK_TFLOPS = {"f32": 157.3, "f16": 2516.6, "bf16": 2516.6}
PEAK_HBM_GBS = 8000.0
# ConvLSTM step measured beside the stack (--workload lstm): one cell per
# encoder level of c2 (hidden channels = the level's channels, 3x3 gate
# filter, same padding), 256 windows, 5 time steps per pass.
LSTM_LEVELS = [(32, 30), (64, 14), (128, 7), (256, 3)]   # (channels, H = W)
LSTM_WINDOWS, LSTM_STEPS = 256, 5
WORKLOAD_TEXT = {
    "c1": "single conv2d fp32 NCHW N=1 3x30x30, 3x3 3->32 s1 p1",
    "lstm": "ConvLSTM cells over the four c2 encoder levels (32x30x30, 64x14x14, 128x7x7, 256x3x3), fp32 "
            "NCHW, 256 windows, 5 time steps, gates from a 3x3 same-padded convolution over concat(x_t, "
            "h_t-1), cell update fused into the contraction",
    "c2": "MSCRED-style encoder stack fp32 NCHW N=1280 (256 windows x 5 steps) of 3x30x30 symmetric signature "
          "matrices: 3x3 3->32 s1p1; 3x3 32->64 s2; 2x2 64->128 s2; 2x2 128->256 s2",
    "c3": "ResNet-style 3x3 fp16 NHWC N=64 C=K=256 14x14 s1 p1",
    "c4": "mixed bf16 NHWC N=128: 7x7 s2p3 3->64 224x224; 1x1 1024->256 14x14; 3x3 512->512 7x7",
    "c5": "kernel-size sweep fp16 NHWC N=32 C=K=128 64x64 same padding R=S in {1,3,5,7,11}",
}
CSRC = os.path.join(ROOT, "cnn_convolution_lowering_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def source_digest() -> str:
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def build_layers(wl, dev, algo):
    import cnn_convolution_lowering_amd as cl
    import torch
    spec = wl.spec
    layers = []
    prev_y = None
    for L in wl.layers:
        x = L.x.to(dev) if L.x is not None else prev_y
        d = cl.Conv2d(*(_x_dims(x.shape, spec.layout)), L.K, L.R, L.S, stride=L.stride, padding=L.padding,
                      dilation=L.dilation, layout=spec.layout, dtype=spec.dtype, algo=algo)
        y = d.new_output(dev)
        layers.append(dict(spec=L, desc=d, x=x, w=L.w.to(dev), b=L.b.to(dev), y=y,
                           flops=2 * spec.N * L.K * d.P * d.Q * L.C * L.R * L.S))
        prev_y = y if spec.chained else None
    ws_bytes = max(l["desc"].workspace_bytes for l in layers)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)
    return layers, ws


def _x_dims(shape, layout):
    if layout == "nchw":
        N, C, H, W = shape
    else:
        N, H, W, C = shape
    return N, C, H, W


STAGES = ("pack", "lower", "contract")


def run_stage(l, stage, ws, stream):
    d = l["desc"]
    if stage == "pack":
        d.pack_filter(l["w"], ws, stream)
    elif stage == "lower":
        d.lower_input(l["x"], ws, stream)
    else:
        d.contract(l["x"], l["w"], l["b"], l["y"], ws, stream)


def stage_launches(l, stage) -> bool:
    info = l["desc"].info
    if stage == "pack":
        return info["ws_filter_bytes"] > 0
    if stage == "lower":
        return info["lowering_elided"] == 0
    return True


def kernel_breakdown(layers, ws, stream, reps=10):
    """Average duration (ms) of every launched kernel, from HIP events on `stream`."""
    import torch
    out = {}
    for i, l in enumerate(layers):
        for st in STAGES:
            if not stage_launches(l, st):
                continue
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
            for a, b in evs:
                for st2 in STAGES:          # keep the data flow of a real step
                    if st2 == st:
                        a.record(stream)
                        run_stage(l, st2, ws, stream)
                        b.record(stream)
                    else:
                        run_stage(l, st2, ws, stream)
            torch.cuda.synchronize()
            out[(i, st)] = sum(a.elapsed_time(b) for a, b in evs) / reps
    return out


def kernel_work(l, stage):
    """(algorithmic flops, algorithmic bytes) of one launch of a stage kernel."""
    info = l["desc"].info
    eb = info["elem_bytes"]
    d = l["desc"]
    p = d.params
    x_bytes = p.N * p.C * p.H * p.W * eb
    w_bytes = p.K * p.C * p.R * p.S * eb
    y_bytes = p.N * p.K * d.P * d.Q * eb
    if stage == "contract":
        a_bytes = x_bytes if info["lowering_elided"] else info["ws_lowered_bytes"]
        b_bytes = info["ws_filter_bytes"] or w_bytes
        return l["flops"], a_bytes + b_bytes + y_bytes + p.K * eb
    if stage == "lower":
        return 0, x_bytes + info["ws_lowered_bytes"]
    return 0, w_bytes + info["ws_filter_bytes"]


CONTRACT_KERNELS = ["conv_gemm_kernel", "conv_gemm_dma_kernel", "conv_gemm_wide_kernel", "conv_nchw_f32_dma_kernel",
                    "conv_strip_kernel", "conv_strip_rb_kernel", "conv_nchw_f32_strip_kernel",
                    "conv_nchw_f32_tile_kernel", "conv_nhwc_tile16_kernel"]


def kernel_symbol(l, stage):
    """Name of the kernel a stage launches (as the kernel trace shows it)."""
    d = l["desc"]
    info = d.info
    if stage == "contract":
        return CONTRACT_KERNELS[info["kernel"]]
    if stage == "pack":
        if info["kernel"] == 5:
            return "pack_filter_frag_kernel"
        return {6: "pack_filter_frag_f32_kernel", 8: "pack_filter_tile16_kernel"}.get(info["kernel"],
                                                                                    "pack_filter_kernel")
    # NHWC with C a whole number of 16-byte vectors: the direct vector copy;
    # otherwise the band kernel (the element-wise fallback, for a one-column
    # tile beyond the LDS budget, occurs in none of the workloads).
    if d.layout == "nhwc" and d.params.C % (16 // info["elem_bytes"]) == 0:
        return "%s_nhwc_vec_kernel" % d.algo
    return "lower_%s_band_kernel" % d.layout


def cpu_baseline(wl, budget_s=10.0):
    """The fp64 reference convolution, as it stands, on a bounded sample of the
    workload's images (every layer, chained as the workload chains them)."""
    import numpy as np
    import torch
    import oracle
    spec = wl.spec
    threads = oracle.default_threads()

    def run(n_img):
        flops = 0
        t0 = time.perf_counter()
        prev = None
        for L in wl.layers:
            x = (L.x[:n_img] if L.x is not None else prev)
            y = oracle.conv2d(x, L.w, L.b, layout=spec.layout, stride=L.stride, padding=L.padding,
                              dilation=L.dilation, nthreads=threads)
            if spec.layout == "nchw":
                _, K, P, Q = y.shape
            else:
                _, P, Q, K = y.shape
            flops += 2 * n_img * K * P * Q * L.C * L.R * L.S
            prev = torch.from_numpy(np.ascontiguousarray(y)).to(wl.dtype) if spec.chained else None
        return flops, time.perf_counter() - t0

    probe = max(1, min(spec.N, 4))
    f, t = run(probe)
    n = int(min(spec.N, max(probe, probe * budget_s / max(t, 1e-6))))
    if n > probe:
        f, t = run(n)
    else:
        n = probe
    return {"value": f / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "sample": "%d of %d images of workload %s, all %d layers, fp64 seven-loop reference, %.1f s"
                      % (n, spec.N, spec.name, len(wl.layers), t)}


def bench_lstm(args, dev):
    """ConvLSTM passes: LSTM_STEPS time steps of the cell at every level,
    h and c carried on the GPU; the value counts the gate convolutions'
    flops.  The dominant level's conv_lstm_step call (pack, lowering,
    contraction) is timed with HIP events inside the timed region."""
    import torch
    import cnn_convolution_lowering_amd as cl
    g = torch.Generator().manual_seed(5)
    levels = []
    for ch, hw in LSTM_LEVELS:
        cell = cl.ConvLSTMCell(LSTM_WINDOWS, ch, ch, hw, hw, 3, 3, padding=1, algo=args.algo)
        xs = [(torch.rand(LSTM_WINDOWS, ch, hw, hw, generator=g) * 2 - 1).to(dev) for _ in range(LSTM_STEPS)]
        w = (torch.randn(4 * ch, 2 * ch, 3, 3, generator=g) / (18 * ch) ** 0.5).to(dev)
        b = (torch.randn(4 * ch, generator=g) * 0.01).to(dev)
        st = [torch.zeros(LSTM_WINDOWS, ch, hw, hw, device=dev) for _ in range(4)]   # h, c, h', c'
        flops = 2.0 * LSTM_WINDOWS * 4 * ch * hw * hw * 2 * ch * 9
        levels.append({"cell": cell, "xs": xs, "w": w, "b": b, "st": st, "ws": cell.new_workspace(dev),
                       "flops": flops, "ch": ch, "hw": hw})
    step_flops = sum(l["flops"] for l in levels) * LSTM_STEPS
    dom = max(range(len(levels)), key=lambda i: levels[i]["flops"])

    def one_pass(rec=None):
        for i, l in enumerate(levels):
            h, c, h2, c2 = l["st"]
            for t in range(LSTM_STEPS):
                if rec is not None and i == dom and t == 0:
                    rec[0].record()
                l["cell"].step(l["xs"][t], h, c, l["w"], l["b"], h_out=h2, c_out=c2, ws=l["ws"])
                if rec is not None and i == dom and t == 0:
                    rec[1].record()
                h, c, h2, c2 = h2, c2, h, c

    for _ in range(args.warmup):
        one_pass()
    torch.cuda.synchronize()
    recs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record()
    for i in range(args.steps):
        one_pass(recs[i])
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / args.steps
    dom_ms = sum(a.elapsed_time(b) for a, b in recs) / args.steps
    achieved = levels[dom]["flops"] / (dom_ms * 1e-3) / 1e12
    out = {"metric": "ConvLSTM step gate-convolution TFLOP/s", "value": step_flops / (ms * 1e-3) / 1e12,
           "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms,
           "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
           "config": {"workload": "lstm: " + WORKLOAD_TEXT["lstm"], "algo": args.algo},
           "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_TFLOPS["f32"], "unit": "TFLOP/s",
                        "frac": achieved / PEAK_TFLOPS["f32"], "traffic": None,
                        "kernel": "conv_lstm_step (pack, lowering, conv_gemm_dma_kernel with the cell epilogue)",
                        "level": "%dx%dx%d" % (levels[dom]["ch"], levels[dom]["hw"], levels[dom]["hw"]),
                        "avg_launch_ms": dom_ms}}
    if not args.no_cpu_baseline:
        import numpy as np
        from oracle.convlstm import convlstm_step
        l = levels[0]

        def run(n):
            x = l["xs"][0][:n].cpu()
            h = torch.zeros(n, l["ch"], l["hw"], l["hw"])
            t = time.perf_counter()
            convlstm_step(x, h, h, l["w"].cpu(), l["b"].cpu(), padding=1)
            return time.perf_counter() - t

        n = 2
        dt = run(n)
        m = int(min(LSTM_WINDOWS, max(n, n * args.cpu_budget / max(dt, 1e-6))))
        if m > n:
            n, dt = m, run(m)
        import oracle
        out["cpu_baseline"] = {"value": l["flops"] * n / LSTM_WINDOWS / dt / 1e12, "unit": "TFLOP/s",
                               "cores": oracle.default_threads(), "kind": "oracle",
                               "sample": "%d of %d windows, one step of the 32x30x30 level, fp64 reference, %.2f s"
                                         % (n, LSTM_WINDOWS, dt)}
    print(json.dumps(out), flush=True)
    return 0


def time_steps(wl, dev, algo, steps, warmup, layer=None):
    """ms per step of the whole path with one lowering, HIP events on the
    current stream; also the largest workspace of its layers."""
    import torch
    layers, ws = build_layers(wl, dev, algo)
    stream = torch.cuda.current_stream(dev)
    if layer is not None:
        for l in layers[:layer]:
            for st in STAGES:
                run_stage(l, st, ws, stream)
        layers = [layers[layer]]
    for _ in range(warmup):
        for l in layers:
            for st in STAGES:
                run_stage(l, st, ws, stream)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(steps):
        for l in layers:
            for st in STAGES:
                run_stage(l, st, ws, stream)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    info = {"ms_per_step": ms,
            "workspace_bytes": max(l["desc"].workspace_bytes for l in layers),
            "lowered_bytes_max": max(l["desc"].info["ws_lowered_bytes"] for l in layers),
            "im2col_bytes_max": max(l["desc"].info["im2col_bytes"] for l in layers)}
    del layers, ws
    return info


def load_traffic(kernel_key: str):
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != source_digest():
        return None      # counters were taken on a different kernel source
    return rec.get("bytes_per_launch")


def gemm_calibration(dev):
    """torch.matmul (hipBLASLt) on A[M x C*R*S] @ B[C*R*S x K] for every layer
    of the 16-bit workloads -- the contraction of each convolution without its
    window gather -- and on 8192^3 in fp16, bf16 and fp32, 20 timed calls each
    after 3 warm-up calls;
    one JSON line per product."""
    import torch
    import cnn_convolution_lowering_amd as cl
    from cnn_convolution_lowering_amd.workloads import workload_spec
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
    torch.backends.cuda.matmul.allow_tf32 = False   # full fp32 products
    shapes = []
    for name in ("c3", "c4", "c5"):
        spec = workload_spec(name)
        H = W = None
        for L in spec.layers:
            if L.H is not None:
                H, W = L.H, L.W
            c = cl.Conv2d(spec.N, L.C, H, W, L.K, L.R, L.S, stride=L.stride, padding=L.padding,
                          layout=spec.layout, dtype=spec.dtype, algo="implicit")
            shapes.append(("%s %s" % (name, L.label), spec.dtype, c.info["M"], L.K, L.C * L.R * L.S))
            if spec.chained:
                H, W = c.P, c.Q
    shapes += [("square 8192", dt, 8192, 8192, 8192) for dt in ("f16", "bf16", "f32")]
    for label, dt, M, N, K in shapes:
        g = torch.Generator(device=dev).manual_seed(7)
        a = torch.randn(M, K, device=dev, generator=g).to(tdt[dt])
        b = torch.randn(K, N, device=dev, generator=g).to(tdt[dt])
        for _ in range(3):
            c = a @ b
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(20):
            c = a @ b
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 20
        tf = 2.0 * M * N * K / (ms * 1e-3) / 1e12
        print(json.dumps({"gemm": label, "dtype": dt, "M": M, "N": N, "K": K, "ms": round(ms, 4),
                          "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_TFLOPS[dt], 3)}), flush=True)
        del a, b, c
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c2", choices=sorted(WORKLOAD_TEXT))
    ap.add_argument("--algo", default="implicit", choices=["im2win", "im2col", "implicit"],
                    help="lowering timed for the headline value (the other two are timed as well, "
                         "unless --only-algo)")
    ap.add_argument("--only-algo", action="store_true", help="time only --algo")
    ap.add_argument("--layer", type=int, default=None,
                    help="time only this layer of the workload (chained inputs are still computed once)")
    ap.add_argument("--tune", action="store_true",
                    help="conv_tune every layer (kernel and tile variant) before timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of reference work to time")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB (5 times), to scale "
                         "the HBM byte counters of a profiler against a transfer of known size")
    ap.add_argument("--gemm-calibration", action="store_true",
                    help="only time the vendor GEMM (torch.matmul, hipBLASLt) on the plain M x K x C*R*S "
                         "products of the 16-bit workloads' layers and on 8192^3 products (fp16, bf16, "
                         "fp32): what the library reaches on this GPU, a measured peak next to the "
                         "published one")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print("bench.py: measures one GPU; --gpus %d is not supported (the convolution would shard over "
              "images, each GPU running the same path on its share with no exchange)" % args.gpus, file=sys.stderr)
        return 2

    import torch
    import cnn_convolution_lowering_amd as cl
    from cnn_convolution_lowering_amd.workloads import make_workload

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    cl.load_library()
    dev = torch.device("cuda:0")
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_per_launch": n, "launches": 5}))
        return 0
    if args.gemm_calibration:
        return gemm_calibration(dev)
    if args.workload == "lstm":
        if args.algo == "implicit":
            args.algo = "im2win"   # the ConvLSTM step reads x and h through the lowering
        return bench_lstm(args, dev)
    wl = make_workload(args.workload)
    spec = wl.spec
    print("bench: workload %s, algo %s, building inputs" % (spec.name, args.algo), file=sys.stderr, flush=True)
    layers, ws = build_layers(wl, dev, args.algo)
    stream = torch.cuda.current_stream(dev)
    tuned = None
    if args.tune:
        print("bench: tuning the layers' kernels", file=sys.stderr, flush=True)
        tuned = []
        for l in layers:   # in order: a chained layer's input is its producer's output
            r = l["desc"].tune(l["x"], l["w"], l["b"], l["y"], ws, reps=5)
            tuned.append({"layer": l["spec"].label, "kernel": r["kernel"], "variant": r["kernel_variant"],
                          "candidates": r["candidates"], "default_ms": r["default_ms"], "best_ms": r["best_ms"]})
    if args.layer is not None:
        # inputs of a chained layer come from one pass of the layers before it
        for l in layers[:args.layer]:
            for st in STAGES:
                run_stage(l, st, ws, stream)
        layers = [layers[args.layer]]
    step_flops = sum(l["flops"] for l in layers)

    # Per-kernel durations (outside the timed region) pick the dominant kernel.
    for _ in range(2):
        for l in layers:
            for st in STAGES:
                run_stage(l, st, ws, stream)
    torch.cuda.synchronize()
    brk = kernel_breakdown(layers, ws, stream)
    dom = max(brk, key=brk.get)
    dom_layer, dom_stage = dom

    def step(rec=None):
        for i, l in enumerate(layers):
            for st in STAGES:
                if rec is not None and (i, st) == dom:
                    rec[0].record(stream)
                    run_stage(l, st, ws, stream)
                    rec[1].record(stream)
                else:
                    run_stage(l, st, ws, stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    print("bench: timing %d steps" % args.steps, file=sys.stderr, flush=True)
    recs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    t_start.record(stream)
    for k in range(args.steps):
        step(recs[k])
    t_end.record(stream)
    torch.cuda.synchronize()
    h1 = time.perf_counter()
    ms_step = t_start.elapsed_time(t_end) / args.steps
    dom_ms = sum(a.elapsed_time(b) for a, b in recs) / args.steps
    tflops = step_flops / (ms_step * 1e-3) / 1e12

    # roofline of the dominant kernel
    dl = layers[dom_layer]
    flops, nbytes = kernel_work(dl, dom_stage)
    peak_f = PEAK_TFLOPS[spec.dtype]
    compute_bound = flops > 0 and flops / (peak_f * 1e12) >= nbytes / (PEAK_HBM_GBS * 1e9)
    kernel_key = "%s/%s/layer%d/%s" % (spec.name, args.algo, dom_layer, dom_stage)
    traffic = load_traffic(kernel_key)
    if compute_bound:
        achieved = flops / (dom_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak_f, "unit": "TFLOP/s", "frac": achieved / peak_f}
    else:
        achieved = nbytes / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
    roof.update({"traffic": traffic, "kernel": kernel_symbol(dl, dom_stage), "kernel_key": kernel_key,
                 "layer": dl["spec"].label, "avg_launch_ms": dom_ms, "algorithmic_flops": flops,
                 "algorithmic_bytes": nbytes})

    per_layer = []
    for i, l in enumerate(layers):
        info = l["desc"].info
        lay_ms = sum(v for (j, _), v in brk.items() if j == i)
        # compulsory traffic B_min = x + w + b + y once, and the layer's bound
        p, eb = l["desc"].params, info["elem_bytes"]
        b_min = (p.N * p.C * p.H * p.W + p.K * p.C * p.R * p.S + p.K + p.N * p.K * l["desc"].P * l["desc"].Q) * eb
        mfma_bound = l["flops"] / (peak_f * 1e12) >= b_min / (PEAK_HBM_GBS * 1e9)
        gbs = b_min / (lay_ms * 1e-3) / 1e9 if lay_ms else None
        tfs = l["flops"] / (lay_ms * 1e-3) / 1e12 if lay_ms else None
        per_layer.append({
            "layer": l["spec"].label, "gflop": l["flops"] / 1e9,
            "kernels_ms": {st: round(brk[(i, st)], 5) for st in STAGES if (i, st) in brk},
            "tflops_isolated": tfs,
            "bound": "mfma" if mfma_bound else "hbm",
            "frac_of_peak": (tfs / peak_f if mfma_bound else gbs / PEAK_HBM_GBS) if lay_ms else None,
            "b_min_bytes": b_min, "b_min_gbs_isolated": gbs,
            "ws_lowered_bytes": info["ws_lowered_bytes"], "im2col_bytes": info["im2col_bytes"],
            "ws_vs_im2col": info["ws_lowered_bytes"] / info["im2col_bytes"],
            "tile": [info["tile_m"], info["tile_n"], info["tile_k"]]})

    out = {
        "metric": METRIC, "value": tflops, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": spec.dtype, "data": "synthetic",
        "config": {"workload": "%s: %s" % (spec.name, WORKLOAD_TEXT[spec.name]), "algo": args.algo,
                   "batch": spec.N, "layers": len(layers), "layout": spec.layout},
        "pct_of_mfma_peak": 100.0 * tflops / peak_f,
        "host_ms_per_step": (h1 - h0) * 1e3 / args.steps,
        "roofline": roof,
        "workspace": {"bytes": max(l["desc"].workspace_bytes for l in layers),
                      "lowered_max_bytes": max(p["ws_lowered_bytes"] for p in per_layer),
                      "im2col_max_bytes": max(p["im2col_bytes"] for p in per_layer),
                      "ratio_max_over_layers": max(p["ws_vs_im2col"] for p in per_layer)},
        "layers": per_layer,
    }
    if tuned is not None:
        out["config"]["tuned"] = True
        out["tuning"] = tuned
    if not args.only_algo:
        flops_total = step_flops
        algos = {}
        for algo in ("implicit", "im2win", "im2col"):
            print("bench: timing the %s lowering" % algo, file=sys.stderr, flush=True)
            r = time_steps(wl, dev, algo, max(5, args.steps // 2), max(2, args.warmup // 2), args.layer)
            r["tflops"] = flops_total / (r["ms_per_step"] * 1e-3) / 1e12
            algos[algo] = r
        out["algorithms"] = algos
    if not args.no_cpu_baseline:
        print("bench: timing the fp64 reference on the host", file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
