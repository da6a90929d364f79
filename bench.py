"""Benchmark: forward convolution through the HIP library on one MI355X.

A step is one pass of the whole path over one workload's batch: for every
layer, the filter pack, the input lowering and the MFMA contraction with its
fused bias epilogue (by default the fused path, whose windows are staged
straight into LDS, so there is no lowering launch); chained layers feed each
other's outputs.  Inputs are resident in device memory before timing starts.

Headline (the default, N=1): the kernel-size sweep -- fp16 NHWC, 32 images of
128 channels at 64x64, R = S in {1, 3, 5, 7, 11}, same padding -- the largest
of the five workloads (880 GFLOP per step).  The other four workloads get a
record each in the same JSON line (--configs).

Timing ("GPU-Accelerating MSCRED with CUDA, im2col, GEMM, and a Custom PyTorch
Extension", section "Timing Methodology": the same input dimensions and batch
for every measurement; "Thousands of (not-so) tiny SVDs: from 15 s to 66 ms on
a GPU": best of several runs after a warm-up):
  cold  every step follows a streaming pass over a 512 MiB buffer, twice the
        256 MB last-level cache, so the step's inputs come from HBM; HIP events
        around each step; the headline value is the median of these steps;
  warm  the same steps back to back;
both give the median over all timed steps and the best step.  The dominant
kernel's launches are timed with HIP events on their own stream inside the
cold timed region.  Measured peaks of this GPU (a register-only MFMA loop per
instruction, the shader clock under it, a streaming copy) are taken in the
same run and every fraction is given against them as well as against the
published MI355X figures.

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "conv2d fwd TFLOPS and % of MFMA peak; workspace bytes vs im2col"
# MI355X published peaks: dense MFMA per storage type, HBM3E bandwidth
PEAK_TFLOPS = {"f32": 157.3, "f16": 2516.6, "bf16": 2516.6}
PEAK_HBM_GBS = 8000.0
FLUSH_BYTES = 512 << 20          # twice the 256 MB last-level cache
# ConvLSTM step measured on its own (--workload lstm): one cell per encoder
# level of c2 (hidden channels = the level's channels, 3x3 gate filter, same
# padding), 256 windows, 5 time steps per pass.
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


# Host-only sources (planner and C ABI; the peak library): not part of any
# convolution kernel's device code.
HOST_ONLY = ("convlower.hip", "peak.hip")


def source_digest() -> str:
    """Digest of the device code of the convolution kernels.  A traffic
    record also names the plan it was taken on, so a planner change that
    picks another kernel for the layer invalidates it as well."""
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        if name in HOST_ONLY:
            continue
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def _x_dims(shape, layout):
    if layout == "nchw":
        N, C, H, W = shape
    else:
        N, H, W, C = shape
    return N, C, H, W


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
    """Average duration (ms) of every launched stage, from HIP events on `stream`."""
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
    """(algorithmic flops, algorithmic bytes) of one launch of a stage.

    contract: 2*C*R*S flops per output element; bytes = the A operand read
    once (x for the fused and in-place paths, else the lowered buffer) + the
    filter (or its packed copy) + y + bias.  lower: x + the lowered buffer.
    pack: the filter + its packed copy."""
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
                    "conv_nchw_f32_tile_kernel", "conv_nhwc_tile16_kernel", "conv_gemm_streamk_kernel",
                    "conv_strip_rb2_kernel", "conv_nchw_f32_taps_kernel", "conv_strip_rb3_kernel",
                    "conv_strip_rb4_kernel", "conv_1x1_stream_kernel"]


def kernel_symbol(l, stage):
    """Name of the kernel a stage launches (as the kernel trace shows it)."""
    d = l["desc"]
    info = d.info
    if stage == "contract":
        return CONTRACT_KERNELS[info["kernel"]]
    if stage == "pack":
        if info["kernel"] in (5, 10):
            return "pack_filter_frag_kernel"
        return {6: "pack_filter_frag_f32_kernel", 11: "pack_filter_frag_f32_kernel",
                8: "pack_filter_tile16_kernel", 12: "pack_filter_frag16_kernel",
                13: "pack_filter_frag16_kernel"}.get(info["kernel"],
                                                                                    "pack_filter_kernel")
    # NHWC with C a whole number of 16-byte vectors: the direct vector copy;
    # fp32 window rows that are not whole vectors: the unpadded element-wise
    # lowering; otherwise the band kernel (the element-wise fallback, for a
    # one-column tile beyond the LDS budget, occurs in none of the workloads).
    p = d.params
    if info["elem_bytes"] == 4 and (p.R * p.C) % 4 and info["RCp"] == p.R * p.C:
        return "lower_unpadded_kernel"
    if d.layout == "nhwc" and d.params.C % (16 // info["elem_bytes"]) == 0:
        return "%s_nhwc_vec_kernel" % d.algo
    return "lower_%s_band_kernel" % d.layout


def load_traffic(kernel_key: str, plan):
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("source_sha256_16") != source_digest() or rec.get("plan") != list(plan):
        return None      # counters were taken on a different kernel source or plan
    return rec.get("bytes_per_launch")


def plan_of(info):
    return [info["kernel"], info["kernel_variant"], info["ksplit"], info["tile_order"]]


class Flusher:
    """A streaming read-modify-write of FLUSH_BYTES (twice the 256 MB
    last-level cache) between cold steps."""

    def __init__(self, dev):
        import torch
        self.buf = torch.zeros(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)

    def __call__(self):
        self.buf.add_(1.0)


def time_steps(step, stream, steps, warmup, flush=None, rec_dom=False):
    """Per-step ms from HIP events on `stream` (warm: back to back; cold:
    `flush` before each step, outside its events), the dominant kernel's
    launch times when `rec_dom`, and host wall seconds of the whole region."""
    import torch
    for _ in range(warmup):
        if flush:
            flush()
        step(None)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    dom = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    h0 = time.perf_counter()
    for k in range(steps):
        if flush:
            flush()
        evs[k][0].record(stream)
        step(dom[k] if rec_dom else None)
        evs[k][1].record(stream)
    torch.cuda.synchronize()
    h1 = time.perf_counter()
    ms = [a.elapsed_time(b) for a, b in evs]
    dms = [a.elapsed_time(b) for a, b in dom] if rec_dom else []
    return ms, dms, h1 - h0


def summary(ms):
    s = sorted(ms)
    return {"median_ms": statistics.median(s), "best_ms": s[0], "best5_mean_ms": sum(s[:5]) / len(s[:5]),
            "steps": len(s)}


def bench_config(name, dev, args, peaks, headline=False):
    """Time one workload: the fused path cold and warm (headline measures),
    per-kernel durations, the roofline of its dominant kernel, and the two
    lowered algorithms."""
    import torch
    from cnn_convolution_lowering_amd.workloads import make_workload
    wl = make_workload(name)
    spec = wl.spec
    say("bench: %s: building inputs" % name)
    layers, ws = build_layers(wl, dev, args.algo)
    stream = torch.cuda.current_stream(dev)
    step_flops = sum(l["flops"] for l in layers)
    peak_f = PEAK_TFLOPS[spec.dtype]
    mpeak_f = peaks.get(spec.dtype) if peaks else None

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

    steps = args.steps if headline else max(30, args.steps // 2)
    warmup = args.warmup if headline else max(3, args.warmup // 2)
    flush = Flusher(dev)
    say("bench: %s: %d cold steps" % (name, steps))
    cold_ms, dom_ms_list, host_s = time_steps(step, stream, steps, warmup, flush=flush, rec_dom=True)
    del flush
    torch.cuda.empty_cache()
    say("bench: %s: %d warm steps" % (name, steps))
    warm_ms, _, _ = time_steps(step, stream, steps, warmup)
    cold, warm = summary(cold_ms), summary(warm_ms)
    dom_ms = sum(dom_ms_list) / len(dom_ms_list)

    dl = layers[dom_layer]
    flops, nbytes = kernel_work(dl, dom_stage)
    compute_bound = flops > 0 and flops / (peak_f * 1e12) >= nbytes / (PEAK_HBM_GBS * 1e9)
    kernel_key = "%s/%s/layer%d/%s" % (spec.name, args.algo, dom_layer, dom_stage)
    if compute_bound:
        achieved = flops / (dom_ms * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": peak_f, "unit": "TFLOP/s", "frac": achieved / peak_f}
        if mpeak_f:
            roof.update({"measured_peak": mpeak_f, "frac_of_measured": achieved / mpeak_f})
    else:
        achieved = nbytes / (dom_ms * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": achieved / PEAK_HBM_GBS}
        if peaks and peaks.get("hbm_gbs"):
            roof.update({"measured_peak": peaks["hbm_gbs"], "frac_of_measured": achieved / peaks["hbm_gbs"]})
    roof.update({"traffic": load_traffic(kernel_key, plan_of(dl["desc"].info)), "kernel": kernel_symbol(dl, dom_stage),
                 "kernel_key": kernel_key, "layer": dl["spec"].label, "avg_launch_ms": dom_ms,
                 "launches_timed": len(dom_ms_list), "algorithmic_flops": flops, "algorithmic_bytes": nbytes})

    per_layer = []
    for i, l in enumerate(layers):
        info = l["desc"].info
        lay_ms = sum(v for (j, _), v in brk.items() if j == i)
        p, eb = l["desc"].params, info["elem_bytes"]
        b_min = (p.N * p.C * p.H * p.W + p.K * p.C * p.R * p.S + p.K + p.N * p.K * l["desc"].P * l["desc"].Q) * eb
        mfma_bound = l["flops"] / (peak_f * 1e12) >= b_min / (PEAK_HBM_GBS * 1e9)
        gbs = b_min / (lay_ms * 1e-3) / 1e9 if lay_ms else None
        tfs = l["flops"] / (lay_ms * 1e-3) / 1e12 if lay_ms else None
        rec = {"layer": l["spec"].label, "gflop": l["flops"] / 1e9,
               "kernels_ms": {st: round(brk[(i, st)], 5) for st in STAGES if (i, st) in brk},
               "contract_kernel": kernel_symbol(l, "contract"),
               "plan": plan_of(info),
               "tflops_isolated": tfs, "bound": "mfma" if mfma_bound else "hbm",
               "frac_of_peak": (tfs / peak_f if mfma_bound else gbs / PEAK_HBM_GBS) if lay_ms else None,
               "b_min_bytes": b_min, "b_min_gbs_isolated": gbs,
               "im2win_bytes": info["im2win_bytes"], "im2col_bytes": info["im2col_bytes"],
               "tile": [info["tile_m"], info["tile_n"], info["tile_k"]]}
        if mfma_bound and mpeak_f and tfs:
            rec["frac_of_measured_peak"] = tfs / mpeak_f
        per_layer.append(rec)
    del layers, ws
    torch.cuda.empty_cache()

    rec = {"workload": "%s: %s" % (spec.name, WORKLOAD_TEXT[spec.name]), "dtype": spec.dtype,
           "gflop_per_step": step_flops / 1e9,
           "tflops": step_flops / (cold["median_ms"] * 1e-3) / 1e12,
           "tflops_warm": step_flops / (warm["median_ms"] * 1e-3) / 1e12,
           "tflops_best": step_flops / (min(cold["best_ms"], warm["best_ms"]) * 1e-3) / 1e12,
           "cold": cold, "warm": warm, "host_s_cold_region": host_s,
           "frac_of_peak": step_flops / (cold["median_ms"] * 1e-3) / 1e12 / peak_f, "roofline": roof,
           "layers": per_layer, "algo": args.algo}
    if mpeak_f:
        rec["frac_of_measured_peak"] = rec["tflops"] / mpeak_f

    # The lowered algorithms: their time and workspace (the im2win / im2col comparison).
    algos = {}
    for algo in (("implicit", "im2win", "im2col") if not args.only_algo else (args.algo,)):
        say("bench: %s: the %s path" % (name, algo))
        lay, w2 = build_layers(wl, dev, algo)

        def step2(rec=None, lay=lay, w2=w2):
            for l in lay:
                for st in STAGES:
                    run_stage(l, st, w2, stream)

        ms2, _, _ = time_steps(step2, stream, max(10, steps // 3), 2)
        s2 = summary(ms2)
        low = max(l["desc"].info["ws_lowered_bytes"] for l in lay)
        col = max(l["desc"].info["im2col_bytes"] for l in lay)
        algos[algo] = {"median_ms": s2["median_ms"], "best_ms": s2["best_ms"],
                       "tflops": step_flops / (s2["median_ms"] * 1e-3) / 1e12,
                       "workspace_bytes": max(l["desc"].workspace_bytes for l in lay),
                       "lowered_max_bytes": low, "im2col_max_bytes": col, "lowered_vs_im2col": low / col}
        del lay, w2
        torch.cuda.empty_cache()
    rec["algorithms"] = algos
    # im2win strips against explicit im2col, max over layers each (the im2win
    # path's own workspace; in-place 1x1 layers lower nothing)
    if "im2win" in algos:
        rec["im2win_vs_im2col"] = algos["im2win"]["lowered_vs_im2col"]
    return rec, wl


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(wl, budget_s=10.0):
    """The fp64 reference convolution, as it stands, on a bounded sample of
    the workload's images (every layer, chained as the workload chains them)
    on every host core the process may use; then one layer of one image on
    one thread (the single-thread baseline)."""
    import numpy as np
    import torch
    import oracle
    spec = wl.spec
    threads = oracle.default_threads()

    def run(n_img, layers, nthreads):
        flops = 0
        t0 = time.perf_counter()
        prev = None
        for L in layers:
            x = (L.x[:n_img] if L.x is not None else prev)
            y = oracle.conv2d(x, L.w, L.b, layout=spec.layout, stride=L.stride, padding=L.padding,
                              dilation=L.dilation, nthreads=nthreads)
            if spec.layout == "nchw":
                _, K, P, Q = y.shape
            else:
                _, P, Q, K = y.shape
            flops += 2 * n_img * K * P * Q * L.C * L.R * L.S
            prev = torch.from_numpy(np.ascontiguousarray(y)).to(wl.dtype) if spec.chained else None
        return flops, time.perf_counter() - t0

    f, t = run(1, wl.layers, threads)
    n = int(min(spec.N, max(1, budget_s / max(t, 1e-6))))
    if n > 1:
        f, t = run(n, wl.layers, threads)
    # single thread: the cheapest compute layer (a chained stack keeps its first layer)
    one = [wl.layers[0]] if spec.chained else [min(wl.layers, key=lambda L: L.C * L.R * L.S * L.K if L.R > 1 else 1e30)]
    f1, t1 = run(1, one, 1)
    return {"value": f / t / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": "%d of %d images of workload %s, all %d layers, fp64 seven-loop reference, %.1f s"
                      % (n, spec.N, spec.name, len(wl.layers), t),
            "single_thread": {"value": f1 / t1 / 1e12, "unit": "TFLOP/s", "cores": 1,
                              "sample": "1 image, layer %s, %.1f s" % (one[0].label, t1)}}


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
    stream = torch.cuda.current_stream(dev)

    def one_pass(rec=None):
        for i, l in enumerate(levels):
            h, c, h2, c2 = l["st"]
            for t in range(LSTM_STEPS):
                if rec is not None and i == dom and t == 0:
                    rec[0].record(stream)
                l["cell"].step(l["xs"][t], h, c, l["w"], l["b"], h_out=h2, c_out=c2, ws=l["ws"])
                if rec is not None and i == dom and t == 0:
                    rec[1].record(stream)
                h, c, h2, c2 = h2, c2, h, c

    ms, dms, host_s = time_steps(one_pass, stream, args.steps, args.warmup, rec_dom=True)
    s = summary(ms)
    dom_ms = sum(dms) / len(dms)
    achieved = levels[dom]["flops"] / (dom_ms * 1e-3) / 1e12
    out = {"metric": "ConvLSTM step gate-convolution TFLOP/s", "value": step_flops / (s["median_ms"] * 1e-3) / 1e12,
           "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
           "ms_per_step": s["median_ms"], "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
           "dtype": "f32", "data": "synthetic", "config": {"workload": "lstm: " + WORKLOAD_TEXT["lstm"],
                                                           "algo": args.algo},
           "warm": s, "host_s": host_s,
           "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_TFLOPS["f32"], "unit": "TFLOP/s",
                        "frac": achieved / PEAK_TFLOPS["f32"], "traffic": None,
                        "kernel": "conv_lstm_step (pack, lowering, conv_gemm_dma_kernel with the cell epilogue)",
                        "level": "%dx%dx%d" % (levels[dom]["ch"], levels[dom]["hw"], levels[dom]["hw"]),
                        "avg_launch_ms": dom_ms}}
    if not args.no_cpu_baseline:
        from oracle.convlstm import convlstm_step
        import oracle
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
        out["cpu_baseline"] = {"value": l["flops"] * n / LSTM_WINDOWS / dt / 1e12, "unit": "TFLOP/s",
                               "cores": oracle.default_threads(), "kind": "oracle", "cpu_model": cpu_model(),
                               "sample": "%d of %d windows, one step of the 32x30x30 level, fp64 reference, %.2f s"
                                         % (n, LSTM_WINDOWS, dt)}
    print(json.dumps(out), flush=True)
    return 0


def say(msg):
    print(msg, file=sys.stderr, flush=True)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50, help="timed steps of the headline workload (>= 30)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="c5", choices=sorted(WORKLOAD_TEXT), help="headline workload")
    ap.add_argument("--configs", default="c1,c2,c3,c4",
                    help="other workloads given a record in the same line (comma list; '' for none)")
    ap.add_argument("--algo", default="implicit", choices=["im2win", "im2col", "implicit"],
                    help="path timed for the headline (the other two are timed as well, unless --only-algo)")
    ap.add_argument("--only-algo", action="store_true", help="time only --algo")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured-peak microbenchmarks")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of reference work to time")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run the library's streaming copy over this many MiB, 5 times: a transfer of known "
                         "size against which a profiler's HBM byte counters are scaled")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print("bench.py: measures one GPU; --gpus %d is not supported (the convolution would shard over "
              "images, each GPU running the same path on its share with no exchange)" % args.gpus, file=sys.stderr)
        return 2
    args.steps = max(30, args.steps)

    import torch
    import cnn_convolution_lowering_amd as cl
    from cnn_convolution_lowering_amd import peak

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    cl.load_library()
    dev = torch.device("cuda:0")
    if args.copy_calibration_mib:
        import ctypes
        lib = peak.load_peak_library()
        n = args.copy_calibration_mib << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        sp = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
        for _ in range(5):
            if lib.convpeak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), n, sp) != 0:
                raise RuntimeError("convpeak_copy failed")
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read_per_launch": n, "copy_bytes_written_per_launch": n, "launches": 5,
                          "kernel": "peak_copy_kernel"}))
        return 0
    if args.workload == "lstm":
        if args.algo == "implicit":
            args.algo = "im2win"   # the ConvLSTM step reads x and h through the lowering
        return bench_lstm(args, dev)

    peaks = None
    if not args.no_peaks:
        say("bench: measured peaks (MFMA loop per instruction, sustained and burst; streaming copy)")
        peaks = peak.measure_peaks(dev)

    head, wl = bench_config(args.workload, dev, args, peaks, headline=True)
    spec = wl.spec
    ms = head["cold"]["median_ms"]
    out = {
        "metric": METRIC, "value": head["tflops"], "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": spec.dtype, "data": "synthetic",
        "config": {"workload": head["workload"], "algo": args.algo, "batch": spec.N, "layers": len(spec.layers),
                   "layout": spec.layout, "timing": "cold (512 MiB streamed between steps), median of %d steps"
                                                    % args.steps},
        "pct_of_mfma_peak": 100.0 * head["frac_of_peak"],
        "roofline": head["roofline"],
        "cold": head["cold"], "warm": head["warm"], "tflops_warm": head["tflops_warm"],
        "tflops_best": head["tflops_best"],
        "measured_peak": peaks,
        "workspace": {"im2win_vs_im2col": head.get("im2win_vs_im2col"),
                      "definition": "largest im2win lowered buffer over the layers / largest explicit im2col "
                                    "matrix over the layers",
                      "fused_path_lowered_bytes": head["algorithms"].get("implicit", {}).get("lowered_max_bytes")},
        "layers": head["layers"], "algorithms": head["algorithms"],
    }
    if peaks:
        out["pct_of_measured_mfma_peak"] = 100.0 * head["frac_of_measured_peak"]
    configs = {}
    for name in [c for c in args.configs.split(",") if c and c != args.workload]:
        rec, _ = bench_config(name, dev, args, peaks)
        configs[name] = rec
    out["configs"] = configs
    if not args.no_cpu_baseline:
        say("bench: timing the fp64 reference on the host")
        out["cpu_baseline"] = cpu_baseline(wl, args.cpu_budget)
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
