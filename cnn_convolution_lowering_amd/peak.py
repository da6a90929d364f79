"""Measured peaks of this GPU (ctypes over ``include/convpeak.h``,
``libconvpeak.so``): MFMA TFLOP/s per instruction from a register-only loop,
the shader clock sustained under that load, and the bandwidth of a plain
16-byte streaming copy.  Marshalling and timing only; the work runs in the
library's kernels.  The convolution path never imports this module.
"""
from __future__ import annotations

import ctypes
import os
import statistics
from typing import Dict

_PKG = os.path.dirname(os.path.abspath(__file__))
PEAK_LIB_PATH = os.path.join(_PKG, "libconvpeak.so")
PEAK_HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "convpeak.h")

# peak_mfma_kind_t
KINDS = {"f32_16x16x4": 0, "f16_32x32x16": 1, "bf16_32x32x16": 2, "f16_16x16x32": 3, "bf16_16x16x32": 4}

_lib = None


def load_peak_library() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(PEAK_LIB_PATH):
        raise ImportError("libconvpeak.so is not built (expected at %s); run __graft_entry__.build()" % PEAK_LIB_PATH)
    lib = ctypes.CDLL(PEAK_LIB_PATH)
    lib.convpeak_mfma_flops_per_iter.argtypes = [ctypes.c_int32]
    lib.convpeak_mfma_flops_per_iter.restype = ctypes.c_int64
    lib.convpeak_mfma.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p]
    lib.convpeak_mfma.restype = ctypes.c_int
    lib.convpeak_wall_clock_khz.argtypes = [ctypes.POINTER(ctypes.c_int64)]
    lib.convpeak_wall_clock_khz.restype = ctypes.c_int
    lib.convpeak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.convpeak_copy.restype = ctypes.c_int
    _lib = lib
    return lib


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError("%s failed (%d)" % (what, rc))


def mfma_peak(kind: str, dev, target_ms: float = 25.0, blocks: int = 1024, reps: int = 3) -> Dict[str, float]:
    """TFLOP/s of one MFMA instruction over the whole GPU (best of ``reps``
    launches of about ``target_ms`` each, after one warm-up launch), and the
    shader clock (MHz) measured inside the launches: shader-clock ticks over
    constant-rate wall-clock ticks, median over workgroups."""
    import torch
    lib = load_peak_library()
    k = KINDS[kind]
    fpi = lib.convpeak_mfma_flops_per_iter(k)
    clocks = torch.zeros(blocks * 8, dtype=torch.int64, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    khz = ctypes.c_int64()
    _check(lib.convpeak_wall_clock_khz(ctypes.byref(khz)), "convpeak_wall_clock_khz")
    # size the launch from a short probe
    iters = 2000
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    _check(lib.convpeak_mfma(k, iters, blocks, ctypes.c_void_p(clocks.data_ptr()), sp), "convpeak_mfma")
    e0.record(stream)
    _check(lib.convpeak_mfma(k, iters, blocks, ctypes.c_void_p(clocks.data_ptr()), sp), "convpeak_mfma")
    e1.record(stream)
    torch.cuda.synchronize(dev)
    ms = e0.elapsed_time(e1)
    iters = max(iters, int(iters * target_ms / max(ms, 1e-3)))
    best_ms, sclk = None, []
    for _ in range(reps):
        e0.record(stream)
        _check(lib.convpeak_mfma(k, iters, blocks, ctypes.c_void_p(clocks.data_ptr()), sp), "convpeak_mfma")
        e1.record(stream)
        torch.cuda.synchronize(dev)
        ms = e0.elapsed_time(e1)
        best_ms = ms if best_ms is None else min(best_ms, ms)
        c = clocks.view(blocks, 8).cpu()
        ratios = [(int(c[b, 1]) - int(c[b, 0])) / max(1, int(c[b, 3]) - int(c[b, 2])) for b in range(blocks)]
        sclk.append(statistics.median(ratios) * khz.value / 1e3)
    flops = float(blocks) * 4 * iters * fpi
    return {"tflops": flops / (best_ms * 1e-3) / 1e12, "sclk_mhz": statistics.median(sclk), "ms": best_ms,
            "iters": iters, "blocks": blocks}


def copy_bandwidth(dev, mib: int = 1024, reps: int = 5) -> Dict[str, float]:
    """GB/s (read + write bytes) of the 16-byte streaming copy over ``mib``
    MiB, best of ``reps`` after one warm-up."""
    import torch
    lib = load_peak_library()
    n = mib << 20
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty(n, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = ctypes.c_void_p(stream.cuda_stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    _check(lib.convpeak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), n, sp), "convpeak_copy")
    best = None
    for _ in range(reps):
        e0.record(stream)
        _check(lib.convpeak_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), n, sp),
               "convpeak_copy")
        e1.record(stream)
        torch.cuda.synchronize(dev)
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    ok = bool(torch.equal(src[:4096], dst[:4096])) and bool(torch.equal(src[-4096:], dst[-4096:]))
    del src, dst
    return {"gbs": 2.0 * n / (best * 1e-3) / 1e9, "bytes": 2 * n, "ms": best, "verified": ok}


def measure_peaks(dev) -> Dict[str, float]:
    """The measured peaks the benchmark reports next to the published ones.

    Sustained (launches of about 25 ms, the regime of back-to-back
    convolution steps; the clock drops under a long MFMA load): f32
    (16x16x4), f16 and bf16 (32x32x16, the strip kernels' instruction, and
    16x16x32, the pipelined kernel's), with the shader clock under the f16
    load.  Burst (launches of about 2 ms): the same 16-bit instructions.  HBM:
    GB/s (read + write) of the streaming copy."""
    sus = {}
    for name in ("f16_32x32x16", "bf16_32x32x16", "f16_16x16x32", "bf16_16x16x32", "f32_16x16x4"):
        sus[name] = mfma_peak(name, dev)
    burst = {}
    for name in ("f16_32x32x16", "f16_16x16x32", "bf16_32x32x16"):
        burst[name] = mfma_peak(name, dev, target_ms=2.0, reps=5)
    cp = copy_bandwidth(dev)
    return {"f16": max(sus["f16_32x32x16"]["tflops"], sus["f16_16x16x32"]["tflops"]),
            "bf16": max(sus["bf16_32x32x16"]["tflops"], sus["bf16_16x16x32"]["tflops"]),
            "f32": sus["f32_16x16x4"]["tflops"], "hbm_gbs": cp["gbs"],
            "sustained": {k: {"tflops": v["tflops"], "sclk_mhz": v["sclk_mhz"], "launch_ms": v["ms"]}
                          for k, v in sus.items()},
            "burst": {k: {"tflops": v["tflops"], "sclk_mhz": v["sclk_mhz"], "launch_ms": v["ms"]}
                      for k, v in burst.items()},
            "copy_verified": cp["verified"],
            "unit": "TFLOP/s (f16, bf16, f32: sustained, best instruction; hbm_gbs: GB/s read+write of a "
                    "streaming copy; sclk: MHz)"}
