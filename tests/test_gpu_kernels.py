"""GPU parity of every compiled contraction kernel and tile variant.

The planner picks one kernel per shape; conv_create_desc_forced with
"<kernel>:<variant>" (the binding's plan=) asks for another one that takes
the shape.  Each variant runs here on shapes
with ragged pixel and channel tiles, strides, dilation and padding, against
the fp64 reference, to the same per-element bound as the default path.
"""
from __future__ import annotations

import os
import sys

import numpy as np
import pytest
import torch

import cnn_convolution_lowering_amd as cl
import oracle
from parity import TORCH_DT, assert_parity, to_f64

pytestmark = pytest.mark.gpu

# kernel name -> (plan_info kernel id, number of compiled variants)
KERNELS = {"reg": (0, 3), "dma": (1, 14), "wide": (2, 9), "nchw": (3, 12), "strip": (4, 5), "striprb": (5, 9), "nchwstrip": (6, 10), "nchwtile": (7, 6), "tile16": (8, 11), "streamk": (9, 12), "striprb2": (10, 2), "nchwtaps": (11, 6), "striprb3": (12, 3), "striprb4": (13, 5), "stream1x1": (14, 4)}
# kernels compiled for some variants only
VARIANTS = {"streamk": (8,)}

# (N, C, H, W, K, R, S, stride, pad, dilation)
SHAPES_C32 = [
    (2, 64, 17, 17, 72, 3, 3, (1, 1), (1, 1), (1, 1)),
    (1, 32, 20, 13, 130, 2, 4, (2, 1), (1, 2), (1, 1)),
    (3, 96, 9, 9, 40, 3, 3, (1, 1), (2, 2), (2, 2)),
    (1, 32, 70, 70, 128, 5, 5, (1, 1), (2, 2), (1, 1)),
    (2, 128, 14, 14, 256, 3, 3, (1, 1), (1, 1), (1, 1)),
]
SHAPES_SMALL_C = [
    (2, 3, 30, 30, 32, 3, 3, (1, 1), (1, 1), (1, 1)),
    (3, 8, 15, 11, 70, 2, 3, (2, 1), (0, 1), (1, 2)),
    (2, 16, 9, 9, 130, 3, 3, (2, 2), (0, 0), (1, 1)),
]
# fp32 NCHW, no horizontal padding, C % 16 == 0: the encoder's strided layers and ragged variants
SHAPES_NCHW_F32 = [
    (3, 32, 30, 30, 64, 3, 3, (2, 2), (0, 0), (1, 1)),
    (2, 64, 14, 14, 128, 2, 2, (2, 2), (0, 0), (1, 1)),
    (2, 128, 7, 7, 256, 2, 2, (2, 2), (0, 0), (1, 1)),
    (2, 16, 13, 22, 40, 3, 4, (1, 1), (1, 0), (1, 1)),
    (1, 48, 20, 17, 70, 2, 3, (1, 2), (0, 0), (2, 1)),
    (2, 32, 9, 40, 33, 3, 2, (2, 1), (2, 0), (1, 3)),
]
# fp32 NCHW tap planes (filter widths 2 and 3, C % 16 == 0, any padding):
# the encoder's strided layers, padding on both axes, dilation on both
# axes, stride 3, ragged pixel and channel tiles, and strip counts (R times
# the 16-channel blocks) that leave a last strip outside the three-buffer
# variants' two-strip passes
SHAPES_NCHW_TAPS = [
    (3, 32, 30, 30, 64, 3, 3, (2, 2), (0, 0), (1, 1)),
    (2, 64, 14, 14, 128, 2, 2, (2, 2), (0, 0), (1, 1)),
    (2, 128, 7, 7, 256, 2, 2, (2, 2), (0, 0), (1, 1)),
    (2, 16, 13, 22, 40, 3, 3, (1, 1), (1, 1), (1, 1)),
    (1, 48, 20, 17, 70, 2, 3, (1, 2), (0, 1), (2, 1)),
    (2, 32, 9, 40, 33, 3, 2, (2, 1), (2, 1), (1, 3)),
    (1, 16, 5, 70, 20, 3, 3, (3, 3), (1, 1), (1, 1)),
]
# fp32 NCHW small windows (C*R*S <= 64, K <= 64): padding, strides, dilation, ragged pixel blocks
SHAPES_SMALL_KG = [
    (3, 3, 30, 30, 32, 3, 3, (1, 1), (1, 1), (1, 1)),
    (2, 3, 17, 23, 20, 3, 3, (2, 1), (1, 2), (1, 1)),
    (2, 2, 9, 11, 64, 3, 2, (1, 2), (2, 0), (2, 3)),
    (1, 1, 40, 33, 50, 1, 5, (3, 1), (0, 2), (1, 1)),
    (2, 7, 12, 12, 16, 3, 3, (1, 1), (1, 1), (1, 1)),
    (1, 4, 70, 9, 33, 2, 2, (1, 1), (1, 0), (1, 1)),
    (2, 1, 25, 27, 24, 3, 5, (1, 1), (1, 2), (1, 1)),
    (1, 5, 11, 13, 40, 3, 3, (1, 1), (0, 1), (1, 1)),
    (1, 3, 14, 16, 48, 3, 3, (2, 2), (1, 1), (1, 1)),
]
# 16-bit NHWC small windows (C*sw and W*C even, unit horizontal dilation):
# odd and even padding (one lead element or none), vertical dilation,
# output rows shorter and longer than a 16-pixel block, K not a multiple of
# 8 or of the lane's channel run, and a batch large enough for several
# output rows per workgroup with a ragged last block of rows
SHAPES_TILE16 = [
    (2, 3, 30, 30, 32, 3, 3, (2, 2), (1, 1), (1, 1)),
    (2, 3, 36, 34, 64, 7, 7, (2, 2), (3, 3), (1, 1)),
    (1, 4, 19, 21, 20, 5, 5, (1, 1), (2, 2), (1, 1)),
    (2, 2, 23, 17, 40, 3, 3, (1, 1), (1, 1), (2, 1)),
    (1, 6, 9, 50, 16, 3, 3, (2, 1), (0, 1), (1, 1)),
    (3, 3, 11, 10, 8, 2, 4, (1, 2), (0, 1), (1, 1)),
    (256, 2, 42, 12, 16, 3, 3, (2, 2), (1, 1), (1, 1)),
    (2, 1, 30, 28, 16, 5, 5, (2, 2), (2, 2), (1, 1)),
    (2, 4, 21, 19, 64, 3, 3, (1, 1), (1, 1), (1, 1)),
]
# (kernel, dtype, layout, algo, shapes)
# the unrolled-tap strip kernel: compiled filter widths, unit horizontal
# dilation; ragged channel tiles, vertical dilation, both strides, padding
SHAPES_RB2 = [
    (2, 64, 17, 19, 72, 3, 3, (1, 1), (1, 1), (1, 1)),
    (1, 32, 20, 33, 40, 5, 5, (1, 1), (2, 2), (2, 1)),
    (3, 96, 9, 70, 130, 7, 7, (2, 1), (3, 3), (1, 1)),
    (2, 64, 12, 64, 64, 11, 11, (1, 1), (5, 5), (1, 1)),
    (1, 32, 16, 64, 32, 9, 9, (1, 1), (4, 4), (1, 1)),
    (2, 32, 10, 60, 160, 3, 5, (1, 1), (1, 2), (1, 1)),
    (1, 32, 6, 64, 96, 7, 7, (1, 1), (3, 3), (1, 1)),
]

# more for the 16x16 forms: a last output-channel tile of one 16-channel
# block, narrow rows for its 256-pixel tiles, one-row filters (a single
# strip of 32 channels; two strips and a partial output-channel tile)
SHAPES_RB3 = [
    (2, 64, 17, 19, 64, 3, 3, (1, 1), (1, 1), (1, 1)),
    (1, 32, 20, 33, 48, 5, 5, (1, 1), (2, 2), (2, 1)),
    (3, 96, 9, 70, 144, 7, 7, (2, 1), (3, 3), (1, 1)),
    (2, 64, 12, 64, 64, 11, 11, (1, 1), (5, 5), (1, 1)),
    (1, 32, 16, 64, 32, 9, 9, (1, 1), (4, 4), (1, 1)),
    (2, 32, 10, 60, 160, 3, 5, (1, 1), (1, 2), (1, 1)),
    (2, 32, 9, 30, 80, 3, 3, (1, 1), (0, 1), (1, 1)),
    (1, 32, 9, 40, 64, 1, 3, (1, 1), (0, 1), (1, 1)),
    (2, 64, 8, 70, 48, 1, 7, (1, 1), (0, 3), (1, 1)),
]

# the streaming 1x1 kernel: pixel counts off the 16-row block, partial and
# odd output-channel counts, each channel count it compiles, and layers
# with several blocks per wave (the persistent loop's passes and its tail,
# the last with a pixel count off the block)
SHAPES_1X1 = [
    (3, 128, 9, 13, 128, 1, 1, (1, 1), (0, 0), (1, 1)),
    (2, 64, 7, 9, 48, 1, 1, (1, 1), (0, 0), (1, 1)),
    (1, 32, 5, 11, 20, 1, 1, (1, 1), (0, 0), (1, 1)),
    (2, 128, 6, 10, 100, 1, 1, (1, 1), (0, 0), (1, 1)),
    (1, 64, 3, 5, 30, 1, 1, (1, 1), (0, 0), (1, 1)),
    (50, 64, 64, 64, 64, 1, 1, (1, 1), (0, 0), (1, 1)),
    (1, 32, 3, 32771, 32, 1, 1, (1, 1), (0, 0), (1, 1)),
]

PLANS = [
    ("reg", "f32", "nhwc", "implicit", SHAPES_SMALL_C + SHAPES_C32[:2]),
    ("reg", "f16", "nchw", "implicit", SHAPES_SMALL_C[:2]),
    ("dma", "f16", "nhwc", "implicit", SHAPES_C32[:3] + SHAPES_SMALL_C[1:]),
    ("dma", "bf16", "nhwc", "im2win", SHAPES_C32[:2] + SHAPES_SMALL_C[:1]),
    ("dma", "f32", "nhwc", "implicit", SHAPES_C32[:2] + SHAPES_SMALL_C[1:2]),
    ("dma", "f32", "nchw", "im2col", SHAPES_SMALL_C[:2]),
    ("wide", "f16", "nhwc", "implicit", SHAPES_C32),
    ("wide", "bf16", "nhwc", "implicit", SHAPES_C32[:3]),
    ("nchw", "f32", "nchw", "implicit", SHAPES_SMALL_C + SHAPES_C32[:2]),
    ("strip", "f16", "nhwc", "implicit", SHAPES_C32),
    ("strip", "bf16", "nhwc", "implicit", SHAPES_C32[:3]),
    ("striprb", "f16", "nhwc", "implicit", SHAPES_C32),
    ("striprb", "bf16", "nhwc", "implicit", SHAPES_C32[:3]),
    ("nchwstrip", "f32", "nchw", "implicit", SHAPES_NCHW_F32),
    ("nchwtaps", "f32", "nchw", "implicit", SHAPES_NCHW_TAPS),
    ("nchwtile", "f32", "nchw", "implicit", SHAPES_SMALL_KG),
    ("tile16", "bf16", "nhwc", "implicit", SHAPES_TILE16),
    ("tile16", "f16", "nhwc", "implicit", SHAPES_TILE16),
    # stream-K: few tiles and short contractions, so that nearly every tile is
    # split between workgroups, some over three or more
    ("streamk", "f16", "nhwc", "implicit", SHAPES_C32 + SHAPES_SMALL_C[1:]),
    ("streamk", "bf16", "nhwc", "im2win", SHAPES_C32[:3] + SHAPES_SMALL_C[:1]),
    ("streamk", "f16", "nhwc", "im2col", SHAPES_C32[:2]),
    ("streamk", "f32", "nhwc", "implicit", SHAPES_C32[:2]),
    ("streamk", "bf16", "nchw", "im2win", SHAPES_SMALL_C[:2]),
    ("striprb2", "f16", "nhwc", "implicit", SHAPES_RB2),
    ("striprb2", "bf16", "nhwc", "implicit", SHAPES_RB2[::2]),
    ("striprb3", "f16", "nhwc", "implicit", SHAPES_RB2 + SHAPES_RB3),
    ("striprb3", "bf16", "nhwc", "implicit", SHAPES_RB3[::2]),
    ("striprb4", "f16", "nhwc", "implicit", SHAPES_RB2 + SHAPES_RB3),
    ("striprb4", "bf16", "nhwc", "implicit", SHAPES_RB3[1::2]),
    ("stream1x1", "f16", "nhwc", "implicit", SHAPES_1X1),
    ("stream1x1", "bf16", "nhwc", "im2col", SHAPES_1X1[:4]),
]


def _cases():
    out = []
    for kind, dt, lay, algo, shapes in PLANS:
        for v in VARIANTS.get(kind, range(KERNELS[kind][1])):
            out.append((kind, v, dt, lay, algo, shapes))
    return out


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cl.load_library()
    return torch.device("cuda:0")


def _perm(t, lay):
    return t.permute(0, 2, 3, 1).contiguous() if lay == "nhwc" else t.contiguous()


@pytest.mark.parametrize("case", _cases(), ids=lambda c: "%s%d-%s-%s-%s" % c[:5])
def test_forced_kernel_parity(dev, case):
    kind, v, dt, lay, algo, shapes = case
    kid = KERNELS[kind][0]
    ran = 0
    for si, (N, C, H, W, K, R, S, st, pd, dl) in enumerate(shapes):
        d = cl.Conv2d(N, C, H, W, K, R, S, stride=st, padding=pd, dilation=dl, layout=lay, dtype=dt, algo=algo,
                      plan="%s:%d" % (kind, v))
        if d.info["kernel"] != kid or d.info["kernel_variant"] != v:
            continue      # this variant does not take the shape
        g = torch.Generator().manual_seed(300 + 17 * v + si)
        x = (torch.rand(N, C, H, W, generator=g) * 2 - 1).to(TORCH_DT[dt])
        w = (torch.randn(K, C, R, S, generator=g) / np.sqrt(C * R * S)).to(TORCH_DT[dt])
        b = (torch.randn(K, generator=g) * 0.1).to(TORCH_DT[dt])
        xl, wl = _perm(x, lay), _perm(w, lay)
        print("case %s:%d %s %s %s shape %s" % (kind, v, dt, lay, algo, shapes[si]), flush=True)
        sys.stdout.flush()
        y = d.forward(xl.to(dev), wl.to(dev), b.to(dev))
        torch.cuda.synchronize()
        ref, yabs = oracle.conv2d(xl, wl, b, layout=lay, stride=st, padding=pd, dilation=dl, with_abs=True)
        assert_parity(to_f64(y.cpu()), ref, yabs, dt, "%s:%d shape %d" % (kind, v, si))
        ran += 1
    assert ran > 0, "no listed shape is taken by %s:%d" % (kind, v)


def test_forced_kernel_integer_exact(dev):
    """Integer inputs through the strip and wide kernels: exact fp32 sums, so
    the result is the reference rounded once to fp16, bit for bit."""
    N, C, H, W, K, R, S = 2, 64, 12, 12, 96, 3, 3
    g = torch.Generator().manual_seed(77)
    x = torch.randint(-2, 3, (N, C, H, W), generator=g).to(torch.float16)
    w = torch.randint(-2, 3, (K, C, R, S), generator=g).to(torch.float16)
    b = torch.randint(-4, 5, (K,), generator=g).to(torch.float16)
    xl, wl = _perm(x, "nhwc"), _perm(w, "nhwc")
    ref = oracle.conv2d(xl, wl, b, layout="nhwc", stride=1, padding=1)
    want = torch.from_numpy(ref).to(torch.float32).to(torch.float16)
    for forced in ("strip:0", "strip:2", "strip:3", "wide:0", "wide:5", "striprb:0", "striprb:3", "striprb:4",
                   "dma:8", "dma:9", "dma:10", "dma:11", "dma:12", "dma:13", "striprb2:0", "striprb2:1", "striprb3:0", "striprb3:1",
                   "striprb4:0"):
        d = cl.Conv2d(N, C, H, W, K, R, S, padding=1, layout="nhwc", dtype="f16", algo="implicit", plan=forced)
        assert d.info["kernel"] == KERNELS[forced.split(":")[0]][0], forced
        print("int case %s" % forced, flush=True)
        y = d.forward(xl.to(dev), wl.to(dev), b.to(dev))
        torch.cuda.synchronize()
        assert torch.equal(y.cpu().view(torch.int16), want.view(torch.int16)), forced


def test_tap_plane_kernel_integer_exact(dev):
    """Integer inputs through every variant of the fp32 tap-plane kernel (a
    strided, padded 3x3 layer and a 2x2 one): exact fp32 sums, so the result
    equals the reference bit for bit."""
    for (N, C, H, W, K, R, S, st, pd) in ((2, 32, 15, 16, 48, 3, 3, 2, 1), (3, 48, 11, 9, 70, 2, 2, 2, 0)):
        g = torch.Generator().manual_seed(79 + R)
        x = torch.randint(-2, 3, (N, C, H, W), generator=g).to(torch.float32)
        w = torch.randint(-2, 3, (K, C, R, S), generator=g).to(torch.float32)
        b = torch.randint(-4, 5, (K,), generator=g).to(torch.float32)
        want = torch.from_numpy(oracle.conv2d(x, w, b, layout="nchw", stride=st, padding=pd)).to(torch.float32)
        for v in range(KERNELS["nchwtaps"][1]):
            d = cl.Conv2d(N, C, H, W, K, R, S, stride=st, padding=pd, layout="nchw", dtype="f32", algo="implicit",
                          plan="nchwtaps:%d" % v)
            assert d.info["kernel"] == KERNELS["nchwtaps"][0] and d.info["kernel_variant"] == v, v
            print("int case nchwtaps:%d R=%d" % (v, R), flush=True)
            y = d.forward(x.to(dev), w.to(dev), b.to(dev))
            torch.cuda.synchronize()
            assert torch.equal(y.cpu(), want), (v, R)


def test_small_window_kernel_integer_exact(dev):
    """Integer inputs through the 16-bit NHWC small-window kernel (the stem
    shape at reduced size, every variant that takes it): exact fp32 sums, so
    the result is the reference rounded once, bit for bit."""
    N, C, H, W, K, R, S = 3, 3, 28, 26, 32, 7, 7
    g = torch.Generator().manual_seed(78)
    x = torch.randint(-2, 3, (N, C, H, W), generator=g).to(torch.bfloat16)
    w = torch.randint(-2, 3, (K, C, R, S), generator=g).to(torch.bfloat16)
    b = torch.randint(-4, 5, (K,), generator=g).to(torch.bfloat16)
    xl, wl = _perm(x, "nhwc"), _perm(w, "nhwc")
    ref = oracle.conv2d(xl, wl, b, layout="nhwc", stride=2, padding=3)
    want = torch.from_numpy(ref).to(torch.float32).to(torch.bfloat16)
    ref0 = oracle.conv2d(xl, wl, None, layout="nhwc", stride=2, padding=3)
    want0 = torch.from_numpy(ref0).to(torch.float32).to(torch.bfloat16)
    ran = 0
    for v in range(KERNELS["tile16"][1]):
        d = cl.Conv2d(N, C, H, W, K, R, S, stride=2, padding=3, layout="nhwc", dtype="bf16", algo="implicit",
                      plan="tile16:%d" % v)
        if d.info["kernel"] != KERNELS["tile16"][0] or d.info["kernel_variant"] != v:
            continue
        print("int case tile16:%d" % v, flush=True)
        y = d.forward(xl.to(dev), wl.to(dev), b.to(dev))
        y0 = d.forward(xl.to(dev), wl.to(dev), None)   # no bias: the accumulators start at zero
        torch.cuda.synchronize()
        assert torch.equal(y.cpu().view(torch.int16), want.view(torch.int16)), v
        assert torch.equal(y0.cpu().view(torch.int16), want0.view(torch.int16)), v
        ran += 1
    assert ran >= 2


# (dtype, layout, algo, shape, forced "dma:<variant>:<ksplit>"): ragged pixel
# and channel tiles, contraction ranges that do not split evenly, NHWC and
# NCHW outputs, fused and lowered operands
SPLIT_CASES = [
    ("f16", "nhwc", "implicit", (2, 64, 17, 17, 72, 3, 3, (1, 1), (1, 1), (1, 1)), "dma:1:2"),
    ("bf16", "nhwc", "implicit", (3, 96, 9, 9, 40, 3, 3, (1, 1), (2, 2), (2, 2)), "dma:0:3"),
    ("f16", "nhwc", "im2win", (2, 64, 17, 17, 130, 3, 3, (2, 1), (1, 1), (1, 1)), "dma:2:4"),
    ("f32", "nchw", "im2col", (2, 16, 13, 11, 33, 3, 3, (1, 1), (1, 1), (1, 1)), "dma:1:3"),
    ("f32", "nhwc", "implicit", (2, 32, 10, 10, 48, 3, 3, (1, 1), (1, 1), (1, 1)), "dma:1:2"),
    ("bf16", "nhwc", "implicit", (4, 256, 7, 7, 256, 3, 3, (1, 1), (1, 1), (1, 1)), "dma:2:5"),
    ("f16", "nhwc", "implicit", (2, 64, 17, 17, 72, 3, 3, (1, 1), (1, 1), (1, 1)), "wide:5:2"),
    ("bf16", "nhwc", "implicit", (3, 96, 9, 9, 300, 3, 3, (1, 1), (2, 2), (2, 2)), "wide:2:3"),
    ("bf16", "nhwc", "implicit", (8, 128, 7, 7, 256, 3, 3, (1, 1), (1, 1), (1, 1)), "wide:0:8"),
    ("f16", "nhwc", "implicit", (3, 96, 9, 9, 300, 3, 3, (1, 1), (2, 2), (2, 2)), "dma:8:3"),
    ("bf16", "nhwc", "implicit", (4, 256, 7, 7, 256, 3, 3, (1, 1), (1, 1), (1, 1)), "dma:9:2"),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=lambda c: "%s-%s-%s-%s" % (c[0], c[1], c[2], c[4]))
def test_split_contraction_parity(dev, case):
    """Contraction split over several workgroups per output tile: fp32
    partials in the workspace, summed in split order with the bias by the
    reduction kernel.  Parity against the oracle with and without a bias, and
    the same bits on a second run (the sum order is fixed)."""
    dt, lay, algo, (N, C, H, W, K, R, S, st, pd, dl), forced = case
    d = cl.Conv2d(N, C, H, W, K, R, S, stride=st, padding=pd, dilation=dl, layout=lay, dtype=dt, algo=algo,
                  plan=forced)
    ks = int(forced.split(":")[2])
    assert d.info["kernel"] == KERNELS[forced.split(":")[0]][0] and d.info["ksplit"] == ks, d.info
    assert d.info["ws_partial_bytes"] == ks * d.info["M"] * K * 4
    g = torch.Generator().manual_seed(91)
    x = (torch.rand(N, C, H, W, generator=g) * 2 - 1).to(TORCH_DT[dt])
    w = (torch.randn(K, C, R, S, generator=g) / np.sqrt(C * R * S)).to(TORCH_DT[dt])
    b = (torch.randn(K, generator=g) * 0.1).to(TORCH_DT[dt])
    xl, wl = _perm(x, lay), _perm(w, lay)
    xd, wd = xl.to(dev), wl.to(dev)
    for bias in (b, None):
        print("split case %s %s %s %s %s bias=%s" % (dt, lay, algo, case[3], forced, bias is not None), flush=True)
        y1 = d.forward(xd, wd, None if bias is None else bias.to(dev))
        y2 = d.forward(xd, wd, None if bias is None else bias.to(dev))
        torch.cuda.synchronize()
        assert torch.equal(y1.cpu().view(-1).view(torch.uint8), y2.cpu().view(-1).view(torch.uint8))
        ref, yabs = oracle.conv2d(xl, wl, bias, layout=lay, stride=st, padding=pd, dilation=dl, with_abs=True)
        assert_parity(to_f64(y1.cpu()), ref, yabs, dt, "split %s" % forced)


ORDER_CASES = [
    # (dtype, layout, algo, shape, plan without the order): tile counts not a
    # multiple of the 8 XCDs, fewer workgroups than XCDs, a split contraction
    ("f16", "nhwc", "implicit", (2, 64, 17, 17, 72, 3, 3, (1, 1), (1, 1), (1, 1)), "dma:8:1"),
    ("bf16", "nhwc", "implicit", (3, 96, 9, 9, 300, 3, 3, (1, 1), (2, 2), (2, 2)), "dma:8:3"),
    ("f16", "nhwc", "im2win", (2, 64, 17, 17, 130, 3, 3, (2, 1), (1, 1), (1, 1)), "dma:2:2"),
    ("bf16", "nhwc", "implicit", (1, 64, 5, 5, 40, 3, 3, (1, 1), (1, 1), (1, 1)), "dma:8:1"),
    ("f32", "nchw", "im2col", (2, 16, 13, 11, 33, 3, 3, (1, 1), (1, 1), (1, 1)), "dma:1:2"),
    ("f16", "nhwc", "implicit", (5, 128, 14, 14, 256, 1, 1, (1, 1), (0, 0), (1, 1)), "dma:11:1"),
]


@pytest.mark.parametrize("case", ORDER_CASES, ids=lambda c: "%s-%s-%s-%s" % (c[0], c[1], c[2], c[4]))
def test_tile_order_parity(dev, case):
    """Every tile order of the pipelined kernel maps the workgroups one to one
    onto the (split, tile) pairs: each order gives the same bits as the plain
    order, which is in parity with the oracle."""
    dt, lay, algo, (N, C, H, W, K, R, S, st, pd, dl), forced = case
    g = torch.Generator().manual_seed(17)
    x = (torch.rand(N, C, H, W, generator=g) * 2 - 1).to(TORCH_DT[dt])
    w = (torch.randn(K, C, R, S, generator=g) / np.sqrt(C * R * S)).to(TORCH_DT[dt])
    b = (torch.randn(K, generator=g) * 0.1).to(TORCH_DT[dt])
    xl, wl = _perm(x, lay), _perm(w, lay)
    xd, wd, bd = xl.to(dev), wl.to(dev), b.to(dev)
    ref, yabs = oracle.conv2d(xl, wl, b, layout=lay, stride=st, padding=pd, dilation=dl, with_abs=True)
    base = None
    for order in range(4):
        plan = "%s:%d" % (forced, order)
        d = cl.Conv2d(N, C, H, W, K, R, S, stride=st, padding=pd, dilation=dl, layout=lay, dtype=dt, algo=algo,
                      plan=plan)
        assert d.info["kernel"] == 1 and d.info["tile_order"] == order, d.info
        assert d.info["ksplit"] == int(forced.split(":")[2]), d.info
        print("tile order case %s %s %s %s %s" % (dt, lay, algo, case[3], plan), flush=True)
        y = d.forward(xd, wd, bd)
        torch.cuda.synchronize()
        yb = y.cpu().view(-1).view(torch.uint8)
        if base is None:
            base = yb
            assert_parity(to_f64(y.cpu()), ref, yabs, dt, "tile order %s" % plan)
        else:
            assert torch.equal(yb, base), plan


@pytest.mark.parametrize("case", [
    ("f32", "nchw", (64, 32, 30, 30, 64, 3, 3, (2, 2), (0, 0), (1, 1))),
    ("f32", "nchw", (16, 3, 30, 30, 32, 3, 3, (1, 1), (1, 1), (1, 1))),
    ("f16", "nhwc", (4, 128, 32, 32, 128, 3, 3, (1, 1), (1, 1), (1, 1))),
    ("bf16", "nhwc", (8, 64, 14, 14, 96, 3, 3, (1, 1), (1, 1), (1, 1))),
    ("bf16", "nhwc", (8, 3, 64, 64, 64, 7, 7, (2, 2), (3, 3), (1, 1))),
    ("bf16", "nhwc", (8, 192, 20, 20, 96, 3, 3, (1, 1), (1, 1), (1, 1))),
], ids=lambda c: "%s-%s" % c[:2])
def test_tune_keeps_a_correct_plan(dev, case):
    """conv_tune times the candidates and returns the fastest as a new
    descriptor, leaving the one it tuned as it was; the kept plan still
    matches the oracle, and is never slower than the default it timed."""
    dt, lay, (N, C, H, W, K, R, S, st, pd, dl) = case
    d = cl.Conv2d(N, C, H, W, K, R, S, stride=st, padding=pd, dilation=dl, layout=lay, dtype=dt, algo="implicit")
    g = torch.Generator().manual_seed(61)
    x = (torch.rand(N, C, H, W, generator=g) * 2 - 1).to(TORCH_DT[dt])
    w = (torch.randn(K, C, R, S, generator=g) / np.sqrt(C * R * S)).to(TORCH_DT[dt])
    b = (torch.randn(K, generator=g) * 0.1).to(TORCH_DT[dt])
    xl, wl = _perm(x, lay), _perm(w, lay)
    xd, wd, bd = xl.to(dev), wl.to(dev), b.to(dev)
    ws = torch.empty(max(d.workspace_bytes, 8 << 20), dtype=torch.uint8, device=dev)
    print("tune %s %s %s" % (dt, lay, case[2]), flush=True)
    before = (d.info["kernel"], d.info["kernel_variant"], d.info["ksplit"])
    r, t = d.tune(xd, wd, bd, ws=ws, reps=3)
    assert r["candidates"] >= 2 and r["best_ms"] <= r["default_ms"]
    assert (r["kernel"], r["kernel_variant"], r["ksplit"]) == (t.info["kernel"], t.info["kernel_variant"],
                                                             t.info["ksplit"])
    assert (d.info["kernel"], d.info["kernel_variant"], d.info["ksplit"]) == before
    assert t.workspace_bytes <= ws.numel()
    y = t.forward(xd, wd, bd, ws=ws)
    torch.cuda.synchronize()
    ref, yabs = oracle.conv2d(xl, wl, b, layout=lay, stride=st, padding=pd, dilation=dl, with_abs=True)
    assert_parity(to_f64(y.cpu()), ref, yabs, dt, "tuned %s" % (r,))
