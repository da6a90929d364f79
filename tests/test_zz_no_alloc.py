"""conv2d_fwd_noalloc (the entry point that allocates nothing, its workspace a
fixed device array inside the library) against conv2d_fwd with a
caller-allocated workspace: the same kernels, so the same bits.  Two calls in
a row per case, the second on a smaller input, through the C ABI."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import cnn_convolution_lowering_amd as cl
from parity import TORCH_DT

pytestmark = pytest.mark.gpu

SCRATCH = 64 << 20


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cl.load_library()
    return torch.device("cuda:0")


def _inputs(N, C, H, W, K, R, S, dt, lay, seed):
    g = torch.Generator().manual_seed(seed)
    x = (torch.rand(N, C, H, W, generator=g) * 2 - 1).to(TORCH_DT[dt])
    w = (torch.randn(K, C, R, S, generator=g) / np.sqrt(C * R * S)).to(TORCH_DT[dt])
    b = (torch.randn(K, generator=g) * 0.1).to(TORCH_DT[dt])
    if lay == "nhwc":
        x, w = x.permute(0, 2, 3, 1).contiguous(), w.permute(0, 2, 3, 1).contiguous()
    return x, w, b


def _bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32)


# (dtype, layout, algo, first shape, second smaller shape, padding, stride,
# plan): the split contraction's partials, the LDS-filter strip kernel's packed
# filter copy (named: by default it reads the KRSC rows), the fp32 strip
# kernel's filter copy, a lowered im2win buffer
CASES = [
    ("bf16", "nhwc", "implicit", (32, 512, 7, 7, 512, 3, 3), (8, 512, 7, 7, 512, 3, 3), 1, 1, None),
    ("f16", "nhwc", "implicit", (32, 128, 64, 64, 128, 11, 11), (4, 128, 32, 32, 128, 11, 11), 5, 1, "striprb4:2"),
    ("f32", "nchw", "implicit", (1280, 32, 30, 30, 64, 3, 3), (64, 32, 30, 30, 64, 3, 3), 0, 2, None),
    ("f16", "nhwc", "im2win", (8, 64, 20, 20, 96, 3, 3), (2, 64, 12, 12, 96, 3, 3), 1, 1, None),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "%s-%s-%s" % c[:3])
def test_noalloc_matches_conv2d_fwd(dev, case):
    dt, lay, algo, first, second, pad, st, plan = case
    for i, shape in enumerate((first, second)):
        N, C, H, W, K, R, S = shape
        d = cl.Conv2d(N, C, H, W, K, R, S, stride=st, padding=pad, layout=lay, dtype=dt, algo=algo, plan=plan)
        assert 0 < d.workspace_bytes <= SCRATCH or (i == 1 and d.workspace_bytes <= SCRATCH), d.info
        x, w, b = _inputs(N, C, H, W, K, R, S, dt, lay, 500 + i)
        xd, wd, bd = x.to(dev), w.to(dev), b.to(dev)
        print("noalloc %s %s %s shape %s kernel %d ws %d" % (dt, lay, algo, shape, d.info["kernel"],
                                                              d.workspace_bytes), flush=True)
        want = d.forward(xd, wd, bd)
        y = torch.full_like(want, float("nan"))
        got = d.forward_noalloc(xd, wd, bd, y=y)
        got2 = d.forward_noalloc(xd, wd, None)
        want2 = d.forward(xd, wd, None)
        torch.cuda.synchronize()
        assert got.data_ptr() == y.data_ptr()
        assert torch.equal(_bits(got.cpu()), _bits(want.cpu())), (shape, "with bias")
        assert torch.equal(_bits(got2.cpu()), _bits(want2.cpu())), (shape, "no bias")


def test_noalloc_rejects_a_workspace_beyond_the_scratch(dev):
    # explicit im2col of an 11x11 layer: 4 GB of lowered rows
    d = cl.Conv2d(32, 128, 64, 64, 128, 11, 11, padding=5, layout="nhwc", dtype="f16", algo="im2col")
    assert d.workspace_bytes > SCRATCH
    x = torch.zeros(32, 64, 64, 128, dtype=torch.float16, device=dev)
    w = torch.zeros(128, 11, 11, 128, dtype=torch.float16, device=dev)
    y = torch.zeros(32, 64, 64, 128, dtype=torch.float16, device=dev)
    with pytest.raises(cl.ConvError) as e:
        d.forward_noalloc(x, w, None, y=y)
    assert e.value.status == -2
    empty = cl.Conv2d(0, 16, 8, 8, 16, 3, 3, padding=1, layout="nhwc", dtype="f16", algo="implicit")
    assert empty.lib.conv2d_fwd_noalloc(empty.handle, None, None, None, None, None) == 0
