"""GPU parity of the ConvLSTM step (conv_lstm_step) against the fp64 oracle
step (oracle/convlstm.py): gate convolution through the lowering and MFMA
contraction, cell update fused into the contraction's epilogue."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import cnn_convolution_lowering_amd as cl
from oracle.convlstm import convlstm_step

pytestmark = pytest.mark.gpu

# (N, Cx, Kh, H, W, R, S, padding, dilation): the four encoder levels of the
# fp32 MSCRED-style stack at a few images, then ragged channel counts, odd
# sizes, a 1x1 gate filter, asymmetric windows and dilation.
SHAPES = [
    (2, 32, 32, 30, 30, 3, 3, 1, 1),
    (3, 64, 64, 14, 14, 3, 3, 1, 1),
    (2, 128, 128, 7, 7, 3, 3, 1, 1),
    (4, 256, 256, 3, 3, 3, 3, 1, 1),
    (3, 5, 16, 9, 11, 3, 3, 1, 1),
    (2, 17, 48, 6, 7, 1, 1, 0, 1),
    (1, 3, 32, 8, 8, 5, 3, (2, 1), 1),
    (2, 8, 16, 10, 10, 3, 3, 2, 2),
]


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cl.load_library()
    return torch.device("cuda:0")


def _bounds(cprev, zabs, c_ref, h_ref, kh):
    """Per-element error bounds of (c_t, h_t).  Each gate pre-activation is
    an fp32-accumulated dot product: |dz| <= 1e-5 * (sum |operand products| +
    |b|) (the convolution tolerance).  sigmoid' <= 1/4, tanh' <= 1 and
    sigmoid, |tanh| <= 1 give |dc| <= (|c_prev|/4 + 1/4 + 1) * dz_max and
    |dh| <= dz_o / 4 + |dc|; fp32 evaluation of the nonlinearities adds a few
    ulp, covered by 2e-6 * (1 + |value|)."""
    z = [zabs[:, g * kh:(g + 1) * kh] for g in range(4)]
    zmax = np.maximum(np.maximum(z[0], z[1]), np.maximum(z[2], z[3]))
    bc = 1e-5 * (0.25 * np.abs(cprev) + 1.25) * zmax + 2e-6 * (1 + np.abs(c_ref))
    bh = 1e-5 * 0.25 * z[3] + bc + 2e-6 * (1 + np.abs(h_ref))
    return bc, bh


def _check(got_h, got_c, x, h, c, w, b, pad, dil, what):
    h_ref, c_ref, zabs = convlstm_step(x, h, c, w, b, padding=pad, dilation=dil, with_abs=True)
    kh = h.shape[1]
    bc, bh = _bounds(c.double().numpy(), zabs, c_ref, h_ref, kh)
    ec = np.abs(got_c.cpu().double().numpy() - c_ref)
    eh = np.abs(got_h.cpu().double().numpy() - h_ref)
    assert (ec <= bc).all(), "%s: c error %.3g over bound (max ratio %.3g)" % (what, ec.max(), (ec / bc).max())
    assert (eh <= bh).all(), "%s: h error %.3g over bound (max ratio %.3g)" % (what, eh.max(), (eh / bh).max())


def _inputs(shape, seed):
    N, Cx, Kh, H, W, R, S, pad, dil = shape
    g = torch.Generator().manual_seed(seed)
    x = torch.rand(N, Cx, H, W, generator=g) * 2 - 1
    h = torch.rand(N, Kh, H, W, generator=g) * 2 - 1
    c = torch.randn(N, Kh, H, W, generator=g)
    w = torch.randn(4 * Kh, Cx + Kh, R, S, generator=g) / np.sqrt((Cx + Kh) * R * S)
    b = torch.randn(4 * Kh, generator=g) * 0.1
    return x, h, c, w, b


@pytest.mark.parametrize("algo", ["im2win", "im2col"])
@pytest.mark.parametrize("si", range(len(SHAPES)))
def test_lstm_step_parity(dev, algo, si):
    shape = SHAPES[si]
    N, Cx, Kh, H, W, R, S, pad, dil = shape
    x, h, c, w, b = _inputs(shape, 40 + si)
    cell = cl.ConvLSTMCell(N, Cx, Kh, H, W, R, S, padding=pad, dilation=dil, algo=algo)
    print("lstm %s shape %s" % (algo, shape), flush=True)
    sys.stdout.flush()
    ho, co = cell.step(x.to(dev), h.to(dev), c.to(dev), w.to(dev), b.to(dev))
    torch.cuda.synchronize()
    _check(ho, co, x, h, c, w, b, pad, dil, "%s shape %d" % (algo, si))


def test_lstm_steps_chain_and_no_bias(dev):
    """Three steps in a row, h and c fed back on the GPU (each step checked
    against the oracle from the GPU's own previous state), no bias."""
    N, Cx, Kh, H, W, R, S, pad, dil = shape = (2, 16, 32, 12, 12, 3, 3, 1, 1)
    cell = cl.ConvLSTMCell(N, Cx, Kh, H, W, R, S, padding=pad, dilation=dil)
    x, h, c, w, _ = _inputs(shape, 7)
    hd, cd, wd = h.to(dev), c.to(dev), w.to(dev)
    ws = cell.new_workspace(dev)
    g = torch.Generator().manual_seed(8)
    for t in range(3):
        xt = torch.rand(N, Cx, H, W, generator=g) * 2 - 1
        print("lstm chain step %d" % t, flush=True)
        hn, cn = cell.step(xt.to(dev), hd, cd, wd, None, ws=ws)
        torch.cuda.synchronize()
        _check(hn, cn, xt, hd.cpu(), cd.cpu(), w, None, pad, dil, "step %d" % t)
        hd, cd = hn, cn


def test_lstm_full_size_level1(dev):
    """The first encoder level at the stack's full batch (1280 images, 32
    channels, 30x30): every output of a sample of images against the oracle."""
    N, Cx, Kh, H, W = 1280, 32, 32, 30, 30
    cell = cl.ConvLSTMCell(N, Cx, Kh, H, W, 3, 3, padding=1)
    x, h, c, w, b = _inputs((N, Cx, Kh, H, W, 3, 3, 1, 1), 99)
    ho, co = cell.step(x.to(dev), h.to(dev), c.to(dev), w.to(dev), b.to(dev))
    torch.cuda.synchronize()
    idx = [0, 1, 637, 1279]
    _check(ho.cpu()[idx], co.cpu()[idx], x[idx], h[idx], c[idx], w, b, 1, 1, "full size")
