"""Pins of the fp64 ConvLSTM step (oracle/convlstm.py) to things other than
itself: torch's LSTMCell (a library routine with the same gate order), the
reduction of a centre-tap 3x3 filter to the 1x1 case, and the closed form
of a zero filter."""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle.convlstm import convlstm_step


def _rand(shape, g, scale=1.0):
    return torch.randn(shape, generator=g, dtype=torch.float64) * scale


def _lstmcell(x, h, c, w, b):
    """Per-pixel torch.nn.LSTMCell (float64) for a 1x1 gate filter."""
    N, Cx, H, W = x.shape
    Kh = h.shape[1]
    cell = torch.nn.LSTMCell(Cx, Kh).double()
    with torch.no_grad():
        cell.weight_ih.copy_(w[:, :Cx, 0, 0])
        cell.weight_hh.copy_(w[:, Cx:, 0, 0])
        cell.bias_ih.copy_(b)
        cell.bias_hh.zero_()
    flat = lambda t: t.permute(0, 2, 3, 1).reshape(-1, t.shape[1])
    with torch.no_grad():
        hn, cn = cell(flat(x), (flat(h), flat(c)))
    back = lambda t: t.reshape(N, H, W, Kh).permute(0, 3, 1, 2).numpy()
    return back(hn), back(cn)


@pytest.mark.parametrize("N,Cx,Kh,H,W", [(2, 3, 4, 3, 5), (1, 8, 16, 2, 2), (3, 1, 2, 1, 1)])
def test_1x1_is_lstmcell(N, Cx, Kh, H, W):
    g = torch.Generator().manual_seed(11 + N + Cx)
    x, h, c = _rand((N, Cx, H, W), g), _rand((N, Kh, H, W), g), _rand((N, Kh, H, W), g)
    w, b = _rand((4 * Kh, Cx + Kh, 1, 1), g, 0.5), _rand((4 * Kh,), g, 0.3)
    ho, co = convlstm_step(x.numpy(), h.numpy(), c.numpy(), w.numpy(), b.numpy())
    hr, cr = _lstmcell(x, h, c, w, b)
    np.testing.assert_allclose(co, cr, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ho, hr, rtol=0, atol=1e-12)


def test_centre_tap_3x3_is_1x1():
    """A 3x3 filter with only its centre tap set, padding 1, is the 1x1 cell."""
    g = torch.Generator().manual_seed(5)
    N, Cx, Kh, H, W = 2, 5, 4, 6, 7
    x, h, c = _rand((N, Cx, H, W), g), _rand((N, Kh, H, W), g), _rand((N, Kh, H, W), g)
    w1, b = _rand((4 * Kh, Cx + Kh, 1, 1), g, 0.5), _rand((4 * Kh,), g, 0.3)
    w3 = torch.zeros(4 * Kh, Cx + Kh, 3, 3, dtype=torch.float64)
    w3[:, :, 1, 1] = w1[:, :, 0, 0]
    ho, co = convlstm_step(x.numpy(), h.numpy(), c.numpy(), w3.numpy(), b.numpy(), padding=1)
    hr, cr = _lstmcell(x, h, c, w1, b)
    np.testing.assert_allclose(co, cr, rtol=0, atol=1e-12)
    np.testing.assert_allclose(ho, hr, rtol=0, atol=1e-12)


def test_zero_filter_closed_form():
    """W = 0: every gate is its bias, so c_t and h_t follow elementwise."""
    g = torch.Generator().manual_seed(9)
    N, Cx, Kh, H, W = 1, 3, 2, 4, 4
    x, h, c = _rand((N, Cx, H, W), g), _rand((N, Kh, H, W), g), _rand((N, Kh, H, W), g)
    b = [0.3, -1.2, 0.7, 2.0, -0.4, 0.1, 1.5, -0.9]   # (i0 i1 f0 f1 g0 g1 o0 o1)
    w = np.zeros((4 * Kh, Cx + Kh, 3, 3))
    ho, co = convlstm_step(x.numpy(), h.numpy(), c.numpy(), w, np.array(b), padding=1)
    s = lambda v: 1.0 / (1.0 + math.exp(-v))
    for j in range(Kh):
        bi, bf, bg, bo = b[j], b[Kh + j], b[2 * Kh + j], b[3 * Kh + j]
        for idx in np.ndindex(N, H, W):
            n, p, q = idx
            cv = s(bf) * float(c[n, j, p, q]) + s(bi) * math.tanh(bg)
            assert abs(co[n, j, p, q] - cv) < 1e-14
            assert abs(ho[n, j, p, q] - s(bo) * math.tanh(cv)) < 1e-14


def test_rejects_a_size_changing_filter():
    x, h, c = np.zeros((1, 2, 5, 5)), np.zeros((1, 1, 5, 5)), np.zeros((1, 1, 5, 5))
    with pytest.raises(ValueError):
        convlstm_step(x, h, c, np.zeros((4, 3, 3, 3)), None, padding=0)
