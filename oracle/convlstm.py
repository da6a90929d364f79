"""One ConvLSTM cell step in fp64 -- TEST INFRASTRUCTURE ONLY.

Same rules as the rest of this package: only the tests, the smoke check and
the benchmark's CPU baseline may import it; the HIP library never does.

"GPU-Accelerating MSCRED with CUDA, im2col, GEMM, and a Custom PyTorch
Extension", sections "MSCRED and ConvLSTM Architecture", "Role of ConvLSTM"
and "Why the Encoder Improved More Than ConvLSTM": after the convolutional
encoder, ConvLSTM layers model how the encoded feature maps change over time
while keeping their spatial layout, and once the encoder is fast they are the
bottleneck.  The pages name the cell (Shi et al., 2015, in their references)
but print no equations.  Reading used here, the plainest one they support:
the four gates come from one convolution over the channel concatenation of
the step's input and the previous hidden state,

    z   = conv(concat(x_t, h_{t-1}), W) + b      4*Kh channels, gate order (i, f, g, o)
    c_t = sigmoid(z_f) * c_{t-1} + sigmoid(z_i) * tanh(z_g)
    h_t = sigmoid(z_o) * tanh(c_t)

with no peephole terms, stride 1 and an output the size of the input (so
h_t can feed the next step), NCHW.  The convolution is this package's fp64
reference; the gate arithmetic is plain numpy in fp64.
"""
from __future__ import annotations

import numpy as np

from . import conv2d, decode


def _f64(a) -> np.ndarray:
    try:
        import torch
        if isinstance(a, torch.Tensor):
            return decode(a)
    except ImportError:
        pass
    return np.asarray(a, dtype=np.float64)


def convlstm_step(x, h, c, w, b, *, padding=0, dilation=1, with_abs=False):
    """(h_t, c_t) in fp64 for NCHW x (N, Cx, H, W), h and c (N, Kh, H, W),
    w (4*Kh, Cx+Kh, R, S), b (4*Kh,) or None.  With ``with_abs`` also the
    per-element sum of |operand products| (plus |b|) of each gate, shape
    (N, 4*Kh, H, W), for error bounds."""
    xf, hf, cf = _f64(x), _f64(h), _f64(c)
    kh = hf.shape[1]
    xh = np.concatenate([xf, hf], axis=1)
    out = conv2d(xh, _f64(w), None if b is None else _f64(b), layout="nchw", stride=1, padding=padding,
                 dilation=dilation, with_abs=with_abs)
    z, zabs = (out if with_abs else (out, None))
    if z.shape[2:] != hf.shape[2:]:
        raise ValueError("the gate convolution must keep the spatial size (got %s for %s)" % (z.shape, hf.shape))
    zi, zf, zg, zo = (z[:, g * kh:(g + 1) * kh] for g in range(4))
    sig = lambda v: 1.0 / (1.0 + np.exp(-v))
    c_t = sig(zf) * cf + sig(zi) * np.tanh(zg)
    h_t = sig(zo) * np.tanh(c_t)
    return (h_t, c_t, zabs) if with_abs else (h_t, c_t)
