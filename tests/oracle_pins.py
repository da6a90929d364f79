"""Pins for the fp64 reference convolution.

Each ``pin_*`` function checks one build of conv_oracle.c (an ``OracleLib``)
against something other than itself: hand-worked values, closed forms
(delta kernels, 1x1 = matrix product, all-ones kernel = box sums from an
integral image), invariants (stride = subsampling, dilation = zero-inserted
kernel, layout permutation, linearity, transposition), brute-force numpy
sliding windows, the independent float64 convolution in torch, and exact
storage decoding.  The tests run every pin on the real oracle, and run them
again on copies of the oracle with a planted mistake to show that each
mistake is caught by at least one pin.

The definition pinned is the cross-correlation with zero padding described
in "GPU-Accelerating MSCRED with CUDA, im2col, GEMM, and a Custom PyTorch
Extension", section "Transforming Conv2D into im2col and GEMM".
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_worked.json")


def _nhwc(x):
    return np.ascontiguousarray(np.transpose(x, (0, 2, 3, 1)))


def _nchw(y):
    return np.ascontiguousarray(np.transpose(y, (0, 3, 1, 2)))


def _store(a: np.ndarray, dtype: str):
    """Round float64 values to a storage dtype (torch CPU, round-to-nearest-even)."""
    t = torch.from_numpy(np.ascontiguousarray(a)).to(torch.float32)
    return {"f32": t, "f16": t.to(torch.float16), "bf16": t.to(torch.bfloat16),
            "f64": torch.from_numpy(np.ascontiguousarray(a))}[dtype]


def _exact64(t: torch.Tensor) -> np.ndarray:
    """fp64 value of a storage tensor via torch's own conversion (independent of the oracle)."""
    return t.to(torch.float64).numpy()


def _close(a, b, scale, tol=1e-12):
    a = np.asarray(a)
    b = np.asarray(b)
    assert a.shape == b.shape, (a.shape, b.shape)
    err = np.max(np.abs(a - b) / (np.asarray(scale) + 1e-300)) if a.size else 0.0
    assert err <= tol, "max scaled error %g > %g" % (err, tol)


def _extent(size, pad, dil, ks, stride):
    """Number of window positions by enumeration (independent of any closed formula)."""
    return len(range(0, size + 2 * pad - dil * (ks - 1), stride))


def brute_force(x, w, b, stride, pad, dil):
    """NCHW float64 convolution by explicit windows of a zero-padded copy."""
    N, C, H, W = x.shape
    K, _, R, S = w.shape
    sh, sw = stride
    ph, pw = pad
    dh, dw = dil
    xp = np.zeros((N, C, H + 2 * ph, W + 2 * pw))
    xp[:, :, ph:ph + H, pw:pw + W] = x
    P = _extent(H, ph, dh, R, sh)
    Q = _extent(W, pw, dw, S, sw)
    y = np.zeros((N, K, P, Q))
    for n in range(N):
        for p in range(P):
            for q in range(Q):
                win = xp[n, :, p * sh:p * sh + dh * (R - 1) + 1:dh, q * sw:q * sw + dw * (S - 1) + 1:dw]
                for k in range(K):
                    y[n, k, p, q] = np.sum(win * w[k]) + (0.0 if b is None else b[k])
    return y


# ---------------------------------------------------------------- the pins

def pin_hand_worked(orc):
    with open(GOLDEN) as f:
        cases = json.load(f)["cases"]
    for case in cases:
        x = np.array(case["x"], dtype=np.float64)
        w = np.array(case["w"], dtype=np.float64)
        b = None if case["b"] is None else np.array(case["b"], dtype=np.float64)
        want = np.array(case["y"], dtype=np.float64)
        kw = dict(stride=case["stride"], padding=case["padding"], dilation=case["dilation"])
        got = orc.conv2d(x, w, b, layout="nchw", **kw)
        np.testing.assert_array_equal(got, want, err_msg=case["name"])
        got = orc.conv2d(_nhwc(x), _nhwc(w), b, layout="nhwc", **kw)
        np.testing.assert_array_equal(_nchw(got), want, err_msg=case["name"] + " nhwc")


def pin_decode(orc):
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.decode(h.view(np.float16))
    want = h.view(np.float16).astype(np.float64)
    nan = np.isnan(want)
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], want[~nan])
    bf = torch.arange(-32768, 32768, dtype=torch.int32).to(torch.int16).view(torch.bfloat16)
    got = orc.decode(bf)
    want = bf.to(torch.float64).numpy()
    nan = np.isnan(want)
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], want[~nan])
    rng = np.random.default_rng(11)
    u = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    u[:8] = [0, 0x80000000, 1, 0x7f7fffff, 0x00800000, 0x007fffff, 0x7f800000, 0xff800000]
    f = u.view(np.float32)
    got = orc.decode(f)
    with np.errstate(invalid="ignore"):
        want = f.astype(np.float64)
    nan = np.isnan(want)
    np.testing.assert_array_equal(np.isnan(got), nan)
    np.testing.assert_array_equal(got[~nan], want[~nan])


def pin_output_dims(orc):
    rng = np.random.default_rng(1)
    for _ in range(300):
        H, W = rng.integers(1, 12, size=2)
        R, S = rng.integers(1, 6, size=2)
        sh, sw, dh, dw = rng.integers(1, 4, size=4)
        ph, pw = rng.integers(0, 4, size=2)
        args = dict(stride=(int(sh), int(sw)), padding=(int(ph), int(pw)), dilation=(int(dh), int(dw)))
        fits = H + 2 * ph >= dh * (R - 1) + 1 and W + 2 * pw >= dw * (S - 1) + 1
        if fits:
            out = torch.nn.functional.conv2d(torch.zeros(1, 1, int(H), int(W)), torch.zeros(1, 1, int(R), int(S)), **args)
            assert orc.output_dims((1, 1, H, W), (1, 1, R, S), **args) == tuple(out.shape[2:])
        else:
            try:
                orc.output_dims((1, 1, H, W), (1, 1, R, S), **args)
            except ValueError:
                pass
            else:
                raise AssertionError("kernel larger than the padded input was accepted")


def pin_delta(orc):
    rng = np.random.default_rng(2)
    for dtype in ("f32", "f16", "bf16"):
        for R in (1, 3, 5):
            x = _store(rng.uniform(-4, 4, size=(2, 3, 7, 6)), dtype)
            w = np.zeros((3, 3, R, R))
            for k in range(3):
                w[k, k, R // 2, R // 2] = 1.0
            w = _store(w, dtype)
            y = orc.conv2d(x, w, None, layout="nchw", padding=R // 2)
            np.testing.assert_array_equal(y, _exact64(x))
            y = orc.conv2d(x.permute(0, 2, 3, 1).contiguous(), w.permute(0, 2, 3, 1).contiguous(), None,
                           layout="nhwc", padding=R // 2)
            np.testing.assert_array_equal(_nchw(y), _exact64(x))
    # off-centre taps and unequal pads: a shifted copy with zero fill
    for (r0, s0, ph, pw) in [(0, 2, 1, 2), (2, 0, 2, 1), (1, 1, 0, 2), (2, 2, 2, 2)]:
        x = rng.uniform(-1, 1, size=(1, 2, 5, 7))
        w = np.zeros((2, 2, 3, 3))
        w[0, 0, r0, s0] = 1.0
        w[1, 1, r0, s0] = 1.0
        y = orc.conv2d(x, w, None, layout="nchw", padding=(ph, pw))
        xp = np.zeros((1, 2, 5 + 2 * ph + 4, 7 + 2 * pw + 4))
        xp[:, :, ph:ph + 5, pw:pw + 7] = x
        P, Q = y.shape[2:]
        np.testing.assert_array_equal(y, xp[:, :, r0:r0 + P, s0:s0 + Q])


def pin_matmul_1x1(orc):
    rng = np.random.default_rng(3)
    for layout in ("nchw", "nhwc"):
        x = rng.standard_normal((3, 5, 4, 6))
        wm = rng.standard_normal((7, 5))
        b = rng.standard_normal(7)
        want = (wm @ x.reshape(3, 5, 24)).reshape(3, 7, 4, 6) + b[None, :, None, None]
        scale = (np.abs(wm) @ np.abs(x.reshape(3, 5, 24))).reshape(3, 7, 4, 6) + np.abs(b)[None, :, None, None]
        if layout == "nchw":
            got = orc.conv2d(x, wm.reshape(7, 5, 1, 1), b, layout="nchw")
        else:
            got = _nchw(orc.conv2d(_nhwc(x), wm.reshape(7, 1, 1, 5), b, layout="nhwc"))
        _close(got, want, scale)


def pin_box_sums(orc):
    rng = np.random.default_rng(4)
    for (R, S, s, p) in [(3, 3, 1, 1), (2, 3, 2, 0), (3, 2, 1, 2), (1, 1, 2, 1), (4, 4, 3, 2)]:
        x = rng.integers(-3, 4, size=(2, 3, 9, 8)).astype(np.float64)
        w = np.ones((2, 3, R, S))
        w[1] *= 2.0
        y = orc.conv2d(x, w, None, layout="nchw", stride=s, padding=p)
        # integral image of the channel-summed, zero-padded input
        xs = np.zeros((2, 9 + 2 * p, 8 + 2 * p))
        xs[:, p:p + 9, p:p + 8] = x.sum(axis=1)
        I = np.zeros((2, xs.shape[1] + 1, xs.shape[2] + 1))
        I[:, 1:, 1:] = xs.cumsum(axis=1).cumsum(axis=2)
        P, Q = y.shape[2:]
        for pp in range(P):
            for qq in range(Q):
                h0, w0 = pp * s, qq * s
                box = I[:, h0 + R, w0 + S] - I[:, h0, w0 + S] - I[:, h0 + R, w0] + I[:, h0, w0]
                np.testing.assert_array_equal(y[:, 0, pp, qq], box)
                np.testing.assert_array_equal(y[:, 1, pp, qq], 2 * box)


def pin_brute_force(orc):
    rng = np.random.default_rng(5)
    combos = [(s, p, d) for s in (1, 2, 3) for p in (0, 1, 2, 3) for d in (1, 2, 3)]
    for i, (s, p, d) in enumerate(combos):
        R, S = int(rng.integers(1, 4)), int(rng.integers(1, 4))
        H, W = int(rng.integers(d * (R - 1) + 1, 9)), int(rng.integers(d * (S - 1) + 1, 9))
        N, C, K = int(rng.integers(1, 3)), int(rng.integers(1, 4)), int(rng.integers(1, 4))
        st = (s, int(rng.integers(1, 4)))
        pd = (p, int(rng.integers(0, 3)))
        dl = (d, int(rng.integers(1, 3)))
        if W + 2 * pd[1] < dl[1] * (S - 1) + 1:
            continue
        x = rng.standard_normal((N, C, H, W))
        w = rng.standard_normal((K, C, R, S))
        b = rng.standard_normal(K)
        want = brute_force(x, w, b, st, pd, dl)
        scale = brute_force(np.abs(x), np.abs(w), np.abs(b), st, pd, dl)
        layout = "nchw" if i % 2 == 0 else "nhwc"
        if layout == "nchw":
            got = orc.conv2d(x, w, b, layout="nchw", stride=st, padding=pd, dilation=dl)
        else:
            got = _nchw(orc.conv2d(_nhwc(x), _nhwc(w), b, layout="nhwc", stride=st, padding=pd, dilation=dl))
        _close(got, want, scale)


def pin_stride_subsample(orc):
    rng = np.random.default_rng(6)
    x = rng.standard_normal((2, 3, 11, 10))
    w = rng.standard_normal((4, 3, 3, 2))
    for s in (2, 3):
        for p in (0, 1, 2):
            y1 = orc.conv2d(x, w, None, layout="nchw", stride=1, padding=p, dilation=(1, 2))
            ys = orc.conv2d(x, w, None, layout="nchw", stride=s, padding=p, dilation=(1, 2))
            np.testing.assert_array_equal(ys, y1[:, :, ::s, ::s])


def pin_dilation_zero_insert(orc):
    rng = np.random.default_rng(7)
    x = rng.standard_normal((2, 3, 12, 11))
    w = rng.standard_normal((2, 3, 3, 2))
    for dh, dw in [(2, 1), (1, 3), (2, 2), (3, 2)]:
        wz = np.zeros((2, 3, dh * 2 + 1, dw * 1 + 1))
        wz[:, :, ::dh, ::dw] = w
        got = orc.conv2d(x, w, None, layout="nchw", padding=1, dilation=(dh, dw))
        want = orc.conv2d(x, wz, None, layout="nchw", padding=1)
        np.testing.assert_array_equal(got, want)


def pin_layout_permutation(orc):
    rng = np.random.default_rng(8)
    for dtype in ("f32", "f16", "bf16"):
        x = _store(rng.uniform(-1, 1, size=(2, 5, 6, 7)), dtype)
        w = _store(rng.standard_normal((3, 5, 3, 2)), dtype)
        b = _store(rng.standard_normal(3), dtype)
        y0 = orc.conv2d(x, w, b, layout="nchw", stride=(2, 1), padding=(1, 0))
        y1 = orc.conv2d(x.permute(0, 2, 3, 1).contiguous(), w.permute(0, 2, 3, 1).contiguous(), b,
                        layout="nhwc", stride=(2, 1), padding=(1, 0))
        np.testing.assert_array_equal(_nchw(y1), y0)


def pin_linearity(orc):
    rng = np.random.default_rng(9)
    x1, x2 = rng.standard_normal((2, 2, 3, 7, 7))
    w1, w2 = rng.standard_normal((2, 4, 3, 3, 3))
    b = rng.standard_normal(4)
    kw = dict(layout="nchw", stride=2, padding=1)
    a, c = 0.75, -1.5
    scale = (orc.conv2d(np.abs(x1), np.abs(w1), None, **kw) + orc.conv2d(np.abs(x2), np.abs(w1), None, **kw)
             + orc.conv2d(np.abs(x1), np.abs(w2), None, **kw))
    _close(orc.conv2d(a * x1 + c * x2, w1, None, **kw),
           a * orc.conv2d(x1, w1, None, **kw) + c * orc.conv2d(x2, w1, None, **kw), 2 * scale)
    _close(orc.conv2d(x1, w1 + w2, None, **kw),
           orc.conv2d(x1, w1, None, **kw) + orc.conv2d(x1, w2, None, **kw), scale)
    _close(orc.conv2d(x1, w1, b, **kw) - orc.conv2d(x1, w1, None, **kw),
           np.broadcast_to(b[None, :, None, None], (2, 4, 4, 4)), scale + np.abs(b)[None, :, None, None])


def pin_transpose(orc):
    rng = np.random.default_rng(10)
    x = rng.standard_normal((2, 3, 9, 9))
    w = rng.standard_normal((2, 3, 3, 3))
    kw = dict(layout="nchw", stride=2, padding=1, dilation=2)
    y = orc.conv2d(x, w, None, **kw)
    yt = orc.conv2d(np.ascontiguousarray(x.transpose(0, 1, 3, 2)), np.ascontiguousarray(w.transpose(0, 1, 3, 2)),
                    None, **kw)
    scale = orc.conv2d(np.abs(x), np.abs(w), None, **kw)
    _close(yt, y.transpose(0, 1, 3, 2), scale.transpose(0, 1, 3, 2))
    # symmetric signature-matrix-like input with a symmetric kernel: y is symmetric itself
    a = rng.uniform(-1, 1, size=(1, 2, 8, 5))
    xs = a @ a.transpose(0, 1, 3, 2)
    ws = w[:, :2] + w[:, :2].transpose(0, 1, 3, 2)
    ys = orc.conv2d(xs, ws, None, layout="nchw", padding=1)
    _close(ys, ys.transpose(0, 1, 3, 2), orc.conv2d(np.abs(xs), np.abs(ws), None, layout="nchw", padding=1))


def pin_torch_float64(orc):
    rng = np.random.default_rng(12)
    for _ in range(12):
        N, C, K = (int(v) for v in rng.integers(1, 4, size=3))
        R, S = (int(v) for v in rng.integers(1, 5, size=2))
        st = tuple(int(v) for v in rng.integers(1, 3, size=2))
        pd = tuple(int(v) for v in rng.integers(0, 3, size=2))
        dl = tuple(int(v) for v in rng.integers(1, 3, size=2))
        H = int(rng.integers(dl[0] * (R - 1) + 1, 12))
        W = int(rng.integers(dl[1] * (S - 1) + 1, 12))
        x = rng.standard_normal((N, C, H, W))
        w = rng.standard_normal((K, C, R, S))
        b = rng.standard_normal(K)
        want = torch.nn.functional.conv2d(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b),
                                          stride=st, padding=pd, dilation=dl).numpy()
        scale = torch.nn.functional.conv2d(torch.from_numpy(np.abs(x)), torch.from_numpy(np.abs(w)),
                                           torch.from_numpy(np.abs(b)), stride=st, padding=pd, dilation=dl).numpy()
        got = orc.conv2d(x, w, b, layout="nchw", stride=st, padding=pd, dilation=dl)
        _close(got, want, scale)


def pin_points_match_full(orc):
    rng = np.random.default_rng(13)
    for layout in ("nchw", "nhwc"):
        x = _store(rng.uniform(-1, 1, size=(3, 4, 8, 9)), "bf16")
        w = _store(rng.standard_normal((5, 4, 3, 3)), "bf16")
        b = _store(rng.standard_normal(5), "bf16")
        if layout == "nhwc":
            x, w = x.permute(0, 2, 3, 1).contiguous(), w.permute(0, 2, 3, 1).contiguous()
        kw = dict(layout=layout, stride=(1, 2), padding=1)
        y, yabs = orc.conv2d(x, w, b, with_abs=True, **kw)
        yn = y if layout == "nchw" else _nchw(y)
        an = yabs if layout == "nchw" else _nchw(yabs)
        pts = np.stack([rng.integers(0, s, size=50) for s in yn.shape], axis=1)
        py, pa = orc.conv2d_points(x, w, b, pts, **kw)
        np.testing.assert_array_equal(py, yn[tuple(pts.T)])
        np.testing.assert_array_equal(pa, an[tuple(pts.T)])


def pin_abs_scale(orc):
    rng = np.random.default_rng(14)
    x = rng.uniform(0, 1, size=(2, 3, 6, 6))
    w = rng.uniform(0, 1, size=(2, 3, 3, 3))
    b = rng.uniform(0, 1, size=2)
    y, ya = orc.conv2d(x, w, b, layout="nchw", padding=1, with_abs=True)
    _close(ya, y, y)
    # |b| + sum |x w| does not see signs, and bounds |y|
    y2, ya2 = orc.conv2d(-x, w, -b, layout="nchw", padding=1, with_abs=True)
    _close(ya2, ya, ya)
    _close(y2, -y, ya)
    xr = rng.standard_normal((2, 3, 6, 6))
    y3, ya3 = orc.conv2d(xr, w, b, layout="nchw", padding=1, with_abs=True)
    assert np.all(np.abs(y3) <= ya3 * (1 + 1e-12))


def pin_thread_count(orc):
    rng = np.random.default_rng(15)
    x = rng.standard_normal((3, 4, 9, 9))
    w = rng.standard_normal((5, 4, 3, 3))
    a = orc.conv2d(x, w, None, layout="nchw", padding=1, nthreads=1)
    b = orc.conv2d(x, w, None, layout="nchw", padding=1, nthreads=7)
    np.testing.assert_array_equal(a, b)


ALL_PINS = [pin_hand_worked, pin_decode, pin_output_dims, pin_delta, pin_matmul_1x1, pin_box_sums,
            pin_brute_force, pin_stride_subsample, pin_dilation_zero_insert, pin_layout_permutation,
            pin_linearity, pin_transpose, pin_torch_float64, pin_points_match_full, pin_abs_scale,
            pin_thread_count]
