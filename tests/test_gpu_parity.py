"""GPU parity: the HIP path (called through the C ABI) against the fp64
reference convolution, on seeded inputs.

Covers: a fuzz over shapes, strides, padding, dilation, layouts, storage types
and both lowerings (several tiles and ragged tails in every GEMM dimension);
integer-valued inputs, where fp32 accumulation is exact and the result must
equal the reference rounded to the storage type bit for bit; delta kernels
(y == x bit for bit); the lowered buffers and packed filter byte for byte;
determinism; the staged entry points; error paths; mid-size layers whose
default plans take the kernels chosen only for many tiles; and every output
of the five workloads at their full sizes in the launch configuration the
benchmark times, under all three algorithms.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import cnn_convolution_lowering_amd as cl
import oracle
from parity import TORCH_DT, assert_parity, expected_im2col, expected_im2win, expected_packed_filter, to_f64

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    cl.load_library()          # raises if the HIP library is not built: there is no other path
    return torch.device("cuda:0")


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _perm_x(x_nchw, layout):
    return x_nchw.permute(0, 2, 3, 1).contiguous() if layout == "nhwc" else x_nchw.contiguous()


def _run(dev, x, w, b, layout, stride, pad, dil, algo):
    d = cl.descriptor(tuple(x.shape), tuple(w.shape), stride=stride, padding=pad, dilation=dil, layout=layout,
                      dtype={torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[x.dtype],
                      algo=algo)
    xd, wd = x.to(dev), w.to(dev)
    bd = None if b is None else b.to(dev)
    y = d.forward(xd, wd, bd)
    torch.cuda.synchronize()
    return y.cpu()


def _check_full(dev, x, w, b, layout, stride, pad, dil, algo, dtype, what):
    _say("case %s" % what)
    y = _run(dev, x, w, b, layout, stride, pad, dil, algo)
    ref, yabs = oracle.conv2d(x, w, b, layout=layout, stride=stride, padding=pad, dilation=dil, with_abs=True)
    return assert_parity(to_f64(y), ref, yabs, dtype, what)


# ---------------------------------------------------------------- fuzz

def _fuzz_cases():
    rng = np.random.default_rng(2024)
    cases = []
    combos = [(dt, lay, algo) for dt in ("f32", "f16", "bf16") for lay in ("nchw", "nhwc")
              for algo in ("im2win", "im2col", "implicit")]
    for i in range(90):
        dt, lay, algo = combos[i % len(combos)]
        R, S = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        st = (int(rng.integers(1, 4)), int(rng.integers(1, 4)))
        dl = (int(rng.integers(1, 3)), int(rng.integers(1, 3))) if i % 3 == 0 else (1, 1)
        pd = (int(rng.integers(0, 4)), int(rng.integers(0, 4)))
        C = int(rng.choice([1, 3, 5, 8, 16, 19, 32, 40, 64]))
        K = int(rng.choice([1, 7, 16, 31, 32, 33, 64, 65, 100, 128, 150]))
        N = int(rng.integers(1, 4))
        H = int(rng.integers(max(1, dl[0] * (R - 1) + 1 - 2 * pd[0]), 24))
        W = int(rng.integers(max(1, dl[1] * (S - 1) + 1 - 2 * pd[1]), 24))
        cases.append((i, dt, lay, algo, N, C, H, W, K, R, S, st, pd, dl))
    return cases


@pytest.mark.parametrize("case", _fuzz_cases(), ids=lambda c: "%d-%s-%s-%s-N%dC%dH%dW%dK%dR%dS%d-s%s-p%s-d%s" % c)
def test_fuzz_parity(dev, case):
    i, dt, lay, algo, N, C, H, W, K, R, S, st, pd, dl = case
    g = torch.Generator().manual_seed(1000 + i)
    x = (torch.rand(N, C, H, W, generator=g) * 2 - 1).to(TORCH_DT[dt])
    w = (torch.randn(K, C, R, S, generator=g) / np.sqrt(C * R * S)).to(TORCH_DT[dt])
    b = (torch.randn(K, generator=g) * 0.1).to(TORCH_DT[dt]) if i % 4 != 3 else None
    _check_full(dev, _perm_x(x, lay), _perm_x(w, lay), b, lay, st, pd, dl, algo, dt, "fuzz %d" % i)


# ------------------------------------------------- default plans, mid-size

# Shapes large enough that the default plan takes the kernels chosen only for
# many tiles, with sizes off their blocks: the LDS-filter strips on 512 x 128
# tiles reading the KRSC rows (3x3 at an output width that does not divide the
# tile, 5x5) and the packed copy (a 1x9 filter), the streaming 1x1 kernel
# (a pixel count off its 16-row blocks, K = 100), and the pipelined kernel's
# one-round tile shapes.  (dtype, N, C, H, W, K, R,
# S, padding, expected kernel, expected variant)
MID_CASES = [
    ("f16", 56, 32, 40, 48, 256, 3, 3, (1, 1), 13, 3),
    ("bf16", 12, 32, 64, 64, 256, 5, 5, (2, 2), 13, 3),
    ("f16", 12, 32, 64, 64, 256, 1, 9, (0, 4), 13, 2),
    ("bf16", 5, 64, 60, 61, 100, 1, 1, (0, 0), 14, 2),
    # one round of the pipelined kernel's 128 x 128 four-stage tiles (164 of
    # them, last row of tiles and last column ragged), and of its 256 x 128
    # tiles on a 1x1 layer the streaming kernel does not take (96 channels;
    # 202 tiles, both ragged)
    ("bf16", 20, 64, 23, 23, 200, 3, 3, (1, 1), 1, 12),
    ("f16", 7, 96, 61, 61, 136, 1, 1, (0, 0), 1, 13),
]


@pytest.mark.parametrize("case", MID_CASES, ids=lambda c: "%s-N%dC%dH%dW%dK%dR%dS%d" % c[:8])
def test_default_plans_mid_size(dev, case):
    dt, N, C, H, W, K, R, S, pd, kern, var = case
    d = cl.Conv2d(N, C, H, W, K, R, S, padding=pd, layout="nhwc", dtype=dt, algo="implicit")
    assert (d.info["kernel"], d.info["kernel_variant"]) == (kern, var), d.info
    g = torch.Generator().manual_seed(4000 + N * 7 + S)
    x = (torch.rand(N, C, H, W, generator=g) * 2 - 1).to(TORCH_DT[dt])
    w = (torch.randn(K, C, R, S, generator=g) / np.sqrt(C * R * S)).to(TORCH_DT[dt])
    b = (torch.randn(K, generator=g) * 0.1).to(TORCH_DT[dt])
    _check_full(dev, _perm_x(x, "nhwc"), _perm_x(w, "nhwc"), b, "nhwc", (1, 1), pd, (1, 1), "implicit", dt,
                "default plan %s" % (case,))


# ---------------------------------------------------------------- exactness

@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("lay", ["nchw", "nhwc"])
@pytest.mark.parametrize("algo", ["im2win", "im2col", "implicit"])
def test_integer_inputs_bit_exact(dev, dt, lay, algo):
    """Integer x, w, b: fp32 accumulation is exact (|partial sums| < 2^24), so y
    must be the reference rounded once to the storage type (RNE), bit for bit."""
    g = torch.Generator().manual_seed(7)
    for (N, C, H, W, K, R, S, st, pd) in [(2, 24, 11, 9, 70, 3, 3, (1, 1), (1, 1)),
                                          (1, 3, 20, 17, 33, 5, 4, (2, 1), (2, 0)),
                                          (3, 64, 6, 6, 130, 1, 1, (1, 1), (0, 0)),
                                          (2, 40, 8, 8, 48, 2, 2, (2, 2), (0, 0))]:
        x = torch.randint(-2, 3, (N, C, H, W), generator=g).to(TORCH_DT[dt])
        w = torch.randint(-2, 3, (K, C, R, S), generator=g).to(TORCH_DT[dt])
        b = torch.randint(-4, 5, (K,), generator=g).to(TORCH_DT[dt])
        xl, wl = _perm_x(x, lay), _perm_x(w, lay)
        _say("int case C%d K%d R%d %s %s %s" % (C, K, R, dt, lay, algo))
        y = _run(dev, xl, wl, b, lay, st, pd, (1, 1), algo)
        ref = oracle.conv2d(xl, wl, b, layout=lay, stride=st, padding=pd)
        assert np.all(np.abs(ref) < 2 ** 24)
        want = torch.from_numpy(ref).to(torch.float32).to(TORCH_DT[dt])
        assert torch.equal(y.view(torch.int16 if dt != "f32" else torch.int32),
                           want.view(torch.int16 if dt != "f32" else torch.int32)), "%s %s %s" % (dt, lay, algo)


@pytest.mark.parametrize("lay", ["nchw", "nhwc"])
@pytest.mark.parametrize("algo", ["im2win", "im2col"])
def test_unpadded_rows_integer_exact(dev, lay, algo):
    """fp32 lowered rows whose R*C is not a whole number of vectors are stored
    unpadded and read element by element; a vector read then crosses into
    the next tap's columns (with horizontal dilation, a different strip
    column).  Integer inputs: the result must be the oracle's bit for bit."""
    g = torch.Generator().manual_seed(29)
    for (N, C, H, W, K, R, S, st, pd, dl) in [(2, 5, 13, 11, 33, 3, 2, (2, 1), (1, 0), (1, 2)),
                                              (3, 3, 30, 30, 32, 3, 3, (1, 1), (1, 1), (1, 1)),
                                              (1, 1, 9, 20, 70, 1, 3, (1, 2), (0, 1), (1, 3)),
                                              (2, 7, 8, 9, 130, 3, 3, (1, 1), (1, 1), (2, 2))]:
        d = cl.Conv2d(N, C, H, W, K, R, S, stride=st, padding=pd, dilation=dl, layout=lay, dtype="f32", algo=algo)
        assert d.info["RCp"] == R * C and d.info["kernel"] == 0, d.info
        x = torch.randint(-2, 3, (N, C, H, W), generator=g).to(torch.float32)
        w = torch.randint(-2, 3, (K, C, R, S), generator=g).to(torch.float32)
        b = torch.randint(-4, 5, (K,), generator=g).to(torch.float32)
        xl, wl = _perm_x(x, lay), _perm_x(w, lay)
        _say("unpadded case C%d R%d S%d dil%s %s %s" % (C, R, S, dl, lay, algo))
        y = _run(dev, xl, wl, b, lay, st, pd, dl, algo)
        ref = oracle.conv2d(xl, wl, b, layout=lay, stride=st, padding=pd, dilation=dl)
        assert np.all(np.abs(ref) < 2 ** 24)
        assert torch.equal(y, torch.from_numpy(ref).to(torch.float32)), (lay, algo, C, R, S)


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("lay", ["nchw", "nhwc"])
def test_delta_kernel_reproduces_input(dev, dt, lay):
    g = torch.Generator().manual_seed(8)
    for R in (1, 3, 5):
        C = 24
        x = (torch.rand(2, C, 13, 10, generator=g) * 8 - 4).to(TORCH_DT[dt])
        w = torch.zeros(C, C, R, R)
        for k in range(C):
            w[k, k, R // 2, R // 2] = 1
        w = w.to(TORCH_DT[dt])
        for algo in ("im2win", "im2col", "implicit"):
            _say("delta R%d %s %s %s" % (R, dt, lay, algo))
            y = _run(dev, _perm_x(x, lay), _perm_x(w, lay), None, lay, 1, R // 2, 1, algo)
            assert torch.equal(y, _perm_x(x, lay)), (R, algo)


# ---------------------------------------------------------------- lowered buffers byte for byte

def _bits(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32).numpy()


@pytest.mark.parametrize("dt", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("lay", ["nchw", "nhwc"])
@pytest.mark.parametrize("shape", [(2, 3, 9, 11, 8, 3, 3, (1, 1), (1, 1), (1, 1)),
                                   (1, 16, 7, 12, 5, 3, 2, (2, 3), (2, 1), (1, 2)),
                                   (2, 8, 10, 10, 4, 2, 5, (1, 2), (0, 2), (2, 1)),
                                   # enough images for bands of several output rows, the last band ragged
                                   (1100, 3, 13, 11, 4, 3, 3, (1, 1), (1, 1), (1, 1)),
                                   (2100, 5, 13, 9, 4, 3, 2, (2, 1), (1, 0), (1, 2)),
                                   # NCHW rows too wide for one staged tile: chunks of output columns
                                   (1, 64, 12, 200, 4, 3, 3, (1, 1), (1, 1), (1, 1)),
                                   (2, 40, 9, 150, 4, 4, 5, (2, 3), (1, 2), (1, 2)),
                                   # NCHW planes on 16-byte boundaries, one chunk across: staged
                                   # with 16-byte loads (bands of one and of several rows)
                                   (3, 5, 12, 12, 4, 3, 3, (1, 1), (1, 1), (1, 1)),
                                   (1100, 3, 12, 12, 4, 3, 3, (1, 1), (1, 1), (1, 1)),
                                   (2, 16, 8, 10, 4, 2, 3, (2, 1), (3, 0), (1, 2)),
                                   # one-column tiles beyond the LDS budget: the element-wise
                                   # kernel (NCHW C*R large; NHWC C=3 rows of 3000 columns),
                                   # and NCHW column chunks with a ragged last chunk
                                   (1, 2048, 6, 6, 4, 5, 5, (1, 1), (1, 1), (1, 1)),
                                   (1, 3, 9, 3000, 4, 7, 7, (1, 1), (0, 3), (1, 1))])
def test_lowered_layouts_exact(dev, dt, lay, shape):
    N, C, H, W, K, R, S, st, pd, dl = shape
    g = torch.Generator().manual_seed(9)
    x = (torch.rand(N, C, H, W, generator=g) * 2 - 1).to(TORCH_DT[dt])
    w = torch.randn(K, C, R, S, generator=g).to(TORCH_DT[dt])
    for algo in ("im2win", "im2col"):
        d = cl.Conv2d(N, C, H, W, K, R, S, stride=st, padding=pd, dilation=dl, layout=lay, dtype=dt, algo=algo)
        info = d.info
        ws = torch.zeros(max(1, d.workspace_bytes), dtype=torch.uint8, device=dev)
        _say("layout %s %s %s %s" % (shape, dt, lay, algo))
        d.pack_filter(_perm_x(w, lay).to(dev), ws)
        d.lower_input(_perm_x(x, lay).to(dev), ws)
        torch.cuda.synchronize()
        wsc = ws.cpu()
        elem = info["elem_bytes"]
        RCp, Kl, P, Q = info["RCp"], info["Kl"], info["P"], info["Q"]
        xb, wb = _bits(x), _bits(w)
        if info["ws_filter_bytes"]:
            o = info["ws_filter_offset"]
            got = wsc[o:o + info["ws_filter_bytes"]].view(x.dtype)
            np.testing.assert_array_equal(_bits(got).reshape(K, Kl), expected_packed_filter(wb, RCp))
        o = info["ws_lowered_offset"]
        got = _bits(wsc[o:o + info["ws_lowered_bytes"]].view(x.dtype))
        win = expected_im2win(xb, R, S, P, Q, st, pd, dl, RCp)
        if algo == "im2win":
            np.testing.assert_array_equal(got.reshape(win.shape), win)
        else:
            np.testing.assert_array_equal(got.reshape(N * P * Q, Kl), expected_im2col(win, Q, S, st[1], dl[1], RCp))


# ---------------------------------------------------------------- properties of the path

def test_deterministic_and_staged_equals_fused(dev):
    g = torch.Generator().manual_seed(10)
    for dt, lay, algo in (("f16", "nhwc", "im2win"), ("f32", "nchw", "im2win"), ("bf16", "nchw", "im2col"),
                          ("f16", "nhwc", "implicit"), ("f32", "nchw", "implicit")):
        x = _perm_x((torch.rand(4, 32, 15, 15, generator=g) * 2 - 1).to(TORCH_DT[dt]), lay).to(dev)
        w = _perm_x(torch.randn(96, 32, 3, 3, generator=g).to(TORCH_DT[dt]), lay).to(dev)
        b = torch.randn(96, generator=g).to(TORCH_DT[dt]).to(dev)
        d = cl.descriptor(tuple(x.shape), tuple(w.shape), padding=1, layout=lay, dtype=dt, algo=algo)
        y1 = d.forward(x, w, b)
        y2 = d.forward(x, w, b)
        ws = d.new_workspace(dev)
        y3 = d.new_output(dev)
        d.pack_filter(w, ws)
        d.lower_input(x, ws)
        d.contract(x, w, b, y3, ws)
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            y4 = d.forward(x, w, b, stream=s)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2) and torch.equal(y1, y3) and torch.equal(y1, y4)


def test_empty_batch(dev):
    d = cl.Conv2d(0, 8, 5, 5, 4, 3, 3, padding=1, layout="nhwc", dtype="f16")
    x = torch.empty(0, 5, 5, 8, dtype=torch.float16, device=dev)
    w = torch.randn(4, 3, 3, 8, device=dev).half()
    y = d.forward(x, w)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (0, 5, 5, 4)


def test_error_paths(dev):
    d = cl.Conv2d(1, 8, 6, 6, 8, 3, 3, padding=1, layout="nhwc", dtype="f16")
    x = torch.randn(1, 6, 6, 8, device=dev).half()
    w = torch.randn(8, 3, 3, 8, device=dev).half()
    with pytest.raises(cl.ConvError) as e:                       # host memory is not accepted
        d.forward(x.cpu(), w)
    assert e.value.status == -4
    big = torch.randn(1 * 6 * 6 * 8 + 8, device=dev).half()
    xm = big[1:1 + 288].view(1, 6, 6, 8)                       # 2-byte offset: misaligned
    with pytest.raises(cl.ConvError) as e:
        d.forward(xm, w)
    assert e.value.status == -5


@pytest.mark.parametrize("lay", ["nchw", "nhwc"])
def test_edge_shapes(dev, lay):
    g = torch.Generator().manual_seed(11)
    cases = [  # N, C, H, W, K, R, S, stride, pad, dil
        (1, 1, 1, 1, 1, 1, 1, (1, 1), (0, 0), (1, 1)),
        (1, 1, 5, 5, 1, 1, 1, (1, 1), (2, 2), (1, 1)),      # padding wider than the kernel: border = bias
        (3, 8, 9, 9, 5, 1, 1, (2, 3), (0, 0), (1, 1)),      # 1x1 strided (read in place for NHWC)
        (2, 5, 4, 30, 9, 1, 7, (1, 4), (0, 3), (1, 1)),     # wide kernel, large stride
        (2, 6, 30, 4, 9, 7, 1, (4, 1), (3, 0), (1, 1)),     # tall kernel
        (1, 8, 12, 12, 3, 3, 3, (5, 5), (0, 0), (1, 1)),    # stride larger than the kernel
        (2, 4, 16, 16, 300, 3, 3, (1, 1), (1, 1), (3, 3)),  # K spans three tiles, dilation 3
        (1, 136, 5, 5, 8, 3, 3, (1, 1), (1, 1), (1, 1)),    # long contraction, ragged K-tile tail
    ]
    for i, (N, C, H, W, K, R, S, st, pd, dl) in enumerate(cases):
        for dt in ("f32", "f16", "bf16"):
            x = (torch.rand(N, C, H, W, generator=g) * 2 - 1).to(TORCH_DT[dt])
            w = (torch.randn(K, C, R, S, generator=g) / np.sqrt(C * R * S)).to(TORCH_DT[dt])
            b = (torch.randn(K, generator=g) * 0.1).to(TORCH_DT[dt])
            for algo in ("im2win", "im2col", "implicit"):
                _check_full(dev, _perm_x(x, lay), _perm_x(w, lay), b, lay, st, pd, dl, algo, dt,
                            "edge %d %s %s %s" % (i, dt, lay, algo))


# ---------------------------------------------------------------- the five workloads, every output

# (workload, layer index) in workload order, so that one layer's reference is
# computed once and shared by the three algorithms
_WORKLOAD_LAYERS = [("c1", 0), ("c2", 0), ("c2", 1), ("c2", 2), ("c2", 3), ("c3", 0), ("c4", 0), ("c4", 1),
                    ("c4", 2), ("c5", 0), ("c5", 1), ("c5", 2), ("c5", 3), ("c5", 4)]


class _WorkloadRefs:
    """The inputs of each layer of one workload and the fp64 reference of its
    whole output, computed once and shared by the three algorithms.  A chained
    layer's input is the previous layer's reference output rounded once to the
    storage type (round to nearest even), so every algorithm sees the same
    input and errors do not compound from layer to layer."""

    def __init__(self):
        self.name = None

    def layer(self, name, i):
        from cnn_convolution_lowering_amd.workloads import make_workload
        if self.name != name:
            self.name, self.wl, self.x, self.ref = name, make_workload(name), {}, {}
        spec = self.wl.spec
        L = self.wl.layers[i]
        if i not in self.x:
            if L.x is not None:
                self.x[i] = L.x
            else:
                prev, _ = self.layer(name, i - 1)[2]
                self.x[i] = torch.from_numpy(prev).to(torch.float32).to(TORCH_DT[spec.dtype]).contiguous()
        if i not in self.ref:
            _say("oracle %s layer %d (%s), %d threads" % (name, i, L.label, oracle.default_threads()))
            self.ref[i] = oracle.conv2d(self.x[i], L.w, L.b, layout=spec.layout, stride=L.stride,
                                        padding=L.padding, dilation=L.dilation, with_abs=True)
        return L, self.x[i], self.ref[i]


@pytest.fixture(scope="module")
def workload_refs():
    return _WorkloadRefs()


@pytest.mark.parametrize("algo", ["implicit", "im2win", "im2col"])
@pytest.mark.parametrize("name,layer", _WORKLOAD_LAYERS, ids=lambda v: str(v))
def test_workload_full_output(dev, workload_refs, name, layer, algo):
    """Every output of every layer of the five workloads at their full sizes,
    through the descriptor the benchmark times (the default plan for the
    algorithm), against the fp64 reference, to the per-element bound."""
    L, x, (ref, yabs) = workload_refs.layer(name, layer)
    spec = workload_refs.wl.spec
    if spec.layout == "nchw":
        N, C, H, W = x.shape
    else:
        N, H, W, C = x.shape
    d = cl.Conv2d(N, C, H, W, L.K, L.R, L.S, stride=L.stride, padding=L.padding, dilation=L.dilation,
                  layout=spec.layout, dtype=spec.dtype, algo=algo)
    assert d.plan is None
    i = d.info
    _say("workload %s layer %d (%s) %s: kernel %d variant %d ksplit %d, %d outputs" % (
        name, layer, L.label, algo, i["kernel"], i["kernel_variant"], i["ksplit"], ref.size))
    y = d.forward(x.to(dev), L.w.to(dev), L.b.to(dev))
    torch.cuda.synchronize()
    got = to_f64(y.cpu())
    assert got.shape == ref.shape
    err = assert_parity(got, ref, yabs, spec.dtype, "%s layer %d %s" % (name, layer, algo))
    # the weaker global reading, for the record
    glob = float(np.max(np.abs(got - ref)) / np.max(yabs))
    _say("  max |err|/sum|x*w| = %.3g (bound %.0e); global max|err| / max sum|x*w| = %.3g" % (
        err, 1e-5 if spec.dtype == "f32" else 4e-3, glob))


@pytest.mark.parametrize("name,batch", [("c2", 6), ("c4", 1), ("c5", 1)])
@pytest.mark.parametrize("algo", ["im2win", "implicit"])
def test_workloads_reduced_batch_full_output(dev, name, batch, algo):
    """The same layers at a small batch (a different plan where the planner
    sizes tiles and splits by the number of output tiles)."""
    from cnn_convolution_lowering_amd.workloads import make_workload
    wl = make_workload(name, batch)
    spec = wl.spec
    x_prev = None
    for i, L in enumerate(wl.layers):
        x = L.x.to(dev) if L.x is not None else x_prev
        d = cl.descriptor(tuple(x.shape), tuple(L.w.shape), stride=L.stride, padding=L.padding,
                          dilation=L.dilation, layout=spec.layout, dtype=spec.dtype, algo=algo)
        _say("workload %s N=%d layer %d (%s) %s" % (name, spec.N, i, L.label, algo))
        y = d.forward(x, L.w.to(dev), L.b.to(dev))
        torch.cuda.synchronize()
        ref, yabs = oracle.conv2d(x.cpu(), L.w, L.b, layout=spec.layout, stride=L.stride, padding=L.padding,
                                  dilation=L.dilation, with_abs=True)
        assert_parity(to_f64(y.cpu()), ref, yabs, spec.dtype, "%s N=%d layer %d" % (name, batch, i))
        x_prev = y
