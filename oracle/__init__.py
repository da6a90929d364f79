"""Reference forward convolution in fp64 -- TEST INFRASTRUCTURE ONLY.

Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, links or calls it, and shares no code with
it.

The arithmetic lives in ``conv_oracle.c`` (seven plain loops, fp64
accumulation, exact decoding of fp32/fp16/bf16 storage); this module only
compiles it with gcc and marshals numpy / torch-CPU arrays into it.

Definition (cross-correlation, zero padding), from "GPU-Accelerating MSCRED
with CUDA, im2col, GEMM, and a Custom PyTorch Extension", sections "Where the
Performance Bottleneck Appeared" and "Transforming Conv2D into im2col and
GEMM":

    y[n,k,p,q] = b[k] + sum_{c,r,s} x[n, c, p*sh-ph+r*dh, q*sw-pw+s*dw] * w[k,c,r,s]

Layouts: "nchw" means x NCHW, w KCRS, y NKPQ; "nhwc" means x NHWC, w KRSC,
y NPQK.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "conv_oracle.c")
_LIB = os.path.join(_HERE, "libconv_oracle.so")

# storage-type codes understood by conv_oracle.c
_DTYPE_CODE = {"f32": 0, "f16": 1, "bf16": 2, "f64": 3}
_LAYOUT_CODE = {"nchw": 0, "nhwc": 1}


class _Problem(ctypes.Structure):
    _fields_ = [(name, ctypes.c_int64) for name in (
        "N", "C", "H", "W", "K", "R", "S",
        "stride_h", "stride_w", "pad_h", "pad_w", "dil_h", "dil_w",
        "layout", "dtype")]


def build(force: bool = True) -> str:
    """Compile conv_oracle.c into libconv_oracle.so next to it (gcc, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


class OracleLib:
    """ctypes view of one build of conv_oracle.c (the default one, or a copy)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.POINTER
        lib.oracle_output_dims.argtypes = [P(_Problem), P(ctypes.c_int64), P(ctypes.c_int64)]
        lib.oracle_output_dims.restype = ctypes.c_int
        lib.oracle_decode.argtypes = [ctypes.c_int64, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        lib.oracle_decode.restype = ctypes.c_int
        lib.oracle_conv2d.argtypes = [P(_Problem), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
        lib.oracle_conv2d.restype = ctypes.c_int
        lib.oracle_conv2d_points.argtypes = [P(_Problem), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_int]
        lib.oracle_conv2d_points.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def output_dims(self, x_shape, w_shape, layout="nchw", stride=1, padding=0, dilation=1):
        pr = _problem(x_shape, w_shape, layout, stride, padding, dilation, "f64")
        P, Q = ctypes.c_int64(), ctypes.c_int64()
        if self.lib.oracle_output_dims(ctypes.byref(pr), ctypes.byref(P), ctypes.byref(Q)) != 0:
            raise ValueError("oracle: invalid convolution parameters")
        return P.value, Q.value

    def decode(self, a) -> np.ndarray:
        """Exact fp64 values of an fp32 / fp16 / bf16 / fp64 array (own bit decoding)."""
        arr, name = _as_storage(a)
        out = np.empty(arr.shape, dtype=np.float64)
        if self.lib.oracle_decode(_DTYPE_CODE[name], arr.ctypes.data, arr.size, out.ctypes.data) != 0:
            raise ValueError("oracle: decode failed")
        return out

    def conv2d(self, x, w, b=None, *, layout="nchw", stride=1, padding=0, dilation=1,
               nthreads: int | None = None, with_abs: bool = False):
        """Full fp64 output (and optionally yabs = |b| + sum|x*w|) in the layout's y order."""
        xa, wa, ba, dt = _operands(x, w, b)
        pr = _problem(xa.shape, wa.shape, layout, stride, padding, dilation, dt)
        P, Q = self.output_dims(xa.shape, wa.shape, layout, stride, padding, dilation)
        N, K = pr.N, pr.K
        shape = (N, K, P, Q) if layout == "nchw" else (N, P, Q, K)
        y = np.empty(shape, dtype=np.float64)
        yabs = np.empty(shape, dtype=np.float64) if with_abs else None
        rc = self.lib.oracle_conv2d(ctypes.byref(pr), xa.ctypes.data, wa.ctypes.data,
                                    None if ba is None else ba.ctypes.data, y.ctypes.data,
                                    None if yabs is None else yabs.ctypes.data,
                                    nthreads or default_threads())
        if rc != 0:
            raise RuntimeError("oracle_conv2d failed (%d)" % rc)
        return (y, yabs) if with_abs else y

    def conv2d_points(self, x, w, b, nkpq, *, layout="nchw", stride=1, padding=0, dilation=1,
                      nthreads: int | None = None):
        """Outputs at the given (n, k, p, q) coordinates, one by one: returns (y, yabs)."""
        xa, wa, ba, dt = _operands(x, w, b)
        pr = _problem(xa.shape, wa.shape, layout, stride, padding, dilation, dt)
        pts = np.ascontiguousarray(np.asarray(nkpq, dtype=np.int64).reshape(-1, 4))
        y = np.empty(len(pts), dtype=np.float64)
        yabs = np.empty(len(pts), dtype=np.float64)
        rc = self.lib.oracle_conv2d_points(ctypes.byref(pr), xa.ctypes.data, wa.ctypes.data,
                                           None if ba is None else ba.ctypes.data, pts.ctypes.data,
                                           len(pts), y.ctypes.data, yabs.ctypes.data,
                                           nthreads or default_threads())
        if rc != 0:
            raise RuntimeError("oracle_conv2d_points failed (%d)" % rc)
        return y, yabs


_default = None


def _load() -> OracleLib:
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build(force=False)
        _default = OracleLib(_LIB)
    return _default


def build_variant(source_text: str, out_path: str) -> OracleLib:
    """Compile a (possibly edited) copy of conv_oracle.c: used by the tests that
    plant a mistake in the oracle and check that the pins catch it."""
    src = out_path + ".c"
    with open(src, "w") as f:
        f.write(source_text)
    subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-pthread",
                           src, "-o", out_path, "-lm"])
    return OracleLib(out_path)


def source_text() -> str:
    with open(_SRC) as f:
        return f.read()


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _pair(v):
    if isinstance(v, (tuple, list)):
        assert len(v) == 2
        return int(v[0]), int(v[1])
    return int(v), int(v)


def _as_storage(a):
    """Return (contiguous numpy array holding the raw storage, dtype code name)."""
    try:
        import torch
        if isinstance(a, torch.Tensor):
            a = a.detach().cpu().contiguous()
            if a.dtype == torch.bfloat16:
                return a.view(torch.int16).numpy(), "bf16"
            a = a.numpy()
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(a)
    name = {np.dtype(np.float32): "f32", np.dtype(np.float16): "f16",
            np.dtype(np.float64): "f64"}.get(a.dtype)
    if name is None:
        raise TypeError("oracle: unsupported storage dtype %s" % a.dtype)
    return a, name


def _problem(x_shape, w_shape, layout, stride, padding, dilation, dtype):
    if layout == "nchw":
        N, C, H, W = x_shape
        K, C2, R, S = w_shape
    elif layout == "nhwc":
        N, H, W, C = x_shape
        K, R, S, C2 = w_shape
    else:
        raise ValueError(layout)
    if C != C2:
        raise ValueError("oracle: channel mismatch %d vs %d" % (C, C2))
    sh, sw = _pair(stride)
    ph, pw = _pair(padding)
    dh, dw = _pair(dilation)
    return _Problem(N, C, H, W, K, R, S, sh, sw, ph, pw, dh, dw, _LAYOUT_CODE[layout], _DTYPE_CODE[dtype])


def _operands(x, w, b):
    xa, xt = _as_storage(x)
    wa, wt = _as_storage(w)
    if xt != wt:
        raise TypeError("oracle: x and w storage types differ (%s, %s)" % (xt, wt))
    ba = None
    if b is not None:
        ba, bt = _as_storage(b)
        if bt != xt:
            raise TypeError("oracle: bias storage type differs")
    return xa, wa, ba, xt


def output_dims(*a, **k):
    return _load().output_dims(*a, **k)


def decode(a) -> np.ndarray:
    return _load().decode(a)


def conv2d(*a, **k):
    return _load().conv2d(*a, **k)


def conv2d_points(*a, **k):
    return _load().conv2d_points(*a, **k)
