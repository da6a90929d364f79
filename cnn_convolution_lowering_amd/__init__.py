"""Forward 2-D convolution lowered to an MFMA contraction on AMD MI355X (gfx950).

A thin ctypes binding over the C ABI in ``include/convlower.h`` (built as
``libconvlower.so`` next to this file).  It only marshals arguments: tensor
shapes and data pointers, the current HIP stream, and -- when the caller does
not pass them -- ``y`` and the workspace allocated with torch.  Every step of
the convolution runs in the library's HIP kernels; there is no other path, and
importing or calling without the built library raises.

    import cnn_convolution_lowering_amd as cl
    y = cl.conv2d(x, w, bias, stride=1, padding=1, layout="nhwc", algo="im2win")
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Dict, Optional, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libconvlower.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "convlower.h")

STATUS = {0: "CONV_OK", -1: "CONV_ERR_INVALID_ARG", -2: "CONV_ERR_UNSUPPORTED", -3: "CONV_ERR_NULL_PTR",
          -4: "CONV_ERR_NOT_DEVICE_PTR", -5: "CONV_ERR_MISALIGNED", -6: "CONV_ERR_HIP", -7: "CONV_ERR_OOM"}
LAYOUTS = {"nchw": 0, "nhwc": 1}
DTYPES = {"f32": 0, "f16": 1, "bf16": 2}
ALGOS = {"im2win": 0, "im2col": 1, "implicit": 2}


class ConvError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        name = STATUS.get(status, str(status))
        super().__init__("%s%s" % (name, (": " + what) if what else ""))


class ConvParams(ctypes.Structure):
    _fields_ = [("N", ctypes.c_int64), ("C", ctypes.c_int64), ("H", ctypes.c_int64), ("W", ctypes.c_int64),
                ("K", ctypes.c_int64), ("R", ctypes.c_int64), ("S", ctypes.c_int64),
                ("stride_h", ctypes.c_int32), ("stride_w", ctypes.c_int32),
                ("pad_h", ctypes.c_int32), ("pad_w", ctypes.c_int32),
                ("dil_h", ctypes.c_int32), ("dil_w", ctypes.c_int32),
                ("layout", ctypes.c_int), ("dtype", ctypes.c_int), ("algo", ctypes.c_int)]


class PlanInfo(ctypes.Structure):
    _fields_ = [("P", ctypes.c_int64), ("Q", ctypes.c_int64), ("M", ctypes.c_int64), ("Kg", ctypes.c_int64),
                ("W_used", ctypes.c_int64), ("RCp", ctypes.c_int64), ("Kl", ctypes.c_int64),
                ("ws_bytes", ctypes.c_uint64), ("ws_filter_offset", ctypes.c_uint64),
                ("ws_filter_bytes", ctypes.c_uint64), ("ws_lowered_offset", ctypes.c_uint64),
                ("ws_lowered_bytes", ctypes.c_uint64), ("im2win_bytes", ctypes.c_uint64),
                ("im2col_bytes", ctypes.c_uint64), ("lowering_elided", ctypes.c_int32),
                ("tile_m", ctypes.c_int32), ("tile_n", ctypes.c_int32), ("tile_k", ctypes.c_int32),
                ("elem_bytes", ctypes.c_int32), ("kernel", ctypes.c_int32), ("kernel_variant", ctypes.c_int32),
                ("ws_partial_offset", ctypes.c_uint64), ("ws_partial_bytes", ctypes.c_uint64),
                ("ksplit", ctypes.c_int32), ("tile_order", ctypes.c_int32)]


class TuneResult(ctypes.Structure):
    _fields_ = [("candidates", ctypes.c_int32), ("kernel", ctypes.c_int32), ("kernel_variant", ctypes.c_int32),
                ("default_ms", ctypes.c_float), ("best_ms", ctypes.c_float), ("ksplit", ctypes.c_int32),
                ("tile_order", ctypes.c_int32)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libconvlower.so; raises if it has not been built."""
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise ImportError("libconvlower.so is not built (expected at %s); run __graft_entry__.build() "
                          "or python cnn_convolution_lowering_amd/build.py" % path)
    lib = ctypes.CDLL(path)
    vp, i64p = ctypes.c_void_p, ctypes.POINTER(ctypes.c_int64)
    sig = {
        "conv_create_desc": [ctypes.POINTER(ConvParams), ctypes.POINTER(vp)],
        "conv_create_desc_forced": [ctypes.POINTER(ConvParams), ctypes.c_char_p, ctypes.POINTER(vp)],
        "conv_destroy_desc": [vp],
        "conv_workspace_size": [vp, ctypes.POINTER(ctypes.c_size_t)],
        "conv_output_dims": [vp, i64p, i64p],
        "conv_plan_info": [vp, ctypes.POINTER(PlanInfo)],
        "conv2d_fwd": [vp, vp, vp, vp, vp, vp, vp],
        "conv2d_fwd_noalloc": [vp, vp, vp, vp, vp, vp],
        "conv_pack_filter": [vp, vp, vp, vp],
        "conv_lower_input": [vp, vp, vp, vp],
        "conv_contract": [vp, vp, vp, vp, vp, vp, vp],
        "conv_lstm_create_desc": [ctypes.POINTER(ConvParams), ctypes.c_int64, ctypes.POINTER(vp)],
        "conv_lstm_step": [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp],
        "conv_tune": [vp, vp, vp, vp, vp, vp, ctypes.c_size_t, ctypes.c_int32, vp, ctypes.POINTER(vp),
                      ctypes.POINTER(TuneResult)],
    }
    for name, args in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    lib.conv_status_string.argtypes = [ctypes.c_int]
    lib.conv_status_string.restype = ctypes.c_char_p
    if path == LIB_PATH:
        _lib = lib
    return lib


def header_functions(path: str = HEADER_PATH):
    """Names of the functions include/convlower.h declares."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_]+\**\s+\**\s*(conv\w*)\s*\(", text, flags=re.M)))


def _pair(v) -> Tuple[int, int]:
    if isinstance(v, (tuple, list)):
        if len(v) != 2:
            raise ValueError("expected an int or a pair, got %r" % (v,))
        return int(v[0]), int(v[1])
    return int(v), int(v)


def _check(status: int, what: str):
    if status != 0:
        raise ConvError(status, what)


def _torch():
    import torch
    return torch


def _dtype_name(t) -> str:
    torch = _torch()
    names = {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}
    if t.dtype not in names:
        raise TypeError("unsupported dtype %s (fp32, fp16 or bf16)" % t.dtype)
    return names[t.dtype]


class Conv2d:
    """One convolution descriptor (a plan); immutable once created.

    ``plan`` asks for a contraction kernel explicitly ("<kernel>:<variant>",
    "<kernel>:<variant>:<ksplit>" or "<kernel>:<variant>:<ksplit>:<tile order>",
    conv_create_desc_forced): for tests and tuning; None is the library's
    default choice."""

    def __init__(self, N, C, H, W, K, R, S, *, stride=1, padding=0, dilation=1, layout="nchw",
                 dtype="f32", algo="im2win", plan: Optional[str] = None, _handle=None):
        self.lib = load_library()
        sh, sw = _pair(stride)
        ph, pw = _pair(padding)
        dh, dw = _pair(dilation)
        if layout not in LAYOUTS or dtype not in DTYPES or algo not in ALGOS:
            raise ValueError("layout/dtype/algo must be one of %s / %s / %s" % (list(LAYOUTS), list(DTYPES), list(ALGOS)))
        self.params = ConvParams(int(N), int(C), int(H), int(W), int(K), int(R), int(S), sh, sw, ph, pw, dh, dw,
                                 LAYOUTS[layout], DTYPES[dtype], ALGOS[algo])
        self.layout, self.dtype, self.algo = layout, dtype, algo
        self.stride, self.padding, self.dilation = (sh, sw), (ph, pw), (dh, dw)
        self.plan = plan
        if _handle is not None:
            self._desc = _handle          # a descriptor conv_tune made for this object
        else:
            self._desc = ctypes.c_void_p()
            if plan is None:
                _check(self.lib.conv_create_desc(ctypes.byref(self.params), ctypes.byref(self._desc)),
                       "conv_create_desc")
            else:
                _check(self.lib.conv_create_desc_forced(ctypes.byref(self.params), plan.encode(),
                                                        ctypes.byref(self._desc)), "conv_create_desc_forced")
        info = PlanInfo()
        _check(self.lib.conv_plan_info(self._desc, ctypes.byref(info)), "conv_plan_info")
        self.info: Dict[str, int] = {name: getattr(info, name) for name, _ in PlanInfo._fields_}
        self.P, self.Q = self.info["P"], self.info["Q"]
        self.workspace_bytes = int(self.info["ws_bytes"])

    def __del__(self):
        desc = getattr(self, "_desc", None)
        if desc is not None and desc.value:
            self.lib.conv_destroy_desc(desc)
            self._desc = None

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._desc

    def x_shape(self):
        p = self.params
        return (p.N, p.C, p.H, p.W) if self.layout == "nchw" else (p.N, p.H, p.W, p.C)

    def w_shape(self):
        p = self.params
        return (p.K, p.C, p.R, p.S) if self.layout == "nchw" else (p.K, p.R, p.S, p.C)

    def y_shape(self):
        p = self.params
        return (p.N, p.K, self.P, self.Q) if self.layout == "nchw" else (p.N, self.P, self.Q, p.K)

    # -- marshalling helpers
    def _tensor(self, t, shape, what):
        if t is None:
            return None
        if tuple(t.shape) != tuple(shape):
            raise ValueError("%s has shape %s, expected %s" % (what, tuple(t.shape), tuple(shape)))
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % what)
        if _dtype_name(t) != self.dtype:
            raise TypeError("%s is %s, descriptor is %s" % (what, t.dtype, self.dtype))
        return t

    @staticmethod
    def _ptr(t) -> Optional[int]:
        return None if t is None else t.data_ptr()

    @staticmethod
    def _stream(stream, device) -> int:
        torch = _torch()
        if stream is None:
            # a host tensor is rejected by the library itself; take the default device's stream then
            stream = torch.cuda.current_stream(device if device.type == "cuda" else None)
        return int(getattr(stream, "cuda_stream", stream))

    def new_workspace(self, device):
        torch = _torch()
        if self.workspace_bytes == 0:
            return None
        return torch.empty(self.workspace_bytes, dtype=torch.uint8, device=device)

    def new_output(self, device):
        torch = _torch()
        dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[self.dtype]
        return torch.empty(self.y_shape(), dtype=dt, device=device)

    def _ws(self, ws, device):
        if ws is None:
            return self.new_workspace(device)
        if ws.numel() * ws.element_size() < self.workspace_bytes:
            raise ValueError("workspace has %d bytes, needs %d" % (ws.numel() * ws.element_size(), self.workspace_bytes))
        return ws

    # -- entry points
    def forward(self, x, w, bias=None, y=None, ws=None, stream=None):
        """conv2d_fwd: y = conv(x, w) + bias, enqueued on ``stream`` (default: current)."""
        self._tensor(x, self.x_shape(), "x")
        self._tensor(w, self.w_shape(), "w")
        self._tensor(bias, (self.params.K,), "bias")
        y = self.new_output(x.device) if y is None else self._tensor(y, self.y_shape(), "y")
        ws = self._ws(ws, x.device)
        _check(self.lib.conv2d_fwd(self._desc, self._ptr(x), self._ptr(w), self._ptr(bias), self._ptr(y),
                                   self._ptr(ws), self._stream(stream, x.device)), "conv2d_fwd")
        return y

    def forward_noalloc(self, x, w, bias=None, y=None, stream=None):
        """conv2d_fwd_noalloc: as forward, with the library's fixed device
        scratch as the workspace (no allocation in the library; ``y`` is
        allocated here with torch only when not given)."""
        self._tensor(x, self.x_shape(), "x")
        self._tensor(w, self.w_shape(), "w")
        self._tensor(bias, (self.params.K,), "bias")
        y = self.new_output(x.device) if y is None else self._tensor(y, self.y_shape(), "y")
        _check(self.lib.conv2d_fwd_noalloc(self._desc, self._ptr(x), self._ptr(w), self._ptr(bias), self._ptr(y),
                                           self._stream(stream, x.device)), "conv2d_fwd_noalloc")
        return y

    def tune(self, x, w, bias=None, y=None, ws=None, reps=5, stream=None):
        """conv_tune: time every kernel / tile variant that takes this
        convolution (within the workspace given) and return (result dict, a
        new Conv2d holding the fastest plan).  This object is not changed, so
        a descriptor shared through ``descriptor()`` keeps its plan."""
        self._tensor(x, self.x_shape(), "x")
        self._tensor(w, self.w_shape(), "w")
        self._tensor(bias, (self.params.K,), "bias")
        y = self.new_output(x.device) if y is None else self._tensor(y, self.y_shape(), "y")
        ws = self._ws(ws, x.device)
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
        res = TuneResult()
        handle = ctypes.c_void_p()
        _check(self.lib.conv_tune(self._desc, self._ptr(x), self._ptr(w), self._ptr(bias), self._ptr(y),
                                  self._ptr(ws), ws_bytes, int(reps), self._stream(stream, x.device),
                                  ctypes.byref(handle), ctypes.byref(res)), "conv_tune")
        p = self.params
        tuned = Conv2d(p.N, p.C, p.H, p.W, p.K, p.R, p.S, stride=self.stride, padding=self.padding,
                       dilation=self.dilation, layout=self.layout, dtype=self.dtype, algo=self.algo,
                       _handle=handle)
        return {name: getattr(res, name) for name, _ in TuneResult._fields_}, tuned

    def pack_filter(self, w, ws, stream=None):
        self._tensor(w, self.w_shape(), "w")
        _check(self.lib.conv_pack_filter(self._desc, self._ptr(w), self._ptr(ws), self._stream(stream, w.device)),
               "conv_pack_filter")

    def lower_input(self, x, ws, stream=None):
        self._tensor(x, self.x_shape(), "x")
        _check(self.lib.conv_lower_input(self._desc, self._ptr(x), self._ptr(ws), self._stream(stream, x.device)),
               "conv_lower_input")

    def contract(self, x, w, bias, y, ws, stream=None):
        self._tensor(y, self.y_shape(), "y")
        _check(self.lib.conv_contract(self._desc, self._ptr(x), self._ptr(w), self._ptr(bias), self._ptr(y),
                                      self._ptr(ws), self._stream(stream, y.device)), "conv_contract")


class ConvLSTMCell:
    """One ConvLSTM step plan (conv_lstm_create_desc): fp32 NCHW, x (N, Cx, H,
    W), h and c (N, Kh, H, W), gate filter w (4*Kh, Cx+Kh, R, S) in gate order
    i, f, g, o, bias (4*Kh,).  Padding / dilation must keep H x W."""

    def __init__(self, N, Cx, Kh, H, W, R, S, *, padding=0, dilation=1, algo="im2win"):
        self.lib = load_library()
        ph, pw = _pair(padding)
        dh, dw = _pair(dilation)
        if algo not in ALGOS:
            raise ValueError("algo must be one of %s" % list(ALGOS))
        self.N, self.Cx, self.Kh, self.H, self.W, self.R, self.S = (int(v) for v in (N, Cx, Kh, H, W, R, S))
        self.params = ConvParams(self.N, self.Cx + self.Kh, self.H, self.W, 4 * self.Kh, self.R, self.S, 1, 1, ph, pw,
                                 dh, dw, LAYOUTS["nchw"], DTYPES["f32"], ALGOS[algo])
        self.algo, self.padding, self.dilation = algo, (ph, pw), (dh, dw)
        self._desc = ctypes.c_void_p()
        _check(self.lib.conv_lstm_create_desc(ctypes.byref(self.params), ctypes.c_int64(self.Cx),
                                              ctypes.byref(self._desc)), "conv_lstm_create_desc")
        info = PlanInfo()
        _check(self.lib.conv_plan_info(self._desc, ctypes.byref(info)), "conv_plan_info")
        self.info: Dict[str, int] = {name: getattr(info, name) for name, _ in PlanInfo._fields_}
        self.workspace_bytes = int(self.info["ws_bytes"])

    def __del__(self):
        desc = getattr(self, "_desc", None)
        if desc is not None and desc.value:
            self.lib.conv_destroy_desc(desc)
            self._desc = None

    def _check_tensor(self, t, shape, what):
        torch = _torch()
        if tuple(t.shape) != tuple(shape):
            raise ValueError("%s has shape %s, expected %s" % (what, tuple(t.shape), tuple(shape)))
        if not t.is_contiguous() or t.dtype != torch.float32:
            raise ValueError("%s must be a contiguous float32 tensor" % what)

    def new_workspace(self, device):
        torch = _torch()
        return None if self.workspace_bytes == 0 else torch.empty(self.workspace_bytes, dtype=torch.uint8,
                                                                   device=device)

    def step(self, x, h, c, w, bias=None, h_out=None, c_out=None, ws=None, stream=None):
        """conv_lstm_step: returns (h_t, c_t)."""
        torch = _torch()
        st = (self.N, self.Kh, self.H, self.W)
        self._check_tensor(x, (self.N, self.Cx, self.H, self.W), "x")
        self._check_tensor(h, st, "h")
        self._check_tensor(c, st, "c")
        self._check_tensor(w, (4 * self.Kh, self.Cx + self.Kh, self.R, self.S), "w")
        if bias is not None:
            self._check_tensor(bias, (4 * self.Kh,), "bias")
        h_out = torch.empty(st, dtype=torch.float32, device=x.device) if h_out is None else h_out
        c_out = torch.empty(st, dtype=torch.float32, device=x.device) if c_out is None else c_out
        self._check_tensor(h_out, st, "h_out")
        self._check_tensor(c_out, st, "c_out")
        if ws is None:
            ws = self.new_workspace(x.device)
        elif ws.numel() * ws.element_size() < self.workspace_bytes:
            raise ValueError("workspace too small")
        p = Conv2d._ptr
        _check(self.lib.conv_lstm_step(self._desc, p(x), p(h), p(c), p(w), p(bias), p(h_out), p(c_out), p(ws),
                                       Conv2d._stream(stream, x.device)), "conv_lstm_step")
        return h_out, c_out


_cache: Dict[tuple, Conv2d] = {}


def descriptor(x_shape, w_shape, *, stride=1, padding=0, dilation=1, layout="nchw", dtype="f32",
               algo="im2win", plan: Optional[str] = None) -> Conv2d:
    """A cached descriptor for the given shapes, parameters and plan request
    (descriptors are immutable, so sharing one is safe)."""
    if layout == "nchw":
        N, C, H, W = x_shape
        K, C2, R, S = w_shape
    elif layout == "nhwc":
        N, H, W, C = x_shape
        K, R, S, C2 = w_shape
    else:
        raise ValueError("layout must be 'nchw' or 'nhwc'")
    if C != C2:
        raise ValueError("x has %d channels, w has %d" % (C, C2))
    key = (N, C, H, W, K, R, S, _pair(stride), _pair(padding), _pair(dilation), layout, dtype, algo, plan)
    d = _cache.get(key)
    if d is None:
        d = Conv2d(N, C, H, W, K, R, S, stride=stride, padding=padding, dilation=dilation, layout=layout,
                   dtype=dtype, algo=algo, plan=plan)
        _cache[key] = d
    return d


def conv2d(x, w, bias=None, *, stride=1, padding=0, dilation=1, layout="nchw", algo="im2win",
           out=None, ws=None, stream=None):
    """Forward convolution of device tensors x and w (layouts per ``layout``)."""
    d = descriptor(tuple(x.shape), tuple(w.shape), stride=stride, padding=padding, dilation=dilation,
                   layout=layout, dtype=_dtype_name(x), algo=algo)
    return d.forward(x, w, bias, y=out, ws=ws, stream=stream)


def status_string(status: int) -> str:
    return load_library().conv_status_string(int(status)).decode()
