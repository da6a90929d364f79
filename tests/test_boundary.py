"""Host-side checks of the C ABI: the library loads and exports what the header
declares; descriptors validate their parameters; extents, workspace sizes and
status codes follow the definitions.  No GPU needed (no compute call is made)."""
import ctypes
import itertools
import os
import zlib

import numpy as np
import pytest

import cnn_convolution_lowering_amd as cl

pytestmark = pytest.mark.skipif(not os.path.exists(cl.LIB_PATH), reason="libconvlower.so not built")


def _params(**kw):
    base = dict(N=2, C=3, H=8, W=8, K=4, R=3, S=3, stride_h=1, stride_w=1, pad_h=1, pad_w=1, dil_h=1, dil_w=1,
                layout=0, dtype=0, algo=0)
    base.update(kw)
    return cl.ConvParams(*[base[n] for n, _ in cl.ConvParams._fields_])


def _create(**kw):
    lib = cl.load_library()
    d = ctypes.c_void_p()
    st = lib.conv_create_desc(ctypes.byref(_params(**kw)), ctypes.byref(d))
    return st, d


def test_exports_every_header_function():
    lib = cl.load_library()
    names = cl.header_functions()
    assert {"conv_create_desc", "conv_workspace_size", "conv2d_fwd", "conv_destroy_desc",
            "conv_status_string", "conv_output_dims", "conv_plan_info", "conv_pack_filter",
            "conv_lower_input", "conv_contract"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_struct_sizes_match_header():
    # conv_params_t: 7 int64 + 6 int32 + 3 enums (int) -> 92 bytes, padded to 96
    assert ctypes.sizeof(cl.ConvParams) == 96
    # conv_plan_info_t: 7 int64 + 7 uint64 + 7 int32 (140, padded to 144),
    # then 2 uint64 + 1 int32 -> 164, padded to 168
    assert ctypes.sizeof(cl.PlanInfo) == 168


@pytest.mark.parametrize("field,value", [
    ("N", -1), ("C", 0), ("H", 0), ("W", -3), ("K", 0), ("R", 0), ("S", -1),
    ("stride_h", 0), ("stride_w", -1), ("dil_h", 0), ("dil_w", -2), ("pad_h", -1), ("pad_w", -1),
    ("layout", 2), ("dtype", 3), ("algo", 3)])
def test_invalid_params(field, value):
    st, d = _create(**{field: value})
    assert st == -1 and not d.value


def test_kernel_larger_than_padded_input():
    st, _ = _create(H=2, W=8, R=3, pad_h=0)
    assert st == -1
    st, _ = _create(H=8, W=4, S=3, dil_w=2, pad_w=0)
    assert st == -1
    st, d = _create(H=2, W=2, R=3, S=3, pad_h=1, pad_w=1)     # exactly fits
    assert st == 0
    cl.load_library().conv_destroy_desc(d)


def test_null_pointers():
    lib = cl.load_library()
    assert lib.conv_create_desc(None, ctypes.byref(ctypes.c_void_p())) == -3
    assert lib.conv_create_desc(ctypes.byref(_params()), None) == -3
    st, d = _create()
    assert lib.conv_workspace_size(d, None) == -3
    assert lib.conv_output_dims(d, None, None) == -3
    assert lib.conv_plan_info(d, None) == -3
    lib.conv_destroy_desc(d)
    assert lib.conv_destroy_desc(None) == 0


def test_foreign_handle_rejected():
    lib = cl.load_library()
    junk = ctypes.create_string_buffer(512)
    h = ctypes.c_void_p(ctypes.addressof(junk))
    size = ctypes.c_size_t()
    assert lib.conv_workspace_size(h, ctypes.byref(size)) == -1
    assert lib.conv2d_fwd(h, None, None, None, None, None, None) == -1
    assert lib.conv_destroy_desc(h) == -1


def test_too_large_is_unsupported():
    st, _ = _create(N=1 << 31)
    assert st == -2
    st, _ = _create(N=4096, C=1024, H=1024, W=1024, K=64, R=11, S=11, pad_h=5, pad_w=5, algo=1)
    assert st == -2


def test_status_strings():
    for code in cl.STATUS:
        assert cl.status_string(code)
    assert cl.status_string(99) == "unknown status"


def test_null_and_misaligned_pointers_rejected_before_any_launch():
    lib = cl.load_library()
    st, d = _create()
    # NULL tensors
    assert lib.conv2d_fwd(d, None, None, None, None, None, None) == -3
    # misaligned (checked before the device query)
    assert lib.conv2d_fwd(d, ctypes.c_void_p(0x1004), ctypes.c_void_p(0x2000), None, ctypes.c_void_p(0x3000),
                          ctypes.c_void_p(0x4000), None) == -5
    lib.conv_destroy_desc(d)


def test_empty_batch_needs_nothing():
    lib = cl.load_library()
    st, d = _create(N=0)
    assert st == 0
    size = ctypes.c_size_t(123)
    assert lib.conv_workspace_size(d, ctypes.byref(size)) == 0 and size.value == 0
    assert lib.conv2d_fwd(d, None, None, None, None, None, None) == 0
    lib.conv_destroy_desc(d)


def _expect_extent(size, pad, dil, ks, stride):
    return len(range(0, size + 2 * pad - dil * (ks - 1), stride))


def test_output_dims_match_enumeration_and_oracle(oracle_mod):
    rng = np.random.default_rng(0)
    n = 0
    while n < 200:
        H, W = (int(v) for v in rng.integers(1, 40, size=2))
        R, S = (int(v) for v in rng.integers(1, 8, size=2))
        sh, sw, dh, dw = (int(v) for v in rng.integers(1, 4, size=4))
        ph, pw = (int(v) for v in rng.integers(0, 4, size=2))
        if H + 2 * ph < dh * (R - 1) + 1 or W + 2 * pw < dw * (S - 1) + 1:
            continue
        n += 1
        c = cl.Conv2d(1, 2, H, W, 3, R, S, stride=(sh, sw), padding=(ph, pw), dilation=(dh, dw))
        want = (_expect_extent(H, ph, dh, R, sh), _expect_extent(W, pw, dw, S, sw))
        assert (c.P, c.Q) == want
        assert (c.P, c.Q) == oracle_mod.output_dims((1, 2, H, W), (3, 2, R, S), stride=(sh, sw),
                                                     padding=(ph, pw), dilation=(dh, dw))


def _round_up(v, a):
    return (v + a - 1) // a * a


@pytest.mark.parametrize("layout,dtype,algo", list(itertools.product(["nchw", "nhwc"], ["f32", "f16", "bf16"],
                                                                       ["im2win", "im2col"])))
def test_workspace_formula(layout, dtype, algo):
    rng = np.random.default_rng(zlib.crc32((layout + dtype + algo).encode()))
    elem = 4 if dtype == "f32" else 2
    vec = 16 // elem
    for _ in range(40):
        N, C, K = int(rng.integers(1, 5)), int(rng.integers(1, 40)), int(rng.integers(1, 70))
        R, S = int(rng.integers(1, 6)), int(rng.integers(1, 6))
        H, W = int(rng.integers(R, 20)), int(rng.integers(S, 20))
        st = (int(rng.integers(1, 3)), int(rng.integers(1, 3)))
        pd = (int(rng.integers(0, 3)), int(rng.integers(0, 3)))
        c = cl.Conv2d(N, C, H, W, K, R, S, stride=st, padding=pd, layout=layout, dtype=dtype, algo=algo)
        P, Q = c.P, c.Q
        # fp32 window rows that are not whole vectors are stored unpadded
        RCp = R * C if dtype == "f32" and (R * C) % vec else _round_up(R * C, vec)
        Kl = S * RCp
        W_used = (Q - 1) * st[1] + S
        info = c.info
        assert info["RCp"] == RCp and info["Kl"] == Kl and info["W_used"] == W_used
        assert info["M"] == N * P * Q and info["Kg"] == C * R * S
        assert info["im2col_bytes"] == N * P * Q * C * R * S * elem
        assert info["im2win_bytes"] == N * P * W_used * RCp * elem
        elided = layout == "nhwc" and R == 1 and S == 1 and pd == (0, 0) and C % vec == 0
        assert info["lowering_elided"] == int(elided)
        packed = not (layout == "nhwc" and C % vec == 0 and (R == 1 or S == 1))
        assert info["ws_filter_bytes"] == (K * Kl * elem if packed else 0)
        low = 0 if elided else (N * P * W_used * RCp * elem if algo == "im2win" else N * P * Q * Kl * elem)
        assert info["ws_lowered_bytes"] == low
        assert info["ws_lowered_offset"] % 256 == 0
        assert c.workspace_bytes >= info["ws_filter_bytes"] + low
        if info["ksplit"] > 1:   # split contraction: the fp32 partials go last
            assert info["ws_partial_offset"] >= info["ws_lowered_offset"] + low
            assert c.workspace_bytes == info["ws_partial_offset"] + info["ws_partial_bytes"]
        elif low:
            assert c.workspace_bytes == info["ws_lowered_offset"] + low


def test_workload_workspace_ratios():
    """im2win strip bytes / explicit-im2col bytes per layer of the five workloads.

    Expected values worked out from the shapes: ratio = W_used*RCp / (Q*C*R*S),
    0 where a 1x1 layer is read in place; the fp32 3-channel layers' window
    rows are unpadded (RCp = R*C = 9), so c1 is 32*9 / (30*27) = 35.6 %."""
    from cnn_convolution_lowering_amd.workloads import workload_spec
    want = {
        "c1": [32 * 9 / (30 * 27)],
        "c2": [32 * 9 / (30 * 27), 29 * 96 / (14 * 288), 14 * 128 / (7 * 256), 6 * 256 / (3 * 512)],
        "c3": [16 * 768 / (14 * 2304)],
        "c4": [229 * 24 / (112 * 147), 0.0, 9 * 1536 / (7 * 4608)],
        "c5": [0.0, 66 * 384 / (64 * 1152), 68 * 640 / (64 * 3200), 70 * 896 / (64 * 6272),
               74 * 1408 / (64 * 15488)],
    }
    for name, expect in want.items():
        spec = workload_spec(name)
        H = W = None
        got = []
        for L in spec.layers:
            if L.H is not None:
                H, W = L.H, L.W
            c = cl.Conv2d(spec.N, L.C, H, W, L.K, L.R, L.S, stride=L.stride, padding=L.padding,
                          layout=spec.layout, dtype=spec.dtype)
            got.append(c.info["ws_lowered_bytes"] / c.info["im2col_bytes"])
            if spec.chained:
                H, W = c.P, c.Q
        np.testing.assert_allclose(got, expect, rtol=1e-12, err_msg=name)


@pytest.mark.parametrize("layout", ["nchw", "nhwc"])
@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_implicit_needs_no_workspace(layout, dtype):
    """The fused path never lowers x: no lowered workspace.  The only
    workspace it may take is the filter copy in MFMA fragment order of the
    register-streamed kernels (K rounded up to 16 or 32, times C*R*S), or of
    the 16-bit NHWC small-window kernel (at most 64 channels by R filter
    rows of ceil((S*C + 1) / 8) 8-element chunks, rounded up to 4 chunks)."""
    for (C, R, S, st, pd) in [(3, 7, 7, 2, 3), (32, 3, 3, 2, 0), (128, 1, 1, 1, 0), (5, 2, 3, 1, 1)]:
        c = cl.Conv2d(4, C, 20, 20, 16, R, S, stride=st, padding=pd, layout=layout, dtype=dtype, algo="implicit")
        assert c.info["ws_lowered_bytes"] == 0 and c.info["lowering_elided"] == 1
        # besides the filter copy, a split contraction's fp32 partials (not lowered input)
        part = c.info["ws_partial_bytes"]
        assert c.info["kernel"] != 9   # stream-K only when named
        assert part == (c.info["ksplit"] * c.info["M"] * 16 * 4 if c.info["ksplit"] > 1 else 0)
        assert c.workspace_bytes == (c.info["ws_partial_offset"] + part if part else c.info["ws_filter_bytes"])
        elem = {"f32": 4, "f16": 2, "bf16": 2}[dtype]
        if c.info["kernel"] == 8:
            assert layout == "nhwc" and dtype != "f32" and C * st % 2 == 0
            chunks = R * ((S * C + 1 + 7) // 8)
            assert 0 < c.info["ws_filter_bytes"] <= 64 * 8 * 4 * ((chunks + 3) // 4) * elem
        else:
            assert c.info["ws_filter_bytes"] <= 32 * C * R * S * elem
            if C % 16 and not part:
                assert c.workspace_bytes == 0


def test_elided_layers_use_no_lowering_workspace():
    c = cl.Conv2d(128, 1024, 14, 14, 256, 1, 1, layout="nhwc", dtype="bf16")
    assert c.info["lowering_elided"] == 1 and c.workspace_bytes == 0
    # named stream-K: its sum slots are the only workspace
    c = cl.Conv2d(128, 1024, 14, 14, 256, 1, 1, layout="nhwc", dtype="bf16", plan="streamk:8")
    assert c.info["kernel"] == 9 and c.info["ws_lowered_bytes"] == 0
    assert c.workspace_bytes == c.info["ws_partial_offset"] + c.info["ws_partial_bytes"]
    c = cl.Conv2d(32, 128, 64, 64, 128, 1, 1, layout="nhwc", dtype="f16", algo="im2col")
    assert c.workspace_bytes == 0


def test_kernel_override_is_host_only_and_checked(monkeypatch):
    """conv_create_desc_forced takes a compiled kernel variant only where that
    kernel takes the shape; otherwise (or when malformed) the planner's choice
    stays.  conv_create_desc never reads the environment."""
    def plan(force=None, **kw):
        args = dict(N=2, C=64, H=17, W=17, K=72, R=3, S=3, padding=1, layout="nhwc", dtype="f16", algo="implicit")
        args.update(kw)
        N, C, H, W, K, R, S = (args.pop(k) for k in ("N", "C", "H", "W", "K", "R", "S"))
        d = cl.Conv2d(N, C, H, W, K, R, S, plan=force, **args)
        return d.info["kernel"], d.info["kernel_variant"], d.info["tile_m"], d.info["tile_n"]

    default = plan()
    monkeypatch.setenv("CONVLOWER_KERNEL", "strip:0")      # the old override: ignored
    assert plan() == default
    monkeypatch.delenv("CONVLOWER_KERNEL")
    assert plan("strip:0")[:3] == (4, 0, 512)
    assert plan("strip:0", R=1, S=1, padding=0)[0] != 4       # a single tap: nothing to share
    assert plan("strip:0", C=48)[0] != 4                       # C not a multiple of 32
    assert plan("strip:0", dtype="f32")[0] != 4                # 16-bit only
    assert plan("wide:2")[:4] == (2, 2, 256, 256)
    assert plan("nchw:1")[0] != 3                              # fp32 NCHW only
    assert plan("nchw:1", layout="nchw", dtype="f32")[:2] == (3, 1)
    for bad in ("strip", "strip:99", "bogus:1", ":", "dma:-1", ""):
        assert plan(bad) == default
    # the cache of shared descriptors keeps forced and default plans apart
    a = cl.descriptor((2, 17, 17, 64), (72, 3, 3, 64), padding=1, layout="nhwc", dtype="f16", algo="implicit")
    b = cl.descriptor((2, 17, 17, 64), (72, 3, 3, 64), padding=1, layout="nhwc", dtype="f16", algo="implicit",
                      plan="wide:2")
    assert a is not b and a.info["kernel"] == default[0] and b.info["kernel"] == 2


def test_lstm_descriptor_validation_and_entry_separation():
    """ConvLSTM descriptors: sizes checked on the host; the plain-convolution
    entry points and conv_lstm_step reject each other's descriptors before
    touching any pointer."""
    import ctypes
    lib = cl.load_library()
    cell = cl.ConvLSTMCell(2, 32, 32, 30, 30, 3, 3, padding=1)
    assert cell.info["ws_lowered_bytes"] > 0 and cell.info["ws_filter_bytes"] == 128 * 64 * 9 * 4
    fake = ctypes.c_void_p(1 << 20)
    assert lib.conv2d_fwd(cell._desc, fake, fake, None, fake, fake, None) == -1
    plain = cl.Conv2d(2, 64, 30, 30, 128, 3, 3, padding=1, layout="nchw", dtype="f32")
    assert lib.conv_lstm_step(plain.handle, fake, fake, fake, fake, None, fake, fake, fake, None) == -1
    bad = [dict(Kh=8), dict(pad=0), dict(algo="implicit")]
    for b in bad:
        kw = dict(Kh=32, pad=1, algo="im2win")
        kw.update(b)
        with pytest.raises(cl.ConvError):
            cl.ConvLSTMCell(2, 32, kw["Kh"], 30, 30, 3, 3, padding=kw["pad"], algo=kw["algo"])
    p = cl.ConvParams(2, 64, 30, 30, 128, 3, 3, 1, 1, 1, 1, 1, 1, 0, 0, 0)
    d = ctypes.c_void_p()
    assert lib.conv_lstm_create_desc(ctypes.byref(p), 31, ctypes.byref(d)) == -1   # C != c_x + K/4
    p.layout = 1
    assert lib.conv_lstm_create_desc(ctypes.byref(p), 32, ctypes.byref(d)) == -2   # NHWC unsupported


def test_tune_argument_checks_on_the_host():
    import ctypes
    lib = cl.load_library()
    d = cl.Conv2d(2, 16, 8, 8, 16, 3, 3, padding=1, layout="nchw", dtype="f32")
    res = cl.TuneResult()
    fake = ctypes.c_void_p(1 << 20)
    out = ctypes.c_void_p(123)
    assert lib.conv_tune(d.handle, fake, fake, None, fake, fake, 1 << 30, 0, None, ctypes.byref(out),
                         ctypes.byref(res)) == -1
    assert not out.value                                     # cleared on every error
    assert lib.conv_tune(d.handle, fake, fake, None, fake, fake, 1 << 30, 3, None, ctypes.byref(out), None) == -3
    assert lib.conv_tune(d.handle, fake, fake, None, fake, fake, 1 << 30, 3, None, None, ctypes.byref(res)) == -3
    cell = cl.ConvLSTMCell(2, 16, 16, 8, 8, 3, 3, padding=1)
    assert lib.conv_tune(cell._desc, fake, fake, None, fake, fake, 1 << 30, 3, None, ctypes.byref(out),
                         ctypes.byref(res)) == -1
    empty = cl.Conv2d(0, 16, 8, 8, 16, 3, 3, padding=1, layout="nchw", dtype="f32")
    assert lib.conv_tune(empty.handle, None, None, None, None, None, 0, 3, None, ctypes.byref(out),
                         ctypes.byref(res)) == 0
    assert out.value and out.value != empty.handle.value     # a new descriptor, same plan
    info = cl.PlanInfo()
    assert lib.conv_plan_info(out, ctypes.byref(info)) == 0
    assert (res.kernel, res.kernel_variant) == (empty.info["kernel"], empty.info["kernel_variant"])
    assert (info.kernel, info.kernel_variant) == (res.kernel, res.kernel_variant)
    assert res.ksplit == empty.info["ksplit"] == 1
    assert lib.conv_destroy_desc(out) == 0

def test_split_contraction_plan():
    """The pipelined kernel splits the contraction in two when the output
    tiles leave most CUs idle or the contraction is very long; the fp32
    partials take ksplit*M*K*4 bytes after the other workspace parts,
    256-byte aligned, and a forced split is honoured (within the contraction
    tiles, every split non-empty)."""
    for a in [(32, 512, 7, 7, 512, 3, 3, 1), (8, 192, 20, 20, 96, 3, 3, 1)]:
        # 4608-long over 100 tiles of 64 x 128; 50 tiles
        c = cl.Conv2d(*a[:7], padding=a[7], layout="nhwc", dtype="bf16", algo="implicit")
        i = c.info
        assert i["kernel"] == 1 and i["ksplit"] == 2, a
        assert i["ws_lowered_bytes"] == 0 and i["ws_partial_bytes"] == 2 * i["M"] * a[4] * 4
        assert i["ws_partial_offset"] % 256 == 0
        assert i["ws_partial_offset"] >= i["ws_filter_offset"] + i["ws_filter_bytes"]
        assert c.workspace_bytes == i["ws_partial_offset"] + i["ws_partial_bytes"]
    # plenty of output tiles, 196 tiles of 128 x 128 taken in one round of the
    # four-stage tiles (a contraction of moderate length or a 4608-long one),
    # or a short contraction: no split
    for a in [(32, 128, 64, 64, 128, 3, 3, 1), (128, 1024, 14, 14, 256, 1, 1, 0), (2, 32, 8, 8, 32, 1, 1, 0),
              (64, 256, 14, 14, 256, 3, 3, 1), (128, 512, 7, 7, 512, 3, 3, 1)]:
        for algo in ("implicit", "im2win", "im2col"):
            c = cl.Conv2d(*a[:7], padding=a[7], layout="nhwc", dtype="f16", algo=algo)
            assert c.info["ksplit"] == 1 and c.info["ws_partial_bytes"] == 0, (a, algo)
    # im2win keeps its lowered part and adds the partials after it
    c = cl.Conv2d(8, 192, 20, 20, 96, 3, 3, padding=1, layout="nhwc", dtype="f16", algo="im2win")
    i = c.info
    if i["ksplit"] > 1:
        assert i["ws_partial_offset"] >= i["ws_lowered_offset"] + i["ws_lowered_bytes"]
    # forced: honoured, clamped to the contraction tiles
    c = cl.Conv2d(2, 64, 17, 17, 72, 3, 3, padding=1, layout="nhwc", dtype="f16", algo="implicit", plan="dma:1:3")
    assert c.info["ksplit"] == 3 and c.info["ws_partial_bytes"] == 3 * c.info["M"] * 72 * 4
    c = cl.Conv2d(2, 16, 9, 9, 24, 1, 1, layout="nhwc", dtype="f16", algo="implicit", plan="dma:1:8")  # one tile
    assert c.info["ksplit"] == 1 and c.info["ws_partial_bytes"] == 0
    # the ConvLSTM step never splits
    cell = cl.ConvLSTMCell(4, 32, 32, 30, 30, 3, 3, padding=1, algo="im2win")
    assert cell.info["ksplit"] == 1 and cell.info["ws_partial_bytes"] == 0


def test_peak_library_exports_and_host_checks():
    """libconvpeak.so (the measured-peak microbenchmarks) exports what
    include/convpeak.h declares; its argument checks run on the host."""
    import re
    from cnn_convolution_lowering_amd import peak
    if not os.path.exists(peak.PEAK_LIB_PATH):
        pytest.skip("libconvpeak.so not built")
    lib = peak.load_peak_library()
    with open(peak.PEAK_HEADER_PATH) as f:
        text = re.sub(r"/\*.*?\*/", " ", f.read(), flags=re.S)
    names = set(re.findall(r"^\s*(?:const\s+)?[a-z0-9_]+\**\s+\**\s*(convpeak\w*)\s*\(", text, flags=re.M))
    assert names == {"convpeak_mfma_flops_per_iter", "convpeak_mfma", "convpeak_wall_clock_khz", "convpeak_copy"}
    for n in names:
        assert hasattr(lib, n), n
    # flops per loop iteration: the instruction's M*N*K*2 times the accumulators per iteration
    assert lib.convpeak_mfma_flops_per_iter(0) == 2 * 16 * 16 * 4 * 8
    assert lib.convpeak_mfma_flops_per_iter(1) == lib.convpeak_mfma_flops_per_iter(2) == 2 * 32 * 32 * 16 * 4
    assert lib.convpeak_mfma_flops_per_iter(3) == lib.convpeak_mfma_flops_per_iter(4) == 2 * 16 * 16 * 32 * 8
    assert lib.convpeak_mfma_flops_per_iter(5) == 0
    fake = ctypes.c_void_p(1 << 20)
    assert lib.convpeak_mfma(1, 0, 4, fake, None) == -1          # iters < 1
    assert lib.convpeak_mfma(1, 10, 0, fake, None) == -1         # no blocks
    assert lib.convpeak_mfma(9, 10, 4, fake, None) == -1         # unknown instruction
    assert lib.convpeak_mfma(1, 10, 4, None, None) == -1         # no clock buffer
    assert lib.convpeak_copy(fake, ctypes.c_void_p((1 << 20) + 4096), 24, None) == -1   # not a multiple of 16
    assert lib.convpeak_copy(ctypes.c_void_p((1 << 20) + 8), fake, 32, None) == -1      # misaligned
    assert lib.convpeak_copy(fake, ctypes.c_void_p((1 << 20) + 16), 64, None) == -1    # overlapping
    assert lib.convpeak_copy(fake, ctypes.c_void_p(1 << 24), 0, None) == 0             # nothing to copy


def test_streamk_plan():
    """Stream-K is taken only when named ("streamk:8", the 128 x 128
    pipelined tiles with early issue) and where its operands allow it; its
    workspace's partial area is one fp32 tile slot and one flag per workgroup
    of a grid of min(tile steps, 512), after the other parts.  The default
    plan of the same layers is the plain pipeline."""
    cases = [((64, 256, 14, 14, 256, 3, 3, 1), "f16", 196 * 36), ((128, 512, 7, 7, 512, 3, 3, 1), "bf16", 196 * 72),
             ((128, 1024, 14, 14, 256, 1, 1, 0), "bf16", 392 * 16)]
    for a, dt, units in cases:
        for algo in ("implicit", "im2win", "im2col"):
            c = cl.Conv2d(*a[:7], padding=a[7], layout="nhwc", dtype=dt, algo=algo)
            assert c.info["kernel"] == 1, (a, algo)
            c = cl.Conv2d(*a[:7], padding=a[7], layout="nhwc", dtype=dt, algo=algo, plan="streamk:8")
            i = c.info
            assert (i["kernel"], i["kernel_variant"], i["ksplit"]) == (9, 8, 1), (a, algo)
            grid = min(units, 512)
            assert i["ws_partial_bytes"] == grid * 128 * 128 * 4 + grid * 4
            assert i["ws_partial_offset"] % 256 == 0
            assert c.workspace_bytes == i["ws_partial_offset"] + i["ws_partial_bytes"]
            low = i["ws_lowered_bytes"]
            if low:
                assert i["ws_partial_offset"] >= i["ws_lowered_offset"] + low
    c = cl.Conv2d(32, 128, 64, 64, 128, 3, 3, padding=1, layout="nhwc", dtype="f16", algo="implicit")
    assert c.info["kernel"] == 13 and c.info["ws_partial_bytes"] == 0   # the LDS-shared-filter strip kernel
    c = cl.Conv2d(64, 256, 14, 14, 256, 3, 3, padding=1, layout="nhwc", dtype="f16", algo="implicit", plan="dma:8")
    assert (c.info["kernel"], c.info["ksplit"], c.info["ws_partial_bytes"]) == (1, 1, 0)
    c = cl.Conv2d(2, 64, 17, 17, 72, 3, 3, padding=1, layout="nhwc", dtype="f16", algo="implicit", plan="streamk:8")
    assert c.info["kernel"] == 9 and c.info["ws_partial_bytes"] == 5 * 9 * 128 * 128 * 4 + 5 * 9 * 4
    # windows whose channels are not whole 64-element stage blocks, fp32 NCHW windows, other shapes: not taken
    for kw in (dict(C=96), dict(layout="nchw", dtype="f32")):
        args = dict(C=64, layout="nhwc", dtype="f16")
        args.update(kw)
        c = cl.Conv2d(2, args["C"], 17, 17, 72, 3, 3, padding=1, layout=args["layout"], dtype=args["dtype"],
                      algo="implicit", plan="streamk:8")
        assert c.info["kernel"] != 9, kw
    for v in (0, 7, 9, 10, 11, 12, 13):
        c = cl.Conv2d(2, 64, 17, 17, 72, 3, 3, padding=1, layout="nhwc", dtype="f16", algo="implicit",
                      plan="streamk:%d" % v)
        assert c.info["kernel"] != 9, v


def test_tile_order_plan():
    """The pipelined kernel's tile order is the fourth field of a forced plan
    and defaults to XCD ranges in serpentine order (2), column-major ranges
    (3) for the one-round 128 x 128 tiles; other kernels ignore it."""
    a = (64, 256, 14, 14, 256, 3, 3)
    c = cl.Conv2d(*a, padding=1, layout="nhwc", dtype="f16", algo="implicit")
    assert (c.info["kernel"], c.info["kernel_variant"], c.info["tile_order"]) == (1, 12, 3)
    c = cl.Conv2d(*a, padding=1, layout="nhwc", dtype="f16", algo="implicit", plan="dma:12:1")
    assert c.info["tile_order"] == 3
    c = cl.Conv2d(128, 1024, 14, 14, 256, 1, 1, layout="nhwc", dtype="bf16", algo="implicit")
    assert (c.info["kernel"], c.info["kernel_variant"], c.info["tile_order"]) == (1, 13, 2)
    c = cl.Conv2d(*a, padding=1, layout="nhwc", dtype="f16", algo="implicit", plan="dma:8:1")
    assert c.info["tile_order"] == 2
    for o in range(4):
        c = cl.Conv2d(*a, padding=1, layout="nhwc", dtype="f16", algo="implicit", plan="dma:8:1:%d" % o)
        assert (c.info["kernel"], c.info["kernel_variant"], c.info["ksplit"], c.info["tile_order"]) == (1, 8, 1, o)
    c = cl.Conv2d(*a, padding=1, layout="nhwc", dtype="f16", algo="implicit", plan="dma:8:2:3")
    assert (c.info["ksplit"], c.info["tile_order"]) == (2, 3)
    for bad in ("dma:8:1:4", "dma:8:1:-1"):
        c = cl.Conv2d(*a, padding=1, layout="nhwc", dtype="f16", algo="implicit", plan=bad)
        assert c.info["tile_order"] == 2, bad
    c = cl.Conv2d(32, 128, 64, 64, 128, 11, 11, padding=5, layout="nhwc", dtype="f16", algo="implicit",
                  plan="striprb:5:1:2")
    assert c.info["kernel"] == 5 and c.info["tile_order"] == 0


def test_tap_plane_plan():
    """fp32 NCHW with C a multiple of 16: 3-wide filters without horizontal
    padding stay on the row-strip kernel (6); 2-wide filters, and 2- or
    3-wide filters with padded columns (which the row strips cannot take),
    go to the tap-plane kernel (11) with its packed filter in the workspace;
    other widths are not compiled there, and a forced plan checks the width."""
    def plan(N, C, H, W, K, R, S, st, pd, forced=None):
        c = cl.Conv2d(N, C, H, W, K, R, S, stride=st, padding=pd, layout="nchw", dtype="f32", algo="implicit",
                      plan=forced)
        return c.info["kernel"], c.info["kernel_variant"], c.info["ws_bytes"]
    assert plan(1280, 32, 30, 30, 64, 3, 3, 2, 0)[0] == 6
    assert plan(1280, 64, 14, 14, 128, 2, 2, 2, 0)[:2] == (11, 5)
    assert plan(1280, 128, 7, 7, 256, 2, 2, 2, 0)[:2] == (11, 3)
    k, v, ws = plan(64, 64, 28, 28, 64, 3, 3, 1, 1)
    assert (k, v) == (11, 3) and ws == 64 * 64 * 9 * 4   # the fp32 fragment copy, K padded to 16
    assert plan(32, 128, 28, 28, 128, 3, 3, 1, 1)[:2] == (11, 5)
    assert plan(8, 32, 20, 20, 64, 5, 5, 1, 2)[0] != 11          # width 5: not compiled
    assert plan(8, 24, 20, 20, 64, 3, 3, 1, 1)[0] != 11          # C not a multiple of 16
    assert plan(8, 32, 20, 20, 64, 5, 5, 1, 2, "nchwtaps:0")[0] != 11
    for v in range(6):
        assert plan(8, 32, 20, 20, 64, 3, 3, 1, 1, "nchwtaps:%d" % v)[:2] == (11, v)
