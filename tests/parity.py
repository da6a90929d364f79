"""Comparison helpers for the GPU parity tests.

Parity rule: for every compared output, |y_gpu - y_ref| <= tol * yabs with
yabs = |b[k]| + sum |x*w| from the fp64 reference (a zero yabs demands an
exact zero).  The bound is the textbook one for a length-n dot product summed
in floating point, |fl(sum) - sum| <= gamma_n * sum |terms| (whose typical
size, about sqrt(n) * 2^-24, is at most 7.4e-6 for the longest contraction
here, n = 15488), plus one rounding of the result to the storage type, at
most 2^-8 = 3.9e-3 of |y| for bf16 (8-bit significand) and 2^-11 for fp16,
and |y| <= yabs; tol = 1e-5 for fp32 storage and 4e-3 for fp16 / bf16
storage (fp32 accumulation in both cases).
"""
from __future__ import annotations

import numpy as np
import torch

TOL = {"f32": 1e-5, "f16": 4e-3, "bf16": 4e-3}
TORCH_DT = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def dtype_name(t: torch.Tensor) -> str:
    return {torch.float32: "f32", torch.float16: "f16", torch.bfloat16: "bf16"}[t.dtype]


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def scaled_error(got: np.ndarray, ref: np.ndarray, yabs: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    diff = np.abs(got - ref)
    zero = yabs == 0
    if np.any(diff[zero] != 0):
        return float("inf")
    if not np.all(np.isfinite(got)):
        return float("inf")
    nz = ~zero
    return float(np.max(diff[nz] / yabs[nz])) if np.any(nz) else 0.0


def assert_parity(got, ref, yabs, dtype: str, what: str = ""):
    err = scaled_error(got, ref, yabs)
    assert err <= TOL[dtype], "%s: max |err|/sum|x*w| = %.3g > %.1g" % (what, err, TOL[dtype])
    return err


# ---------------------------------------------------------------- expected lowered layouts (numpy)

def padded_nchw(x_nchw: np.ndarray, ph: int, pw: int, extra_h: int, extra_w: int) -> np.ndarray:
    N, C, H, W = x_nchw.shape
    out = np.zeros((N, C, H + 2 * ph + extra_h, W + 2 * pw + extra_w), dtype=x_nchw.dtype)
    out[:, :, ph:ph + H, pw:pw + W] = x_nchw
    return out


def expected_im2win(x_nchw, R, S, P, Q, stride, pad, dil, RCp):
    """Win[n][p][j][t]: t = r*C + c < R*C -> x at (h = p*sh-ph+r*dh, w = j-pw), zero padding."""
    N, C, H, W = x_nchw.shape
    sh, sw = stride
    ph, pw = pad
    dh, dw = dil
    W_used = (Q - 1) * sw + (S - 1) * dw + 1
    xp = padded_nchw(x_nchw, ph, pw, dh * R + sh * P, W_used)
    win = np.zeros((N, P, W_used, RCp), dtype=x_nchw.dtype)
    for r in range(R):
        rows = xp[:, :, np.arange(P) * sh + r * dh, :W_used]          # N, C, P, W_used
        win[:, :, :, r * C:(r + 1) * C] = np.transpose(rows, (0, 2, 3, 1))
    return win


def expected_im2col(win, Q, S, stride_w, dil_w, RCp):
    N, P, W_used, _ = win.shape
    col = np.zeros((N, P, Q, S * RCp), dtype=win.dtype)
    for s in range(S):
        col[:, :, :, s * RCp:(s + 1) * RCp] = win[:, :, np.arange(Q) * stride_w + s * dil_w, :]
    return col.reshape(N * P * Q, S * RCp)


def expected_packed_filter(w_kcrs, RCp):
    K, C, R, S = w_kcrs.shape
    out = np.zeros((K, S, RCp), dtype=w_kcrs.dtype)
    for r in range(R):
        out[:, :, r * C:(r + 1) * C] = np.transpose(w_kcrs[:, :, r, :], (0, 2, 1))
    return out.reshape(K, S * RCp)
