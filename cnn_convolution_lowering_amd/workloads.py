"""Seeded synthetic inputs for the five convolution workloads.

This module only draws numbers: it holds no convolution arithmetic (no output
extents, no lowering, no contraction), so that both the GPU path and the fp64
reference checker can take their inputs from it without sharing any of the
method.

The pages' own data is not available: the MSCRED signals are confidential
("GPU-Accelerating MSCRED with CUDA, im2col, GEMM, and a Custom PyTorch
Extension", section "Limitations and Data-Privacy Considerations"), and the
twelve CNN layers of "Enabling Memory-efficient Im2win Convolution with
Multi-precision Support on GPU CUDA and Tensor Cores" (abstract) are not
listed.  These workloads stand in for them:

  c1  fp32 NCHW, one 3x30x30 image, 3x3 conv 3->32, stride 1, pad 1
  c2  fp32 NCHW, 1280 images of 3 symmetric 30x30 signature matrices (30
      features, as in the article's experimental setup), through four chained
      convolutions 3x3 3->32 s1 p1; 3x3 32->64 s2; 2x2 64->128 s2; 2x2 128->256 s2
  c3  fp16 NHWC, N=64, 3x3 256->256 at 14x14, stride 1, pad 1
  c4  bf16 NHWC, N=128, three independent layers: 7x7 s2 p3 3->64 at 224x224;
      1x1 1024->256 at 14x14; 3x3 512->512 p1 at 7x7
  c5  fp16 NHWC, N=32, 128->128 at 64x64, R=S in {1,3,5,7,11}, pad R//2

Recipe: ``torch.Generator('cpu').manual_seed(seed)``; every tensor is drawn in
fp32 (signature matrices in fp64) in logical NCHW / KCRS order -- the first
layer's x, then per layer (w, b), or (x, w, b) for independent layers --
rounded to the storage dtype (round-to-nearest-even), then permuted to
NHWC / KRSC where the workload says so.  x ~ U[-1, 1), w ~ N(0, sigma) with
sigma = 0.1 (c1, c2) or He-normal sqrt(2 / (C R S)) (c3-c5), b ~ N(0, 0.01).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional, Tuple

import torch

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


@dataclass
class LayerSpec:
    C: int
    K: int
    R: int
    S: int
    stride: Tuple[int, int] = (1, 1)
    padding: Tuple[int, int] = (0, 0)
    dilation: Tuple[int, int] = (1, 1)
    H: Optional[int] = None      # input extent; None when the input is the previous layer's output
    W: Optional[int] = None
    w_std: float = 0.1
    b_std: float = 0.01
    label: str = ""


@dataclass
class WorkloadSpec:
    name: str
    dtype: str
    layout: str
    N: int
    seed: int
    layers: List[LayerSpec]
    chained: bool = False        # layer i+1 consumes layer i's output
    shared_x: bool = False       # every layer reads the same x
    signature_x: bool = False    # x is 3 symmetric signature matrices per image


@dataclass
class LayerInputs:
    spec: LayerSpec
    x: Optional[torch.Tensor]    # None for chained layers after the first
    w: torch.Tensor
    b: torch.Tensor

    def __getattr__(self, name):
        # shape fields (C, K, R, S, stride, padding, dilation, label) come from the spec
        if name != "spec" and "spec" in self.__dict__:
            return getattr(self.spec, name)
        raise AttributeError(name)


@dataclass
class Workload:
    spec: WorkloadSpec
    layers: List[LayerInputs] = field(default_factory=list)

    @property
    def dtype(self) -> torch.dtype:
        return DTYPES[self.spec.dtype]


def _he(C, R, S):
    return math.sqrt(2.0 / (C * R * S))


def workload_spec(name: str, batch: Optional[int] = None) -> WorkloadSpec:
    """The named workload; ``batch`` overrides N for reduced-size test runs."""
    name = name.lower()
    if name == "c1":
        spec = WorkloadSpec("c1", "f32", "nchw", 1, 0, [
            LayerSpec(3, 32, 3, 3, (1, 1), (1, 1), H=30, W=30, w_std=0.1, label="3x3 3->32 s1p1 30x30")])
    elif name == "c2":
        spec = WorkloadSpec("c2", "f32", "nchw", 1280, 1, [
            LayerSpec(3, 32, 3, 3, (1, 1), (1, 1), H=30, W=30, w_std=0.1, label="L1 3x3 3->32 s1p1"),
            LayerSpec(32, 64, 3, 3, (2, 2), (0, 0), w_std=0.1, label="L2 3x3 32->64 s2"),
            LayerSpec(64, 128, 2, 2, (2, 2), (0, 0), w_std=0.1, label="L3 2x2 64->128 s2"),
            LayerSpec(128, 256, 2, 2, (2, 2), (0, 0), w_std=0.1, label="L4 2x2 128->256 s2"),
        ], chained=True, signature_x=True)
    elif name == "c3":
        spec = WorkloadSpec("c3", "f16", "nhwc", 64, 2, [
            LayerSpec(256, 256, 3, 3, (1, 1), (1, 1), H=14, W=14, w_std=_he(256, 3, 3),
                      label="3x3 256->256 s1p1 14x14")])
    elif name == "c4":
        spec = WorkloadSpec("c4", "bf16", "nhwc", 128, 3, [
            LayerSpec(3, 64, 7, 7, (2, 2), (3, 3), H=224, W=224, w_std=_he(3, 7, 7), label="7x7 s2p3 3->64 224x224"),
            LayerSpec(1024, 256, 1, 1, (1, 1), (0, 0), H=14, W=14, w_std=_he(1024, 1, 1), label="1x1 1024->256 14x14"),
            LayerSpec(512, 512, 3, 3, (1, 1), (1, 1), H=7, W=7, w_std=_he(512, 3, 3), label="3x3 512->512 s1p1 7x7"),
        ])
    elif name == "c5":
        spec = WorkloadSpec("c5", "f16", "nhwc", 32, 4, [
            LayerSpec(128, 128, R, R, (1, 1), (R // 2, R // 2), H=64, W=64, w_std=_he(128, R, R),
                      label="%dx%d 128->128 same 64x64" % (R, R))
            for R in (1, 3, 5, 7, 11)], shared_x=True)
    else:
        raise ValueError("unknown workload %r" % name)
    if batch is not None:
        spec.N = int(batch)
    return spec


def _to_layout_x(x: torch.Tensor, layout: str) -> torch.Tensor:
    return x.permute(0, 2, 3, 1).contiguous() if layout == "nhwc" else x.contiguous()


def _to_layout_w(w: torch.Tensor, layout: str) -> torch.Tensor:
    return w.permute(0, 2, 3, 1).contiguous() if layout == "nhwc" else w.contiguous()


def uniform(g: torch.Generator, shape, lo=-1.0, hi=1.0) -> torch.Tensor:
    return torch.rand(shape, generator=g, dtype=torch.float32) * (hi - lo) + lo


def normal(g: torch.Generator, shape, std: float) -> torch.Tensor:
    return torch.randn(shape, generator=g, dtype=torch.float32) * std


def signature_matrices(g: torch.Generator, n: int, features: int = 30,
                       widths=(10, 30, 60)) -> torch.Tensor:
    """[n, len(widths), features, features] symmetric matrices A A^T / w_c.

    Stand-in for MSCRED's multi-scale signature matrices (pairwise relations of
    ``features`` signals over windows of ``widths`` steps): for each scale c, a
    fresh A ~ U[-1, 1]^(features x w_c) per image, product taken in fp64.
    """
    out = torch.empty(n, len(widths), features, features, dtype=torch.float64)
    for c, wc in enumerate(widths):
        a = torch.rand((n, features, wc), generator=g, dtype=torch.float64) * 2.0 - 1.0
        out[:, c] = torch.bmm(a, a.transpose(1, 2)) / wc
    return out.to(torch.float32)


def make_workload(name: str, batch: Optional[int] = None) -> Workload:
    """Draw the workload's tensors on the CPU (storage dtype, workload layout)."""
    spec = workload_spec(name, batch)
    dt = DTYPES[spec.dtype]
    g = torch.Generator(device="cpu").manual_seed(spec.seed)
    wl = Workload(spec)
    x0 = None
    for i, L in enumerate(spec.layers):
        x = None
        need_x = (i == 0) or not (spec.chained or spec.shared_x)
        if need_x:
            if spec.signature_x:
                assert L.C == 3 and L.H == 30 and L.W == 30
                x = signature_matrices(g, spec.N)
            else:
                x = uniform(g, (spec.N, L.C, L.H, L.W))
            x = _to_layout_x(x.to(dt), spec.layout)
            x0 = x
        elif spec.shared_x:
            x = x0
        w = _to_layout_w(normal(g, (L.K, L.C, L.R, L.S), L.w_std).to(dt), spec.layout)
        b = normal(g, (L.K,), L.b_std).to(dt)
        wl.layers.append(LayerInputs(L, x, w, b))
    return wl

