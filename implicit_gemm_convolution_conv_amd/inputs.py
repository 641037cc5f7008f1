"""Seeded synthetic inputs for the convolution workloads.

This module only draws random tensors (torch generators, fp32 draws rounded to
bf16 by torch) and names the workload shapes. It holds none of the
convolution's arithmetic and imports neither the product library nor the
oracle, so both sides of every parity check can take their inputs from here.

Workloads (shapes and distributions as the FlyDSL and MIOpen pages measure
them; the draws themselves are synthetic):

* ``c1``  conv3d bf16, N=1 C=64 D=4 H=W=16, K=64, 3x3x3, stride 1, pad 1;
  x, w ~ U(-1, 1).
* ``c2``  point-output patch-embed conv2d bf16 (MIOpen PR #10912 measurement):
  N=9500 C=3 H=W=14, K=1280, filter 14x14, stride 14, pad 0 -> one GEMM
  9500 x 1280 x 588; x, w ~ N(0, 1).
* ``c3``  conv3d bf16, N=1 C=2048 D=60 H=80 W=45, K=2048, 3x3x3, stride 1,
  pad 1 (FlyDSL PR #860 headline shape, M = 216000); x ~ N(0, 1) stored
  NDHWC, w ~ N(0, 1/sqrt(C*27)).
* ``c4``  the c3 shape in fp8-e4m3: x drawn NCDHW bf16, packed to fp8 NDHWC
  with a per-tensor scale.
* ``c4t`` c4's temporal 3x1x1 variant, pad (1, 0, 0); w ~ N(0, 1/sqrt(3C)).
* ``c5``  large conv3d bf16 (x and y above 2^31 elements): N=1 C=1024 D=240
  H=160 W=90, K=1024, 3x1x1, pad (1, 0, 0); x ~ U(-1, 1),
  w ~ N(0, 1/sqrt(3C)).
* ``c3s`` one GPU's share of c3 split 8 ways over output channels: the c3
  activations with a 256-channel filter slice (no exchange between GPUs).
* ``c5s`` one GPU's share of c5 split 8 ways over time: 30 output planes,
  read from 32 input planes (its 30 plus the (T - 1) * dd = 2 halo planes a
  neighbour would send), no padding (an interior shard).
* ``pw``  1x1x1 conv3d bf16 on NCDHW activations, C=512 -> K=48 over
  D=240 H=320 W=180 (14 GB of activations): the shape the FlyDSL page's
  1x1x1 measurement implies (its description gives the 14 GB A operand and
  K=48); x ~ N(0, 1), w ~ N(0, 1/sqrt(C)).

"N(0, 1/sqrt(R))" is read as standard deviation 1/sqrt(R).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch


@dataclass(frozen=True)
class Workload:
    name: str
    x_shape: tuple  # (N, C, D, H, W), logical
    w_shape: tuple  # (K, C, T, R, S)
    stride: tuple = (1, 1, 1)
    pad: tuple = (0, 0, 0)
    dil: tuple = (1, 1, 1)
    dtype: str = "bf16"  # arithmetic the conv runs in: "bf16" or "fp8"
    x_layout: str = "NCDHW"  # memory layout x is drawn in
    x_dist: tuple = ("uniform", 1.0)  # ("uniform", a) = U(-a, a); ("normal", sigma)
    w_dist: tuple = ("uniform", 1.0)
    seed: int = 0
    note: str = field(default="", compare=False)

    @property
    def reduction(self) -> int:
        k, c, t, r, s = self.w_shape
        return c * t * r * s


def _R(c, t, r, s):
    return c * t * r * s


WORKLOADS = {
    "c1": Workload("c1", (1, 64, 4, 16, 16), (64, 64, 3, 3, 3), pad=(1, 1, 1),
                   x_dist=("uniform", 1.0), w_dist=("uniform", 1.0), seed=1,
                   note="conv3d fwd bf16 N=1 C=64 D=4 H=16 W=16 K=64 3x3x3 s1 p1"),
    "c2": Workload("c2", (9500, 3, 1, 14, 14), (1280, 3, 1, 14, 14), stride=(1, 14, 14),
                   x_dist=("normal", 1.0), w_dist=("normal", 1.0), seed=2,
                   note="point-output patch-embed conv2d fwd bf16 N=9500 C=3 H=W=14 K=1280 14x14 s14"),
    "c3": Workload("c3", (1, 2048, 60, 80, 45), (2048, 2048, 3, 3, 3), pad=(1, 1, 1), x_layout="NDHWC",
                   x_dist=("normal", 1.0), w_dist=("normal", 1.0 / math.sqrt(_R(2048, 3, 3, 3))), seed=3,
                   note="conv3d fwd bf16 NDHWC N=1 C=2048 D=60 H=80 W=45 K=2048 3x3x3 s1 p1"),
    "c4": Workload("c4", (1, 2048, 60, 80, 45), (2048, 2048, 3, 3, 3), pad=(1, 1, 1), dtype="fp8",
                   x_dist=("normal", 1.0), w_dist=("normal", 1.0 / math.sqrt(_R(2048, 3, 3, 3))), seed=4,
                   note="conv3d fwd fp8-e4m3 N=1 C=2048 D=60 H=80 W=45 K=2048 3x3x3 s1 p1"),
    "c4t": Workload("c4t", (1, 2048, 60, 80, 45), (2048, 2048, 3, 1, 1), pad=(1, 0, 0), dtype="fp8",
                    x_dist=("normal", 1.0), w_dist=("normal", 1.0 / math.sqrt(_R(2048, 3, 1, 1))), seed=4,
                    note="conv3d fwd fp8-e4m3 N=1 C=2048 D=60 H=80 W=45 K=2048 3x1x1 pad (1,0,0)"),
    "c5": Workload("c5", (1, 1024, 240, 160, 90), (1024, 1024, 3, 1, 1), pad=(1, 0, 0),
                   x_dist=("uniform", 1.0), w_dist=("normal", 1.0 / math.sqrt(_R(1024, 3, 1, 1))), seed=5,
                   note="large conv3d fwd bf16 N=1 C=1024 D=240 H=160 W=90 K=1024 3x1x1 pad (1,0,0)"),
    "c3s": Workload("c3s", (1, 2048, 60, 80, 45), (256, 2048, 3, 3, 3), pad=(1, 1, 1), x_layout="NDHWC",
                    x_dist=("normal", 1.0), w_dist=("normal", 1.0 / math.sqrt(_R(2048, 3, 3, 3))), seed=3,
                    note="c3 share of one of 8 GPUs (output channels 256 of 2048): conv3d fwd bf16 NDHWC "
                         "N=1 C=2048 D=60 H=80 W=45 K=256 3x3x3 s1 p1"),
    "c5s": Workload("c5s", (1, 1024, 32, 160, 90), (1024, 1024, 3, 1, 1),
                    x_dist=("uniform", 1.0), w_dist=("normal", 1.0 / math.sqrt(_R(1024, 3, 1, 1))), seed=5,
                    note="c5 share of one of 8 GPUs (30 of 240 output planes, 2 halo planes): conv3d fwd bf16 "
                         "N=1 C=1024 D=32 H=160 W=90 K=1024 3x1x1 pad 0"),
    "pw": Workload("pw", (1, 512, 240, 320, 180), (48, 512, 1, 1, 1),
                   x_dist=("normal", 1.0), w_dist=("normal", 1.0 / math.sqrt(512)), seed=6,
                   note="1x1x1 conv3d fwd bf16 NCDHW (no transpose) N=1 C=512 D=240 H=320 W=180 K=48"),
}

_CHUNK = 1 << 27  # draw large tensors in 128 Mi-element pieces to bound fp32 scratch


def _fill(out: torch.Tensor, dist: tuple, gen: torch.Generator) -> torch.Tensor:
    """Fill a contiguous bf16 tensor with fp32 draws rounded to bf16 (RNE, by torch)."""
    flat = out.view(-1)
    kind, a = dist
    for i in range(0, flat.numel(), _CHUNK):
        n = min(_CHUNK, flat.numel() - i)
        if kind == "uniform":
            v = torch.rand(n, generator=gen, device=out.device, dtype=torch.float32).mul_(2 * a).sub_(a)
        elif kind == "normal":
            v = torch.randn(n, generator=gen, device=out.device, dtype=torch.float32).mul_(a)
        else:
            raise ValueError(kind)
        flat[i:i + n] = v.to(torch.bfloat16)
    return out


def draw(shape, dist: tuple, gen: torch.Generator, device="cpu") -> torch.Tensor:
    return _fill(torch.empty(shape, dtype=torch.bfloat16, device=device), dist, gen)


def generator(seed: int, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def make(wl: Workload | str, device="cpu"):
    """(x, w) as bf16 tensors: x in wl.x_layout memory order (logical NCDHW dims
    reported by x_shape), w as KCTRS. x is drawn first, then w."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    g = generator(wl.seed, device)
    n, c, d, h, w_ = wl.x_shape
    if wl.x_layout == "NDHWC":
        x = draw((n, d, h, w_, c), wl.x_dist, g, device)
    else:
        x = draw((n, c, d, h, w_), wl.x_dist, g, device)
    w = draw(wl.w_shape, wl.w_dist, g, device)
    return x, w


def int_valued(shape, lo: int, hi: int, gen: torch.Generator, device="cpu") -> torch.Tensor:
    """Integers drawn uniformly from [lo, hi], stored as bf16 (exact for |v| <= 256)."""
    return torch.randint(lo, hi + 1, shape, generator=gen, device=device).to(torch.bfloat16)


def sparse_ternary(shape, nnz_per_row: int, gen: torch.Generator, device="cpu") -> torch.Tensor:
    """Filter (K, ...) with exactly min(nnz_per_row, row size) entries per output
    channel drawn from {-1, +1} at random positions, the rest 0 (bf16)."""
    k = shape[0]
    row = 1
    for v in shape[1:]:
        row *= v
    nnz = min(nnz_per_row, row)
    out = torch.zeros((k, row), dtype=torch.float32, device=device)
    scores = torch.rand((k, row), generator=gen, device=device)
    idx = scores.topk(nnz, dim=1).indices
    signs = torch.randint(0, 2, (k, nnz), generator=gen, device=device).float() * 2 - 1
    out.scatter_(1, idx, signs)
    return out.view(shape).to(torch.bfloat16)


def bf16_bits(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (host copy)."""
    import numpy as np
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
