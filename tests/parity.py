"""Shared helpers for the GPU parity tests: run the HIP path through the C ABI,
evaluate the CPU oracle on the same seeded inputs, compare.

Tolerance for random data (both dtypes), on the compared set of outputs:
    relative L2  ||y_gpu - y_ref|| / ||y_ref||       <= 1e-2
    max abs      max |y_gpu - y_ref| <= 2e-2 * sqrt(R) * max|x| * max|w|
with R = C*T*R*S and, for fp8, the maxima of the dequantised operands. The
fp8 codes are the same on both sides (checked bit for bit), so only fp32
accumulation order and the final bf16 rounding differ.
"""

from __future__ import annotations

import math

import numpy as np
import torch

from implicit_gemm_convolution_conv_amd import binding as B
from implicit_gemm_convolution_conv_amd import inputs as I
from oracle import oracle as O

DEV = "cuda"
REL_L2 = 1e-2
ABS_FACTOR = 2e-2


def bits(t: torch.Tensor) -> np.ndarray:
    return I.bf16_bits(t)


def y_values(y: torch.Tensor) -> np.ndarray:
    return y.detach().float().cpu().double().numpy()


def check_close(y_gpu: np.ndarray, y_ref: np.ndarray, R: int, max_x: float, max_w: float, what=""):
    assert y_gpu.shape == y_ref.shape, (y_gpu.shape, y_ref.shape)
    assert np.all(np.isfinite(y_gpu)), f"{what}: non-finite output"
    diff = y_gpu - y_ref
    den = np.linalg.norm(y_ref)
    rel = np.linalg.norm(diff) / den if den > 0 else np.linalg.norm(diff)
    mabs = np.abs(diff).max() if diff.size else 0.0
    bound = ABS_FACTOR * math.sqrt(R) * max_x * max_w
    assert rel <= REL_L2, f"{what}: rel L2 {rel:.3e} > {REL_L2}"
    assert mabs <= bound, f"{what}: max abs {mabs:.3e} > {bound:.3e}"
    return rel, mabs


class Fp8Operands:
    """The GPU's fp8 preparation of (x, w), plus the oracle's own, checked bit for bit."""

    def __init__(self, x_ncdhw: torch.Tensor, w: torch.Tensor, check_codes=True, stream=None):
        self.amax = torch.empty(2, dtype=torch.float32, device=DEV)
        self.scales = torch.empty(4, dtype=torch.float32, device=DEV)
        B.conv_amax(x_ncdhw, x_ncdhw.numel(), self.amax[0:1], stream)
        B.conv_fp8_scales(self.amax[0:1], self.scales[0:2], stream)
        B.conv_amax(w, w.numel(), self.amax[1:2], stream)
        B.conv_fp8_scales(self.amax[1:2], self.scales[2:4], stream)
        n, c, d, h, wd = x_ncdhw.shape
        self.xq = torch.empty((n, d, h, wd, c), dtype=torch.uint8, device=DEV)
        B.conv_pack_x(x_ncdhw, self.xq, x_ncdhw.shape, B.IGC_FP8_E4M3FN, self.scales[0:2], stream)
        cols = B.conv_packed_w_cols(w.shape, B.IGC_FP8_E4M3FN)
        self.wq = torch.empty((w.shape[0], cols), dtype=torch.uint8, device=DEV)
        B.conv_pack_w(w, self.wq, w.shape, B.IGC_FP8_E4M3FN, B.IGC_NDHWC, self.scales[2:4], stream)
        torch.cuda.synchronize()
        # oracle side, from the same bf16 bits
        xb, wb = bits(x_ncdhw), bits(w)
        self.ref_amax = (O.amax_bf16(xb), O.amax_bf16(wb))
        sx, ix = O.fp8_scales(self.ref_amax[0])
        sw, iw = O.fp8_scales(self.ref_amax[1])
        self.ref_scales = np.array([sx, ix, sw, iw], np.float32)
        got = self.scales.cpu().numpy()
        assert np.array_equal(got.view(np.uint32), self.ref_scales.view(np.uint32)), (got, self.ref_scales)
        assert np.array_equal(self.amax.cpu().numpy(), np.array(self.ref_amax, np.float32))
        self.ref_wq = O.quantize_e4m3(wb, iw)  # KCTRS codes
        if check_codes:
            self.ref_xq = O.quantize_e4m3(xb, ix)  # NCDHW codes
            got_x = self.xq.cpu().numpy()
            assert np.array_equal(got_x, np.moveaxis(self.ref_xq, 1, -1)), "fp8 activation codes differ"
        k = w.shape[0]
        rk = int(np.prod(w.shape[1:]))
        ref_packed = np.zeros((k, cols), np.uint8)
        ref_packed[:, :rk] = np.moveaxis(self.ref_wq, 1, -1).reshape(k, rk)  # (t, r, s, c) order
        assert np.array_equal(self.wq.cpu().numpy(), ref_packed), "fp8 filter codes differ"


def run_bf16(x_ncdhw, w, stride, pad, dil, x_layout="NDHWC", out=None, workspace=None, bias=None, amax=None):
    """HIP path for bf16: pack (if needed) + conv, returns y (bf16, GPU). With a
    workspace tensor the conv goes through conv_fwd_ws (split reduction), with a
    bias (fp32 [K]) or an amax output (fp32 [1]) through conv_fwd_ex."""
    xshape, wshape = tuple(x_ncdhw.shape), tuple(w.shape)
    if out is None:
        out = torch.empty((xshape[0], wshape[0]) + B.conv_out_dims(xshape, wshape, stride, pad, dil),
                          dtype=torch.bfloat16, device=DEV)
    lay = B.IGC_NDHWC if x_layout == "NDHWC" else B.IGC_NCDHW
    cols = B.conv_packed_w_cols(wshape, B.IGC_BF16)
    wp = torch.empty((wshape[0], cols), dtype=torch.bfloat16, device=DEV)
    B.conv_pack_w(w, wp, wshape, B.IGC_BF16, lay)
    if x_layout == "NDHWC" and xshape[1] % 8 == 0:
        n, c, d, h, wd = xshape
        xp = torch.empty((n, d, h, wd, c), dtype=torch.bfloat16, device=DEV)
        B.conv_pack_x(x_ncdhw, xp, xshape, B.IGC_BF16)
    elif x_layout == "NDHWC":  # channel counts the pack kernel does not take: channel-last input as given
        xp = x_ncdhw.permute(0, 2, 3, 4, 1).contiguous()
    else:
        xp = x_ncdhw
    if bias is not None or amax is not None:
        B.conv_fwd_ex(xp, wp, out, xshape, wshape, stride, pad, dil, B.IGC_BF16, lay, bias=bias, y_amax=amax,
                      workspace=workspace)
    elif workspace is None:
        B.conv_fwd(xp, wp, out, xshape, wshape, stride, pad, dil, B.IGC_BF16, lay)
    else:
        B.conv_fwd_ws(xp, wp, out, xshape, wshape, stride, pad, dil, B.IGC_BF16, lay, workspace=workspace)
    torch.cuda.synchronize()
    return out


def run_fp8(ops: Fp8Operands, xshape, wshape, stride, pad, dil, out=None, workspace=None, bias=None, amax=None):
    if out is None:
        out = torch.empty((xshape[0], wshape[0]) + B.conv_out_dims(xshape, wshape, stride, pad, dil),
                          dtype=torch.bfloat16, device=DEV)
    if bias is not None or amax is not None:
        B.conv_fwd_ex(ops.xq, ops.wq, out, xshape, wshape, stride, pad, dil, B.IGC_FP8_E4M3FN, B.IGC_NDHWC,
                      ops.scales, bias=bias, y_amax=amax, workspace=workspace)
    elif workspace is None:
        B.conv_fwd(ops.xq, ops.wq, out, xshape, wshape, stride, pad, dil, B.IGC_FP8_E4M3FN, B.IGC_NDHWC, ops.scales)
    else:
        B.conv_fwd_ws(ops.xq, ops.wq, out, xshape, wshape, stride, pad, dil, B.IGC_FP8_E4M3FN, B.IGC_NDHWC,
                      ops.scales, workspace=workspace)
    torch.cuda.synchronize()
    return out


def sample_points(n, k, do, ho, wo, rng, n_random=400, extra_d=(), extra_k=()):
    """Output positions to check at full size: corners, edges and face centres of
    the output box and their neighbours (several channels each), chosen planes
    and channels, plus uniform draws. Rows of (n, k, od, oh, ow)."""
    def marks(m):
        return sorted({v for v in (0, 1, m // 2, m - 2, m - 1) if 0 <= v < m})

    pts = []
    for od in sorted(set(marks(do)) | {d for d in extra_d if 0 <= d < do}):
        for oh in marks(ho):
            for ow in marks(wo):
                ks = {0, k - 1, int(rng.integers(0, k))} | {kk for kk in extra_k if 0 <= kk < k}
                for kk in ks:
                    pts.append((int(rng.integers(0, n)), kk, od, oh, ow))
    for _ in range(n_random):
        pts.append(tuple(int(rng.integers(0, m)) for m in (n, k, do, ho, wo)))
    return np.array(pts, np.int64)


def gather(y: torch.Tensor, pts: np.ndarray) -> np.ndarray:
    idx = torch.from_numpy(pts).to(y.device)
    return y[idx[:, 0], idx[:, 1], idx[:, 2], idx[:, 3], idx[:, 4]].float().cpu().double().numpy()
