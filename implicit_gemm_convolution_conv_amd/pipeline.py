"""Convenience sequences of the C-ABI calls, with torch allocating the buffers.

This module only orders calls into the library (amax -> scales -> pack ->
conv) and allocates their outputs; it performs no arithmetic of its own.
"""

from __future__ import annotations

import torch

from . import binding as B

DTYPES = {"bf16": B.IGC_BF16, "fp8": B.IGC_FP8_E4M3FN}
LAYOUTS = {"NCDHW": B.IGC_NCDHW, "NDHWC": B.IGC_NDHWC}


def _code(dtype):
    return DTYPES[dtype] if isinstance(dtype, str) else int(dtype)


def packed_weight(w_kctrs: torch.Tensor, dtype="bf16", x_layout="NDHWC", scale_pair=None, stream=None):
    """Pack a bf16 KCTRS filter (fp8: scale_pair must hold its {s, inv})."""
    dt = _code(dtype)
    cols = B.conv_packed_w_cols(w_kctrs.shape, dt)
    out = torch.empty((w_kctrs.shape[0], cols), dtype=torch.uint8 if dt == B.IGC_FP8_E4M3FN else torch.bfloat16,
                      device=w_kctrs.device)
    B.conv_pack_w(w_kctrs, out, w_kctrs.shape, dt, LAYOUTS[x_layout], scale_pair, stream)
    return out


def packed_input(x_ncdhw: torch.Tensor, dtype="bf16", scale_pair=None, stream=None):
    """NCDHW bf16 -> NDHWC (bf16 or fp8 codes), returned as a (N, D, H, W, C) tensor."""
    dt = _code(dtype)
    n, c, d, h, w = x_ncdhw.shape
    out = torch.empty((n, d, h, w, c), dtype=torch.uint8 if dt == B.IGC_FP8_E4M3FN else torch.bfloat16,
                      device=x_ncdhw.device)
    B.conv_pack_x(x_ncdhw, out, x_ncdhw.shape, dt, scale_pair, stream)
    return out


def fp8_scales(x_bf16: torch.Tensor, w_bf16: torch.Tensor, stream=None):
    """Device float[4] = {s_x, inv_x, s_w, inv_w} from the two tensors' amax."""
    amax = torch.empty(2, dtype=torch.float32, device=x_bf16.device)
    scales = torch.empty(4, dtype=torch.float32, device=x_bf16.device)
    B.conv_amax(x_bf16, x_bf16.numel(), amax[0:1], stream)
    B.conv_fp8_scales(amax[0:1], scales[0:2], stream)
    B.conv_amax(w_bf16, w_bf16.numel(), amax[1:2], stream)
    B.conv_fp8_scales(amax[1:2], scales[2:4], stream)
    return scales


def output(xshape, wshape, stride, pad, dil, device):
    do, ho, wo = B.conv_out_dims(xshape, wshape, stride, pad, dil)
    return torch.empty((xshape[0], wshape[0], do, ho, wo), dtype=torch.bfloat16, device=device)


def conv3d(x_ncdhw: torch.Tensor, w_kctrs: torch.Tensor, stride=(1, 1, 1), pad=(0, 0, 0), dil=(1, 1, 1),
           dtype="bf16", stream=None):
    """y = conv3d(x, w) from bf16 NCDHW x and bf16 KCTRS w, all on the GPU.

    Point-output shapes and bf16 1x1x1 filters read x as is; other shapes pack
    x to NDHWC first. fp8 quantises both operands with per-tensor amax/448
    scales."""
    dt = _code(dtype)
    xshape, wshape = tuple(x_ncdhw.shape), tuple(w_kctrs.shape)
    direct = dt == B.IGC_BF16 and direct_ncdhw(xshape, wshape, stride, pad, dil)
    scales = fp8_scales(x_ncdhw, w_kctrs, stream) if dt == B.IGC_FP8_E4M3FN else None
    sx = scales[0:2] if scales is not None else None
    sw = scales[2:4] if scales is not None else None
    y = output(xshape, wshape, stride, pad, dil, x_ncdhw.device)
    if direct:
        wp = packed_weight(w_kctrs, dt, "NCDHW", sw, stream)
        B.conv_fwd(x_ncdhw, wp, y, xshape, wshape, stride, pad, dil, dt, B.IGC_NCDHW, scales, stream)
        return y
    xp = packed_input(x_ncdhw, dt, sx, stream)
    wp = packed_weight(w_kctrs, dt, "NDHWC", sw, stream)
    B.conv_fwd(xp, wp, y, xshape, wshape, stride, pad, dil, dt, B.IGC_NDHWC, scales, stream)
    return y


def direct_ncdhw(xshape, wshape, stride, pad, dil) -> bool:
    """True when the library reads bf16 NCDHW x as it is for this shape (point output, or the 1x1x1 pointwise
    path) instead of needing the NDHWC pack."""
    try:
        plan = B.conv_plan(xshape, wshape, stride, pad, dil, B.IGC_BF16, B.IGC_NCDHW)
    except B.IgcError:
        return False
    return plan.startswith("path=point")
