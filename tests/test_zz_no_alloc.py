"""conv_fwd_noalloc: the forward convolution with its workspace in the library's static device scratch.

It must give conv_fwd_ws's (conv_fwd_ex's) output bit for bit on the same inputs, since it runs the same plan
with the same partial sums, on two calls in a row, the second with a smaller input (the scratch keeps the first
call's partial sums, which the second call must overwrite before it reads them). Both calls go through the C
ABI; the first uses a tail split (partial sums of 76 tiles in 3 splits), the second a split reduction with a
bias and the amax of y.
"""

import pytest
import torch

from implicit_gemm_convolution_conv_amd import binding as B
from implicit_gemm_convolution_conv_amd import inputs as I
from implicit_gemm_convolution_conv_amd import pipeline as PL

import parity as P

pytestmark = pytest.mark.gpu


def _announce(name):
    print(f"[case] {name}", flush=True)


def _nan(shape):
    return torch.full(shape, float("nan"), dtype=torch.bfloat16, device=P.DEV)


def test_noalloc_matches_workspace_call_twice():
    # call 1: c3's one-GPU share (K = 256): 844 tiles of 256x256, the last 76 split three ways
    wl = I.WORKLOADS["c3s"]
    xs, ws = wl.x_shape, wl.w_shape
    args = (xs, ws, wl.stride, wl.pad, wl.dil, B.IGC_BF16, B.IGC_NDHWC)
    _announce("noalloc call 1: c3s, tail split through the static scratch")
    nws = B.conv_fwd_workspace_bytes(*args)
    assert nws == 76 * 3 * 256 * 256 * 4
    assert "tail=76/3" in B.conv_plan_ws(*args, nws)
    x, w = I.make(wl, P.DEV)
    wp = PL.packed_weight(w, "bf16", "NDHWC")
    yshape = (xs[0], ws[0]) + B.conv_out_dims(xs, ws, wl.stride, wl.pad, wl.dil)
    y_ref = _nan(yshape)
    wsb = torch.full((nws // 4,), float("nan"), dtype=torch.float32, device=P.DEV)
    B.conv_fwd_ws(x, wp, y_ref, *args, workspace=wsb)
    y = _nan(yshape)
    B.conv_fwd_noalloc(x, wp, y, *args)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    del x, w, wp, y, y_ref, wsb
    torch.cuda.empty_cache()

    # call 2, smaller: the 64-channel 3x3x3 conv on 4x16x16, 16 tiles of 64x64 in 5 reduction splits, with a
    # bias and the amax of y
    wl = I.WORKLOADS["c1"]
    xs, ws = wl.x_shape, wl.w_shape
    args = (xs, ws, wl.stride, wl.pad, wl.dil, B.IGC_BF16, B.IGC_NDHWC)
    _announce("noalloc call 2: c1, split reduction with bias and amax through the static scratch")
    nws = B.conv_fwd_workspace_bytes(*args)
    assert nws == 5 * 1024 * 64 * 4
    x, w = I.make(wl, P.DEV)
    xk = PL.packed_input(x, "bf16")
    wp = PL.packed_weight(w, "bf16", "NDHWC")
    bias = I.draw((ws[0],), ("uniform", 2.0), I.generator(77, P.DEV), P.DEV).float()
    yshape = (xs[0], ws[0]) + B.conv_out_dims(xs, ws, wl.stride, wl.pad, wl.dil)
    y_ref, y = _nan(yshape), _nan(yshape)
    amax_ref = torch.full((1,), float("nan"), dtype=torch.float32, device=P.DEV)
    amax = torch.full((1,), float("nan"), dtype=torch.float32, device=P.DEV)
    wsb = torch.full((nws // 4,), float("nan"), dtype=torch.float32, device=P.DEV)
    B.conv_fwd_ex(xk, wp, y_ref, *args, bias=bias, y_amax=amax_ref, workspace=wsb)
    B.conv_fwd_noalloc(xk, wp, y, *args, bias=bias, y_amax=amax)
    torch.cuda.synchronize()
    assert not torch.isnan(y).any()
    assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))
    assert float(amax) == float(amax_ref)

    # a plan without any split needs no scratch: the same output as conv_fwd
    _announce("noalloc call 3: no split, as conv_fwd")
    xs3, ws3 = (1, 64, 6, 10, 12), (96, 64, 3, 1, 1)
    args3 = (xs3, ws3, (1, 1, 1), (1, 0, 0), (1, 1, 1), B.IGC_BF16, B.IGC_NDHWC)
    assert B.conv_fwd_workspace_bytes(*args3) == 0
    g = I.generator(78, P.DEV)
    x3 = I.draw((1, 6, 10, 12, 64), ("uniform", 1.0), g, P.DEV)
    w3 = I.draw(ws3, ("uniform", 1.0), g, P.DEV)
    wp3 = PL.packed_weight(w3, "bf16", "NDHWC")
    yshape3 = (1, 96) + B.conv_out_dims(*args3[:5])
    y3_ref, y3 = _nan(yshape3), _nan(yshape3)
    B.conv_fwd(x3, wp3, y3_ref, *args3)
    B.conv_fwd_noalloc(x3, wp3, y3, *args3)
    torch.cuda.synchronize()
    assert torch.equal(y3.view(torch.int16), y3_ref.view(torch.int16))
