"""GPU parity of the fused epilogue extras (conv_fwd_ex): the per-channel bias
against the oracle's bias term, and the fused amax of y, on every kernel
family (register, global-address direct-to-LDS, input window, buffer-addressed,
ping-pong, tap-shared windows, 1x1x1 NCDHW, point output, split reduction).

The fused amax must equal max |y| over the bf16 values the same call wrote, bit
for bit: that holds at any size and needs no oracle. Every case prints its name
before touching the GPU.
"""

import numpy as np
import pytest
import torch

from implicit_gemm_convolution_conv_amd import binding as B
from implicit_gemm_convolution_conv_amd import inputs as I
from oracle import oracle as O

import parity as P

pytestmark = pytest.mark.gpu


def _announce(name):
    print(f"[case] {name}", flush=True)


class forced:
    def __init__(self, tile=-1, splits=0, path=B.IGC_PATH_AUTO):
        self.tile, self.splits, self.path = tile, splits, path

    def __enter__(self):
        B.conv_debug_force(self.path, self.tile, 0)
        B.conv_debug_force_splits(self.splits)

    def __exit__(self, *exc):
        B.conv_debug_force(B.IGC_PATH_AUTO, -1, 0)
        B.conv_debug_force_splits(0)


def _amax_of(y):
    return float(y.float().abs().max())


def _out(xs, ws, st, pd, dl):
    return torch.full((xs[0], ws[0]) + B.conv_out_dims(xs, ws, st, pd, dl), float("nan"), dtype=torch.bfloat16,
                      device=P.DEV)


# name, x, w, stride, pad, dil, layout, tile, splits
CASES = [
    ("dma_256", (1, 64, 5, 9, 11), (96, 64, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), "NDHWC", B.IGC_TILE_DMA_256, 0),
    ("dma_128_linear_strided", (2, 24, 5, 7, 9), (40, 24, 3, 3, 3), (1, 2, 1), (1, 1, 2), (1, 1, 2), "NDHWC",
     B.IGC_TILE_DMA_128, 0),
    ("dma_64", (1, 64, 4, 16, 16), (64, 64, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), "NDHWC", B.IGC_TILE_DMA_64, 1),
    ("dma_256_temporal", (2, 64, 9, 6, 7), (96, 64, 3, 1, 1), (1, 1, 1), (1, 0, 0), (1, 1, 1), "NDHWC",
     B.IGC_TILE_DMA_256, 1),
    ("buffer", (2, 128, 6, 10, 12), (200, 128, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), "NDHWC", B.IGC_TILE_BUF, 0),
    ("buffer_ahead", (1, 64, 4, 18, 20), (72, 64, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), "NDHWC",
     B.IGC_TILE_BUF_AHEAD, 0),
    # whole 256x256 tiles inside one image with 16-byte aligned rows: the outputs go through LDS
    ("buffer_lds_epilogue", (1, 128, 4, 16, 16), (256, 128, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), "NDHWC",
     B.IGC_TILE_BUF, 0),
    ("buffer_ahead_lds_epilogue", (1, 128, 4, 16, 16), (256, 128, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), "NDHWC",
     B.IGC_TILE_BUF_AHEAD, 0),
    ("pingpong", (1, 128, 5, 9, 11), (136, 128, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), "NDHWC",
     B.IGC_TILE_BUF_PINGPONG, 0),
    ("pingpong_lds_epilogue", (1, 128, 4, 16, 16), (256, 128, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), "NDHWC",
     B.IGC_TILE_BUF_PINGPONG, 0),
    ("pointwise_ncdhw", (2, 48, 3, 7, 8), (80, 48, 1, 1, 1), (1, 1, 1), (0, 0, 0), (1, 1, 1), "NCDHW", -1, 0),
    ("point_output", (40, 3, 1, 14, 14), (68, 3, 1, 14, 14), (1, 14, 14), (0, 0, 0), (1, 1, 1), "NCDHW", -1, 0),
    ("point_output_lds", (200, 3, 1, 14, 14), (256, 3, 1, 14, 14), (1, 14, 14), (0, 0, 0), (1, 1, 1), "NCDHW",
     B.IGC_TILE_DMA_64, 0),
    ("split_c1", (1, 64, 4, 16, 16), (64, 64, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), "NDHWC", B.IGC_TILE_DMA_64, 5),
    ("split_point", (40, 3, 1, 14, 14), (68, 3, 1, 14, 14), (1, 14, 14), (0, 0, 0), (1, 1, 1), "NCDHW",
     B.IGC_TILE_DMA_64, 4),
    ("split_odd_tails", (1, 16, 3, 5, 7), (25, 16, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), "NDHWC",
     B.IGC_TILE_DMA_64, 2),
]


def _workspace(xs, ws, st, pd, dl, splits):
    if splits <= 1:
        return None
    ynum = xs[0] * ws[0] * int(np.prod(B.conv_out_dims(xs, ws, st, pd, dl)))
    return torch.full((splits * ynum,), float("nan"), dtype=torch.float32, device=P.DEV)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_bias_and_amax_bf16(case):
    name, xs, ws, st, pd, dl, layout, tile, splits = case
    _announce(f"epilogue bf16 {name}")
    g = I.generator(70 + len(name), P.DEV)
    x = I.draw(xs, ("uniform", 1.0), g, P.DEV)
    w = I.draw(ws, ("uniform", 1.0), g, P.DEV)
    bias = I.draw((ws[0],), ("uniform", 4.0), g, P.DEV).float()
    amax = torch.full((1,), float("nan"), dtype=torch.float32, device=P.DEV)
    with forced(tile, splits):
        y = P.run_bf16(x, w, st, pd, dl, x_layout=layout, out=_out(xs, ws, st, pd, dl),
                       workspace=_workspace(xs, ws, st, pd, dl, splits), bias=bias, amax=amax)
        y0 = P.run_bf16(x, w, st, pd, dl, x_layout=layout, workspace=_workspace(xs, ws, st, pd, dl, splits))
        y_noextra = torch.empty_like(y0)
        P.run_bf16(x, w, st, pd, dl, x_layout=layout, out=y_noextra)  # conv_fwd (never splits)
    assert not torch.isnan(y).any()
    ref = O.conv3d(P.bits(x), P.bits(w), st, pd, dl, bias=bias.cpu().numpy())
    R = int(np.prod(ws[1:]))
    # the bias widens the value range: bound with max|x| max|w| + max|b| / sqrt(R) folded in
    mx, mw = float(x.abs().max()), float(w.abs().max())
    P.check_close(P.y_values(y), ref, R, mx, mw + float(bias.abs().max()) / (R ** 0.5 * mx), name)
    assert float(amax) == _amax_of(y)
    if splits <= 1:
        assert torch.equal(y0.view(torch.int16), y_noextra.view(torch.int16))


@pytest.mark.parametrize("case", [c for c in CASES if c[0] in ("dma_256", "dma_64", "buffer", "buffer_ahead",
                                                               "buffer_lds_epilogue", "buffer_ahead_lds_epilogue",
                                                               "pingpong", "pingpong_lds_epilogue", "pointwise_ncdhw",
                                                               "point_output", "point_output_lds", "split_c1",
                                                               "split_odd_tails")],
                         ids=lambda c: c[0])
def test_bias_integer_bit_exact(case):
    name, xs, ws, st, pd, dl, layout, tile, splits = case
    _announce(f"epilogue integer {name}")
    g = I.generator(90, P.DEV)
    x = I.int_valued(xs, -2, 2, g, P.DEV)
    w = I.sparse_ternary(ws, 128, g, P.DEV)
    bias = I.int_valued((ws[0],), -8, 8, g, P.DEV).float()  # |y| <= 264: exact in fp32 and bf16
    amax = torch.zeros(1, dtype=torch.float32, device=P.DEV)
    with forced(tile, splits):
        y = P.run_bf16(x, w, st, pd, dl, x_layout=layout, out=_out(xs, ws, st, pd, dl),
                       workspace=_workspace(xs, ws, st, pd, dl, splits), bias=bias, amax=amax)
    ref = O.conv3d(P.bits(x), P.bits(w), st, pd, dl, bias=bias.cpu().numpy())
    assert np.array_equal(P.y_values(y), ref)
    assert float(amax) == float(np.abs(ref).max())


@pytest.mark.parametrize("tile,splits,kout", [(-1, 0, 136), (B.IGC_TILE_BUF_PINGPONG, 0, 136), (B.IGC_TILE_BUF, 0, 136),
                                              (B.IGC_TILE_DMA_64, 1, 136), (B.IGC_TILE_DMA_64, 3, 136),
                                              (B.IGC_TILE_BUF, 0, 256), (B.IGC_TILE_BUF_AHEAD, 0, 256),
                                              (B.IGC_TILE_BUF_PINGPONG, 0, 256)])
def test_bias_and_amax_fp8(tile, splits, kout):
    # kout = 256 on 4 x 16 x 16 outputs: whole tiles inside the image, the LDS-staged epilogue of the buffer tiles
    _announce(f"epilogue fp8 tile {tile} splits {splits} K {kout}")
    if kout == 256:
        xs, ws, st, pd, dl = (1, 128, 4, 16, 16), (256, 128, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)
    else:
        xs, ws, st, pd, dl = (1, 128, 5, 9, 11), (136, 128, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)
    g = I.generator(91, P.DEV)
    x = I.draw(xs, ("normal", 1.0), g, P.DEV)
    w = I.draw(ws, ("normal", 1.0 / np.sqrt(np.prod(ws[1:]))), g, P.DEV)
    bias = I.draw((ws[0],), ("normal", 1.0), g, P.DEV).float()
    ops = P.Fp8Operands(x, w)
    amax = torch.full((1,), float("nan"), dtype=torch.float32, device=P.DEV)
    with forced(tile, splits):
        y = P.run_fp8(ops, xs, ws, st, pd, dl, out=_out(xs, ws, st, pd, dl),
                      workspace=_workspace(xs, ws, st, pd, dl, splits), bias=bias, amax=amax)
    torch.cuda.synchronize()
    sx, sw = float(ops.ref_scales[0]), float(ops.ref_scales[2])
    ref = O.conv3d(ops.ref_xq, ops.ref_wq, st, pd, dl, sx=sx, sw=sw, bias=bias.cpu().numpy())
    R = int(np.prod(ws[1:]))
    mx = float(np.abs(O.e4m3_decode(ops.ref_xq)).max()) * sx
    mw = float(np.abs(O.e4m3_decode(ops.ref_wq)).max()) * sw
    P.check_close(P.y_values(y), ref, R, mx, mw + float(bias.abs().max()) / (R ** 0.5 * mx), "fp8 bias")
    assert float(amax) == _amax_of(y)


def test_fused_amax_feeds_next_fp8_layer():
    # y of one conv is the next fp8 conv's x: the fused amax gives the same scales as a separate conv_amax pass
    _announce("fused amax vs conv_amax")
    xs, ws, st, pd, dl = (1, 64, 6, 10, 12), (128, 64, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)
    g = I.generator(92, P.DEV)
    x = I.draw(xs, ("normal", 1.0), g, P.DEV)
    w = I.draw(ws, ("normal", 1.0 / np.sqrt(np.prod(ws[1:]))), g, P.DEV)
    amax = torch.empty(1, dtype=torch.float32, device=P.DEV)
    y = P.run_bf16(x, w, st, pd, dl, amax=amax)
    sep = torch.empty(1, dtype=torch.float32, device=P.DEV)
    B.conv_amax(y, y.numel(), sep)
    torch.cuda.synchronize()
    assert float(amax) == float(sep) == _amax_of(y)
    pair_fused = torch.empty(2, dtype=torch.float32, device=P.DEV)
    pair_sep = torch.empty(2, dtype=torch.float32, device=P.DEV)
    B.conv_fp8_scales(amax, pair_fused)
    B.conv_fp8_scales(sep, pair_sep)
    torch.cuda.synchronize()
    assert torch.equal(pair_fused.view(torch.int32), pair_sep.view(torch.int32))
