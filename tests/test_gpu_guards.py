"""Guard bands and canaries around every operand of the HIP path.

x, the packed filter and the workspace sit inside larger buffers whose margins hold NaN (bf16 0x7fc0, E4M3FN
0x7f): a kernel that reads even one element before or past an operand, and uses it, puts a NaN into y. y sits
between two canary margins of a fixed, finite bit pattern, and starts as NaN: every element must be written and
nothing around y may change. The margins of the inputs must come back unchanged too (no kernel writes them).
Buffer-addressed tiles clamp GEMM rows past M (or past K) to the last valid row, so these cases use ragged M and
K on every tile family, both dtypes, the point-output and pointwise paths, the split reduction and the tail
split. Results are compared with the oracle: bit for bit on integer-valued inputs.
"""

import numpy as np
import pytest
import torch

from implicit_gemm_convolution_conv_amd import binding as B
from implicit_gemm_convolution_conv_amd import inputs as I
from oracle import oracle as O

import parity as P

pytestmark = pytest.mark.gpu

GUARD = 8192  # elements (bf16) or bytes (fp8) of margin on each side: 16-byte aligned views
NAN_BF16, NAN_E4M3, CANARY = 0x7FC0, 0x7F, 0x3C5A


def _announce(name):
    print(f"[case] {name}", flush=True)


_INT_OF = {torch.bfloat16: torch.int16, torch.uint8: torch.uint8, torch.float32: torch.int32}


class Guarded:
    """A contiguous view of `shape` inside a buffer with GUARD elements of the bit pattern `fill` on each side."""

    def __init__(self, shape, dtype, fill):
        n = int(np.prod(shape))
        self.whole = torch.empty(n + 2 * GUARD, dtype=dtype, device=P.DEV)
        self.raw = self.whole.view(_INT_OF[dtype])
        signed, unsigned = {torch.int16: (np.int16, np.uint16), torch.uint8: (np.uint8, np.uint8),
                            torch.int32: (np.int32, np.uint32)}[self.raw.dtype]
        self.fill = int(np.array(fill, unsigned).view(signed))
        self.raw.fill_(self.fill)
        self.view = self.whole[GUARD:GUARD + n].view(shape)

    def margins_intact(self):
        return bool((self.raw[:GUARD] == self.fill).all()) and bool((self.raw[-GUARD:] == self.fill).all())


class forced:
    def __init__(self, tile=-1, splits=0, cus=0):
        self.tile, self.splits, self.cus = tile, splits, cus

    def __enter__(self):
        B.conv_debug_force(B.IGC_PATH_AUTO, self.tile, 0)
        B.conv_debug_force_splits(self.splits)
        B.conv_debug_force_grid(self.cus)

    def __exit__(self, *exc):
        B.conv_debug_force(B.IGC_PATH_AUTO, -1, 0)
        B.conv_debug_force_splits(0)
        B.conv_debug_force_grid(0)


def _run(xs, ws, st, pd, dl, layout, dtype, x_vals, w_vals, scales=None, bias=None):
    """Packs x (NDHWC unless the layout is NCDHW) and w into guarded buffers, runs the conv (conv_fwd_ex with a
    guarded NaN workspace when the plan wants one) into a guarded NaN-filled y and checks every margin."""
    lay = B.IGC_NDHWC if layout == "NDHWC" else B.IGC_NCDHW
    fp8 = dtype == B.IGC_FP8_E4M3FN
    tdt, nan = (torch.uint8, NAN_E4M3) if fp8 else (torch.bfloat16, NAN_BF16)
    n, c, d, h, w = xs
    xg = Guarded((n, d, h, w, c) if lay == B.IGC_NDHWC else xs, tdt, nan)
    if lay == B.IGC_NDHWC:
        B.conv_pack_x(x_vals, xg.view, xs, dtype, None if scales is None else scales[0:2])
    else:
        xg.view.copy_(x_vals)
    cols = B.conv_packed_w_cols(ws, dtype)
    wg = Guarded((ws[0], cols), tdt, nan)
    B.conv_pack_w(w_vals, wg.view, ws, dtype, lay, None if scales is None else scales[2:4])
    yshape = (n, ws[0]) + B.conv_out_dims(xs, ws, st, pd, dl)
    yg = Guarded(yshape, torch.bfloat16, CANARY)
    yg.view.fill_(float("nan"))
    nws = B.conv_fwd_workspace_bytes(xs, ws, st, pd, dl, dtype, lay)
    wsg = Guarded((max(nws, 16) // 4,), torch.float32, 0x7FC00001) if nws > 0 else None
    if wsg is not None:
        wsg.view.fill_(float("nan"))
    plan = B.conv_plan_ws(xs, ws, st, pd, dl, dtype, lay, max(nws, 0))
    B.conv_fwd_ex(xg.view, wg.view, yg.view, xs, ws, st, pd, dl, dtype, lay, scales, bias=bias,
                  workspace=None if wsg is None else wsg.view)
    torch.cuda.synchronize()
    assert yg.margins_intact(), f"a write landed next to y ({plan})"
    assert xg.margins_intact() and wg.margins_intact(), f"a write landed next to x or w ({plan})"
    if wsg is not None:
        assert wsg.margins_intact(), f"a write landed next to the workspace ({plan})"
    assert not torch.isnan(yg.view).any(), f"NaN in y: an element unwritten or a guard read ({plan})"
    return yg.view, plan


# name, x (N,C,D,H,W), w (K,C,T,R,S), stride, pad, dil, tile, splits, CUs stood in for
CASES = [
    # 990 rows (3 full M tiles + 222), 200 output channels: ragged in both GEMM dimensions
    ("buf_ragged", (2, 128, 5, 9, 11), (200, 128, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), B.IGC_TILE_BUF, 0, 0),
    ("buf_ahead_ragged", (2, 128, 5, 9, 11), (200, 128, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1),
     B.IGC_TILE_BUF_AHEAD, 0, 0),
    ("pingpong_ragged", (2, 128, 5, 9, 11), (200, 128, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1),
     B.IGC_TILE_BUF_PINGPONG, 0, 0),
    ("buf_temporal_ragged", (1, 128, 7, 10, 13), (136, 128, 3, 1, 1), (1, 1, 1), (1, 0, 0), (1, 1, 1),
     B.IGC_TILE_BUF, 0, 0),
    # the last input plane is the last element of x: taps past it must read as zero, not the margin
    ("buf_strided_dilated", (1, 64, 7, 12, 13), (72, 64, 2, 3, 3), (2, 2, 1), (1, 2, 2), (2, 2, 2),
     B.IGC_TILE_BUF, 0, 0),
    ("dma256_ragged", (2, 128, 5, 9, 11), (200, 128, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1),
     B.IGC_TILE_DMA_256, 0, 0),
    ("dma64_linear_c24", (2, 24, 5, 7, 9), (40, 24, 3, 3, 3), (1, 2, 1), (1, 1, 2), (1, 1, 2), B.IGC_TILE_DMA_64, 0,
     0),
    ("split_reduction", (1, 64, 4, 16, 16), (64, 64, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), -1, 0, 0),
    ("tail_split", (2, 256, 3, 11, 29), (300, 256, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), B.IGC_TILE_BUF_AHEAD,
     0, 12),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_guards_bf16_integer(case):
    name, xs, ws, st, pd, dl, tile, splits, cus = case
    _announce(f"guards bf16 {name}")
    g = I.generator(300, P.DEV)
    x = I.int_valued(xs, -2, 2, g, P.DEV)
    w = I.sparse_ternary(ws, 128, g, P.DEV)
    with forced(tile, splits, cus):
        y, plan = _run(xs, ws, st, pd, dl, "NDHWC", B.IGC_BF16, x, w)
    if name == "tail_split":
        assert "tail=4/3" in plan, plan
    if name == "split_reduction":
        assert "splits=5" in plan, plan
    ref = O.conv3d(P.bits(x), P.bits(w), st, pd, dl)
    assert np.array_equal(P.y_values(y), ref)


@pytest.mark.parametrize("case", [c for c in CASES if c[0] in ("buf_ragged", "pingpong_ragged", "buf_temporal_ragged",
                                                               "dma256_ragged", "tail_split")], ids=lambda c: c[0])
def test_guards_fp8_integer(case):
    name, xs, ws, st, pd, dl, tile, splits, cus = case
    _announce(f"guards fp8 {name}")
    g = I.generator(301, P.DEV)
    x = I.int_valued(xs, -2, 2, g, P.DEV)
    w = I.sparse_ternary(ws, 128, g, P.DEV)
    unit = torch.ones(4, dtype=torch.float32, device=P.DEV)  # integers |v| <= 2 are exact codes at unit scale
    with forced(tile, splits, cus):
        y, _ = _run(xs, ws, st, pd, dl, "NDHWC", B.IGC_FP8_E4M3FN, x, w, scales=unit)
    ref = O.conv3d(P.bits(x), P.bits(w), st, pd, dl)
    assert np.array_equal(P.y_values(y), ref)


@pytest.mark.parametrize("tile", [-1, B.IGC_TILE_DMA_64])
@pytest.mark.parametrize("layout", ["NCDHW", "NDHWC"])
def test_guards_point_output(layout, tile):
    # 130 images of 588 elements (rows only 8-byte aligned), 68 channels: the last image row ends at the margin
    _announce(f"guards point output {layout} tile {tile}")
    xs, ws, st, pd, dl = (130, 3, 1, 14, 14), (68, 3, 1, 14, 14), (1, 14, 14), (0, 0, 0), (1, 1, 1)
    g = I.generator(302, P.DEV)
    x = I.int_valued(xs, -2, 2, g, P.DEV)
    w = I.sparse_ternary(ws, 128, g, P.DEV)
    xin = x if layout == "NCDHW" else x.permute(0, 2, 3, 4, 1).contiguous()
    lay = B.IGC_NCDHW if layout == "NCDHW" else B.IGC_NDHWC
    # x as it is (no pack), inside NaN margins
    xg = Guarded(tuple(xin.shape), torch.bfloat16, NAN_BF16)
    xg.view.copy_(xin)
    wg = Guarded((ws[0], B.conv_packed_w_cols(ws, B.IGC_BF16)), torch.bfloat16, NAN_BF16)
    B.conv_pack_w(w, wg.view, ws, B.IGC_BF16, lay)
    yg = Guarded((xs[0], ws[0], 1, 1, 1), torch.bfloat16, CANARY)
    yg.view.fill_(float("nan"))
    with forced(tile):
        B.conv_fwd(xg.view, wg.view, yg.view, xs, ws, st, pd, dl, B.IGC_BF16, lay)
    torch.cuda.synchronize()
    assert yg.margins_intact() and xg.margins_intact() and wg.margins_intact()
    ref = O.conv3d(P.bits(x), P.bits(w), st, pd, dl)
    assert np.array_equal(P.y_values(yg.view), ref)


def test_guards_pointwise_ncdhw():
    # 1x1x1 on NCDHW: 2 images of 48 channels x 168 positions, 80 output channels (ragged against 512 x 64 tiles)
    _announce("guards pointwise NCDHW")
    xs, ws, one, zero = (2, 48, 3, 7, 8), (80, 48, 1, 1, 1), (1, 1, 1), (0, 0, 0)
    g = I.generator(303, P.DEV)
    x = I.int_valued(xs, -2, 2, g, P.DEV)
    w = I.sparse_ternary(ws, 128, g, P.DEV)
    assert B.conv_plan(xs, ws, one, zero, one, B.IGC_BF16, B.IGC_NCDHW).startswith("path=pointwise")
    y, _ = _run(xs, ws, one, zero, one, "NCDHW", B.IGC_BF16, x, w)
    ref = O.conv3d(P.bits(x), P.bits(w), one, zero, one)
    assert np.array_equal(P.y_values(y), ref)


def test_guards_random_bf16_with_bias():
    # random operands and a bias on the default plan of a ragged shape, against the oracle's tolerance
    _announce("guards random bf16 with bias")
    xs, ws, st, pd, dl = (2, 128, 5, 9, 11), (200, 128, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)
    g = I.generator(304, P.DEV)
    x = I.draw(xs, ("uniform", 1.0), g, P.DEV)
    w = I.draw(ws, ("uniform", 1.0), g, P.DEV)
    bias = I.draw((ws[0],), ("uniform", 1.0), g, P.DEV).float()
    y, _ = _run(xs, ws, st, pd, dl, "NDHWC", B.IGC_BF16, x, w, bias=bias)
    ref = O.conv3d(P.bits(x), P.bits(w), st, pd, dl, bias=bias.cpu().numpy())
    R = int(np.prod(ws[1:]))
    mx, mw = float(x.abs().max()), float(w.abs().max())
    P.check_close(P.y_values(y), ref, R, mx, mw + float(bias.abs().max()) / (R ** 0.5 * mx), "guards random")
