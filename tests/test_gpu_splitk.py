"""GPU parity of the split reduction (conv_fwd_ws): every split count and start
position against the oracle, integer-valued inputs bit for bit, fp8, tails
that take the scalar stores, and a workspace too small for the planned split.

Every case prints its name before touching the GPU.
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
    """Force a tile and a split count for the duration of a with-block."""

    def __init__(self, tile=-1, splits=0, path=B.IGC_PATH_AUTO):
        self.tile, self.splits, self.path = tile, splits, path

    def __enter__(self):
        B.conv_debug_force(self.path, self.tile, 0)
        B.conv_debug_force_splits(self.splits)

    def __exit__(self, *exc):
        B.conv_debug_force(B.IGC_PATH_AUTO, -1, 0)
        B.conv_debug_force_splits(0)


def _workspace(xs, ws, st, pd, dl, splits, dtype=B.IGC_BF16):
    """NaN-filled fp32 workspace with room for `splits` slices of y."""
    ynum = xs[0] * ws[0] * int(np.prod(B.conv_out_dims(xs, ws, st, pd, dl)))
    return torch.full((splits * ynum,), float("nan"), dtype=torch.float32, device=P.DEV)


def _nan_out(xs, ws, st, pd, dl):
    return torch.full((xs[0], ws[0]) + B.conv_out_dims(xs, ws, st, pd, dl), float("nan"), dtype=torch.bfloat16,
                      device=P.DEV)


def _plan_splits(xs, ws, st, pd, dl, lay, nbytes, dtype=B.IGC_BF16):
    plan = B.conv_plan_ws(xs, ws, st, pd, dl, dtype, lay, nbytes)
    kv = dict(item.split("=") for item in plan.split())
    return int(kv["splits"]), int(kv["ksplit"]), int(kv["nk"]), plan


# name, x (N,C,D,H,W), w (K,C,T,R,S), stride, pad, dil, layout, tile, splits
SPLIT_CASES = [
    # linear reduction order (C % 64 != 0): a split starts mid-tap
    ("linear_c24", (2, 24, 5, 7, 9), (40, 24, 3, 3, 3), (1, 2, 1), (1, 1, 2), (1, 1, 2), "NDHWC", B.IGC_TILE_DMA_64, 3),
    # channel-block order over two channel blocks, 128x128 tiles
    ("cblock_c128", (2, 128, 6, 10, 12), (200, 128, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), "NDHWC",
     B.IGC_TILE_DMA_128, 5),
    # channel-block order, 11 steps per split: the second split starts mid-way through the taps of a block
    ("cblock_mid_taps", (1, 128, 5, 9, 11), (96, 128, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), "NDHWC",
     B.IGC_TILE_DMA_64, 5),
    # temporal decode, one step per split
    ("temporal", (2, 64, 9, 6, 7), (96, 64, 3, 1, 1), (1, 1, 1), (1, 0, 0), (1, 1, 1), "NDHWC", B.IGC_TILE_DMA_64, 3),
    # point output: image rows of 588 elements, the chunk straddling a row end belongs to the last split
    ("point_tail", (40, 3, 1, 14, 14), (68, 3, 1, 14, 14), (1, 14, 14), (0, 0, 0), (1, 1, 1), "NCDHW",
     B.IGC_TILE_DMA_64, 4),
    # the 256x192 point tile split 3 ways (4, 4 and 2 steps; the straddling chunks in the last split)
    ("point_256x192_split", (300, 3, 1, 14, 14), (200, 3, 1, 14, 14), (1, 14, 14), (0, 0, 0), (1, 1, 1), "NCDHW",
     B.IGC_TILE_DMA_256x192, 3),
    # Do*Ho*Wo = 105 (scalar partial stores) and an odd element count (scalar reduction)
    ("odd_tails", (1, 16, 3, 5, 7), (25, 16, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), "NDHWC", B.IGC_TILE_DMA_64, 2),
    # the 256x256 tile, many splits of a short grid
    ("tile256_c1", (1, 64, 4, 16, 16), (64, 64, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), "NDHWC",
     B.IGC_TILE_DMA_256, 9),
    # 4-stage ring, fewer steps per split than stages
    ("ring4_short", (1, 32, 4, 8, 8), (48, 32, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), "NDHWC",
     B.IGC_TILE_DMA_64, 12),
    # more splits than steps: capped at one step each
    ("splits_beyond_steps", (1, 64, 3, 6, 6), (32, 64, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), "NDHWC",
     B.IGC_TILE_DMA_64, 1000),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_split_bf16(case):
    name, xs, ws, st, pd, dl, layout, tile, splits = case
    _announce(f"split bf16 {name}")
    lay = B.IGC_NDHWC if layout == "NDHWC" else B.IGC_NCDHW
    g = I.generator(40 + len(name), P.DEV)
    x = I.draw(xs, ("uniform", 1.0), g, P.DEV)
    w = I.draw(ws, ("uniform", 1.0), g, P.DEV)
    ref = O.conv3d(P.bits(x), P.bits(w), st, pd, dl)
    with forced(tile, splits):
        ws_t = _workspace(xs, ws, st, pd, dl, min(splits, 64))
        got_splits, ksplit, nk, plan = _plan_splits(xs, ws, st, pd, dl, lay, ws_t.numel() * 4)
        want = min(splits, nk, 64)
        assert ksplit == -(-nk // want) and got_splits == -(-nk // ksplit) and got_splits > 1, plan
        y = P.run_bf16(x, w, st, pd, dl, x_layout=layout, out=_nan_out(xs, ws, st, pd, dl), workspace=ws_t)
        y2 = P.run_bf16(x, w, st, pd, dl, x_layout=layout, out=_nan_out(xs, ws, st, pd, dl), workspace=ws_t)
    assert not torch.isnan(y).any()
    assert torch.equal(y.view(torch.int16), y2.view(torch.int16)), "split result not deterministic"
    R = int(np.prod(ws[1:]))
    P.check_close(P.y_values(y), ref, R, float(x.abs().max()), float(w.abs().max()), name)


@pytest.mark.parametrize("case", [c for c in SPLIT_CASES if c[0] in ("linear_c24", "cblock_mid_taps", "point_tail",
                                                                       "point_256x192_split",
                                                                       "odd_tails", "cblock_c128")],
                         ids=lambda c: c[0])
def test_split_integer_bit_exact(case):
    name, xs, ws, st, pd, dl, layout, tile, splits = case
    _announce(f"split integer {name}")
    g = I.generator(60, P.DEV)
    x = I.int_valued(xs, -2, 2, g, P.DEV)
    w = I.sparse_ternary(ws, 128, g, P.DEV)  # |y| <= 256: every partial sum and their total exact in fp32
    with forced(tile, splits):
        y = P.run_bf16(x, w, st, pd, dl, x_layout=layout, out=_nan_out(xs, ws, st, pd, dl),
                       workspace=_workspace(xs, ws, st, pd, dl, min(splits, 64)))
    ref = O.conv3d(P.bits(x), P.bits(w), st, pd, dl)
    assert np.array_equal(P.y_values(y), ref)


def test_split_auto_on_c1_shape():
    wl = I.WORKLOADS["c1"]
    _announce("split auto c1")
    xs, ws = wl.x_shape, wl.w_shape
    nbytes = B.conv_fwd_workspace_bytes(xs, ws, wl.stride, wl.pad, wl.dil, B.IGC_BF16, B.IGC_NDHWC)
    assert nbytes > 0
    splits, _, _, plan = _plan_splits(xs, ws, wl.stride, wl.pad, wl.dil, B.IGC_NDHWC, nbytes)
    assert splits > 1 and nbytes == splits * 1024 * 64 * 4, plan
    x, w = I.make(wl, P.DEV)
    ws_t = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=P.DEV)
    y = P.run_bf16(x, w, wl.stride, wl.pad, wl.dil, out=_nan_out(xs, ws, wl.stride, wl.pad, wl.dil), workspace=ws_t)
    ref = O.conv3d(P.bits(x), P.bits(w), wl.stride, wl.pad, wl.dil)
    P.check_close(P.y_values(y), ref, wl.reduction, float(x.abs().max()), float(w.abs().max()), "c1 split")
    # without a workspace conv_fwd_ws is conv_fwd, bit for bit
    y_plain = P.run_bf16(x, w, wl.stride, wl.pad, wl.dil)
    y_nows = P.run_bf16(x, w, wl.stride, wl.pad, wl.dil, workspace=torch.empty(0, device=P.DEV))
    assert torch.equal(y_plain.view(torch.int16), y_nows.view(torch.int16))


def test_split_workspace_too_small_lowers_splits():
    wl = I.WORKLOADS["c1"]
    _announce("split small workspace")
    xs, ws, st, pd, dl = wl.x_shape, wl.w_shape, wl.stride, wl.pad, wl.dil
    full = B.conv_fwd_workspace_bytes(xs, ws, st, pd, dl, B.IGC_BF16, B.IGC_NDHWC)
    small = 2 * 1024 * 64 * 4 + 100  # room for two slices
    assert small < full
    splits, _, _, plan = _plan_splits(xs, ws, st, pd, dl, B.IGC_NDHWC, small)
    assert splits == 2, plan
    x, w = I.make(wl, P.DEV)
    ws_t = torch.full((small // 4 + 1,), float("nan"), dtype=torch.float32, device=P.DEV)
    guard = ws_t[small // 4:].clone()
    y = P.run_bf16(x, w, st, pd, dl, out=_nan_out(xs, ws, st, pd, dl), workspace=ws_t)
    # nothing past workspace_bytes is touched (here: past the two slices)
    assert torch.equal(ws_t[2 * 1024 * 64:].isnan(), torch.ones_like(ws_t[2 * 1024 * 64:], dtype=torch.bool))
    assert guard.isnan().all()
    ref = O.conv3d(P.bits(x), P.bits(w), st, pd, dl)
    P.check_close(P.y_values(y), ref, wl.reduction, float(x.abs().max()), float(w.abs().max()), "c1 two slices")


@pytest.mark.parametrize("tile,splits", [(-1, 0), (B.IGC_TILE_DMA_64, 3), (B.IGC_TILE_DMA_256, 9)])
def test_split_fp8(tile, splits):
    _announce(f"split fp8 tile {tile} splits {splits}")
    xs, ws, st, pd, dl = (1, 64, 4, 16, 16), (64, 64, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)
    g = I.generator(61, P.DEV)
    x = I.draw(xs, ("normal", 1.0), g, P.DEV)
    w = I.draw(ws, ("normal", 1.0 / np.sqrt(np.prod(ws[1:]))), g, P.DEV)
    ops = P.Fp8Operands(x, w)
    with forced(tile, splits):
        nbytes = B.conv_fwd_workspace_bytes(xs, ws, st, pd, dl, B.IGC_FP8_E4M3FN, B.IGC_NDHWC)
        got, _, _, plan = _plan_splits(xs, ws, st, pd, dl, B.IGC_NDHWC, nbytes, B.IGC_FP8_E4M3FN)
        assert got > 1, plan
        ws_t = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=P.DEV)
        y = P.run_fp8(ops, xs, ws, st, pd, dl, out=_nan_out(xs, ws, st, pd, dl), workspace=ws_t)
    torch.cuda.synchronize()
    sx, sw = float(ops.ref_scales[0]), float(ops.ref_scales[2])
    ref = O.conv3d(ops.ref_xq, ops.ref_wq, st, pd, dl, sx=sx, sw=sw)
    mx = float(np.abs(O.e4m3_decode(ops.ref_xq)).max()) * sx
    mw = float(np.abs(O.e4m3_decode(ops.ref_wq)).max()) * sw
    P.check_close(P.y_values(y), ref, int(np.prod(ws[1:])), mx, mw, "fp8 split")


def test_split_fp8_integer_bit_exact():
    _announce("split fp8 integer, unit scales")
    xs, ws, st, pd, dl = (1, 64, 5, 9, 11), (80, 64, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)
    g = I.generator(62, P.DEV)
    x = I.int_valued(xs, -2, 2, g, P.DEV)
    w = I.sparse_ternary(ws, 128, g, P.DEV)
    ones = torch.ones(4, dtype=torch.float32, device=P.DEV)
    n, c, d, h, wd = xs
    xq = torch.empty((n, d, h, wd, c), dtype=torch.uint8, device=P.DEV)
    B.conv_pack_x(x, xq, xs, B.IGC_FP8_E4M3FN, ones[0:2])
    wq = torch.empty((ws[0], B.conv_packed_w_cols(ws, B.IGC_FP8_E4M3FN)), dtype=torch.uint8, device=P.DEV)
    B.conv_pack_w(w, wq, ws, B.IGC_FP8_E4M3FN, B.IGC_NDHWC, ones[2:4])
    y = _nan_out(xs, ws, st, pd, dl)
    with forced(B.IGC_TILE_DMA_64, 4):
        B.conv_fwd_ws(xq, wq, y, xs, ws, st, pd, dl, B.IGC_FP8_E4M3FN, B.IGC_NDHWC, ones,
                      workspace=_workspace(xs, ws, st, pd, dl, 4))
    torch.cuda.synchronize()
    ref = O.conv3d(P.bits(x), P.bits(w), st, pd, dl)
    assert np.array_equal(P.y_values(y), ref)


# ------------------------------------------------------------------ tail split of the buffer-addressed tiles

class capped_cus:
    """Plan the tail split for `n` CUs (and cap persistent grids), for the duration of a with-block."""

    def __init__(self, n):
        self.n = n

    def __enter__(self):
        B.conv_debug_force_grid(self.n)

    def __exit__(self, *exc):
        B.conv_debug_force_grid(0)


def _tail(plan):
    kv = dict(item.split("=") for item in plan.split())
    r, s = kv["tail"].split("/")
    return int(r), int(s)


# name, x, w, stride, pad, dil, CUs stood in for, expected (tail tiles, splits); every reduction has >= 96 steps
TAIL_CASES = [
    # 6 tiles of 256 x 256 on 4 "CUs": 2 tail tiles in 2 splits of 54 steps; tiles stay inside one image
    ("tail_generic_6_tiles", (1, 256, 4, 16, 24), (256, 256, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), 4, (2, 2)),
    # 8 M tiles x 2 K tiles on 12: 4 tail tiles in 3 splits of 36 steps; ragged M, K = 300, two images
    ("tail_ragged_two_images", (2, 256, 3, 11, 29), (300, 256, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), 12,
     (4, 3)),
    # temporal 3x1x1 with C = 2048 (96 steps): 5 tiles on 4, one tail tile in 4 splits of 24 steps
    ("tail_temporal", (1, 2048, 5, 16, 16), (256, 2048, 3, 1, 1), (1, 1, 1), (1, 0, 0), (1, 1, 1), 4, (1, 4)),
    # 17 tiles on 16: one tail tile in 8 splits of its 108 steps, which start mid-way through a channel block's taps
    ("tail_one_tile_8_splits", (1, 256, 4, 17, 64), (256, 256, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), 16, (1, 8)),
]


@pytest.mark.parametrize("tile", [B.IGC_TILE_BUF, B.IGC_TILE_BUF_AHEAD, B.IGC_TILE_BUF_PINGPONG])
@pytest.mark.parametrize("case", TAIL_CASES, ids=[c[0] for c in TAIL_CASES])
def test_tail_split_bf16(case, tile):
    name, xs, ws, st, pd, dl, cus, want = case
    _announce(f"tail split bf16 tile {tile} {name}")
    g = I.generator(95, P.DEV)
    x = I.draw(xs, ("uniform", 1.0), g, P.DEV)
    w = I.draw(ws, ("uniform", 1.0), g, P.DEV)
    with forced(tile=tile), capped_cus(cus):
        nbytes = B.conv_fwd_workspace_bytes(xs, ws, st, pd, dl, B.IGC_BF16, B.IGC_NDHWC)
        assert _tail(B.conv_plan_ws(xs, ws, st, pd, dl, B.IGC_BF16, B.IGC_NDHWC, nbytes)) == want
        assert nbytes == want[0] * want[1] * 256 * 256 * 4
        wsp = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=P.DEV)
        y = P.run_bf16(x, w, st, pd, dl, out=_nan_out(xs, ws, st, pd, dl), workspace=wsp)
        y_plain = P.run_bf16(x, w, st, pd, dl)
    assert not torch.isnan(y).any()
    ref = O.conv3d(P.bits(x), P.bits(w), st, pd, dl)
    P.check_close(P.y_values(y), ref, int(np.prod(ws[1:])), float(x.abs().max()), float(w.abs().max()), name)
    # outside the tail tiles the bits are conv_fwd's; inside, another summation order
    differ = (y.view(torch.int16) != y_plain.view(torch.int16)).float().mean().item()
    assert differ < 0.5


@pytest.mark.parametrize("tile", [B.IGC_TILE_BUF, B.IGC_TILE_BUF_AHEAD, B.IGC_TILE_BUF_PINGPONG])
@pytest.mark.parametrize("case", TAIL_CASES, ids=[c[0] for c in TAIL_CASES])
def test_tail_split_integer_bit_exact(case, tile):
    name, xs, ws, st, pd, dl, cus, want = case
    _announce(f"tail split integer tile {tile} {name}")
    g = I.generator(96, P.DEV)
    x = I.int_valued(xs, -2, 2, g, P.DEV)
    w = I.sparse_ternary(ws, 128, g, P.DEV)
    bias = I.int_valued((ws[0],), -8, 8, g, P.DEV).float()
    amax = torch.full((1,), float("nan"), dtype=torch.float32, device=P.DEV)
    with forced(tile=tile), capped_cus(cus):
        nbytes = B.conv_fwd_workspace_bytes(xs, ws, st, pd, dl, B.IGC_BF16, B.IGC_NDHWC)
        wsp = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=P.DEV)
        y = P.run_bf16(x, w, st, pd, dl, out=_nan_out(xs, ws, st, pd, dl), workspace=wsp, bias=bias, amax=amax)
    ref = O.conv3d(P.bits(x), P.bits(w), st, pd, dl, bias=bias.cpu().numpy())
    assert np.array_equal(P.y_values(y), ref)
    assert float(amax) == float(np.abs(ref).max())


@pytest.mark.parametrize("tile", [B.IGC_TILE_BUF, B.IGC_TILE_BUF_AHEAD, B.IGC_TILE_BUF_PINGPONG])
def test_tail_split_fp8(tile):
    # C = 512 in fp8: 108 steps of 128 channels, 4 tail tiles in 3 splits
    name, xs, ws, st, pd, dl, cus, want = ("tail_fp8_ragged", (2, 512, 3, 11, 29), (300, 512, 3, 3, 3), (1, 1, 1),
                                           (1, 1, 1), (1, 1, 1), 12, (4, 3))
    _announce(f"tail split fp8 tile {tile} {name}")
    g = I.generator(97, P.DEV)
    x = I.draw(xs, ("normal", 1.0), g, P.DEV)
    w = I.draw(ws, ("normal", 1.0 / np.sqrt(np.prod(ws[1:]))), g, P.DEV)
    ops = P.Fp8Operands(x, w)
    with forced(tile=tile), capped_cus(cus):
        nbytes = B.conv_fwd_workspace_bytes(xs, ws, st, pd, dl, B.IGC_FP8_E4M3FN, B.IGC_NDHWC)
        plan = B.conv_plan_ws(xs, ws, st, pd, dl, B.IGC_FP8_E4M3FN, B.IGC_NDHWC, nbytes)
        assert _tail(plan) == want, plan
        wsp = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=P.DEV)
        y = P.run_fp8(ops, xs, ws, st, pd, dl, out=_nan_out(xs, ws, st, pd, dl), workspace=wsp)
    sx, sw = float(ops.ref_scales[0]), float(ops.ref_scales[2])
    ref = O.conv3d(ops.ref_xq, ops.ref_wq, st, pd, dl, sx=sx, sw=sw)
    mx = float(np.abs(O.e4m3_decode(ops.ref_xq)).max()) * sx
    mw = float(np.abs(O.e4m3_decode(ops.ref_wq)).max()) * sw
    P.check_close(P.y_values(y), ref, int(np.prod(ws[1:])), mx, mw, name)


def test_tail_split_needs_its_workspace():
    # 16 bytes short of the tail split's need: the call runs as conv_fwd, bit for bit
    name, xs, ws, st, pd, dl, cus, want = TAIL_CASES[0]
    _announce("tail split, workspace 16 bytes short")
    g = I.generator(98, P.DEV)
    x = I.draw(xs, ("uniform", 1.0), g, P.DEV)
    w = I.draw(ws, ("uniform", 1.0), g, P.DEV)
    with forced(tile=B.IGC_TILE_BUF), capped_cus(cus):
        nbytes = B.conv_fwd_workspace_bytes(xs, ws, st, pd, dl, B.IGC_BF16, B.IGC_NDHWC)
        assert _tail(B.conv_plan_ws(xs, ws, st, pd, dl, B.IGC_BF16, B.IGC_NDHWC, nbytes - 16)) == (0, 1)
        wsp = torch.full(((nbytes - 16) // 4,), float("nan"), dtype=torch.float32, device=P.DEV)
        y_ws = P.run_bf16(x, w, st, pd, dl, workspace=wsp)
        y_plain = P.run_bf16(x, w, st, pd, dl)
    assert torch.equal(y_ws.view(torch.int16), y_plain.view(torch.int16))


# The 128x128 buffer tile runs two workgroups per CU, so a round holds twice the CUs' tiles. 34 x 2 tiles of
# 128 x 128 on 16 CUs (32 slots): 64 in two full rounds, 4 tail tiles in 8 splits of the 108 steps (which start
# mid-way through a channel block's taps), for bf16 (C = 256) and fp8 (C = 512).
TAIL_128_CASES = [
    ("bf16", B.IGC_BF16, (1, 256, 4, 17, 64), (256, 256, 3, 3, 3), (4, 8)),
    ("fp8", B.IGC_FP8_E4M3FN, (1, 512, 4, 17, 64), (256, 512, 3, 3, 3), (4, 8)),
]


@pytest.mark.parametrize("case", TAIL_128_CASES, ids=[c[0] for c in TAIL_128_CASES])
def test_tail_split_128_tile_integer_bit_exact(case):
    name, dt, xs, ws, want = case
    st, pd, dl, cus = (1, 1, 1), (1, 1, 1), (1, 1, 1), 16
    _announce(f"tail split, 128x128 buffer tile, {name}")
    g = I.generator(99, P.DEV)
    x = I.int_valued(xs, -2, 2, g, P.DEV)
    w = I.sparse_ternary(ws, 128, g, P.DEV)
    with forced(tile=B.IGC_TILE_BUF_128), capped_cus(cus):
        nbytes = B.conv_fwd_workspace_bytes(xs, ws, st, pd, dl, dt, B.IGC_NDHWC)
        plan = B.conv_plan_ws(xs, ws, st, pd, dl, dt, B.IGC_NDHWC, nbytes)
        assert _tail(plan) == want, plan
        assert nbytes == want[0] * want[1] * 128 * 128 * 4
        wsp = torch.full((nbytes // 4,), float("nan"), dtype=torch.float32, device=P.DEV)
        if dt == B.IGC_BF16:
            y = P.run_bf16(x, w, st, pd, dl, out=_nan_out(xs, ws, st, pd, dl), workspace=wsp)
        else:
            ones = torch.ones(4, dtype=torch.float32, device=P.DEV)  # integers |v| <= 2 are exact E4M3FN codes
            n, c, d, h, wd = xs
            xq = torch.empty((n, d, h, wd, c), dtype=torch.uint8, device=P.DEV)
            B.conv_pack_x(x, xq, xs, dt, ones[0:2])
            wq = torch.empty((ws[0], B.conv_packed_w_cols(ws, dt)), dtype=torch.uint8, device=P.DEV)
            B.conv_pack_w(w, wq, ws, dt, B.IGC_NDHWC, ones[2:4])
            y = _nan_out(xs, ws, st, pd, dl)
            B.conv_fwd_ws(xq, wq, y, xs, ws, st, pd, dl, dt, B.IGC_NDHWC, ones, workspace=wsp)
            torch.cuda.synchronize()
    ref = O.conv3d(P.bits(x), P.bits(w), st, pd, dl)
    assert np.array_equal(P.y_values(y), ref)
