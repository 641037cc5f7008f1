"""GPU parity of the HIP path against the CPU oracle at sizes the oracle finishes
in seconds (several tiles and ragged tails), plus the exact cases.

Every case prints its name before touching the GPU so that a failing run
names it.
"""

import zlib

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from implicit_gemm_convolution_conv_amd import binding as B
from implicit_gemm_convolution_conv_amd import inputs as I
from oracle import oracle as O

import parity as P

pytestmark = pytest.mark.gpu


def _announce(name):
    print(f"[case] {name}", flush=True)


class forced:
    """Force a path / tile / raster group for the duration of a with-block."""

    def __init__(self, path=B.IGC_PATH_AUTO, tile=-1, group_m=0):
        self.args = (path, tile, group_m)

    def __enter__(self):
        B.conv_debug_force(*self.args)

    def __exit__(self, *exc):
        B.conv_debug_force(B.IGC_PATH_AUTO, -1, 0)


def _bf16_case(name, xs, ws, st, pd, dl, seed, dist=("uniform", 1.0), x_layout="NDHWC"):
    _announce(name)
    g = I.generator(seed, P.DEV)
    x = I.draw(xs, dist, g, P.DEV)
    w = I.draw(ws, dist, g, P.DEV)
    y = P.run_bf16(x, w, st, pd, dl, x_layout=x_layout)
    ref = O.conv3d(P.bits(x), P.bits(w), st, pd, dl)
    R = int(np.prod(ws[1:]))
    P.check_close(P.y_values(y), ref, R, float(x.abs().max()), float(w.abs().max()), name)
    return x, w, y


def test_c1_full_bf16():
    wl = I.WORKLOADS["c1"]
    _announce("c1 full")
    x, w = I.make(wl, P.DEV)
    y = P.run_bf16(x, w, wl.stride, wl.pad, wl.dil)
    ref = O.conv3d(P.bits(x), P.bits(w), wl.stride, wl.pad, wl.dil)
    P.check_close(P.y_values(y), ref, wl.reduction, float(x.abs().max()), float(w.abs().max()), "c1")


GEOMS = [
    # name, x (N,C,D,H,W), w (K,C,T,R,S), stride, pad, dil
    ("ragged_linear_c24", (2, 24, 5, 7, 9), (40, 24, 3, 3, 3), (1, 2, 1), (1, 1, 2), (1, 1, 2)),
    ("ragged_c72_k136", (1, 72, 4, 9, 11), (136, 72, 2, 3, 3), (2, 1, 1), (1, 1, 1), (1, 2, 1)),
    ("c8_tiny", (3, 8, 3, 5, 6), (16, 8, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)),
    ("c128_cblock_multi_tile", (2, 128, 6, 10, 12), (200, 128, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)),
    ("asym_pad_stride2", (1, 64, 7, 13, 10), (72, 64, 3, 5, 1), (2, 2, 1), (0, 2, 0), (1, 1, 1)),
    ("temporal_3x1x1", (2, 64, 9, 6, 7), (96, 64, 3, 1, 1), (1, 1, 1), (1, 0, 0), (1, 1, 1)),
    ("temporal_strided_dilated", (1, 32, 11, 5, 9), (48, 32, 3, 1, 1), (2, 1, 1), (2, 0, 0), (2, 1, 1)),
    ("pointwise_1x1x1", (2, 48, 3, 7, 5), (80, 48, 1, 1, 1), (1, 1, 1), (0, 0, 0), (1, 1, 1)),
    # NDHWC 1x1x1, stride 1: the flat [N*D*H*W, C] x [C, K] GEMM, 9 row tiles and 2 column tiles, both ragged
    ("pointwise_1x1x1_flat_multi_tile", (2, 96, 5, 17, 13), (300, 96, 1, 1, 1), (1, 1, 1), (0, 0, 0), (1, 1, 1)),
    ("odd_spatial_vec_off", (1, 16, 3, 5, 7), (24, 16, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)),
]


@pytest.mark.parametrize("case", GEOMS, ids=[g[0] for g in GEOMS])
def test_bf16_shapes(case):
    name, xs, ws, st, pd, dl = case
    _bf16_case(name, xs, ws, st, pd, dl, seed=zlib.crc32(name.encode()) % 1000)


@pytest.mark.parametrize("layout", ["NCDHW", "NDHWC"])
@pytest.mark.parametrize("k", [200, 198])
def test_point_output_bf16(layout, k):
    # patch-embed geometry at a reduced batch: 14x14 filter, stride 14, C=3 (R = 588, not a multiple of 64)
    _bf16_case(f"point_{layout}_k{k}", (300, 3, 1, 14, 14), (k, 3, 1, 14, 14), (1, 14, 14), (0, 0, 0), (1, 1, 1),
               seed=7, dist=("normal", 1.0), x_layout=layout)


DMA_TILES = [B.IGC_TILE_DMA_256, B.IGC_TILE_DMA_128, B.IGC_TILE_DMA_64, B.IGC_TILE_DMA_256x192]
DMA_TILES_FP8 = [B.IGC_TILE_DMA_256, B.IGC_TILE_DMA_128, B.IGC_TILE_DMA_64]
BUF_TILES_BF16 = [B.IGC_TILE_BUF, B.IGC_TILE_BUF_AHEAD, B.IGC_TILE_BUF_PINGPONG, B.IGC_TILE_BUF_128]
BUF_TILES_FP8 = BUF_TILES_BF16
POINT_TILES = DMA_TILES  # bf16 point-output GEMMs


@pytest.mark.parametrize("tile", POINT_TILES)
def test_point_output_whole_tiles(tile):
    # 512 output channels over 600 images: whole tiles leave through the LDS-staged epilogue (256x192, 128x128,
    # 64x64), the image tiles past 600 and every 256x256 tile (its ring is too small to stage a tile) store directly
    with forced(tile=tile):
        _bf16_case(f"point whole tiles, tile {tile}", (600, 3, 1, 14, 14), (512, 3, 1, 14, 14), (1, 14, 14),
                   (0, 0, 0), (1, 1, 1), seed=8, dist=("normal", 1.0), x_layout="NCDHW")
        _announce(f"point whole tiles integer, tile {tile}")
        _int_case((600, 3, 1, 14, 14), (512, 3, 1, 14, 14), (1, 14, 14), (0, 0, 0), (1, 1, 1), seed=9,
                  x_layout="NCDHW")


def test_2d_and_1d_through_3d():
    _announce("conv2d / conv1d as D=T=1 (and H=R=1)")
    g = I.generator(11, P.DEV)
    x2 = I.draw((2, 16, 1, 12, 10), ("uniform", 1.0), g, P.DEV)
    w2 = I.draw((24, 16, 1, 3, 3), ("uniform", 1.0), g, P.DEV)
    y = P.run_bf16(x2, w2, (1, 1, 2), (0, 1, 1), (1, 1, 1))
    ref = F.conv2d(x2[:, :, 0].double().cpu(), w2[:, :, 0].double().cpu(), stride=(1, 2), padding=1).numpy()
    P.check_close(P.y_values(y)[:, :, 0], ref, 16 * 9, float(x2.abs().max()), float(w2.abs().max()), "conv2d")
    x1 = I.draw((3, 32, 1, 1, 40), ("uniform", 1.0), g, P.DEV)
    w1 = I.draw((8, 32, 1, 1, 5), ("uniform", 1.0), g, P.DEV)
    y = P.run_bf16(x1, w1, (1, 1, 2), (0, 0, 2), (1, 1, 1))
    ref = F.conv1d(x1[:, :, 0, 0].double().cpu(), w1[:, :, 0, 0].double().cpu(), stride=2, padding=2).numpy()
    P.check_close(P.y_values(y)[:, :, 0, 0], ref, 32 * 5, float(x1.abs().max()), float(w1.abs().max()), "conv1d")


def test_temporal_path_matches_generic_bitwise():
    _announce("temporal vs generic, bitwise")
    g = I.generator(12, P.DEV)
    xs, ws, st, pd, dl = (2, 64, 9, 6, 7), (96, 64, 3, 1, 1), (1, 1, 1), (1, 0, 0), (1, 1, 1)
    x = I.draw(xs, ("uniform", 1.0), g, P.DEV)
    w = I.draw(ws, ("uniform", 1.0), g, P.DEV)
    assert B.conv_plan(xs, ws, st, pd, dl, B.IGC_BF16, B.IGC_NDHWC).startswith("path=temporal")
    y_fast = P.run_bf16(x, w, st, pd, dl)
    try:
        B.conv_debug_force(B.IGC_PATH_GENERIC, -1, 0)
        y_gen = P.run_bf16(x, w, st, pd, dl)
    finally:
        B.conv_debug_force(B.IGC_PATH_AUTO, -1, 0)
    assert torch.equal(y_fast.view(torch.int16), y_gen.view(torch.int16))


def test_every_tile_gives_identical_bits():
    # the reduction order over k (channel block outer, tap, 16x16 MFMA k-slices in order) is the same for every
    # tile shape, global-address or buffer-addressed
    _announce("every tile bitwise")
    g = I.generator(13, P.DEV)
    xs, ws, st, pd, dl = (1, 128, 5, 18, 20), (264, 128, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)
    x = I.draw(xs, ("uniform", 1.0), g, P.DEV)
    w = I.draw(ws, ("uniform", 1.0), g, P.DEV)
    outs = {}
    for tile in DMA_TILES + BUF_TILES_BF16:
        with forced(tile=tile):
            outs[tile] = P.run_bf16(x, w, st, pd, dl).clone()
    ref = O.conv3d(P.bits(x), P.bits(w), st, pd, dl)
    first = outs[DMA_TILES[0]]
    P.check_close(P.y_values(first), ref, 128 * 27, float(x.abs().max()), float(w.abs().max()), "tile 0")
    for tile, o in outs.items():
        assert torch.equal(o.view(torch.int16), first.view(torch.int16)), tile


def test_every_output_written_and_deterministic():
    _announce("NaN-prefilled output, repeat runs")
    g = I.generator(14, P.DEV)
    xs, ws, st, pd, dl = (2, 40, 5, 9, 7), (72, 40, 3, 3, 3), (1, 2, 1), (1, 1, 1), (1, 1, 1)
    x = I.draw(xs, ("uniform", 1.0), g, P.DEV)
    w = I.draw(ws, ("uniform", 1.0), g, P.DEV)
    shape = (2, 72) + B.conv_out_dims(xs, ws, st, pd, dl)
    y1 = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=P.DEV)
    y2 = torch.full(shape, float("nan"), dtype=torch.bfloat16, device=P.DEV)
    P.run_bf16(x, w, st, pd, dl, out=y1)
    P.run_bf16(x, w, st, pd, dl, out=y2)
    assert not torch.isnan(y1).any()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


# ------------------------------------------------------------------ exact (integer-valued) cases

def _int_case(xs, ws, st, pd, dl, seed, x_layout="NDHWC"):
    g = I.generator(seed, P.DEV)
    x = I.int_valued(xs, -2, 2, g, P.DEV)
    w = I.sparse_ternary(ws, 128, g, P.DEV)  # |y| <= 2 * 128: every partial sum exact in fp32, y exact in bf16
    y = P.run_bf16(x, w, st, pd, dl, x_layout=x_layout)
    ref = O.conv3d(P.bits(x), P.bits(w), st, pd, dl)
    assert np.array_equal(P.y_values(y), ref)


@pytest.mark.parametrize("case", [
    ((2, 64, 5, 9, 11), (96, 64, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)),
    ((1, 24, 6, 7, 8), (40, 24, 3, 2, 3), (2, 1, 2), (1, 0, 2), (1, 2, 1)),
    ((2, 128, 7, 5, 6), (64, 128, 3, 1, 1), (1, 1, 1), (1, 0, 0), (1, 1, 1)),
])
def test_integer_inputs_bit_exact_bf16(case):
    _announce(f"integer bf16 {case}")
    _int_case(*case, seed=21)


@pytest.mark.parametrize("layout", ["NCDHW", "NDHWC"])
def test_integer_inputs_bit_exact_point(layout):
    _announce(f"integer point {layout}")
    _int_case((130, 3, 1, 14, 14), (68, 3, 1, 14, 14), (1, 14, 14), (0, 0, 0), (1, 1, 1), seed=22, x_layout=layout)


def test_integer_inputs_bit_exact_fp8():
    # integers |v| <= 2 are exact E4M3FN codes with unit scales, so the fp8 path is exact too
    _announce("integer fp8, unit scales")
    g = I.generator(23, P.DEV)
    xs, ws, st, pd, dl = (1, 64, 5, 9, 11), (80, 64, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)
    x = I.int_valued(xs, -2, 2, g, P.DEV)
    w = I.sparse_ternary(ws, 128, g, P.DEV)
    ones = torch.ones(4, dtype=torch.float32, device=P.DEV)
    n, c, d, h, wd = xs
    xq = torch.empty((n, d, h, wd, c), dtype=torch.uint8, device=P.DEV)
    B.conv_pack_x(x, xq, xs, B.IGC_FP8_E4M3FN, ones[0:2])
    wq = torch.empty((ws[0], B.conv_packed_w_cols(ws, B.IGC_FP8_E4M3FN)), dtype=torch.uint8, device=P.DEV)
    B.conv_pack_w(w, wq, ws, B.IGC_FP8_E4M3FN, B.IGC_NDHWC, ones[2:4])
    y = torch.empty((n, ws[0]) + B.conv_out_dims(xs, ws, st, pd, dl), dtype=torch.bfloat16, device=P.DEV)
    B.conv_fwd(xq, wq, y, xs, ws, st, pd, dl, B.IGC_FP8_E4M3FN, B.IGC_NDHWC, ones)
    torch.cuda.synchronize()
    ref = O.conv3d(P.bits(x), P.bits(w), st, pd, dl)
    assert np.array_equal(P.y_values(y), ref)


# ------------------------------------------------------------------ fp8

FP8_GEOMS = [
    ("c1_shape_fp8", (1, 64, 4, 16, 16), (64, 64, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)),
    ("fp8_c48_linear", (2, 48, 5, 6, 7), (40, 48, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)),
    ("fp8_c256_k300", (1, 256, 4, 9, 10), (300, 256, 3, 3, 3), (1, 2, 1), (1, 1, 1), (1, 1, 1)),
    ("fp8_temporal", (1, 128, 8, 9, 10), (136, 128, 3, 1, 1), (1, 1, 1), (1, 0, 0), (1, 1, 1)),
    ("fp8_c16_tiny", (2, 16, 3, 5, 6), (24, 16, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)),
]


@pytest.mark.parametrize("case", FP8_GEOMS, ids=[g[0] for g in FP8_GEOMS])
def test_fp8_shapes(case):
    name, xs, ws, st, pd, dl = case
    _announce(name)
    g = I.generator(31, P.DEV)
    x = I.draw(xs, ("normal", 1.0), g, P.DEV)
    w = I.draw(ws, ("normal", 1.0 / np.sqrt(np.prod(ws[1:]))), g, P.DEV)
    ops = P.Fp8Operands(x, w)
    y = P.run_fp8(ops, xs, ws, st, pd, dl)
    sx, sw = float(ops.ref_scales[0]), float(ops.ref_scales[2])
    ref = O.conv3d(ops.ref_xq, ops.ref_wq, st, pd, dl, sx=sx, sw=sw)
    mx = float(np.abs(O.e4m3_decode(ops.ref_xq)).max()) * sx
    mw = float(np.abs(O.e4m3_decode(ops.ref_wq)).max()) * sw
    P.check_close(P.y_values(y), ref, int(np.prod(ws[1:])), mx, mw, name)


def test_pack_bf16_is_a_transpose():
    _announce("bf16 pack bit-exact, ragged spatial")
    g = I.generator(41, P.DEV)
    for xs in [(2, 72, 3, 5, 7), (1, 64, 4, 16, 16), (3, 8, 2, 3, 5)]:
        x = I.draw(xs, ("normal", 1.0), g, P.DEV)
        n, c, d, h, wd = xs
        out = torch.empty((n, d, h, wd, c), dtype=torch.bfloat16, device=P.DEV)
        B.conv_pack_x(x, out, xs, B.IGC_BF16)
        torch.cuda.synchronize()
        assert np.array_equal(P.bits(out), np.moveaxis(P.bits(x), 1, -1))


@pytest.mark.parametrize("order", ["sorted", "shuffled"])
def test_fp8_pack_every_bf16_pattern(order):
    # Every bf16 bit pattern (NaNs, infinities, subnormals and both zeros included), packed to fp8 under
    # several inverse scales and compared code for code with the oracle's encoder. "sorted" puts 128
    # neighbouring patterns in each lane's 16 channels x 8 positions, so most lanes hold no value that
    # can saturate; "shuffled" mixes magnitudes in every lane.
    _announce(f"fp8 pack, all 65536 bf16 patterns, {order}")
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    if order == "shuffled":
        pats = pats[np.random.default_rng(43).permutation(65536)]
    xb = np.ascontiguousarray(pats.reshape(4096, 16).T)  # x[0, c, 0, 0, s] = pats[16 s + c]
    xs = (1, 16, 1, 1, 4096)
    x = torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16).reshape(xs).to(P.DEV)
    for inv in (1.0, 448.0 / 3.0, 2.0 ** -7, 1.5, 3.0e38, 1.0e-30):
        inv32 = np.float32(inv)
        pair = torch.tensor([1.0, float(inv32)], dtype=torch.float32, device=P.DEV)
        xq = torch.empty((1, 1, 1, 4096, 16), dtype=torch.uint8, device=P.DEV)
        B.conv_pack_x(x, xq, xs, B.IGC_FP8_E4M3FN, pair)
        torch.cuda.synchronize()
        ref = O.quantize_e4m3(xb, inv32)  # (16, 4096) codes
        got = xq.cpu().numpy().reshape(4096, 16).T
        bad = np.nonzero(got != ref)
        assert bad[0].size == 0, (f"inv={inv32}: {bad[0].size} codes differ, e.g. bf16 {xb[bad][:4]} -> "
                                  f"{got[bad][:4]} vs oracle {ref[bad][:4]}")


def test_amax_handles_tails_and_zero():
    _announce("amax tails / zero tensor")
    g = I.generator(42, P.DEV)
    amax = torch.empty(1, dtype=torch.float32, device=P.DEV)
    for n in (1, 7, 8, 9, 1000003):
        t = I.draw((n,), ("normal", 3.0), g, P.DEV)
        B.conv_amax(t, n, amax)
        torch.cuda.synchronize()
        assert float(amax) == O.amax_bf16(P.bits(t))
    z = torch.zeros(100, dtype=torch.bfloat16, device=P.DEV)
    pair = torch.empty(2, dtype=torch.float32, device=P.DEV)
    B.conv_amax(z, 100, amax)
    B.conv_fp8_scales(amax, pair)
    torch.cuda.synchronize()
    assert pair.tolist() == [1.0, 1.0]


# ------------------------------------------------------------------ global-address direct-to-LDS tiles

DMA_CASES = [g for g in GEOMS if g[0] in ("ragged_linear_c24", "c128_cblock_multi_tile", "asym_pad_stride2",
                                           "temporal_3x1x1", "temporal_strided_dilated", "c8_tiny")]


@pytest.mark.parametrize("tile", DMA_TILES)
@pytest.mark.parametrize("case", DMA_CASES, ids=[g[0] for g in DMA_CASES])
def test_dma_tiles_bf16(tile, case):
    name, xs, ws, st, pd, dl = case
    with forced(tile=tile):
        _bf16_case(f"dma tile {tile} {name}", xs, ws, st, pd, dl, seed=zlib.crc32(name.encode()) % 1000)


@pytest.mark.parametrize("tile", DMA_TILES)
def test_dma_tiles_integer_bit_exact(tile):
    _announce(f"dma tile {tile} integer")
    with forced(tile=tile):
        _int_case((2, 64, 5, 9, 11), (96, 64, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), seed=24)
        _int_case((1, 24, 6, 7, 8), (40, 24, 3, 2, 3), (2, 1, 2), (1, 0, 2), (1, 2, 1), seed=25)


@pytest.mark.parametrize("tile", DMA_TILES_FP8)
@pytest.mark.parametrize("case", FP8_GEOMS, ids=[g[0] for g in FP8_GEOMS])
def test_dma_tiles_fp8(tile, case):
    name, xs, ws, st, pd, dl = case
    _announce(f"dma tile {tile} {name}")
    g = I.generator(32, P.DEV)
    x = I.draw(xs, ("normal", 1.0), g, P.DEV)
    w = I.draw(ws, ("normal", 1.0 / np.sqrt(np.prod(ws[1:]))), g, P.DEV)
    ops = P.Fp8Operands(x, w)
    with forced(tile=tile):
        y = P.run_fp8(ops, xs, ws, st, pd, dl)
    sx, sw = float(ops.ref_scales[0]), float(ops.ref_scales[2])
    ref = O.conv3d(ops.ref_xq, ops.ref_wq, st, pd, dl, sx=sx, sw=sw)
    mx = float(np.abs(O.e4m3_decode(ops.ref_xq)).max()) * sx
    mw = float(np.abs(O.e4m3_decode(ops.ref_wq)).max()) * sw
    P.check_close(P.y_values(y), ref, int(np.prod(ws[1:])), mx, mw, name)


@pytest.mark.parametrize("tile", POINT_TILES)
@pytest.mark.parametrize("layout", ["NCDHW", "NDHWC"])
def test_point_output_dma_tiles(tile, layout):
    with forced(tile=tile):
        _bf16_case(f"point dma tile {tile} {layout}", (300, 3, 1, 14, 14), (200, 3, 1, 14, 14), (1, 14, 14),
                   (0, 0, 0), (1, 1, 1), seed=8, dist=("normal", 1.0), x_layout=layout)
        _bf16_case(f"point dma tile {tile} {layout} k198 odd R", (77, 6, 1, 3, 7), (198, 6, 1, 3, 7), (1, 3, 7),
                   (0, 0, 0), (1, 1, 1), seed=9, dist=("normal", 1.0), x_layout=layout)


@pytest.mark.parametrize("tile", POINT_TILES)
def test_point_output_dma_integer_bit_exact(tile):
    _announce(f"integer point dma tile {tile}")
    with forced(tile=tile):
        _int_case((130, 3, 1, 14, 14), (68, 3, 1, 14, 14), (1, 14, 14), (0, 0, 0), (1, 1, 1), seed=26,
                  x_layout="NCDHW")


@pytest.mark.parametrize("tile", [-1] + DMA_TILES_FP8)
def test_point_output_fp8(tile):
    # channel-last fp8 patch embed: 7x7 filter, stride 7, C=16 (the fp8 pack needs C % 16 == 0)
    name = f"fp8 point tile {tile}"
    _announce(name)
    xs, ws, st, pd, dl = (100, 16, 1, 7, 7), (72, 16, 1, 7, 7), (1, 7, 7), (0, 0, 0), (1, 1, 1)
    g = I.generator(33, P.DEV)
    x = I.draw(xs, ("normal", 1.0), g, P.DEV)
    w = I.draw(ws, ("normal", 1.0 / np.sqrt(np.prod(ws[1:]))), g, P.DEV)
    ops = P.Fp8Operands(x, w)
    with forced(tile=tile):
        assert B.conv_plan(xs, ws, st, pd, dl, B.IGC_FP8_E4M3FN, B.IGC_NDHWC).startswith("path=point")
        y = P.run_fp8(ops, xs, ws, st, pd, dl)
    sx, sw = float(ops.ref_scales[0]), float(ops.ref_scales[2])
    ref = O.conv3d(ops.ref_xq, ops.ref_wq, st, pd, dl, sx=sx, sw=sw)
    mx = float(np.abs(O.e4m3_decode(ops.ref_xq)).max()) * sx
    mw = float(np.abs(O.e4m3_decode(ops.ref_wq)).max()) * sw
    P.check_close(P.y_values(y), ref, int(np.prod(ws[1:])), mx, mw, name)


# ------------------------------------------------------------------ buffer-addressed tiles

BUF_CASES = [g for g in GEOMS if g[0] in ("c128_cblock_multi_tile", "asym_pad_stride2", "temporal_3x1x1")] + [
    ("dilated_c64", (1, 64, 6, 11, 13), (80, 64, 3, 3, 3), (1, 1, 1), (2, 1, 2), (2, 1, 2)),
    ("c192_k300_two_col_tiles", (1, 192, 4, 9, 10), (300, 192, 3, 3, 3), (1, 2, 1), (1, 1, 1), (1, 1, 1)),
    ("pointwise_c64_one_step", (2, 64, 3, 7, 5), (80, 64, 1, 1, 1), (1, 1, 1), (0, 0, 0), (1, 1, 1)),
    ("generic_1x1x2_two_steps", (1, 64, 3, 6, 9), (48, 64, 1, 1, 2), (1, 1, 1), (0, 0, 1), (1, 1, 1)),
    ("temporal_c128_t1", (1, 128, 3, 5, 6), (40, 128, 1, 1, 1), (1, 1, 1), (0, 0, 0), (1, 1, 1)),
    # windows that cross output planes and images, strided and dilated columns, odd output rows
    ("windows_cross_planes_images", (3, 64, 3, 5, 21), (72, 64, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)),
    ("windows_stride2_dilated", (1, 64, 7, 12, 37), (64, 64, 2, 3, 3), (2, 2, 1), (1, 2, 2), (2, 2, 2)),
    ("windows_2d_5x5", (2, 128, 1, 19, 37), (96, 128, 1, 5, 5), (1, 1, 1), (0, 2, 2), (1, 1, 1)),
    # time padding beyond the filter's reach: a tile's first input plane clamps to its image's last plane
    ("pad_beyond_reach_images", (3, 64, 4, 5, 6), (40, 64, 2, 2, 2), (1, 1, 1), (3, 1, 1), (1, 1, 1)),
    # whole 256x256 tiles inside each image (P = 1024, K = 256): the LDS-staged epilogue; a second image
    ("lds_epilogue_two_images", (2, 128, 4, 16, 16), (256, 128, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)),
    # P = 1800: 7 whole tiles per image through LDS, the tile across the image boundary stored directly
    ("lds_epilogue_straddle", (2, 64, 5, 18, 20), (256, 64, 3, 1, 1), (1, 1, 1), (1, 0, 0), (1, 1, 1)),
]


@pytest.mark.parametrize("tile", BUF_TILES_BF16)
@pytest.mark.parametrize("case", BUF_CASES, ids=[g[0] for g in BUF_CASES])
def test_buffer_tiles_bf16(tile, case):
    name, xs, ws, st, pd, dl = case
    with forced(tile=tile):
        assert "loads=buffer-lds" in B.conv_plan(xs, ws, st, pd, dl, B.IGC_BF16, B.IGC_NDHWC)
        _bf16_case(f"buffer tile {tile} {name}", xs, ws, st, pd, dl, seed=zlib.crc32(name.encode()) % 1000)


@pytest.mark.parametrize("tile", BUF_TILES_BF16)
def test_buffer_tiles_integer_bit_exact(tile):
    _announce(f"buffer tile {tile} integer")
    with forced(tile=tile):
        _int_case((2, 64, 5, 9, 11), (96, 64, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), seed=29)
        _int_case((1, 128, 6, 7, 8), (40, 128, 3, 2, 3), (2, 1, 2), (1, 0, 2), (1, 2, 1), seed=30)


@pytest.mark.parametrize("tile", BUF_TILES_FP8)
@pytest.mark.parametrize("case", [g for g in FP8_GEOMS if g[0] in ("fp8_c256_k300", "fp8_temporal")],
                         ids=lambda g: g[0])
def test_buffer_tiles_fp8(tile, case):
    name, xs, ws, st, pd, dl = case
    _announce(f"buffer tile {tile} {name}")
    g = I.generator(35, P.DEV)
    x = I.draw(xs, ("normal", 1.0), g, P.DEV)
    w = I.draw(ws, ("normal", 1.0 / np.sqrt(np.prod(ws[1:]))), g, P.DEV)
    ops = P.Fp8Operands(x, w)
    with forced(tile=tile):
        y = P.run_fp8(ops, xs, ws, st, pd, dl)
    sx, sw = float(ops.ref_scales[0]), float(ops.ref_scales[2])
    ref = O.conv3d(ops.ref_xq, ops.ref_wq, st, pd, dl, sx=sx, sw=sw)
    mx = float(np.abs(O.e4m3_decode(ops.ref_xq)).max()) * sx
    mw = float(np.abs(O.e4m3_decode(ops.ref_wq)).max()) * sw
    P.check_close(P.y_values(y), ref, int(np.prod(ws[1:])), mx, mw, name)


@pytest.mark.parametrize("dtype", ["bf16", "fp8"])
def test_temporal_tap_raster(dtype):
    # 3x1x1 over 8 planes of 32 x 32: taps 1024 rows (4 tiles) apart, 32 M tiles x 4 K tiles, raster groups of
    # 8: one block of 8 groups whose members are one tap apart. Each tile is still computed once: the output
    # equals the consecutive raster's bit for bit, and the oracle within tolerance.
    _announce(f"temporal tap raster {dtype}")
    xs, ws, st, pd, dl = (1, 128, 8, 32, 32), (1024, 128, 3, 1, 1), (1, 1, 1), (1, 0, 0), (1, 1, 1)
    g = I.generator(37, P.DEV)
    x = I.draw(xs, ("normal", 1.0), g, P.DEV)
    w = I.draw(ws, ("normal", 1.0 / np.sqrt(np.prod(ws[1:]))), g, P.DEV)
    dt = B.IGC_BF16 if dtype == "bf16" else B.IGC_FP8_E4M3FN
    if dtype == "bf16":
        run = lambda: P.run_bf16(x, w, st, pd, dl)
    else:
        ops = P.Fp8Operands(x, w)
        run = lambda: P.run_fp8(ops, xs, ws, st, pd, dl)
    with forced(tile=B.IGC_TILE_BUF):  # the 128-tile grid would otherwise take the 128x128 direct-to-LDS tile
        kv = dict(item.split("=") for item in B.conv_plan(xs, ws, st, pd, dl, dt, B.IGC_NDHWC).split())
        assert (kv["path"], kv["tap"], kv["group_m"], kv["grid"]) == ("temporal", "4", "8", "128"), kv
        y_tap = run().clone()
        try:
            B.conv_debug_force_tap_raster(-1)
            assert "tap=0" in B.conv_plan(xs, ws, st, pd, dl, dt, B.IGC_NDHWC)
            y_off = run().clone()
        finally:
            B.conv_debug_force_tap_raster(0)
    assert torch.equal(y_tap.view(torch.int16), y_off.view(torch.int16))
    if dtype == "bf16":
        ref = O.conv3d(P.bits(x), P.bits(w), st, pd, dl)
        P.check_close(P.y_values(y_tap), ref, int(np.prod(ws[1:])), float(x.abs().max()), float(w.abs().max()),
                      "tap raster")
    else:
        sx, sw = float(ops.ref_scales[0]), float(ops.ref_scales[2])
        ref = O.conv3d(ops.ref_xq, ops.ref_wq, st, pd, dl, sx=sx, sw=sw)
        mx = float(np.abs(O.e4m3_decode(ops.ref_xq)).max()) * sx
        mw = float(np.abs(O.e4m3_decode(ops.ref_wq)).max()) * sw
        P.check_close(P.y_values(y_tap), ref, int(np.prod(ws[1:])), mx, mw, "tap raster fp8")


# ------------------------------------------------------------------ 1x1x1 filters on NCDHW activations (no transpose)

PW_CASES = [
    ("pw_c64_k48_two_position_tiles", (1, 64, 4, 8, 16), (48, 64, 1, 1, 1)),
    ("pw_c40_k100_ragged", (2, 40, 3, 5, 8), (100, 40, 1, 1, 1)),      # C < 64, two channel tiles, S = 120
    ("pw_c512_k48_three_images", (3, 512, 2, 6, 20), (48, 512, 1, 1, 1)),  # 8 reduction steps
    ("pw_c200_k64_tail", (1, 200, 5, 7, 24), (64, 200, 1, 1, 1)),      # C % 64 != 0, S = 840
    ("pw_c8_k16_tiny", (1, 8, 1, 1, 8), (16, 8, 1, 1, 1)),
    ("pw_2d", (2, 96, 1, 12, 30), (72, 96, 1, 1, 1)),
]


@pytest.mark.parametrize("case", PW_CASES, ids=[c[0] for c in PW_CASES])
def test_pointwise_ncdhw(case):
    name, xs, ws = case
    one, zero = (1, 1, 1), (0, 0, 0)
    assert B.conv_plan(xs, ws, one, zero, one, B.IGC_BF16, B.IGC_NCDHW).startswith("path=pointwise")
    _bf16_case(f"pointwise {name}", xs, ws, one, zero, one, seed=zlib.crc32(name.encode()) % 1000,
               dist=("normal", 1.0), x_layout="NCDHW")


def test_pointwise_integer_bit_exact():
    _announce("pointwise integer")
    _int_case((2, 72, 3, 4, 10), (80, 72, 1, 1, 1), (1, 1, 1), (0, 0, 0), (1, 1, 1), seed=31, x_layout="NCDHW")


def test_pointwise_matches_transposed_path_bitwise():
    # same reduction order as the NDHWC temporal path (64-channel steps, two 32-channel MFMA slices), same bits;
    # the NaN-prefilled output checks that every element is written
    _announce("pointwise vs pack + temporal path, bitwise")
    g = I.generator(17, P.DEV)
    xs, ws, one, zero = (2, 192, 3, 10, 24), (88, 192, 1, 1, 1), (1, 1, 1), (0, 0, 0)
    x = I.draw(xs, ("normal", 1.0), g, P.DEV)
    w = I.draw(ws, ("normal", 0.1), g, P.DEV)
    y1 = torch.full((xs[0], ws[0]) + xs[2:], float("nan"), dtype=torch.bfloat16, device=P.DEV)
    P.run_bf16(x, w, one, zero, one, x_layout="NCDHW", out=y1)
    y2 = P.run_bf16(x, w, one, zero, one, x_layout="NDHWC")
    assert not torch.isnan(y1).any()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
