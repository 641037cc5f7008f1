"""C-ABI library: loads, exports every declared symbol, host-side logic (no GPU work)."""

import os
import re

import pytest

from implicit_gemm_convolution_conv_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    text = open(os.path.join(ROOT, "include", "igconv.h")).read()
    return sorted(set(re.findall(r"IGC_API\s+[\w\s\*]*?\b(conv_\w+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert _declared() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = B.load()
    for name in _declared():
        assert hasattr(lib, name), name


def test_header_constants_match_binding():
    text = open(os.path.join(ROOT, "include", "igconv.h")).read()
    consts = dict(re.findall(r"#define (IGC_\w+)\s+\(?(-?\d+)\)?", text))
    for name, value in consts.items():
        assert getattr(B, name) == int(value), name


@pytest.mark.parametrize("geom", [
    ((2, 3, 4, 5, 6), (2, 3, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)),
    ((1, 3, 5, 4, 7), (4, 3, 2, 3, 1), (1, 2, 1), (0, 1, 0), (1, 1, 1)),
    ((2, 2, 6, 7, 5), (3, 2, 3, 2, 3), (2, 1, 2), (2, 0, 1), (1, 2, 1)),
    ((1, 4, 7, 6, 8), (2, 4, 2, 2, 3), (1, 1, 2), (1, 2, 0), (2, 1, 2)),
])
def test_out_dims_match_torch(geom):
    import torch
    import torch.nn.functional as F
    xs, ws, st, pd, dl = geom
    y = F.conv3d(torch.zeros(xs), torch.zeros(ws), stride=st, padding=pd, dilation=dl)
    assert B.conv_out_dims(xs, ws, st, pd, dl) == tuple(y.shape[2:])


def test_packed_cols():
    assert B.conv_packed_w_cols((64, 64, 3, 3, 3), B.IGC_BF16) == 1728
    assert B.conv_packed_w_cols((1280, 3, 1, 14, 14), B.IGC_BF16) == 640
    assert B.conv_packed_w_cols((1280, 3, 1, 14, 14), B.IGC_FP8_E4M3FN) == 640
    assert B.conv_packed_w_cols((8, 16, 1, 1, 1), B.IGC_FP8_E4M3FN) == 128
    assert B.conv_packed_w_cols((2048, 2048, 3, 3, 3), B.IGC_FP8_E4M3FN) == 55296


def _plan(x, w, st=(1, 1, 1), pd=(0, 0, 0), dl=(1, 1, 1), dt=B.IGC_BF16, lay=B.IGC_NDHWC):
    return dict(kv.split("=") for kv in B.conv_plan(x, w, st, pd, dl, dt, lay).split())


def test_path_selection():
    assert _plan((9500, 3, 1, 14, 14), (1280, 3, 1, 14, 14), (1, 14, 14), lay=B.IGC_NCDHW)["path"] == "point"
    assert _plan((2, 16, 1, 14, 14), (32, 16, 1, 14, 14), (1, 14, 14))["path"] == "point"
    # input larger than the filter: still one output position, but not a plain GEMM over the batch
    assert _plan((2, 16, 1, 15, 15), (32, 16, 1, 14, 14), (1, 14, 14))["path"] == "generic"
    p = _plan((1, 2048, 60, 80, 45), (2048, 2048, 3, 1, 1), pd=(1, 0, 0), dt=B.IGC_FP8_E4M3FN)
    assert p["path"] == "temporal" and p["order"] == "cblock" and p["kstep"] == "128"
    assert (p["schedule"], p["tile_id"]) == ("lockstep", str(B.IGC_TILE_BUF))  # fp8, a short reduction (48 steps)
    p4 = _plan((1, 2048, 60, 80, 45), (2048, 2048, 3, 3, 3), pd=(1, 1, 1), dt=B.IGC_FP8_E4M3FN)
    # fp8, long reduction: the lockstep buffer tile (the swept table's winner and the size rule's choice)
    assert (p4["schedule"], p4["tile_id"], p4["nk"]) == ("lockstep", str(B.IGC_TILE_BUF), "432")
    assert _plan((1, 2048, 60, 80, 45), (2048, 2048, 3, 3, 3), pd=(1, 1, 1))["schedule"] == "lockstep"
    p = _plan((1, 2048, 60, 80, 45), (2048, 2048, 3, 3, 3), pd=(1, 1, 1))
    assert (p["path"], p["tile"], p["grid"], p["nk"], p["stages"], p["bstages"]) == ("generic", "256x256", "6752", "864", "3", "2")
    assert (p["loads"], p["tile_id"]) == ("buffer-lds", str(B.IGC_TILE_BUF))  # the swept table's winner
    # beyond 2^31 bytes: each tile rebases its buffer at the first input plane it reads (4 planes = 118 MB here)
    p = _plan((1, 1024, 240, 160, 90), (1024, 1024, 3, 1, 1), pd=(1, 0, 0))
    assert (p["big"], p["loads"]) == ("1", "buffer-lds")
    # a single input plane of 2 GB cannot fit one buffer window: 64-bit global-address loads
    p = _plan((1, 128, 3, 4096, 2049), (128, 128, 3, 3, 3), pd=(1, 1, 1))
    assert (p["big"], p["loads"]) == ("1", "global-lds")
    # point output: the tile that fills one round of the GPU best, 256x192 (5 x 50 = 250 tiles) for the patch embed
    p = _plan((9500, 3, 1, 14, 14), (1280, 3, 1, 14, 14), (1, 14, 14), lay=B.IGC_NCDHW)
    assert (p["tile"], p["grid"], p["group_m"]) == ("256x192", "250", "5")
    p = _plan((9500, 3, 1, 14, 14), (1280, 3, 1, 14, 14), (1, 14, 14), lay=B.IGC_NCDHW, dt=B.IGC_FP8_E4M3FN)
    assert (p["tile"], p["grid"]) == ("256x256", "190")  # 256x192 is a bf16-only tile
    assert _plan((1, 1024, 240, 160, 90), (1024, 1024, 3, 1, 1), pd=(1, 0, 0))["big"] == "1"
    p = _plan((1, 64, 4, 16, 16), (64, 64, 3, 3, 3), pd=(1, 1, 1))
    assert (p["tile"], p["stages"]) == ("64x64", "4")
    assert _plan((1, 24, 4, 16, 16), (64, 24, 3, 3, 3), pd=(1, 1, 1))["order"] == "linear"
    # 1x1x1 filters on NCDHW bf16 activations: one GEMM per image, no transpose
    p = _plan((1, 512, 240, 320, 180), (48, 512, 1, 1, 1), lay=B.IGC_NCDHW)
    assert (p["path"], p["tile"], p["nk"], p["grid"]) == ("pointwise", "512x64", "16", str(240 * 320 * 180 // 512))
    assert _plan((2, 64, 4, 6, 10), (48, 64, 1, 1, 1))["path"] == "temporal"   # NDHWC: the flat GEMM of the temporal path
    with pytest.raises(B.IgcError) as e:  # D*H*W % 8 != 0: NCDHW activations need the pack
        _plan((2, 64, 3, 5, 7), (48, 64, 1, 1, 1), lay=B.IGC_NCDHW)
    assert e.value.status == B.IGC_ERR_UNSUPPORTED
    with pytest.raises(B.IgcError) as e:  # fp8 operands come from the NDHWC pack
        _plan((1, 64, 4, 6, 10), (48, 64, 1, 1, 1), dt=B.IGC_FP8_E4M3FN, lay=B.IGC_NCDHW)
    assert e.value.status == B.IGC_ERR_UNSUPPORTED


def _swept_entries():
    """(esz, path, tile) of every entry of the generated tile table, in the sweep's shape order."""
    path = os.path.join(os.path.dirname(B.__file__), "csrc", "tile_table.h")
    rows = re.findall(r"^    \{(\d+), (\d+), [0-9.]+, \d+, \d+, (\d+), ", open(path).read(), re.M)
    return [tuple(int(v) for v in r) for r in rows]


def test_swept_table_drives_the_plan():
    from implicit_gemm_convolution_conv_amd import sweep as S
    entries = _swept_entries()
    assert len(entries) == len(S.SHAPES) and entries
    for (esz, path, tile), (name, dtype, xs, ws, pad) in zip(entries, S.SHAPES):
        assert esz == (1 if dtype == S.FP8 else 2), name
        dt = B.IGC_FP8_E4M3FN if dtype == S.FP8 else B.IGC_BF16
        p = _plan(xs, ws, pd=pad, dt=dt)
        assert p["path"] == ("temporal" if path == S.PATH_TEMPORAL else "generic"), name
        assert p["tile_id"] == str(tile), (name, p["tile_id"], tile)  # each swept shape plans onto its winner
    # the c1 shape's winner (64x64 with a split reduction) and a grid of 8 large tiles' winner (128x128)
    assert _plan((1, 64, 4, 16, 16), (64, 64, 3, 3, 3), pd=(1, 1, 1))["tile_id"] == str(B.IGC_TILE_DMA_64)
    assert _plan((1, 256, 8, 16, 16), (256, 256, 3, 3, 3), pd=(1, 1, 1))["tile_id"] == str(B.IGC_TILE_DMA_128)
    # beyond the table's reach the size rule decides: 3x3x3 over 16384 channels (6912 steps) on 8 tiles of
    # 256x256: 128 tiles of 64x64 would fill half the CUs, too many to split, so 128x128 with its split
    p = _plan((1, 16384, 4, 16, 32), (256, 16384, 3, 3, 3), pd=(1, 1, 1))
    assert p["tile_id"] == str(B.IGC_TILE_DMA_128), p
    # and a short reduction keeps 64x64: 3x3x3 over 64 channels on the same grid (27 steps)
    p = _plan((1, 64, 4, 16, 32), (256, 64, 3, 3, 3), pd=(1, 1, 1))
    assert p["tile_id"] == str(B.IGC_TILE_DMA_64), p


def test_forced_path_and_tile():
    try:
        B.conv_debug_force(B.IGC_PATH_GENERIC, B.IGC_TILE_DMA_128, 0)
        p = _plan((1, 64, 8, 8, 8), (64, 64, 3, 1, 1), pd=(1, 0, 0))
        assert (p["path"], p["tile"], p["tile_id"]) == ("generic", "128x128", str(B.IGC_TILE_DMA_128))
        B.conv_debug_force(B.IGC_PATH_POINT, -1, 0)
        with pytest.raises(B.IgcError) as e:
            _plan((1, 64, 8, 8, 8), (64, 64, 3, 1, 1), pd=(1, 0, 0))
        assert e.value.status == B.IGC_ERR_UNSUPPORTED
        B.conv_debug_force(B.IGC_PATH_AUTO, B.IGC_TILE_DMA_256x192, 0)  # a bf16-only tile
        with pytest.raises(B.IgcError) as e:
            _plan((1, 64, 8, 8, 8), (64, 64, 3, 3, 3), pd=(1, 1, 1), dt=B.IGC_FP8_E4M3FN)
        assert e.value.status == B.IGC_ERR_UNSUPPORTED
        B.conv_debug_force(B.IGC_PATH_AUTO, B.IGC_TILE_BUF, 0)  # buffer-addressed tiles: im2col paths, whole channel blocks
        p = _plan((1, 64, 8, 8, 8), (64, 64, 3, 3, 3), pd=(1, 1, 1))
        assert (p["loads"], p["stages"], p["bstages"]) == ("buffer-lds", "3", "2")
        for xs, ws in (((2, 16, 1, 14, 14), (32, 16, 1, 14, 14)), ((1, 96, 4, 4, 4), (8, 96, 3, 3, 3))):
            with pytest.raises(B.IgcError) as e:
                _plan(xs, ws, (1, 14, 14) if xs[0] == 2 else (1, 1, 1), pd=(0, 0, 0) if xs[0] == 2 else (1, 1, 1))
            assert e.value.status == B.IGC_ERR_UNSUPPORTED
        B.conv_debug_force(B.IGC_PATH_AUTO, B.IGC_TILE_BUF_PINGPONG, 0)  # ping-pong tile: tap masks of 32 bits
        assert _plan((1, 64, 8, 8, 8), (64, 64, 3, 3, 3), pd=(1, 1, 1))["schedule"] == "pingpong"
        with pytest.raises(B.IgcError) as e:
            _plan((1, 64, 8, 8, 8), (64, 64, 4, 3, 3), pd=(1, 1, 1))
        assert e.value.status == B.IGC_ERR_UNSUPPORTED
        B.conv_debug_force(B.IGC_PATH_AUTO, B.IGC_TILE_PW, 0)  # the pointwise kernel serves the pointwise path only
        with pytest.raises(B.IgcError) as e:
            _plan((1, 64, 8, 8, 8), (64, 64, 3, 3, 3), pd=(1, 1, 1))
        assert e.value.status == B.IGC_ERR_UNSUPPORTED
        B.conv_debug_force(B.IGC_PATH_AUTO, B.IGC_TILE_DMA_64, 5)
        p = _plan((1, 64, 8, 8, 8), (64, 64, 3, 3, 3), pd=(1, 1, 1), dt=B.IGC_FP8_E4M3FN)
        assert (p["stages"], p["kstep"], p["group_m"]) == ("4", "128", "5")
        with pytest.raises(B.IgcError) as e:  # tile ids past the table
            B.conv_debug_force(B.IGC_PATH_AUTO, B.IGC_TILE_BUF_128 + 1, 0)
        assert e.value.status == B.IGC_ERR_INVALID
    finally:
        B.conv_debug_force(B.IGC_PATH_AUTO, -1, 0)


def test_debug_hooks_are_per_thread():
    # a tile forced in one thread leaves the plans of another thread alone
    import threading
    geom = ((1, 64, 8, 8, 8), (64, 64, 3, 3, 3))
    auto = _plan(*geom, pd=(1, 1, 1))
    seen = {}

    def other():
        seen["plan"] = _plan(*geom, pd=(1, 1, 1))

    try:
        B.conv_debug_force(B.IGC_PATH_AUTO, B.IGC_TILE_DMA_128, 0)
        B.conv_debug_force_splits(1)
        assert _plan(*geom, pd=(1, 1, 1))["tile_id"] == str(B.IGC_TILE_DMA_128)
        t = threading.Thread(target=other)
        t.start()
        t.join()
    finally:
        B.conv_debug_force(B.IGC_PATH_AUTO, -1, 0)
        B.conv_debug_force_splits(0)
    assert seen["plan"] == auto


@pytest.mark.parametrize("args,status", [
    (((1, 64, 4, 4, 4), (64, 32, 3, 3, 3)), B.IGC_ERR_INVALID),          # channel mismatch
    (((1, 64, 2, 4, 4), (64, 64, 3, 3, 3)), B.IGC_ERR_INVALID),          # filter does not fit (pad 0)
    (((0, 64, 4, 4, 4), (64, 64, 3, 3, 3)), B.IGC_ERR_INVALID),          # empty batch
    (((1, 60, 4, 4, 4), (64, 60, 3, 3, 3)), B.IGC_ERR_UNSUPPORTED),      # C % 8 != 0 on the im2col path
])
def test_invalid_geometry_is_rejected(args, status):
    with pytest.raises(B.IgcError) as e:
        B.conv_plan(args[0], args[1], (1, 1, 1), (0, 0, 0), (1, 1, 1), B.IGC_BF16, B.IGC_NDHWC)
    assert e.value.status == status
    assert B.conv_last_error()


def test_fp8_channel_requirement_and_layout():
    with pytest.raises(B.IgcError) as e:
        B.conv_plan((1, 24, 4, 4, 4), (8, 24, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), B.IGC_FP8_E4M3FN,
                    B.IGC_NDHWC)
    assert e.value.status == B.IGC_ERR_UNSUPPORTED
    with pytest.raises(B.IgcError) as e:  # im2col needs channel-last activations
        B.conv_plan((1, 64, 4, 4, 4), (8, 64, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1), B.IGC_BF16, B.IGC_NCDHW)
    assert e.value.status == B.IGC_ERR_UNSUPPORTED


def test_null_pointers_rejected_before_any_launch():
    lib = B.load()
    xs = (B._i64((1, 64, 4, 4, 4), 5), B._i64((64, 64, 3, 3, 3), 5))
    one = B._i32((1, 1, 1))
    rc = lib.conv_fwd(None, None, None, xs[0], xs[1], one, one, one, B.IGC_BF16, B.IGC_NDHWC, None, None)
    assert rc == B.IGC_ERR_INVALID
    assert lib.conv_amax(None, 10, None, None) == B.IGC_ERR_INVALID
    assert lib.conv_pack_x(None, None, xs[0], B.IGC_BF16, None, None) == B.IGC_ERR_INVALID
    rc = lib.conv_fwd(16, 32, 48, xs[0], xs[1], one, one, one, B.IGC_FP8_E4M3FN, B.IGC_NDHWC, None, None)
    assert rc == B.IGC_ERR_INVALID  # fp8 without scales
    rc = lib.conv_fwd(8, 32, 48, xs[0], xs[1], one, one, one, B.IGC_BF16, B.IGC_NDHWC, None, None)
    assert rc == B.IGC_ERR_ALIGN


def _tile_reach(xs, ws, st, pd, dl, esz, bm=256):
    """Brute force over every 256-row tile: the byte range its valid im2col reads cover (every input pixel of
    every output row the tile touches, plus one more output row, a superset of its rows' reads), relative to the
    tile's buffer base, the first input plane its first row can read."""
    n_, c, d, h, w = xs
    _, _, t_, r_, s_ = ws
    do = (d + 2 * pd[0] - dl[0] * (t_ - 1) - 1) // st[0] + 1
    ho = (h + 2 * pd[1] - dl[1] * (r_ - 1) - 1) // st[1] + 1
    wo = (w + 2 * pd[2] - dl[2] * (s_ - 1) - 1) // st[2] + 1
    P, M, rows_total = do * ho * wo, n_ * do * ho * wo, n_ * do * ho
    pix = c * esz
    worst_lo, worst_hi = 0, 0
    for m0 in range(0, M, bm):
        n0, od0 = m0 // P, (m0 % P) // (ho * wo)
        base = (n0 * d + min(max(0, od0 * st[0] - pd[0]), d - 1)) * h * w * pix
        g0, g1 = m0 // wo, min(rows_total - 1, (min(m0 + bm, M) - 1) // wo + 1)
        for g in range(g0, g1 + 1):  # output rows (n, od, oh); every column of each
            n, od, oh = g // (do * ho), (g // ho) % do, g % ho
            for t in range(t_):
                idd = od * st[0] - pd[0] + t * dl[0]
                for r in range(r_):
                    ih = oh * st[1] - pd[1] + r * dl[1]
                    if not (0 <= idd < d and 0 <= ih < h):
                        continue
                    row = ((n * d + idd) * h + ih) * w * pix
                    worst_lo = min(worst_lo, row - base)
                    worst_hi = max(worst_hi, row + w * pix - base)
    return worst_lo, worst_hi


@pytest.mark.parametrize("geom", [
    ((1, 8, 9, 6, 7), (8, 8, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)),
    ((3, 8, 5, 6, 7), (8, 8, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)),     # tiles hold whole images
    ((2, 8, 9, 12, 30), (8, 8, 3, 3, 3), (2, 1, 1), (2, 1, 1), (2, 1, 1)),   # crossing into the next image
    ((4, 8, 7, 5, 5), (8, 8, 2, 1, 1), (1, 1, 1), (1, 0, 0), (3, 1, 1)),     # temporal, dilated
    ((2, 8, 11, 20, 20), (8, 8, 3, 3, 3), (2, 2, 2), (0, 1, 1), (1, 2, 2)),
    ((5, 8, 3, 4, 3), (8, 8, 3, 2, 2), (1, 2, 1), (2, 0, 1), (1, 1, 1)),
    ((3, 8, 4, 5, 6), (8, 8, 2, 2, 2), (1, 1, 1), (3, 1, 1), (1, 1, 1)),     # padding beyond the filter's reach
])
def test_buffer_span_bound_covers_every_tile(geom):
    xs, ws, st, pd, dl = geom
    lo, hi = _tile_reach(xs, ws, st, pd, dl, esz=2)
    p = _plan(xs, ws, st, pd, dl)
    assert lo >= 0, "a valid read lies below the tile's buffer base"
    assert hi <= int(p["xspan"]), (hi, p["xspan"])


def _plan_ws(x, w, nbytes, st=(1, 1, 1), pd=(1, 1, 1), dl=(1, 1, 1), dt=B.IGC_BF16, lay=B.IGC_NDHWC):
    return dict(kv.split("=") for kv in B.conv_plan_ws(x, w, st, pd, dl, dt, lay, nbytes).split())


def test_split_reduction_plan():
    c1x, c1w = (1, 64, 4, 16, 16), (64, 64, 3, 3, 3)
    ynum = 1024 * 64
    nbytes = B.conv_fwd_workspace_bytes(c1x, c1w, (1, 1, 1), (1, 1, 1), (1, 1, 1), B.IGC_BF16, B.IGC_NDHWC)
    p = _plan_ws(c1x, c1w, nbytes)
    # 16 tiles of 64x64, 27 steps: splits of >= 5 steps, at most about 256 workgroups
    assert (p["tile"], p["grid"], p["nk"]) == ("64x64", "16", "27")
    s, k = int(p["splits"]), int(p["ksplit"])
    assert (s, k) == (5, 6) and nbytes == s * ynum * 4
    assert s * 16 <= 256
    # conv_fwd (no workspace) never splits; conv_plan describes it
    assert _plan(c1x, c1w, pd=(1, 1, 1))["splits"] == "1"
    assert _plan_ws(c1x, c1w, 0)["splits"] == "1"
    # a workspace for two slices gives two splits, one byte short of two gives none
    assert _plan_ws(c1x, c1w, 2 * ynum * 4)["splits"] == "2"
    assert _plan_ws(c1x, c1w, 2 * ynum * 4 - 1)["splits"] == "1"
    # full grids do not split the reduction; c3's last round (96 of 6752 tiles) takes the tail split: 2 workgroups
    # per tile, 2 * 96 fp32 tiles of 256 x 256 of workspace
    big = ((1, 2048, 60, 80, 45), (2048, 2048, 3, 3, 3))
    assert B.conv_fwd_workspace_bytes(*big, (1, 1, 1), (1, 1, 1), (1, 1, 1), B.IGC_BF16, B.IGC_NDHWC) == 96 * 2 * 256 * 256 * 4
    assert _plan_ws(*big, 1 << 40)["splits"] == "1"
    assert _plan_ws(*big, 1 << 40)["tail"] == "96/2"
    assert _plan_ws(*big, 96 * 2 * 256 * 256 * 4 - 1)["tail"] == "0/1"
    # c3's one-GPU share: 844 tiles = 3 rounds + 76, 3 splits each; a 3x1x1 filter over 54000 tiles (last round
    # 240 of 256 CUs) does not split, nor does its 48-step share (6752 tiles, a last round of 96)
    assert _plan_ws((1, 2048, 60, 80, 45), (256, 2048, 3, 3, 3), 1 << 40)["tail"] == "76/3"
    assert _plan_ws((1, 1024, 240, 160, 90), (1024, 1024, 3, 1, 1), 1 << 40, pd=(1, 0, 0))["tail"] == "0/1"
    assert _plan_ws((1, 1024, 32, 160, 90), (1024, 1024, 3, 1, 1), 1 << 40, pd=(0, 0, 0))["tail"] == "0/1"
    # few reduction steps: no split (temporal c1-like, 3 steps)
    assert B.conv_fwd_workspace_bytes((1, 64, 4, 16, 16), (64, 64, 3, 1, 1), (1, 1, 1), (1, 0, 0), (1, 1, 1),
                                      B.IGC_BF16, B.IGC_NDHWC) == 0
    with pytest.raises(B.IgcError):
        B.conv_fwd_workspace_bytes((1, 64, 4, 4, 4), (64, 32, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1),
                                   B.IGC_BF16, B.IGC_NDHWC)


def test_forced_splits():
    c1x, c1w = (1, 64, 4, 16, 16), (64, 64, 3, 3, 3)
    try:
        B.conv_debug_force_splits(5)
        p = _plan_ws(c1x, c1w, 1 << 30)
        assert (p["splits"], p["ksplit"]) == ("5", "6")  # ceil(27 / 5) = 6 steps, ceil(27 / 6) = 5 splits
        B.conv_debug_force_splits(4)
        p = _plan_ws(c1x, c1w, 1 << 30)
        assert (p["splits"], p["ksplit"]) == ("4", "7")
        B.conv_debug_force_splits(100)  # capped at one step per split
        p = _plan_ws(c1x, c1w, 1 << 30)
        assert (p["splits"], p["ksplit"]) == ("27", "1")
        B.conv_debug_force_splits(1)
        assert B.conv_fwd_workspace_bytes(c1x, c1w, (1, 1, 1), (1, 1, 1), (1, 1, 1), B.IGC_BF16, B.IGC_NDHWC) == 0
        B.conv_debug_force_splits(3)
        B.conv_debug_force(B.IGC_PATH_AUTO, B.IGC_TILE_BUF, 0)  # buffer-addressed tile: no split
        with pytest.raises(B.IgcError) as e:
            _plan_ws(c1x, c1w, 1 << 30)
        assert e.value.status == B.IGC_ERR_UNSUPPORTED
        with pytest.raises(B.IgcError) as e:
            B.conv_debug_force_splits(-1)
        assert e.value.status == B.IGC_ERR_INVALID
    finally:
        B.conv_debug_force(B.IGC_PATH_AUTO, -1, 0)
        B.conv_debug_force_splits(0)


def test_workspace_arguments_checked_before_any_launch():
    lib = B.load()
    xs = (B._i64((1, 64, 4, 16, 16), 5), B._i64((64, 64, 3, 3, 3), 5))
    one = B._i32((1, 1, 1))
    rc = lib.conv_fwd_ws(16, 32, 48, xs[0], xs[1], one, one, one, B.IGC_BF16, B.IGC_NDHWC, None, None, 64, None)
    assert rc == B.IGC_ERR_INVALID  # bytes without a workspace
    rc = lib.conv_fwd_ws(16, 32, 48, xs[0], xs[1], one, one, one, B.IGC_BF16, B.IGC_NDHWC, None, 8, 64, None)
    assert rc == B.IGC_ERR_ALIGN


def test_point_gradient_entry_points():
    xs, ws, st = (9500, 3, 1, 14, 14), (1280, 3, 1, 14, 14), (1, 14, 14)
    z, one = (0, 0, 0), (1, 1, 1)
    assert B.conv_packed_w_t_cols(ws) == 1280
    assert B.conv_packed_w_t_cols((18, 5, 1, 3, 7)) == 64
    ldn = 9536  # 9500 images rounded up to 64
    base = (588 * ldn * 2 + 255) // 256 * 256 + (1280 * ldn * 2 + 255) // 256 * 256
    # a 149-step reduction: 128x128 tiles over 588 x 1280 (50 tiles), 10 splits of 15 steps, fp32 slices
    assert B.conv_bwd_weight_workspace_bytes(xs, ws, st, z, one, B.IGC_BF16, B.IGC_NCDHW) == \
        base + 10 * 1280 * 588 * 4
    # 37 images of 5 x 3 x 7 -> 18 channels: one reduction step over 64 (padded) images, too short to split
    small = B.conv_bwd_weight_workspace_bytes((37, 5, 1, 3, 7), (18, 5, 1, 3, 7), (1, 3, 7), z, one, B.IGC_BF16,
                                              B.IGC_NDHWC)
    assert small == 13568 + 2304  # x^T 105 x 64 and dy^T 18 x 64 bf16, each rounded up to 256 bytes
    # a long batch on a small grid splits: 4000 images, 2 tiles, 63 steps of 64 images
    split = B.conv_bwd_weight_workspace_bytes((4000, 5, 1, 3, 7), (18, 5, 1, 3, 7), (1, 3, 7), z, one, B.IGC_BF16,
                                              B.IGC_NCDHW)
    ldn = 4032
    tr = (105 * ldn * 2 + 255) // 256 * 256 + (18 * ldn * 2 + 255) // 256 * 256
    assert split > tr and (split - tr) % (18 * 105 * 4) == 0 and (split - tr) // (18 * 105 * 4) > 1
    for fn in (lambda: B.conv_bwd_weight_workspace_bytes((1, 3, 4, 14, 14), ws, st, z, one, B.IGC_BF16,
                                                         B.IGC_NCDHW),  # input deeper than the filter
               lambda: B.conv_bwd_weight_workspace_bytes(xs, ws, st, (0, 1, 1), one, B.IGC_BF16, B.IGC_NCDHW),
               lambda: B.conv_bwd_weight_workspace_bytes(xs, ws, st, z, one, B.IGC_FP8_E4M3FN, B.IGC_NCDHW)):
        with pytest.raises(B.IgcError) as e:
            fn()
        assert e.value.status == B.IGC_ERR_UNSUPPORTED
    lib = B.load()
    a, b = B._i64(xs, 5), B._i64(ws, 5)
    odd = B._i64((9500, 3, 1, 14, 14), 5), B._i64((1279, 3, 1, 14, 14), 5)
    rc = lib.conv_bwd_data(16, 32, 48, odd[0], odd[1], B._i32(st), B._i32(z), B._i32(one), B.IGC_BF16,
                           B.IGC_NCDHW, None)
    assert rc == B.IGC_ERR_UNSUPPORTED  # dy rows of an odd K are not 4-byte aligned
    rc = lib.conv_bwd_weight(16, 32, 48, a, b, B._i32(st), B._i32(z), B._i32(one), B.IGC_BF16, B.IGC_NCDHW, 64,
                             base - 1, None)
    assert rc == B.IGC_ERR_INVALID  # workspace below the two transposes


def test_noalloc_rejects_a_workspace_beyond_its_scratch_before_any_launch():
    # a forced 64-way split of a 1024 x 1280 output (64 x 5 MiB of fp32 partials) needs more than the 64 MiB
    # static scratch: rejected with a message, nothing enqueued (null tensors are never touched)
    xs, ws = (1, 64, 4, 16, 16), (1280, 64, 3, 3, 3)
    lib = B.load()
    one = B._i32((1, 1, 1))
    try:
        B.conv_debug_force(B.IGC_PATH_AUTO, B.IGC_TILE_DMA_64, 0)
        B.conv_debug_force_splits(64)
        need = B.conv_fwd_workspace_bytes(xs, ws, (1, 1, 1), (1, 1, 1), (1, 1, 1), B.IGC_BF16, B.IGC_NDHWC)
        assert need > 64 << 20
        rc = lib.conv_fwd_noalloc(16, 32, 48, B._i64(xs, 5), B._i64(ws, 5), one, one, one, B.IGC_BF16,
                                  B.IGC_NDHWC, None, None, None, None)
        assert rc == B.IGC_ERR_UNSUPPORTED
        assert "static scratch" in B.conv_last_error()
    finally:
        B.conv_debug_force(B.IGC_PATH_AUTO, -1, 0)
        B.conv_debug_force_splits(0)


def test_fast_division_matches_integer_division(tmp_path):
    """The multiply-high division the kernels use for the tile walk and the row decode (FastDiv, the
    round-up method of Granlund and Montgomery) against plain integer division, compiled for the host."""
    import shutil
    import subprocess
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    if not os.path.exists(hipcc) and shutil.which("hipcc") is None:
        pytest.skip("hipcc is not installed")
    exe = tmp_path / "fastdiv_check"
    src = os.path.join(ROOT, "tests", "fastdiv_check.cpp")
    inc = os.path.join(ROOT, "implicit_gemm_convolution_conv_amd", "csrc")
    subprocess.run([hipcc, "-O2", "-std=c++17", "-x", "hip", "--cuda-host-only", "-I", inc, src, "-o", str(exe)],
                   check=True, capture_output=True)
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert " 0 mismatches" in r.stdout
