"""GPU parity at the full workload sizes, through the calls bench.py times.

bench.py times conv_fwd_ws with a workspace of conv_fwd_workspace_bytes: on
the 256x256 buffer tiles the last, partial round of tiles then runs split along
the reduction (the tail split), and a second pass adds the partial sums. Every
full-size check here makes that same call (`_timed_call`) and asserts the plan
it runs; conv_fwd (no workspace) runs beside it where the plan splits.

Random data: the oracle evaluates sampled output elements one by one (box
corners, edges, faces and their neighbours, chosen planes and channels,
uniform draws, and for split plans several elements of every tail tile) and
the relative-L2 / max-abs tolerance applies over the sample. The tail tiles
are found from the outputs themselves: outside them conv_fwd_ws and conv_fwd
run the same instructions and agree bit for bit, inside them the summation
order differs. Exact checks at full size: a delta filter (output = shifted
copy of the input, bit for bit) and all-ones operands (output = C x number
of valid taps, a closed form), which exercise every address the kernels
compute, for bf16 and for fp8 with unit scales.
"""

import numpy as np
import pytest
import torch

from implicit_gemm_convolution_conv_amd import binding as B
from implicit_gemm_convolution_conv_amd import inputs as I
from implicit_gemm_convolution_conv_amd import pipeline as PL
from oracle import oracle as O

import parity as P

pytestmark = pytest.mark.gpu


def _announce(name):
    print(f"[case] {name}", flush=True)


def _free():
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def _valid_taps(size, ksz, pad, dev):
    o = torch.arange(size + 2 * pad - ksz + 1, device=dev)
    t = torch.arange(ksz, device=dev)
    pos = o[:, None] - pad + t[None, :]
    return ((pos >= 0) & (pos < size)).sum(1).to(torch.float64)


def _plan_kv(plan):
    return dict(item.split("=") for item in plan.split())


def _timed_call(xk, wp, y, wl, dtype, scales=None):
    """The call bench.py times for workload `wl`: conv_fwd_ws with a NaN-filled workspace of
    conv_fwd_workspace_bytes (conv_fwd where the plan needs none). Returns the plan string it ran."""
    args = (wl.x_shape, wl.w_shape, wl.stride, wl.pad, wl.dil, dtype, B.IGC_NDHWC)
    nws = B.conv_fwd_workspace_bytes(*args)
    plan = B.conv_plan_ws(*args, max(nws, 0))
    if nws > 0:
        wsb = torch.full((nws // 4,), float("nan"), dtype=torch.float32, device=P.DEV)
        B.conv_fwd_ws(xk, wp, y, *args, scales, workspace=wsb)
        torch.cuda.synchronize()
        del wsb
    else:
        B.conv_fwd(xk, wp, y, *args, scales)
        torch.cuda.synchronize()
    return plan


def _tail_split(plan):
    r, s = _plan_kv(plan)["tail"].split("/")
    return int(r), int(s)


def _tile_of_workgroup(bid, tiles_m, tiles_n, group_m, tap_stride):
    """The output tile (m-tile, k-tile) that workgroup `bid` of a launch computes: the kernels' tile schedule
    restated (workgroups dealt to the 8 XCDs in turn and renumbered so that consecutive tiles share one; tiles
    walked in groups of group_m tile rows, every column of a group before the next; the temporal raster
    spreads a group's rows one time tap apart)."""
    nblk = tiles_m * tiles_n
    xcd, idx = bid & 7, bid >> 3
    q, r = nblk >> 3, nblk & 7
    lin = xcd * q + min(xcd, r) + idx
    gsz = group_m * tiles_n
    g = lin // gsz
    first = g * group_m
    rows = min(tiles_m - first, group_m)
    inn = lin - g * gsz
    tm, tn = first + inn % rows, inn // rows
    if tap_stride > 0:
        blk = group_m * tap_stride
        if tm < tiles_m // blk * blk:
            b, rr = divmod(tm, blk)
            gi, c = divmod(rr, group_m)
            tm = b * blk + c * tap_stride + gi
    return tm, tn


def _tail_tiles(plan, y_shape, tm=256, tn=256):
    """The (m-tile, k-tile) pairs the tail split computes: the tiles of workgroups tail_first .. ntiles - 1."""
    kv = _plan_kv(plan)
    r, _ = _tail_split(plan)
    _, k, do, ho, wo = y_shape
    tiles_m, tiles_n = -(-do * ho * wo // tm), -(-k // tn)
    ntiles = tiles_m * tiles_n
    assert int(kv["grid"]) == ntiles
    return {_tile_of_workgroup(b, tiles_m, tiles_n, int(kv["group_m"]), int(kv["tap"]))
            for b in range(ntiles - r, ntiles)}


def _tiles_that_differ(y_ws, y_plain, tm=256, tn=256):
    """(m-tile, k-tile) pairs of a one-image output where the two results differ in any bit."""
    n, k = y_ws.shape[:2]
    assert n == 1
    diff = (y_ws.view(torch.int16) != y_plain.view(torch.int16)).view(k, -1)
    idx = diff.nonzero()
    if idx.numel() == 0:
        return set()
    tiles = torch.unique(torch.stack([idx[:, 1] // tm, idx[:, 0] // tn], 1), dim=0)
    return {(int(a), int(b)) for a, b in tiles.cpu().numpy()}


def _points_in_tiles(tiles, y_shape, per_tile, rng, tm=256, tn=256):
    """`per_tile` random output elements (n, k, od, oh, ow) inside each (m-tile, k-tile) of a one-image output."""
    _, k, do, ho, wo = y_shape
    m_total = do * ho * wo
    pts = []
    for mt, nt in sorted(tiles):
        for _ in range(per_tile):
            m = int(rng.integers(mt * tm, min(m_total, (mt + 1) * tm)))
            kk = int(rng.integers(nt * tn, min(k, (nt + 1) * tn)))
            pts.append((0, kk, m // (ho * wo), (m // wo) % ho, m % wo))
    return np.array(pts, np.int64).reshape(-1, 5)


def _check_tail_split(y_ws, y_plain, plan, R, max_x, max_w, rng, what, expect_most_differ=True):
    """conv_fwd_ws against conv_fwd on the same inputs: they may differ only inside the tail tiles, and there
    only by summation order (within the tolerance). Returns oracle points, several in every tail tile.
    bf16 products round in fp32, so another summation order changes some output bits in nearly every tail
    tile; fp8 products are exact in fp32 and a tile's bits often come out the same either way."""
    r, s = _tail_split(plan)
    assert r > 0 and s >= 2, f"{what}: the timed plan has no tail split: {plan}"
    tail = _tail_tiles(plan, tuple(y_ws.shape))
    assert len(tail) == r
    differ = _tiles_that_differ(y_ws, y_plain)
    assert differ <= tail, f"{what}: tiles outside the tail differ from conv_fwd: {sorted(differ - tail)[:8]}"
    if expect_most_differ:
        assert len(differ) >= r // 2, f"{what}: only {len(differ)} of {r} tail tiles differ from conv_fwd"
    mdiff = float((y_ws.float() - y_plain.float()).abs().max())
    assert mdiff <= P.ABS_FACTOR * np.sqrt(R) * max_x * max_w, f"{what}: conv_fwd_ws vs conv_fwd {mdiff}"
    pts = _points_in_tiles(tail, tuple(y_ws.shape), max(1, -(-400 // r)), rng)
    assert len(pts) >= 400
    return pts


def test_c2_point_output_full():
    wl = I.WORKLOADS["c2"]
    _announce("c2 point-output, all 9500 x 1280 outputs")
    x, w = I.make(wl, P.DEV)
    assert B.conv_plan(wl.x_shape, wl.w_shape, wl.stride, wl.pad, wl.dil, B.IGC_BF16,
                       B.IGC_NCDHW).startswith("path=point")
    y = P.run_bf16(x, w, wl.stride, wl.pad, wl.dil, x_layout="NCDHW")
    ref = O.conv3d(P.bits(x), P.bits(w), wl.stride, wl.pad, wl.dil)
    P.check_close(P.y_values(y), ref, wl.reduction, float(x.abs().max()), float(w.abs().max()), "c2")
    _free()


def _delta_filter(ws, tap, seed):
    """One-hot filter: output channel k reads input channel perm[k] at filter tap `tap` (bf16)."""
    k, c = ws[0], ws[1]
    perm = torch.randperm(c, generator=torch.Generator().manual_seed(seed))[:k].to(P.DEV)
    wd = torch.zeros(ws, dtype=torch.bfloat16, device=P.DEV)
    wd[torch.arange(k, device=P.DEV), perm, tap[0], tap[1], tap[2]] = 1.0
    return wd, perm


def _all_ones_counts(xs, c, dev):
    """C x the number of valid taps of a 3x3x3 filter with pad 1 at every output position (D, H, W)."""
    d, h, w = xs[2:]
    return (_valid_taps(d, 3, 1, dev)[:, None, None] * _valid_taps(h, 3, 1, dev)[None, :, None]
            * _valid_taps(w, 3, 1, dev)[None, None, :]) * c


def test_c3_sampled_and_exact():
    wl = I.WORKLOADS["c3"]
    _announce("c3 bf16 through conv_fwd_ws (the timed call), sampled and tail tiles vs oracle")
    x, w = I.make(wl, P.DEV)  # x drawn NDHWC
    xs, ws = wl.x_shape, wl.w_shape
    wp = PL.packed_weight(w, "bf16", "NDHWC")
    y = torch.full((1, ws[0]) + tuple(B.conv_out_dims(xs, ws, wl.stride, wl.pad, wl.dil)), float("nan"),
                   dtype=torch.bfloat16, device=P.DEV)
    plan = _timed_call(x, wp, y, wl, B.IGC_BF16)
    kv = _plan_kv(plan)
    assert (kv["path"], kv["tile"], kv["loads"], kv["tail"]) == ("generic", "256x256", "buffer-lds", "96/2"), plan
    assert not torch.isnan(y).any()
    y_plain = PL.output(xs, ws, wl.stride, wl.pad, wl.dil, P.DEV)
    B.conv_fwd(x, wp, y_plain, xs, ws, wl.stride, wl.pad, wl.dil, B.IGC_BF16, B.IGC_NDHWC)
    torch.cuda.synchronize()
    mx, mw = float(x.abs().max()), float(w.abs().max())
    rng = np.random.default_rng(3)
    tail_pts = _check_tail_split(y, y_plain, plan, wl.reduction, mx, mw, rng, "c3")
    del y_plain
    pts = np.concatenate([P.sample_points(1, ws[0], *y.shape[2:], rng, n_random=600, extra_k=(1023, 1024)),
                          tail_pts])
    ref = O.conv3d_points(P.bits(x), P.bits(w), pts, wl.stride, wl.pad, wl.dil, x_layout="NDHWC")
    P.check_close(P.gather(y, pts), ref, wl.reduction, mx, mw, "c3")
    n_tail = len(tail_pts)
    P.check_close(P.gather(y, tail_pts), ref[-n_tail:], wl.reduction, mx, mw, "c3 tail tiles")

    _announce("c3 bf16 delta filter, full size, conv_fwd_ws")
    k, c = ws[0], ws[1]
    tap = (2, 0, 1)
    wd, perm = _delta_filter(ws, tap, 0)
    wpd = PL.packed_weight(wd, "bf16", "NDHWC")
    y.fill_(float("nan"))
    _timed_call(x, wpd, y, wl, B.IGC_BF16)
    xpad = torch.nn.functional.pad(x, (0, 0, 1, 1, 1, 1, 1, 1))  # zero halo on D, H, W of NDHWC
    d, h, wdt = xs[2:]
    shifted = xpad[:, tap[0]:tap[0] + d, tap[1]:tap[1] + h, tap[2]:tap[2] + wdt, :]  # (N, D, H, W, C)
    expect = shifted[..., perm].permute(0, 4, 1, 2, 3)
    assert torch.equal(y.view(torch.int16), expect.contiguous().view(torch.int16))
    del xpad, shifted, expect, wd, wpd

    _announce("c3 bf16 all-ones, full size, conv_fwd_ws")
    x.fill_(1.0)
    wones = torch.ones(ws, dtype=torch.bfloat16, device=P.DEV)
    wp = PL.packed_weight(wones, "bf16", "NDHWC")
    y.fill_(float("nan"))
    _timed_call(x, wp, y, wl, B.IGC_BF16)
    assert torch.equal(y.double(), _all_ones_counts(xs, c, P.DEV).expand(1, k, d, h, wdt))
    _free()


@pytest.mark.parametrize("name", ["c4", "c4t"])
def test_fp8_sampled(name):
    wl = I.WORKLOADS[name]
    _announce(f"{name} fp8 pack (all codes) and sampled conv through the timed call")
    x, w = I.make(wl, P.DEV)  # x drawn NCDHW bf16
    xs, ws = wl.x_shape, wl.w_shape
    ops = P.Fp8Operands(x, w, check_codes=True)
    y = torch.full((1, ws[0]) + tuple(B.conv_out_dims(xs, ws, wl.stride, wl.pad, wl.dil)), float("nan"),
                   dtype=torch.bfloat16, device=P.DEV)
    plan = _timed_call(ops.xq, ops.wq, y, wl, B.IGC_FP8_E4M3FN, ops.scales)
    kv = _plan_kv(plan)
    assert not torch.isnan(y).any()
    sx, sw = float(ops.ref_scales[0]), float(ops.ref_scales[2])
    mx = float(np.abs(O.e4m3_decode(ops.ref_xq)).max()) * sx
    mw = float(np.abs(O.e4m3_decode(ops.ref_wq)).max()) * sw
    rng = np.random.default_rng(4)
    pts = P.sample_points(1, ws[0], *y.shape[2:], rng, n_random=600)
    if name == "c4":  # the swept table's winner, the lockstep buffer tile, with its tail split: 96 tiles in 2 splits
        assert (kv["schedule"], kv["tile_id"], kv["tail"]) == ("lockstep", str(B.IGC_TILE_BUF), "96/2"), plan
        y_plain = PL.output(xs, ws, wl.stride, wl.pad, wl.dil, P.DEV)
        B.conv_fwd(ops.xq, ops.wq, y_plain, xs, ws, wl.stride, wl.pad, wl.dil, B.IGC_FP8_E4M3FN, B.IGC_NDHWC,
                   ops.scales)
        torch.cuda.synchronize()
        pts = np.concatenate([pts, _check_tail_split(y, y_plain, plan, wl.reduction, mx, mw, rng, name,
                                                      expect_most_differ=False)])
        del y_plain
    else:  # 48 steps: no tail split, the lockstep buffer tile with the temporal raster
        assert (kv["path"], kv["schedule"], kv["tail"]) == ("temporal", "lockstep", "0/1"), plan
    ref = O.conv3d_points(ops.ref_xq, ops.ref_wq, pts, wl.stride, wl.pad, wl.dil, sx=sx, sw=sw)
    P.check_close(P.gather(y, pts), ref, wl.reduction, mx, mw, name)
    _free()


def test_c4_fp8_exact_full_size():
    """fp8 at full size with unit scales: integer activations in [-2, 2] and a one-hot or all-ones filter are
    exact E4M3FN codes, so the timed call must give a shifted copy of x, and C x the valid taps, bit for bit."""
    wl = I.WORKLOADS["c4"]
    xs, ws = wl.x_shape, wl.w_shape
    k, c = ws[0], ws[1]
    d, h, wdt = xs[2:]
    unit = torch.ones(4, dtype=torch.float32, device=P.DEV)
    _announce("c4 fp8 delta filter, full size, conv_fwd_ws (tile 4, tail split)")
    xi = I.int_valued(xs, -2, 2, I.generator(40, P.DEV), P.DEV)  # NCDHW bf16
    xq = PL.packed_input(xi, "fp8", unit[0:2])
    tap = (0, 2, 1)
    wd, perm = _delta_filter(ws, tap, 4)
    wq = PL.packed_weight(wd, "fp8", "NDHWC", unit[2:4])
    del wd
    y = torch.full((1, k, d, h, wdt), float("nan"), dtype=torch.bfloat16, device=P.DEV)
    plan = _timed_call(xq, wq, y, wl, B.IGC_FP8_E4M3FN, unit)
    assert (_plan_kv(plan)["tile_id"], _plan_kv(plan)["tail"]) == (str(B.IGC_TILE_BUF), "96/2"), plan
    xpad = torch.nn.functional.pad(xi, (1, 1, 1, 1, 1, 1))  # zero halo on D, H, W of NCDHW
    for k0 in range(0, k, 512):
        expect = xpad[:, perm[k0:k0 + 512], tap[0]:tap[0] + d, tap[1]:tap[1] + h, tap[2]:tap[2] + wdt]
        assert torch.equal(y[:, k0:k0 + 512].view(torch.int16), expect.contiguous().view(torch.int16)), k0
    del xpad, expect, xi, wq

    _announce("c4 fp8 all-ones, full size, conv_fwd_ws")
    xq.fill_(0x38)  # E4M3FN code of 1.0
    wq = PL.packed_weight(torch.ones(ws, dtype=torch.bfloat16, device=P.DEV), "fp8", "NDHWC", unit[2:4])
    y.fill_(float("nan"))
    _timed_call(xq, wq, y, wl, B.IGC_FP8_E4M3FN, unit)
    assert torch.equal(y.double(), _all_ones_counts(xs, c, P.DEV).expand(1, k, d, h, wdt))
    _free()


def test_c5_large_tensor():
    wl = I.WORKLOADS["c5"]
    xs, ws = wl.x_shape, wl.w_shape
    n, c, d, h, wdt = xs
    k = ws[0]
    _announce("c5 >2^31 elements: transpose bit-exact")
    x, w = I.make(wl, P.DEV)  # NCDHW, 3.5e9 elements
    assert x.numel() > 2 ** 31
    plan = B.conv_plan(xs, ws, wl.stride, wl.pad, wl.dil, B.IGC_BF16, B.IGC_NDHWC)
    assert "path=temporal" in plan and "big=1" in plan
    xt = PL.packed_input(x, "bf16")
    torch.cuda.synchronize()
    for dd in range(0, d, 16):  # compare plane blocks to bound the scratch
        assert torch.equal(xt[:, dd:dd + 16].view(torch.int16),
                           x[:, :, dd:dd + 16].permute(0, 2, 3, 4, 1).contiguous().view(torch.int16))

    _announce("c5 sampled vs oracle (planes across the 2^31 / 2^32 offsets), the timed call")
    wp = PL.packed_weight(w, "bf16", "NDHWC")
    y = torch.full((1, k) + tuple(B.conv_out_dims(xs, ws, wl.stride, wl.pad, wl.dil)), float("nan"),
                   dtype=torch.bfloat16, device=P.DEV)
    plan = _timed_call(xt, wp, y, wl, B.IGC_BF16)
    assert (_plan_kv(plan)["loads"], _plan_kv(plan)["tail"]) == ("buffer-lds", "0/1"), plan
    assert y.numel() > 2 ** 31
    rng = np.random.default_rng(5)
    pts = P.sample_points(1, k, *y.shape[2:], rng, n_random=800, extra_d=(145, 146, 147, 238),
                          extra_k=(621, 622, 1023))
    xb = P.bits(x)  # 7 GB host copy, NCDHW
    ref = O.conv3d_points(xb, P.bits(w), pts, wl.stride, wl.pad, wl.dil)
    del xb
    P.check_close(P.gather(y, pts), ref, wl.reduction, float(x.abs().max()), float(w.abs().max()), "c5")

    # delta filters on the first and the last time tap: y[:, k, od] = x[:, perm[k], od - 1 + t]
    for t, seed in ((0, 1), (2, 11)):
        _announce(f"c5 delta filter on tap t={t}, full size (bit-exact)")
        wd, perm = _delta_filter(ws, (t, 0, 0), seed)
        wpd = PL.packed_weight(wd, "bf16", "NDHWC")
        del wd
        y.fill_(float("nan"))
        _timed_call(xt, wpd, y, wl, B.IGC_BF16)
        zero_plane = 0 if t == 0 else d - 1
        assert torch.equal(y[:, :, zero_plane].view(torch.int16),
                           torch.zeros_like(y[:, :, zero_plane]).view(torch.int16))
        lo, hi = (1, d) if t == 0 else (0, d - 1)
        for kk in range(0, k, 128):
            src = x[:, perm[kk:kk + 128], lo - 1 + t: hi - 1 + t]
            assert torch.equal(y[:, kk:kk + 128, lo:hi].view(torch.int16), src.view(torch.int16)), (t, kk)
        del wpd

    _announce("c5 all-ones, full size: 2C on the first and last planes, 3C inside")
    del x
    torch.cuda.empty_cache()
    xt.fill_(1.0)
    wp = PL.packed_weight(torch.ones(ws, dtype=torch.bfloat16, device=P.DEV), "bf16", "NDHWC")
    y.fill_(float("nan"))
    _timed_call(xt, wp, y, wl, B.IGC_BF16)
    del xt
    for kk in range(0, k, 128):
        blk = y[:, kk:kk + 128]
        assert bool((blk[:, :, 1:d - 1] == 3 * c).all()), kk
        assert bool((blk[:, :, 0] == 2 * c).all()) and bool((blk[:, :, d - 1] == 2 * c).all()), kk
    _free()


def test_two_images_above_2_31_elements():
    """N = 2 with x above 2^31 elements: the pages' large-input fix admits one image only, here each tile's buffer
    window is rebased at the first input plane it can read, in whichever image. A 3x3x3 bf16 conv over
    2 x 1024 x 80 x 161 x 89 activations (2.35 G elements, P % 256 = 208, so tiles straddle the two images)
    through the conv_fwd_ws call: random operands on sampled elements on both sides of the image boundary and
    across the 2^31-element offset, then a delta filter bit for bit over the whole output."""
    wl = I.Workload("two images", (2, 1024, 80, 161, 89), (256, 1024, 3, 3, 3), pad=(1, 1, 1), x_layout="NDHWC",
                    x_dist=("normal", 1.0), w_dist=("normal", 1.0 / np.sqrt(1024 * 27)), seed=9)
    xs, ws = wl.x_shape, wl.w_shape
    n, c, d, h, wdt = xs
    k = ws[0]
    _announce("two images > 2^31 elements, 3x3x3 bf16: sampled vs oracle")
    x, w = I.make(wl, P.DEV)  # x drawn NDHWC
    assert x.numel() > 2 ** 31
    wp = PL.packed_weight(w, "bf16", "NDHWC")
    y = torch.full((n, k) + tuple(B.conv_out_dims(xs, ws, wl.stride, wl.pad, wl.dil)), float("nan"),
                   dtype=torch.bfloat16, device=P.DEV)
    plan = _timed_call(x, wp, y, wl, B.IGC_BF16)
    kv = _plan_kv(plan)
    assert (kv["path"], kv["loads"], kv["big"]) == ("generic", "buffer-lds", "1"), plan
    assert not torch.isnan(y).any()
    rng = np.random.default_rng(9)
    pts = P.sample_points(n, k, *y.shape[2:], rng, n_random=600, extra_d=(0, 1, d - 2, d - 1))
    # both sides of the image boundary, in the tile that straddles it, and around element offset 2^31 of x
    edge = [(0, int(rng.integers(0, k)), d - 1, h - 1, wdt - 1 - i) for i in range(40)]
    edge += [(1, int(rng.integers(0, k)), 0, 0, i) for i in range(40)]
    m31 = (2 ** 31) // c  # the input row holding element 2^31 of NDHWC x
    for dm in range(-20, 20):
        m = m31 + dm
        img, sp = divmod(m, d * h * wdt)
        edge.append((img, int(rng.integers(0, k)), sp // (h * wdt), (sp // wdt) % h, sp % wdt))
    pts = np.concatenate([pts, np.array(edge, np.int64)])
    xb = P.bits(x)
    ref = O.conv3d_points(xb, P.bits(w), pts, wl.stride, wl.pad, wl.dil, x_layout="NDHWC")
    del xb
    P.check_close(P.gather(y, pts), ref, wl.reduction, float(x.abs().max()), float(w.abs().max()), "two images")

    _announce("two images > 2^31 elements: delta filter, full size, bit-exact")
    tap = (0, 2, 1)
    wd, perm = _delta_filter(ws, tap, 4)
    wpd = PL.packed_weight(wd, "bf16", "NDHWC")
    y.fill_(float("nan"))
    _timed_call(x, wpd, y, wl, B.IGC_BF16)
    for img in range(n):
        xpad = torch.nn.functional.pad(x[img:img + 1], (0, 0, 1, 1, 1, 1, 1, 1))  # zero halo on D, H, W
        shifted = xpad[:, tap[0]:tap[0] + d, tap[1]:tap[1] + h, tap[2]:tap[2] + wdt, :]
        expect = shifted[..., perm].permute(0, 4, 1, 2, 3).contiguous()
        assert torch.equal(y[img:img + 1].view(torch.int16), expect.view(torch.int16)), img
        del xpad, shifted, expect
    _free()


def test_pointwise_ncdhw_page_workload():
    """1x1x1 conv on 14 GB of NCDHW activations, read without a transpose: sampled positions against the oracle
    (a 1x1x1 conv of the gathered columns), then a one-hot filter that must copy channels bit for bit."""
    wl = I.WORKLOADS["pw"]
    xs, ws = wl.x_shape, wl.w_shape
    n, c, d, h, wdt = xs
    k = ws[0]
    one, zero = (1, 1, 1), (0, 0, 0)
    _announce("pw 1x1x1 NCDHW, 14 GB: sampled vs oracle")
    assert B.conv_plan(xs, ws, one, zero, one, B.IGC_BF16, B.IGC_NCDHW).startswith("path=pointwise")
    x, w = I.make(wl, P.DEV)
    wp = PL.packed_weight(w, "bf16", "NCDHW")
    y = PL.output(xs, ws, one, zero, one, P.DEV)
    B.conv_fwd(x, wp, y, xs, ws, one, zero, one, B.IGC_BF16, B.IGC_NCDHW)
    torch.cuda.synchronize()
    S = d * h * wdt
    rng = np.random.default_rng(6)
    pos = np.unique(np.concatenate([rng.integers(0, S, 2000), [0, 1, 255, 256, S - 256, S - 1]]))
    pos_t = torch.as_tensor(pos, device=P.DEV)
    cols = x.view(n, c, S)[:, :, pos_t].contiguous().view(n, c, 1, 1, len(pos))
    ref = O.conv3d(P.bits(cols), P.bits(w), one, zero, one)            # (n, k, 1, 1, len(pos))
    got = y.view(n, k, S)[:, :, pos_t].contiguous().view(n, k, 1, 1, len(pos))
    P.check_close(P.y_values(got), ref, c, float(x.abs().max()), float(w.abs().max()), "pw")

    _announce("pw one-hot filter, full size (bit-exact)")
    perm = torch.randperm(c, generator=torch.Generator().manual_seed(2))[:k].to(P.DEV)
    wd = torch.zeros(ws, dtype=torch.bfloat16, device=P.DEV)
    wd[torch.arange(k, device=P.DEV), perm, 0, 0, 0] = 1.0
    B.conv_fwd(x, PL.packed_weight(wd, "bf16", "NCDHW"), y, xs, ws, one, zero, one, B.IGC_BF16, B.IGC_NCDHW)
    torch.cuda.synchronize()
    for kk in range(k):
        assert torch.equal(y[:, kk].view(torch.int16), x[:, perm[kk]].view(torch.int16)), kk
    _free()


@pytest.mark.parametrize("name", ["c3s", "c5s"])
def test_one_gpu_share_sampled(name):
    # one GPU's share of an 8-way split, at its real shape: the kernel that GPU would run, through the call
    # bench.py times (c3s: 844 tiles = 3 rounds of 256 + 76 tail tiles in 3 splits)
    wl = I.WORKLOADS[name]
    _announce(f"{name} one-GPU share, sampled vs oracle, the timed call")
    x, w = I.make(wl, P.DEV)
    xs, ws = wl.x_shape, wl.w_shape
    wp = PL.packed_weight(w, "bf16", "NDHWC")
    xk = x if wl.x_layout == "NDHWC" else PL.packed_input(x, "bf16")
    y = torch.full((1, ws[0]) + tuple(B.conv_out_dims(xs, ws, wl.stride, wl.pad, wl.dil)), float("nan"),
                   dtype=torch.bfloat16, device=P.DEV)
    plan = _timed_call(xk, wp, y, wl, B.IGC_BF16)
    assert not torch.isnan(y).any()
    mx, mw = float(x.abs().max()), float(w.abs().max())
    rng = np.random.default_rng(7)
    pts = P.sample_points(1, ws[0], *y.shape[2:], rng, n_random=400)
    if name == "c3s":
        assert _plan_kv(plan)["tail"] == "76/3", plan
        y_plain = PL.output(xs, ws, wl.stride, wl.pad, wl.dil, P.DEV)
        B.conv_fwd(xk, wp, y_plain, xs, ws, wl.stride, wl.pad, wl.dil, B.IGC_BF16, B.IGC_NDHWC)
        torch.cuda.synchronize()
        pts = np.concatenate([pts, _check_tail_split(y, y_plain, plan, wl.reduction, mx, mw, rng, name)])
        del y_plain
    ref = O.conv3d_points(P.bits(x), P.bits(w), pts, wl.stride, wl.pad, wl.dil, x_layout=wl.x_layout)
    P.check_close(P.gather(y, pts), ref, wl.reduction, mx, mw, name)
    _free()


def test_shards_reassemble_the_full_output():
    # the two splits the path shards along, on a reduced c3 / c5 geometry: output channels (each GPU a
    # filter slice, no exchange) and time (each GPU its output planes from its input planes plus the halo
    # planes its neighbours send, zero planes at the ends); every launch runs the same tile, so the shards'
    # outputs are the full output's slices bit for bit
    _announce("shards reassemble the full output")
    g = I.generator(8, P.DEV)
    xs, ws = (1, 256, 12, 20, 18), (192, 256, 3, 3, 3)
    x = I.draw(xs, ("normal", 1.0), g, P.DEV)
    w = I.draw(ws, ("normal", 0.02), g, P.DEV)
    one, pad1 = (1, 1, 1), (1, 1, 1)
    B.conv_debug_force(B.IGC_PATH_AUTO, B.IGC_TILE_DMA_128, 0)
    try:
        xk = PL.packed_input(x, "bf16")
        full = PL.output(xs, ws, one, pad1, one, P.DEV)
        B.conv_fwd(xk, PL.packed_weight(w, "bf16", "NDHWC"), full, xs, ws, one, pad1, one, B.IGC_BF16, B.IGC_NDHWC)
        for k0 in range(0, 192, 64):  # 3 GPUs, 64 output channels each
            wsh = (64,) + ws[1:]
            part = PL.output(xs, wsh, one, pad1, one, P.DEV)
            B.conv_fwd(xk, PL.packed_weight(w[k0:k0 + 64].contiguous(), "bf16", "NDHWC"), part, xs, wsh, one,
                       pad1, one, B.IGC_BF16, B.IGC_NDHWC)
            torch.cuda.synchronize()
            assert torch.equal(part.view(torch.int16), full[:, k0:k0 + 64].contiguous().view(torch.int16)), k0
        # time split of a 3x1x1 conv with pad (1, 0, 0): 3 GPUs of 4 output planes; GPU g reads padded
        # input planes 4g .. 4g + 5 (its own 4 and one halo plane per side), with no padding of its own
        wt = I.draw((128, 256, 3, 1, 1), ("normal", 0.03), g, P.DEV)
        wtp = PL.packed_weight(wt, "bf16", "NDHWC")
        tpad = (1, 0, 0)
        full = PL.output(xs, wt.shape, one, tpad, one, P.DEV)
        B.conv_fwd(xk, wtp, full, xs, wt.shape, one, tpad, one, B.IGC_BF16, B.IGC_NDHWC)
        xpad = torch.nn.functional.pad(xk, (0, 0, 0, 0, 0, 0, 1, 1))  # zero plane before and after (NDHWC)
        for d0 in range(0, 12, 4):
            xsh = xpad[:, d0:d0 + 6].contiguous()
            shp = (1, 256, 6, 20, 18)
            part = PL.output(shp, wt.shape, one, (0, 0, 0), one, P.DEV)
            B.conv_fwd(xsh, wtp, part, shp, wt.shape, one, (0, 0, 0), one, B.IGC_BF16, B.IGC_NDHWC)
            torch.cuda.synchronize()
            assert part.shape[2] == 4
            assert torch.equal(part.view(torch.int16), full[:, :, d0:d0 + 4].contiguous().view(torch.int16)), d0
    finally:
        B.conv_debug_force(B.IGC_PATH_AUTO, -1, 0)
    _free()
