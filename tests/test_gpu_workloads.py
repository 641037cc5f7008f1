"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

Random data: the oracle evaluates sampled output elements one by one (box
corners, edges, faces and their neighbours, chosen planes and channels, plus
uniform draws) and the relative-L2 / max-abs tolerance applies over the
sample. Exact checks at full size: a delta filter (output = shifted copy of
the input, bit for bit) and all-ones operands (output = C x number of valid
taps, a closed form), which exercise every address the kernels compute.
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


def test_c3_sampled_and_exact():
    wl = I.WORKLOADS["c3"]
    _announce("c3 bf16 sampled")
    x, w = I.make(wl, P.DEV)  # x drawn NDHWC
    xs, ws = wl.x_shape, wl.w_shape
    wp = PL.packed_weight(w, "bf16", "NDHWC")
    y = PL.output(xs, ws, wl.stride, wl.pad, wl.dil, P.DEV)
    B.conv_fwd(x, wp, y, xs, ws, wl.stride, wl.pad, wl.dil, B.IGC_BF16, B.IGC_NDHWC)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    pts = P.sample_points(1, ws[0], *y.shape[2:], rng, n_random=600, extra_k=(1023, 1024))
    ref = O.conv3d_points(P.bits(x), P.bits(w), pts, wl.stride, wl.pad, wl.dil, x_layout="NDHWC")
    P.check_close(P.gather(y, pts), ref, wl.reduction, float(x.abs().max()), float(w.abs().max()), "c3")

    _announce("c3 bf16 delta filter, full size")
    k, c = ws[0], ws[1]
    perm = torch.randperm(c, generator=torch.Generator().manual_seed(0))[:k].to(P.DEV)
    wd = torch.zeros(ws, dtype=torch.bfloat16, device=P.DEV)
    tap = (2, 0, 1)
    wd[torch.arange(k, device=P.DEV), perm, tap[0], tap[1], tap[2]] = 1.0
    wpd = PL.packed_weight(wd, "bf16", "NDHWC")
    B.conv_fwd(x, wpd, y, xs, ws, wl.stride, wl.pad, wl.dil, B.IGC_BF16, B.IGC_NDHWC)
    xpad = torch.nn.functional.pad(x, (0, 0, 1, 1, 1, 1, 1, 1))  # zero halo on D, H, W of NDHWC
    d, h, wdt = xs[2:]
    shifted = xpad[:, tap[0]:tap[0] + d, tap[1]:tap[1] + h, tap[2]:tap[2] + wdt, :]  # (N, D, H, W, C)
    expect = shifted[..., perm].permute(0, 4, 1, 2, 3)
    assert torch.equal(y.view(torch.int16), expect.contiguous().view(torch.int16))
    del xpad, shifted, expect, wd, wpd

    _announce("c3 bf16 all-ones, full size")
    x.fill_(1.0)
    wones = torch.ones(ws, dtype=torch.bfloat16, device=P.DEV)
    wp = PL.packed_weight(wones, "bf16", "NDHWC")
    B.conv_fwd(x, wp, y, xs, ws, wl.stride, wl.pad, wl.dil, B.IGC_BF16, B.IGC_NDHWC)
    cnt = (_valid_taps(d, 3, 1, P.DEV)[:, None, None] * _valid_taps(h, 3, 1, P.DEV)[None, :, None]
           * _valid_taps(wdt, 3, 1, P.DEV)[None, None, :]) * c
    assert torch.equal(y.double(), cnt.expand(1, k, d, h, wdt))
    _free()


@pytest.mark.parametrize("name", ["c4", "c4t"])
def test_fp8_sampled(name):
    wl = I.WORKLOADS[name]
    _announce(f"{name} fp8 pack (all codes) and sampled conv")
    x, w = I.make(wl, P.DEV)  # x drawn NCDHW bf16
    xs, ws = wl.x_shape, wl.w_shape
    ops = P.Fp8Operands(x, w, check_codes=True)
    y = P.run_fp8(ops, xs, ws, wl.stride, wl.pad, wl.dil)
    rng = np.random.default_rng(4)
    pts = P.sample_points(1, ws[0], *y.shape[2:], rng, n_random=600)
    sx, sw = float(ops.ref_scales[0]), float(ops.ref_scales[2])
    ref = O.conv3d_points(ops.ref_xq, ops.ref_wq, pts, wl.stride, wl.pad, wl.dil, sx=sx, sw=sw)
    mx = float(np.abs(O.e4m3_decode(ops.ref_xq)).max()) * sx
    mw = float(np.abs(O.e4m3_decode(ops.ref_wq)).max()) * sw
    P.check_close(P.gather(y, pts), ref, wl.reduction, mx, mw, name)
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

    _announce("c5 sampled vs oracle (planes across the 2^31 / 2^32 offsets)")
    wp = PL.packed_weight(w, "bf16", "NDHWC")
    y = PL.output(xs, ws, wl.stride, wl.pad, wl.dil, P.DEV)
    B.conv_fwd(xt, wp, y, xs, ws, wl.stride, wl.pad, wl.dil, B.IGC_BF16, B.IGC_NDHWC)
    torch.cuda.synchronize()
    assert y.numel() > 2 ** 31
    rng = np.random.default_rng(5)
    pts = P.sample_points(1, k, *y.shape[2:], rng, n_random=800, extra_d=(145, 146, 147, 238),
                          extra_k=(621, 622, 1023))
    xb = P.bits(x)  # 7 GB host copy, NCDHW
    ref = O.conv3d_points(xb, P.bits(w), pts, wl.stride, wl.pad, wl.dil)
    del xb
    P.check_close(P.gather(y, pts), ref, wl.reduction, float(x.abs().max()), float(w.abs().max()), "c5")

    _announce("c5 delta filter, full size (bit-exact)")
    perm = torch.randperm(c, generator=torch.Generator().manual_seed(1))[:k].to(P.DEV)
    wd = torch.zeros(ws, dtype=torch.bfloat16, device=P.DEV)
    wd[torch.arange(k, device=P.DEV), perm, 0, 0, 0] = 1.0  # tap t=0: y[:, k, od] = x[:, perm[k], od - 1]
    wpd = PL.packed_weight(wd, "bf16", "NDHWC")
    B.conv_fwd(xt, wpd, y, xs, ws, wl.stride, wl.pad, wl.dil, B.IGC_BF16, B.IGC_NDHWC)
    torch.cuda.synchronize()
    del xt
    assert torch.equal(y[:, :, 0].view(torch.int16), torch.zeros_like(y[:, :, 0]).view(torch.int16))
    for kk in range(0, k, 128):
        src = x[:, perm[kk:kk + 128], : d - 1]
        assert torch.equal(y[:, kk:kk + 128, 1:].view(torch.int16), src.view(torch.int16)), kk
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
    # one GPU's share of an 8-way split, at its real shape: the kernel that GPU would run
    wl = I.WORKLOADS[name]
    _announce(f"{name} one-GPU share, sampled vs oracle")
    x, w = I.make(wl, P.DEV)
    xs, ws = wl.x_shape, wl.w_shape
    wp = PL.packed_weight(w, "bf16", "NDHWC")
    xk = x if wl.x_layout == "NDHWC" else PL.packed_input(x, "bf16")
    y = PL.output(xs, ws, wl.stride, wl.pad, wl.dil, P.DEV)
    B.conv_fwd(xk, wp, y, xs, ws, wl.stride, wl.pad, wl.dil, B.IGC_BF16, B.IGC_NDHWC)
    torch.cuda.synchronize()
    rng = np.random.default_rng(7)
    pts = P.sample_points(1, ws[0], *y.shape[2:], rng, n_random=400)
    ref = O.conv3d_points(P.bits(x), P.bits(w), pts, wl.stride, wl.pad, wl.dil, x_layout=wl.x_layout)
    P.check_close(P.gather(y, pts), ref, wl.reduction, float(x.abs().max()), float(w.abs().max()), name)
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
    B.conv_debug_force(B.IGC_PATH_AUTO, 24, 0)
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
