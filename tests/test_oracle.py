"""Pins for the CPU oracle (no GPU).

The oracle is checked against things other than itself: torch's own conv
routines in float64 (the routine FlyDSL PR #860 validates its kernels
against), an independent numpy im2col . matmul, closed forms (delta filter,
all-ones), linearity, the point-output == matmul identity of MIOpen PR #10912,
and for the encodings torch's bf16 / float8_e4m3fn casts plus the format's
fixed points. Shapes use distinct sizes on every axis so that a transposed
index or a dropped term shows up.
"""

import itertools
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _torch_conv3d(x, w, stride, pad, dil):
    return F.conv3d(torch.from_numpy(x), torch.from_numpy(w), stride=stride, padding=pad, dilation=dil).numpy()


def _im2col_conv3d(x, w, stride, pad, dil):
    """Independent reference: explicit zero-padded input, im2col matrix, one matmul."""
    n, c, d, h, wd = x.shape
    k, _, t, r, s = w.shape
    xp = np.zeros((n, c, d + 2 * pad[0], h + 2 * pad[1], wd + 2 * pad[2]))
    xp[:, :, pad[0]:pad[0] + d, pad[1]:pad[1] + h, pad[2]:pad[2] + wd] = x
    do = (d + 2 * pad[0] - dil[0] * (t - 1) - 1) // stride[0] + 1
    ho = (h + 2 * pad[1] - dil[1] * (r - 1) - 1) // stride[1] + 1
    wo = (wd + 2 * pad[2] - dil[2] * (s - 1) - 1) // stride[2] + 1
    cols = np.empty((n, do, ho, wo, c, t, r, s))
    for a, b, e in itertools.product(range(t), range(r), range(s)):
        sl = xp[:, :,
                a * dil[0]: a * dil[0] + stride[0] * (do - 1) + 1: stride[0],
                b * dil[1]: b * dil[1] + stride[1] * (ho - 1) + 1: stride[1],
                e * dil[2]: e * dil[2] + stride[2] * (wo - 1) + 1: stride[2]]
        cols[..., a, b, e] = np.moveaxis(sl, 1, -1)
    y = cols.reshape(n * do * ho * wo, -1) @ w.reshape(k, -1).T
    return np.moveaxis(y.reshape(n, do, ho, wo, k), -1, 1)


GEOMS = [
    # x (N,C,D,H,W), w (K,C,T,R,S), stride, pad, dil
    ((2, 3, 4, 5, 6), (2, 3, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)),
    ((1, 3, 5, 4, 7), (4, 3, 2, 3, 1), (1, 2, 1), (0, 1, 0), (1, 1, 1)),
    ((2, 2, 6, 7, 5), (3, 2, 3, 2, 3), (2, 1, 2), (2, 0, 1), (1, 2, 1)),
    ((1, 4, 7, 6, 8), (2, 4, 2, 2, 3), (1, 1, 2), (1, 2, 0), (2, 1, 2)),
    ((3, 2, 3, 4, 4), (5, 2, 3, 1, 1), (1, 1, 1), (1, 0, 0), (1, 1, 1)),
    ((1, 5, 1, 6, 6), (3, 5, 1, 3, 3), (1, 3, 3), (0, 0, 0), (1, 1, 1)),
]


@pytest.mark.parametrize("geom", GEOMS)
def test_bruteforce_matches_torch_and_im2col(geom):
    xs, ws, st, pd, dl = geom
    x = _rand(xs, 1)
    w = _rand(ws, 2)
    y = O.conv3d(x, w, st, pd, dl)
    yt = _torch_conv3d(x, w, st, pd, dl)
    yi = _im2col_conv3d(x, w, st, pd, dl)
    assert y.shape == yt.shape == yi.shape
    scale = np.abs(yt).max()
    assert np.abs(y - yt).max() <= 1e-12 * scale
    assert np.abs(y - yi).max() <= 1e-12 * scale


@pytest.mark.parametrize("geom", GEOMS[:3])
def test_ndhwc_layout_is_the_same_conv(geom):
    xs, ws, st, pd, dl = geom
    x = _rand(xs, 3)
    w = _rand(ws, 4)
    y = O.conv3d(x, w, st, pd, dl)
    y2 = O.conv3d(np.ascontiguousarray(np.moveaxis(x, 1, -1)), w, st, pd, dl, x_layout="NDHWC")
    assert np.array_equal(y, y2)


def test_out_dims_match_torch():
    for xs, ws, st, pd, dl in GEOMS:
        yt = _torch_conv3d(_rand(xs, 0), _rand(ws, 0), st, pd, dl)
        assert O.out_dims(xs, ws, st, pd, dl) == yt.shape[2:]


def test_points_equal_full_output():
    xs, ws, st, pd, dl = GEOMS[2]
    x = _rand(xs, 5)
    w = _rand(ws, 6)
    y = O.conv3d(x, w, st, pd, dl)
    rng = np.random.default_rng(0)
    pts = np.stack([rng.integers(0, m, 40) for m in (y.shape[0], y.shape[1], y.shape[2], y.shape[3], y.shape[4])], 1)
    yp = O.conv3d_points(x, w, pts, st, pd, dl)
    assert np.array_equal(yp, y[tuple(pts.T)])


@pytest.mark.parametrize("tap", [(0, 0, 0), (1, 1, 1), (2, 0, 1), (0, 2, 2)])
def test_delta_filter_is_a_shifted_copy(tap):
    n, c, d, h, wd = 2, 4, 5, 6, 7
    k = 3
    perm = [2, 0, 3]  # output channel k copies input channel perm[k]
    x = _rand((n, c, d, h, wd), 7)
    w = np.zeros((k, c, 3, 3, 3))
    for kk in range(k):
        w[kk, perm[kk], tap[0], tap[1], tap[2]] = 1.0
    y = O.conv3d(x, w, (1, 1, 1), (1, 1, 1), (1, 1, 1))
    expect = np.zeros_like(y)
    for kk in range(k):
        for od, oh, ow in itertools.product(range(d), range(h), range(wd)):
            i, j, l = od + tap[0] - 1, oh + tap[1] - 1, ow + tap[2] - 1
            if 0 <= i < d and 0 <= j < h and 0 <= l < wd:
                expect[:, kk, od, oh, ow] = x[:, perm[kk], i, j, l]
    assert np.array_equal(y, expect)


def _valid_taps(size, ksz, pad):
    """Per output index, how many of the ksz taps land inside [0, size) (stride 1, dil 1)."""
    out = size + 2 * pad - ksz + 1
    return np.array([sum(0 <= o - pad + t < size for t in range(ksz)) for o in range(out)])


@pytest.mark.parametrize("ks,pad", [((3, 3, 3), (1, 1, 1)), ((3, 1, 1), (1, 0, 0)), ((2, 3, 1), (1, 2, 0))])
def test_all_ones_closed_form(ks, pad):
    c = 5
    x = np.ones((1, c, 4, 5, 6))
    w = np.ones((2, c) + ks)
    y = O.conv3d(x, w, (1, 1, 1), pad, (1, 1, 1))
    vd, vh, vw = (_valid_taps(s, k, p) for s, k, p in zip((4, 5, 6), ks, pad))
    expect = c * vd[:, None, None] * vh[None, :, None] * vw[None, None, :]
    assert np.array_equal(y[0, 0], expect) and np.array_equal(y[0, 1], expect)
    if ks == (3, 3, 3):  # corner / edge / face / interior counts 8C, 12C, 18C, 27C
        assert {y[0, 0, 0, 0, 0], y[0, 0, 0, 0, 1], y[0, 0, 0, 1, 1], y[0, 0, 1, 1, 1]} == {8 * c, 12 * c, 18 * c, 27 * c}


def test_linearity():
    xs, ws, st, pd, dl = GEOMS[3]
    x1, x2 = _rand(xs, 8), _rand(xs, 9)
    w1, w2 = _rand(ws, 10), _rand(ws, 11)
    a, b = 0.75, -1.25
    lhs = O.conv3d(a * x1 + b * x2, w1, st, pd, dl)
    rhs = a * O.conv3d(x1, w1, st, pd, dl) + b * O.conv3d(x2, w1, st, pd, dl)
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)
    lhs = O.conv3d(x1, a * w1 + b * w2, st, pd, dl)
    rhs = a * O.conv3d(x1, w1, st, pd, dl) + b * O.conv3d(x1, w2, st, pd, dl)
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("geom", GEOMS[:4])
def test_bias_matches_torch(geom):
    # the bias term of a convolution layer: torch's conv3d with bias (an independent implementation)
    xs, ws, st, pd, dl = geom
    x, w = _rand(xs, 12), _rand(ws, 13)
    b = _rand((ws[0],), 14).astype(np.float32)
    ref = F.conv3d(torch.from_numpy(x), torch.from_numpy(w), torch.from_numpy(b.astype(np.float64)), stride=st,
                   padding=pd, dilation=dl).numpy()
    assert np.allclose(O.conv3d(x, w, st, pd, dl, bias=b), ref, rtol=1e-12, atol=1e-12)


def test_bias_closed_forms():
    xs, ws, st, pd, dl = GEOMS[2]
    x = _rand(xs, 15)
    b = np.array([0.5, -3.0, 1.0e3], np.float32)
    # zero filter: y is the bias of its channel, everywhere, exactly
    y = O.conv3d(x, np.zeros(ws), st, pd, dl, bias=b)
    assert np.array_equal(y, np.broadcast_to(b.astype(np.float64)[None, :, None, None, None], y.shape))
    # with a filter: exactly bias[k] more than without (integer-valued data, every sum exact)
    xi = np.random.default_rng(16).integers(-2, 3, xs).astype(np.float64)
    wi = np.random.default_rng(17).integers(-1, 2, ws).astype(np.float64)
    d = O.conv3d(xi, wi, st, pd, dl, bias=b) - O.conv3d(xi, wi, st, pd, dl)
    assert np.array_equal(d, np.broadcast_to(b.astype(np.float64)[None, :, None, None, None], d.shape))
    # sampled points carry the same bias
    pts = np.array([[0, 0, 0, 0, 0], [1, 2, 1, 3, 1], [1, 1, 0, 2, 2]], np.int64)
    full = O.conv3d(xi, wi, st, pd, dl, bias=b)
    got = O.conv3d_points(xi, wi, pts, st, pd, dl, bias=b)
    assert np.array_equal(got, full[tuple(pts.T)])


@pytest.mark.parametrize("layout", ["NCDHW", "NDHWC"])
def test_point_output_equals_matmul(layout):
    # patch-embed geometry (stride == kernel, pad 0, input == filter extent): y = X . W^T
    n, c, h, wd, k = 7, 3, 14, 14, 5
    x = _rand((n, c, 1, h, wd), 12)
    w = _rand((k, c, 1, h, wd), 13)
    if layout == "NDHWC":
        xo = np.ascontiguousarray(np.moveaxis(x, 1, -1))
        y = O.conv3d(xo, w, (1, 14, 14), (0, 0, 0), (1, 1, 1), x_layout="NDHWC")
        # channel-last: both operands enumerate (t, r, s, c)
        ref = xo.reshape(n, -1) @ np.moveaxis(w, 1, -1).reshape(k, -1).T
    else:
        y = O.conv3d(x, w, (1, 14, 14), (0, 0, 0), (1, 1, 1))
        ref = x.reshape(n, -1) @ w.reshape(k, -1).T
    assert y.shape == (n, k, 1, 1, 1)
    assert np.allclose(y.reshape(n, k), ref, rtol=1e-12, atol=1e-12)


def test_1x1x1_equals_matmul():
    x = _rand((2, 6, 3, 4, 5), 14)
    w = _rand((4, 6, 1, 1, 1), 15)
    y = O.conv3d(x, w)
    ref = np.einsum("ncs,kc->nks", x.reshape(2, 6, -1), w.reshape(4, 6)).reshape(y.shape)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_temporal_3x1x1_equals_unfold_matmul():
    # FlyDSL PR #860 reverted unfold route: A = unfold over time (kernel 3, pad 1), y = A . W^T
    n, c, d, h, wd, k = 1, 4, 6, 3, 5, 3
    x = _rand((n, c, d, h, wd), 16)
    w = _rand((k, c, 3, 1, 1), 17)
    y = O.conv3d(x, w, (1, 1, 1), (1, 0, 0), (1, 1, 1))
    xt = torch.from_numpy(x).reshape(n * c, 1, d, h * wd)
    cols = F.unfold(xt, kernel_size=(3, 1), padding=(1, 0))  # (n*c, 3, d*h*wd)
    a = cols.reshape(n, c * 3, d * h * wd).permute(0, 2, 1).numpy()  # column order (c, t)
    ref = (a @ w.reshape(k, c * 3).T).transpose(0, 2, 1).reshape(y.shape)
    assert np.allclose(y, ref, rtol=1e-12, atol=1e-12)


def test_2d_and_1d_are_degenerate_3d():
    x2 = _rand((2, 3, 7, 6), 18)
    w2 = _rand((4, 3, 3, 2), 19)
    y = O.conv3d(x2[:, :, None], w2[:, :, None], (1, 2, 1), (0, 1, 1), (1, 1, 2))
    ref = F.conv2d(torch.from_numpy(x2), torch.from_numpy(w2), stride=(2, 1), padding=(1, 1), dilation=(1, 2)).numpy()
    assert np.allclose(y[:, :, 0], ref, rtol=1e-12, atol=1e-12)
    x1 = _rand((2, 3, 9), 20)
    w1 = _rand((4, 3, 3), 21)
    y = O.conv3d(x1[:, :, None, None], w1[:, :, None, None], (1, 1, 2), (0, 0, 1), (1, 1, 1))
    ref = F.conv1d(torch.from_numpy(x1), torch.from_numpy(w1), stride=2, padding=1).numpy()
    assert np.allclose(y[:, :, 0, 0], ref, rtol=1e-12, atol=1e-12)


def test_bf16_operands_are_exact_values():
    g = torch.Generator().manual_seed(3)
    xb = (torch.rand((1, 3, 4, 5, 6), generator=g) * 2 - 1).to(torch.bfloat16)
    wb = (torch.rand((2, 3, 3, 3, 3), generator=g) * 2 - 1).to(torch.bfloat16)
    xbits = xb.view(torch.int16).numpy().view(np.uint16)
    wbits = wb.view(torch.int16).numpy().view(np.uint16)
    y = O.conv3d(xbits, wbits, (1, 1, 1), (1, 1, 1), (1, 1, 1))
    ref = _torch_conv3d(xb.double().numpy(), wb.double().numpy(), (1, 1, 1), (1, 1, 1), (1, 1, 1))
    assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max()


# ------------------------------------------------------------------ encodings

def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    f = rng.standard_normal(100000).astype(np.float32) * np.float32(3.0)
    # exact ties at the 16 dropped bits, both parities, plus carries into the exponent
    ties = (rng.integers(0, 1 << 15, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    edge = np.array([0.0, -0.0, 1.0, -1.0, 3.3895314e38, 1e-40, -1e-40, 65504.0, np.inf, -np.inf], np.float32)
    allf = np.concatenate([f, ties, edge])
    ours = O.bf16_round(allf)
    ref = torch.from_numpy(allf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    nan = np.isnan(allf)  # NaN payloads are not compared, only that NaN stays NaN
    assert np.array_equal(ours[~nan], ref[~nan])
    assert np.all((ours[nan] & 0x7F80) == 0x7F80) and np.all((ours[nan] & 0x7F) != 0)


def _golden_e4m3():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3fn_fixed_points.txt")) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if line:
                code, val = line.split()
                rows.append((int(code, 16), float(val)))
    return rows


def test_e4m3_decode_fixed_points():
    for code, val in _golden_e4m3():
        got = O.e4m3_decode(np.array([code], np.uint8))[0]
        if math.isnan(val):
            assert math.isnan(got)
        else:
            assert got == val, hex(code)


def test_e4m3_decode_matches_torch_for_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    fin = ~np.isnan(ref)
    assert np.array_equal(ours[fin], ref[fin])


def test_e4m3_round_trip_and_order():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    vals = O.e4m3_decode(codes)
    back = O.e4m3_encode(vals.astype(np.float32))
    # -0.0 encodes back to 0x80, so the round trip is exact on every finite code
    assert np.array_equal(back, codes)
    pos = O.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(pos) > 0)


def test_e4m3_ties_go_to_even_and_saturate():
    pos = O.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)  # midpoints are exact in fp32
    got = O.e4m3_encode(mids)
    lo = np.arange(0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, expect.astype(np.uint8))
    assert np.array_equal(O.e4m3_encode(-mids), (expect | 0x80).astype(np.uint8))
    big = np.array([448.0, 460.0, 464.0, 1e6, np.inf, -500.0], np.float32)
    assert np.array_equal(O.e4m3_encode(big), np.array([0x7E] * 5 + [0xFE], np.uint8))
    assert O.e4m3_encode(np.array([np.nan], np.float32))[0] & 0x7F == 0x7F
    assert O.e4m3_encode(np.array([2.0 ** -10], np.float32))[0] == 0x00  # half the smallest subnormal: tie -> 0
    assert O.e4m3_encode(np.array([2.0 ** -10 * 1.5], np.float32))[0] == 0x01


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(1)
    f = np.concatenate([rng.standard_normal(200000) * 60, rng.standard_normal(20000) * 1e-3]).astype(np.float32)
    f = f[np.abs(f) < 464]  # torch's cast is not saturating; below 464 both round to nearest even
    ours = O.e4m3_encode(f)
    ref = torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


def test_amax_and_scales():
    g = torch.Generator().manual_seed(5)
    t = torch.randn(12345, generator=g).to(torch.bfloat16)
    bits = t.view(torch.int16).numpy().view(np.uint16)
    amax = O.amax_bf16(bits)
    assert amax == float(t.float().abs().max())
    s, inv = O.fp8_scales(amax)
    assert s == np.float32(amax) / np.float32(448.0)
    assert inv == np.float32(448.0) / np.float32(amax)
    assert O.fp8_scales(0.0) == (1.0, 1.0)
    q = O.quantize_e4m3(bits, inv)
    ref = (t.float() * torch.tensor(inv)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q, ref)
    assert np.abs(O.e4m3_decode(q)).max() <= 448.0


def test_fp8_conv_is_conv_of_dequantised_values():
    g = torch.Generator().manual_seed(6)
    xb = torch.randn((1, 4, 3, 5, 4), generator=g).to(torch.bfloat16)
    wb = (torch.randn((3, 4, 3, 1, 2), generator=g) * 0.1).to(torch.bfloat16)
    xq, sx, _ = O.quantize_tensor_e4m3(xb.view(torch.int16).numpy().view(np.uint16))
    wq, sw, _ = O.quantize_tensor_e4m3(wb.view(torch.int16).numpy().view(np.uint16))
    y = O.conv3d(xq, wq, (1, 1, 1), (1, 0, 1), (1, 1, 1), sx=sx, sw=sw)
    xd = torch.from_numpy(xq).view(torch.float8_e4m3fn).double() * float(sx)
    wd = torch.from_numpy(wq).view(torch.float8_e4m3fn).double() * float(sw)
    ref = F.conv3d(xd, wd, padding=(1, 0, 1)).numpy()
    assert np.abs(y - ref).max() <= 1e-12 * np.abs(ref).max()


# ------------------------------------------------------------------ gradients

@pytest.mark.parametrize("geom", GEOMS)
def test_gradients_match_torch_autograd(geom):
    # torch's autograd of conv3d in float64 is an independent implementation of both adjoints
    xs, ws, st, pd, dl = geom
    x, w = _rand(xs, 20), _rand(ws, 21)
    xt = torch.from_numpy(x).requires_grad_()
    wt = torch.from_numpy(w).requires_grad_()
    y = F.conv3d(xt, wt, stride=st, padding=pd, dilation=dl)
    dy = _rand(tuple(y.shape), 22)
    gx, gw = torch.autograd.grad(y, (xt, wt), torch.from_numpy(dy))
    assert np.allclose(O.conv3d_bwd_data(dy, w, xs, st, pd, dl), gx.numpy(), rtol=1e-12, atol=1e-12)
    assert np.allclose(O.conv3d_bwd_weight(x, dy, ws, st, pd, dl), gw.numpy(), rtol=1e-12, atol=1e-12)
    # channel-last x: the same gradients, dx laid out NDHWC
    xl = np.ascontiguousarray(np.moveaxis(x, 1, -1))
    assert np.allclose(O.conv3d_bwd_data(dy, w, xs, st, pd, dl, x_layout="NDHWC"),
                       np.moveaxis(gx.numpy(), 1, -1), rtol=1e-12, atol=1e-12)
    assert np.allclose(O.conv3d_bwd_weight(xl, dy, ws, st, pd, dl, x_layout="NDHWC"), gw.numpy(),
                       rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("geom", GEOMS)
def test_gradients_are_the_adjoints(geom):
    # <conv(x, w), dy> = <x, dgrad(dy, w)> = <w, wgrad(x, dy)>; integer data keeps every sum exact
    xs, ws, st, pd, dl = geom
    rng = np.random.default_rng(23)
    x = rng.integers(-3, 4, xs).astype(np.float64)
    w = rng.integers(-3, 4, ws).astype(np.float64)
    y = O.conv3d(x, w, st, pd, dl)
    dy = rng.integers(-3, 4, y.shape).astype(np.float64)
    lhs = float(np.sum(y * dy))
    assert float(np.sum(x * O.conv3d_bwd_data(dy, w, xs, st, pd, dl))) == lhs
    assert float(np.sum(w * O.conv3d_bwd_weight(x, dy, ws, st, pd, dl))) == lhs


@pytest.mark.parametrize("layout", ["NCDHW", "NDHWC"])
def test_point_output_gradients_are_gemms(layout):
    # point output (input extent == filter extent, stride == filter): both gradients are one GEMM over the
    # batch in the layout's own element order (MIOpen PR #10912, PR body)
    xs, ws, st = (7, 3, 2, 4, 4), (5, 3, 2, 4, 4), (2, 4, 4)
    x, w = _rand(xs, 24), _rand(ws, 25)
    dy = _rand((7, 5, 1, 1, 1), 26)
    n, k = 7, 5
    if layout == "NDHWC":
        xl = np.ascontiguousarray(np.moveaxis(x, 1, -1))
        wl = np.moveaxis(w, 1, -1).reshape(k, -1)
    else:
        xl, wl = x, w.reshape(k, -1)
    dx = O.conv3d_bwd_data(dy, w, xs, st, x_layout=layout)
    assert np.allclose(dx.reshape(n, -1), dy.reshape(n, k) @ wl, rtol=1e-12, atol=1e-12)
    dw = O.conv3d_bwd_weight(xl, dy, ws, st, x_layout=layout)
    dwl = np.moveaxis(dw, 1, -1).reshape(k, -1) if layout == "NDHWC" else dw.reshape(k, -1)
    assert np.allclose(dwl, dy.reshape(n, k).T @ xl.reshape(n, -1), rtol=1e-12, atol=1e-12)


def test_gradients_of_bf16_operands_are_exact_values():
    # bf16 bit patterns widen exactly: gradients of the bit patterns equal gradients of their values
    xs, ws, st, pd, dl = GEOMS[0]
    xb = O.bf16_round(_rand(xs, 27).astype(np.float32))
    wb = O.bf16_round(_rand(ws, 28).astype(np.float32))
    dyb = O.bf16_round(_rand((2, 2, 4, 5, 6), 29).astype(np.float32))
    xv, wv, dyv = O.bf16_value(xb), O.bf16_value(wb), O.bf16_value(dyb)
    assert np.array_equal(O.conv3d_bwd_data(dyb, wb, xs, st, pd, dl), O.conv3d_bwd_data(dyv, wv, xs, st, pd, dl))
    assert np.array_equal(O.conv3d_bwd_weight(xb, dyb, ws, st, pd, dl), O.conv3d_bwd_weight(xv, dyv, ws, st, pd, dl))
