"""HIP-graph capture of the library's calls. Every entry point takes the caller's stream and only enqueues
kernels (no memset, copy, allocation or synchronisation), so a sequence of calls can be captured once and
replayed. Each case captures a sequence with torch.cuda.CUDAGraph (the binding passes torch's current stream,
which is the capture stream inside the capture), then replays it several times: new inputs are copied into
the graph's static tensors before each replay, other eager GPU work and synchronisations run between the
replays, and every replay must equal the same calls run eagerly on the same inputs, bit for bit. Torch
operations that could record memsets stay outside the captures."""

import numpy as np
import pytest
import torch

from implicit_gemm_convolution_conv_amd import binding as B
from implicit_gemm_convolution_conv_amd import inputs as I

import parity as P

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _announce(name):
    print(f"[case] {name}", flush=True)


def _same(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


def _check_graph(name, static_inputs, new_inputs, run, outputs):
    """run(outs) enqueues the sequence writing into the tensors `outs`; `outputs` are the graph's static
    outputs. new_inputs(i) returns fresh values for every static input (same shapes)."""
    run(outputs)  # eager warm-up: first-call set-up happens outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(outputs)
    torch.cuda.synchronize()
    eager_out = [torch.empty_like(o) for o in outputs]
    other = torch.randn(512, 512, device=P.DEV)
    for i in range(REPLAYS):
        for dst, src in zip(static_inputs, new_inputs(i)):
            dst.copy_(src)
        torch.cuda.synchronize()
        for o in outputs:
            o.fill_(float("nan")) if o.is_floating_point() else o.zero_()
        g.replay()
        other = other @ other.T / 512  # eager work between replays
        torch.cuda.synchronize()
        run(eager_out)
        torch.cuda.synchronize()
        for k, (o, e) in enumerate(zip(outputs, eager_out)):
            assert _same(o, e), f"{name}: replay {i}, output {k} differs from the eager calls"
    del g


def _bf16(shape, seed):
    return I.draw(shape, ("normal", 1.0), I.generator(seed, P.DEV), P.DEV)


def test_graph_split_reduction():
    _announce("graph: conv_fwd_ws with a split reduction (conv + reduction pass)")
    xs, ws, st, pd, dl = (1, 64, 4, 16, 16), (64, 64, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)
    args = (xs, ws, st, pd, dl, B.IGC_BF16, B.IGC_NDHWC)
    nws = B.conv_fwd_workspace_bytes(*args)
    assert "splits=1 " not in B.conv_plan_ws(*args, nws)
    n, c, d, h, w = xs
    x = torch.empty((n, d, h, w, c), dtype=torch.bfloat16, device=P.DEV)
    wt = _bf16(ws, 1)
    wp = torch.empty((ws[0], B.conv_packed_w_cols(ws, B.IGC_BF16)), dtype=torch.bfloat16, device=P.DEV)
    B.conv_pack_w(wt, wp, ws, B.IGC_BF16, B.IGC_NDHWC)
    wsb = torch.empty(nws // 4, dtype=torch.float32, device=P.DEV)
    y = torch.empty((n, ws[0]) + B.conv_out_dims(xs, ws, st, pd, dl), dtype=torch.bfloat16, device=P.DEV)
    _check_graph("split reduction", [x], lambda i: [_bf16(x.shape, 10 + i)],
                 lambda outs: B.conv_fwd_ws(x, wp, outs[0], *args, workspace=wsb), [y])


def test_graph_tail_split_buffer_tile():
    _announce("graph: buffer tile with a tail split (6 tiles planned for 4 CUs: 2 tail tiles in 2 splits)")
    xs, ws, st, pd, dl = (1, 256, 4, 16, 24), (256, 256, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)
    args = (xs, ws, st, pd, dl, B.IGC_BF16, B.IGC_NDHWC)
    B.conv_debug_force(B.IGC_PATH_AUTO, B.IGC_TILE_BUF, 0)
    B.conv_debug_force_grid(4)
    try:
        nws = B.conv_fwd_workspace_bytes(*args)
        plan = B.conv_plan_ws(*args, nws)
        assert "tail=2/2" in plan, plan
        n, c, d, h, w = xs
        x = torch.empty((n, d, h, w, c), dtype=torch.bfloat16, device=P.DEV)
        wt = _bf16(ws, 2)
        wp = torch.empty((ws[0], B.conv_packed_w_cols(ws, B.IGC_BF16)), dtype=torch.bfloat16, device=P.DEV)
        B.conv_pack_w(wt, wp, ws, B.IGC_BF16, B.IGC_NDHWC)
        wsb = torch.empty(nws // 4, dtype=torch.float32, device=P.DEV)
        y = torch.empty((n, ws[0]) + B.conv_out_dims(xs, ws, st, pd, dl), dtype=torch.bfloat16, device=P.DEV)
        _check_graph("tail split", [x], lambda i: [_bf16(x.shape, 20 + i)],
                     lambda outs: B.conv_fwd_ws(x, wp, outs[0], *args, workspace=wsb), [y])
    finally:
        B.conv_debug_force(B.IGC_PATH_AUTO, -1, 0)
        B.conv_debug_force_grid(0)


def test_graph_fp8_pipeline():
    _announce("graph: fp8 amax -> scales -> pack x, pack w -> conv_fwd_ws")
    xs, ws, st, pd, dl = (1, 128, 6, 20, 20), (160, 128, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)
    args = (xs, ws, st, pd, dl, B.IGC_FP8_E4M3FN, B.IGC_NDHWC)
    nws = B.conv_fwd_workspace_bytes(*args)
    wsb = torch.empty(max(nws, 16) // 4, dtype=torch.float32, device=P.DEV)
    x = torch.empty(xs, dtype=torch.bfloat16, device=P.DEV)
    w = torch.empty(ws, dtype=torch.bfloat16, device=P.DEV)
    n, c, d, h, wd = xs
    amax = torch.empty(2, dtype=torch.float32, device=P.DEV)
    scales = torch.empty(4, dtype=torch.float32, device=P.DEV)
    xq = torch.empty((n, d, h, wd, c), dtype=torch.uint8, device=P.DEV)
    wq = torch.empty((ws[0], B.conv_packed_w_cols(ws, B.IGC_FP8_E4M3FN)), dtype=torch.uint8, device=P.DEV)
    y = torch.empty((n, ws[0]) + B.conv_out_dims(xs, ws, st, pd, dl), dtype=torch.bfloat16, device=P.DEV)

    def run(outs):
        yo, so = outs
        B.conv_amax(x, x.numel(), amax[0:1])
        B.conv_fp8_scales(amax[0:1], so[0:2])
        B.conv_amax(w, w.numel(), amax[1:2])
        B.conv_fp8_scales(amax[1:2], so[2:4])
        B.conv_pack_x(x, xq, xs, B.IGC_FP8_E4M3FN, so[0:2])
        B.conv_pack_w(w, wq, ws, B.IGC_FP8_E4M3FN, B.IGC_NDHWC, so[2:4])
        if nws > 0:
            B.conv_fwd_ws(xq, wq, yo, *args, so, workspace=wsb)
        else:
            B.conv_fwd(xq, wq, yo, *args, so)

    _check_graph("fp8 pipeline", [x, w],
                 lambda i: [_bf16(xs, 30 + i) * (1 + i), _bf16(ws, 40 + i) * 0.02], run, [y, scales])


def test_graph_bias_and_amax_epilogue():
    _announce("graph: conv_fwd_ex with bias and the amax of y")
    xs, ws, st, pd, dl = (2, 64, 5, 9, 11), (96, 64, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)
    args = (xs, ws, st, pd, dl, B.IGC_BF16, B.IGC_NDHWC)
    n, c, d, h, w = xs
    x = torch.empty((n, d, h, w, c), dtype=torch.bfloat16, device=P.DEV)
    wt = _bf16(ws, 3)
    wp = torch.empty((ws[0], B.conv_packed_w_cols(ws, B.IGC_BF16)), dtype=torch.bfloat16, device=P.DEV)
    B.conv_pack_w(wt, wp, ws, B.IGC_BF16, B.IGC_NDHWC)
    bias = torch.empty(ws[0], dtype=torch.float32, device=P.DEV)
    y = torch.empty((n, ws[0]) + B.conv_out_dims(xs, ws, st, pd, dl), dtype=torch.bfloat16, device=P.DEV)
    amax = torch.empty(1, dtype=torch.float32, device=P.DEV)
    _check_graph("bias + amax", [x, bias], lambda i: [_bf16(x.shape, 50 + i), torch.randn(ws[0], device=P.DEV)],
                 lambda outs: B.conv_fwd_ex(x, wp, outs[0], *args, bias=bias, y_amax=outs[1]), [y, amax])


def test_graph_point_output_and_gradients():
    _announce("graph: point-output forward, backward data and backward weights")
    xs, ws, st, pd, dl = (300, 3, 1, 14, 14), (200, 3, 1, 14, 14), (1, 14, 14), (0, 0, 0), (1, 1, 1)
    args = (xs, ws, st, pd, dl, B.IGC_BF16, B.IGC_NCDHW)
    x = torch.empty(xs, dtype=torch.bfloat16, device=P.DEV)
    w = _bf16(ws, 4) * 0.05
    wp = torch.empty((ws[0], B.conv_packed_w_cols(ws, B.IGC_BF16)), dtype=torch.bfloat16, device=P.DEV)
    B.conv_pack_w(w, wp, ws, B.IGC_BF16, B.IGC_NCDHW)
    wt = torch.empty((int(np.prod(ws[1:])), B.conv_packed_w_t_cols(ws)), dtype=torch.bfloat16, device=P.DEV)
    B.conv_pack_w_t(w, wt, ws, B.IGC_NCDHW)
    dy = torch.empty((xs[0], ws[0], 1, 1, 1), dtype=torch.bfloat16, device=P.DEV)
    nws = B.conv_bwd_weight_workspace_bytes(*args)
    wsb = torch.empty(max(nws, 16) // 4, dtype=torch.float32, device=P.DEV)
    y = torch.empty((xs[0], ws[0], 1, 1, 1), dtype=torch.bfloat16, device=P.DEV)
    dx = torch.empty(xs, dtype=torch.bfloat16, device=P.DEV)
    dw = torch.empty(ws, dtype=torch.bfloat16, device=P.DEV)

    def run(outs):
        yo, dxo, dwo = outs
        B.conv_fwd(x, wp, yo, *args)
        B.conv_bwd_data(dy, wt, dxo, *args)
        B.conv_bwd_weight(x, dy, dwo, *args, wsb)

    _check_graph("point output + gradients", [x, dy], lambda i: [_bf16(xs, 60 + i), _bf16(dy.shape, 70 + i)],
                 run, [y, dx, dw])


def test_graph_no_alloc_entry():
    _announce("graph: conv_fwd_noalloc (partial sums in the library's static scratch)")
    xs, ws, st, pd, dl = (1, 64, 4, 16, 16), (64, 64, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)
    args = (xs, ws, st, pd, dl, B.IGC_BF16, B.IGC_NDHWC)
    n, c, d, h, w = xs
    x = torch.empty((n, d, h, w, c), dtype=torch.bfloat16, device=P.DEV)
    wt = _bf16(ws, 5)
    wp = torch.empty((ws[0], B.conv_packed_w_cols(ws, B.IGC_BF16)), dtype=torch.bfloat16, device=P.DEV)
    B.conv_pack_w(wt, wp, ws, B.IGC_BF16, B.IGC_NDHWC)
    y = torch.empty((n, ws[0]) + B.conv_out_dims(xs, ws, st, pd, dl), dtype=torch.bfloat16, device=P.DEV)
    _check_graph("no-alloc", [x], lambda i: [_bf16(x.shape, 80 + i)],
                 lambda outs: B.conv_fwd_noalloc(x, wp, outs[0], *args), [y])
