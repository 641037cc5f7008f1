#!/usr/bin/env python3
"""Forward implicit-GEMM conv benchmark on one MI355X.

Step = one forward convolution of the headline workload, conv3d bf16 NDHWC
N=1 C=2048 D=60 H=80 W=45, K=2048, 3x3x3, stride 1, pad 1 (GEMM
216000 x 2048 x 55296, 4.892e13 flop), with x already resident in HBM in
NDHWC and the filter packed once beforehand (it is a layer's constant). The
call is conv_fwd_ws with a workspace allocated once beforehand: its last,
partial round of tiles (96 of 6752) runs split along the reduction, so a step
is the conv kernel plus the small pass that adds those tiles' partial sums.
Throughput = 2*M*N*R / time (TFLOPS).

Printed as ONE JSON line on stdout (everything else goes to stderr):
  value          TFLOPS of the timed steps (W untimed warm-up steps first)
  roofline       the conv kernel against dense bf16 MFMA peak, its duration
                 taken with HIP events on the stream it is launched on
  cpu_baseline   the fp64 CPU oracle timed on a bounded sample of the same
                 workload's outputs, in the same unit
  extra          the other workloads (fp8 kernel-only and end-to-end with
                 amax + scales + pack, the 3x1x1 temporal variant, the
                 point-output patch embed, the >2^31-element 3x1x1 conv)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}  # dense MFMA, MI355X published figures
PEAK_HBM_GBS = 8000.0
# sources that decide the headline kernel's code and launch configuration
KERNEL_SOURCES = ["implicit_gemm_convolution_conv_amd/csrc/conv_igemm.h",
                  "implicit_gemm_convolution_conv_amd/csrc/conv_igemm_dma.h",
                  "implicit_gemm_convolution_conv_amd/csrc/conv_igemm_buf.h",
                  "implicit_gemm_convolution_conv_amd/csrc/conv_igemm_pp.h",
                  "implicit_gemm_convolution_conv_amd/csrc/conv_buf_bf16.hip",
                  "implicit_gemm_convolution_conv_amd/csrc/splitk.hip",
                  "implicit_gemm_convolution_conv_amd/csrc/igconv_internal.h",
                  "implicit_gemm_convolution_conv_amd/csrc/api.hip",
                  "implicit_gemm_convolution_conv_amd/csrc/tile_table.h"]
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "conv_igemm_c3_bf16_traffic.json")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def conv_flops(xshape, wshape, stride, pad, dil):
    """2 * M * K * R, R = C*T*R*S, M = N*Do*Ho*Wo (padding taps included)."""
    n, c, d, h, w = xshape
    k, _, t, r, s = wshape
    do = (d + 2 * pad[0] - dil[0] * (t - 1) - 1) // stride[0] + 1
    ho = (h + 2 * pad[1] - dil[1] * (r - 1) - 1) // stride[1] + 1
    wo = (w + 2 * pad[2] - dil[2] * (s - 1) - 1) // stride[2] + 1
    return 2 * n * do * ho * wo * k * c * t * r * s


def kernel_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


_SPIN = {}


def spin_cycles(torch, ms):
    """Argument of torch.cuda._sleep (a bounded spin kernel) that keeps the stream busy for about `ms`."""
    if "per_ms" not in _SPIN:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        torch.cuda._sleep(1_000_000)
        b.record()
        b.synchronize()
        _SPIN["per_ms"] = 1e6 / max(a.elapsed_time(b), 1e-3)
    return int(_SPIN["per_ms"] * ms)


def time_launches(fn, steps, warmup, torch, stats=None, between=None, queued=False):
    """Run fn warmup times, then `steps` times with an event pair around each call
    on the current stream (the one the library launches on). Returns (wall ms per
    step, mean event ms per call); `stats`, if a dict, also receives the median
    and minimum event ms. `between`, if given, runs before every timed call
    outside its events (the cold-cache figure evicts the caches with it).

    With `queued`, a spin kernel holds the stream while the host enqueues every
    timed call, so that no call waits for the host's launch of the next one:
    the events then time the GPU's work alone, which is what a kernel of a few
    microseconds needs (without it a call's events also span the host time of
    its launch whenever the GPU had drained the queue). The wall time is then
    not a throughput and is returned as None; stats["gap"] is the time per call
    between the calls' event pairs (near zero when the queue never drained)."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    if queued:
        spin = spin_cycles(torch, 2.0 + 0.25 * steps)
    t0 = time.perf_counter()
    if queued:
        torch.cuda._sleep(spin)
    for a, b in evs:
        if between is not None:
            between()
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    times = sorted(a.elapsed_time(b) for a, b in evs)
    ev = sum(times) / steps
    if stats is not None:
        stats["median"] = times[len(times) // 2] if len(times) % 2 else 0.5 * (times[len(times) // 2 - 1] +
                                                                                times[len(times) // 2])
        stats["min"] = times[0]
        if queued:
            stats["gap"] = (evs[0][0].elapsed_time(evs[-1][1]) - sum(times)) / steps
            # and the calls back to back with one event pair around them all: the per-call time of a
            # stream of calls, with no timestamp work between the kernels; nine such batches, their
            # per-call times' mean and median
            per_call = []
            for _ in range(9):
                a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                torch.cuda._sleep(spin)
                a.record(stream)
                for _ in range(steps):
                    fn()
                b.record(stream)
                torch.cuda.synchronize()
                per_call.append(a.elapsed_time(b) / steps)
            stats["b2b"] = sum(per_call) / len(per_call)
            stats["b2b_median"] = sorted(per_call)[len(per_call) // 2]
    return (None if queued else wall), ev


def bench_workload(name, steps, warmup, torch, B, I, PL):
    """Returns a dict of timings for one workload (GPU tensors freed after)."""
    wl = I.WORKLOADS[name]
    x, w = I.make(wl, "cuda")
    xshape, wshape = wl.x_shape, wl.w_shape
    flops = conv_flops(xshape, wshape, wl.stride, wl.pad, wl.dil)
    y = PL.output(xshape, wshape, wl.stride, wl.pad, wl.dil, "cuda")
    res = {"workload": wl.note, "flop": flops}
    if wl.dtype == "bf16":
        if name in ("c2", "pw"):  # point output / 1x1x1: x read as is (NCDHW), filter in (c, t, r, s) order
            wp = PL.packed_weight(w, "bf16", "NCDHW")
            lay, xk = B.IGC_NCDHW, x
        else:
            wp = PL.packed_weight(w, "bf16", "NDHWC")
            lay = B.IGC_NDHWC
            xk = x if wl.x_layout == "NDHWC" else PL.packed_input(x, "bf16")
        # The step is the library's call for this workload: conv_fwd_ws with a preallocated workspace where
        # the plan uses one (split reduction of an under-filled grid, or the tail split of a partial last
        # round), conv_fwd otherwise; conv_fwd without the workspace is timed beside it.
        nws = B.conv_fwd_workspace_bytes(xshape, wshape, wl.stride, wl.pad, wl.dil, B.IGC_BF16, lay)
        wsb = torch.empty(nws // 4, dtype=torch.float32, device="cuda") if nws > 0 else None
        res["plan"] = B.conv_plan_ws(xshape, wshape, wl.stride, wl.pad, wl.dil, B.IGC_BF16, lay, max(nws, 0))
        res["workspace_bytes"] = max(nws, 0)

        def plain_step():
            B.conv_fwd(xk, wp, y, xshape, wshape, wl.stride, wl.pad, wl.dil, B.IGC_BF16, lay)

        def step():
            if wsb is None:
                plain_step()
            else:
                B.conv_fwd_ws(xk, wp, y, xshape, wshape, wl.stride, wl.pad, wl.dil, B.IGC_BF16, lay, workspace=wsb)

        st = {}
        wall, ev = time_launches(step, steps, warmup, torch, st)
        res.update(ms=wall, kernel_ms=ev, kernel_ms_median=st["median"], kernel_ms_min=st["min"],
                   tflops=flops / (wall * 1e-3) / 1e12, kernel_tflops=flops / (ev * 1e-3) / 1e12)
        if name in ("c1", "c2"):  # a few microseconds: the GPU's own time per call, with the calls queued
            qst = {}
            _, qev = time_launches(step, steps, warmup, torch, qst, queued=True)
            res.update(queued_kernel_ms=qev, queued_kernel_ms_median=qst["median"], queued_kernel_ms_min=qst["min"],
                       queued_gap_ms=qst["gap"], queued_kernel_tflops=flops / (qst["median"] * 1e-3) / 1e12,
                       back_to_back_ms=qst["b2b"], back_to_back_tflops=flops / (qst["b2b"] * 1e-3) / 1e12,
                       back_to_back_ms_median=qst["b2b_median"],
                       kernel_time_note="an event pair around a lone call adds 2-3 us of GPU-side timestamp work; "
                                        "back_to_back_ms_median (median over 9 batches of calls issued back to "
                                        "back, one event pair per batch) is the per-call kernel time and agrees "
                                        "with rocprofv3's kernel durations")
        if name in ("c1", "c2"):  # working set fits the MALL: also with the caches evicted before every call
            scratch = torch.empty(1 << 28, dtype=torch.int16, device="cuda")  # 512 MB
            cst = {}
            time_launches(step, steps, warmup, torch, cst, between=lambda: scratch.fill_(1))
            res.update(cold_kernel_ms_median=cst["median"], cold_kernel_ms_min=cst["min"])
            del scratch
        if wsb is not None:
            res["plain_plan"] = B.conv_plan(xshape, wshape, wl.stride, wl.pad, wl.dil, B.IGC_BF16, lay)
            pst = {}
            _, pev = time_launches(plain_step, steps, warmup, torch, pst)
            res.update(plain_kernel_ms=pev, plain_kernel_ms_median=pst["median"], plain_kernel_ms_min=pst["min"])
            del wsb
        if name == "pw":  # HBM-bound: x and y once, the filter per 64 output channels
            nbytes = 2 * (x.numel() + y.numel() + w.numel())
            res.update(kernel_gbs=nbytes / (ev * 1e-3) / 1e9, hbm_frac=nbytes / (ev * 1e-3) / 1e9 / PEAK_HBM_GBS)
        if name not in ("c2", "pw") and wl.x_layout != "NDHWC":  # also the bf16 transpose that feeds it
            xt = torch.empty((xshape[0],) + tuple(xshape[2:]) + (xshape[1],), dtype=torch.bfloat16, device="cuda")
            _, ev_t = time_launches(lambda: B.conv_pack_x(x, xt, xshape, B.IGC_BF16), steps, warmup, torch)
            nbytes = 4 * x.numel()
            res.update(transpose_ms=ev_t, transpose_gbs=nbytes / (ev_t * 1e-3) / 1e9)
            del xt
    else:
        scales = PL.fp8_scales(x, w)
        wq = PL.packed_weight(w, "fp8", "NDHWC", scales[2:4])
        n, c, d, h, wd = xshape
        xq = torch.empty((n, d, h, wd, c), dtype=torch.uint8, device="cuda")
        amax = torch.empty(1, dtype=torch.float32, device="cuda")
        fargs = (xshape, wshape, wl.stride, wl.pad, wl.dil, B.IGC_FP8_E4M3FN, B.IGC_NDHWC)
        nws = B.conv_fwd_workspace_bytes(*fargs)  # the tail split of a partial last round, when planned
        wsb = torch.empty(nws // 4, dtype=torch.float32, device="cuda") if nws > 0 else None
        res["plan"] = B.conv_plan_ws(*fargs, max(nws, 0))
        res["workspace_bytes"] = max(nws, 0)

        def prep():
            B.conv_amax(x, x.numel(), amax)
            B.conv_fp8_scales(amax, scales[0:2])
            B.conv_pack_x(x, xq, xshape, B.IGC_FP8_E4M3FN, scales[0:2])

        def plain_conv():
            B.conv_fwd(xq, wq, y, *fargs, scales)

        def conv():
            if wsb is None:
                plain_conv()
            else:
                B.conv_fwd_ws(xq, wq, y, *fargs, scales, workspace=wsb)

        def e2e():
            prep()
            conv()

        st = {}
        _, ev_k = time_launches(conv, steps, warmup, torch, st)
        res.update(kernel_ms_median=st["median"], kernel_ms_min=st["min"])
        wall_e, ev_e = time_launches(e2e, steps, warmup, torch)
        _, ev_p = time_launches(lambda: B.conv_pack_x(x, xq, xshape, B.IGC_FP8_E4M3FN, scales[0:2]), steps,
                                warmup, torch)
        _, ev_a = time_launches(lambda: B.conv_amax(x, x.numel(), amax), steps, warmup, torch)
        res.update(kernel_ms=ev_k, kernel_tflops=flops / (ev_k * 1e-3) / 1e12, e2e_ms=ev_e,
                   e2e_tflops=flops / (ev_e * 1e-3) / 1e12, pack_ms=ev_p,
                   pack_gbs=3 * x.numel() / (ev_p * 1e-3) / 1e9, amax_ms=ev_a,
                   amax_gbs=2 * x.numel() / (ev_a * 1e-3) / 1e9)
        if wsb is not None:
            pst = {}
            _, pev = time_launches(plain_conv, steps, warmup, torch, pst)
            res.update(plain_kernel_ms=pev, plain_kernel_ms_median=pst["median"], plain_kernel_ms_min=pst["min"])
        del xq, wq, scales, wsb
    del x, w, y
    torch.cuda.empty_cache()
    return res


def bench_epilogue(steps, warmup, torch, B, I, PL):
    """The headline conv with the fused epilogue extras (bias + amax of y, conv_fwd_ex)
    against the plain conv followed by a separate amax pass over y."""
    wl = I.WORKLOADS["c3"]
    x, w = I.make(wl, "cuda")
    xs, ws = wl.x_shape, wl.w_shape
    y = PL.output(xs, ws, wl.stride, wl.pad, wl.dil, "cuda")
    wp = PL.packed_weight(w, "bf16", "NDHWC")
    bias = torch.randn(ws[0], generator=I.generator(33, "cuda"), device="cuda", dtype=torch.float32)
    amax = torch.empty(1, dtype=torch.float32, device="cuda")
    args = (xs, ws, wl.stride, wl.pad, wl.dil, B.IGC_BF16, B.IGC_NDHWC)

    def fused():
        B.conv_fwd_ex(x, wp, y, *args, bias=bias, y_amax=amax)

    def plain():
        B.conv_fwd(x, wp, y, *args)

    def separate():
        plain()
        B.conv_amax(y, y.numel(), amax)

    res = {"workload": wl.note + " + bias + amax(y)"}
    for key, fn in (("fused", fused), ("plain", plain), ("separate", separate)):
        st = {}
        _, ev = time_launches(fn, steps, warmup, torch, st)
        res.update({f"{key}_ms": ev, f"{key}_ms_median": st["median"]})
    _, ev_a = time_launches(lambda: B.conv_amax(y, y.numel(), amax), steps, warmup, torch)
    res.update(amax_pass_ms=ev_a, amax_pass_gbs=2 * y.numel() / (ev_a * 1e-3) / 1e9)
    del x, w, y, wp
    torch.cuda.empty_cache()
    return res


def bench_grad(steps, warmup, torch, B, I, PL):
    """Gradients of the point-output patch embed (c2 shape): backward data and backward weights."""
    wl = I.WORKLOADS["c2"]
    x, w = I.make(wl, "cuda")
    xs, ws = wl.x_shape, wl.w_shape
    st, pd, dl = wl.stride, wl.pad, wl.dil
    dy = torch.randn((xs[0], ws[0], 1, 1, 1), generator=I.generator(34, "cuda"), device="cuda").to(torch.bfloat16)
    wt = torch.empty((int(w[0].numel()), B.conv_packed_w_t_cols(ws)), dtype=torch.bfloat16, device="cuda")
    B.conv_pack_w_t(w, wt, ws, B.IGC_NCDHW)
    dx = torch.empty_like(x)
    dw = torch.empty_like(w)
    nws = B.conv_bwd_weight_workspace_bytes(xs, ws, st, pd, dl, B.IGC_BF16, B.IGC_NCDHW)
    wsb = torch.empty(nws, dtype=torch.uint8, device="cuda")
    flops = 2 * xs[0] * ws[0] * int(w[0].numel())
    res = {"workload": wl.note + ": backward data and backward weights", "flop": flops, "workspace_bytes": nws}
    for key, fn in (("dgrad", lambda: B.conv_bwd_data(dy, wt, dx, xs, ws, st, pd, dl, B.IGC_BF16, B.IGC_NCDHW)),
                    ("wgrad", lambda: B.conv_bwd_weight(x, dy, dw, xs, ws, st, pd, dl, B.IGC_BF16, B.IGC_NCDHW,
                                                       wsb))):
        stt, cst, qst = {}, {}, {}
        _, ev = time_launches(fn, steps, warmup, torch, stt)
        time_launches(fn, steps, warmup, torch, qst, queued=True)
        res.update({f"{key}_queued_ms_median": qst["median"], f"{key}_queued_gap_ms": qst["gap"],
                    f"{key}_back_to_back_ms": qst["b2b"], f"{key}_back_to_back_ms_median": qst["b2b_median"]})
        scratch = torch.empty(1 << 28, dtype=torch.int16, device="cuda")
        time_launches(fn, steps, warmup, torch, cst, between=lambda: scratch.fill_(1))
        del scratch
        res.update({f"{key}_ms": ev, f"{key}_ms_median": stt["median"], f"{key}_ms_min": stt["min"],
                    f"{key}_cold_ms_median": cst["median"], f"{key}_tflops": flops / (stt["median"] * 1e-3) / 1e12})
    del x, w, dy, wt, dx, dw, wsb
    torch.cuda.empty_cache()
    return res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_threads():
    """Threads the oracle runs on: every core of the process's affinity mask, within the OMP_NUM_THREADS budget
    of the host when it sets one (the GPU hosts give one GPU's process a share of their cores that way)."""
    affinity = len(os.sched_getaffinity(0))
    budget = int(os.environ.get("OMP_NUM_THREADS", "0") or 0)
    return min(affinity, budget) if budget > 0 else affinity, affinity


def cpu_baseline(seconds: float, I):
    """The fp64 oracle on a bounded random sample of the headline workload's outputs, and on the whole of the two
    small workloads (c1, c2)."""
    import numpy as np
    import torch
    from oracle import oracle as O

    threads, affinity = oracle_threads()
    O.set_threads(threads)
    full = {}
    for name in ("c1", "c2"):  # evaluated in full: every output element
        wl = I.WORKLOADS[name]
        x, w = I.make(wl, "cpu")
        xb, wb = I.bf16_bits(x), I.bf16_bits(w)
        flop = conv_flops(wl.x_shape, wl.w_shape, wl.stride, wl.pad, wl.dil)
        t0 = time.perf_counter()
        O.conv3d(xb, wb, wl.stride, wl.pad, wl.dil)
        t = time.perf_counter() - t0
        full[name] = {"seconds": round(t, 3), "tflops": round(flop / t / 1e12, 6), "workload": wl.note}

    wl = I.WORKLOADS["c3"]
    x, w = I.make(wl, "cuda")  # same seeded draw as the GPU run
    xb, wb = I.bf16_bits(x), I.bf16_bits(w)
    del x, w
    torch.cuda.empty_cache()
    n, c, d, h, wd = wl.x_shape
    k = wl.w_shape[0]
    do, ho, wo = O.out_dims(wl.x_shape, wl.w_shape, wl.stride, wl.pad, wl.dil)
    rng = np.random.default_rng(0)
    R = wl.reduction

    def run(npts):
        pts = np.stack([rng.integers(0, m, npts) for m in (n, k, do, ho, wo)], 1)
        t0 = time.perf_counter()
        O.conv3d_points(xb, wb, pts, wl.stride, wl.pad, wl.dil, x_layout="NDHWC")
        return time.perf_counter() - t0

    npts = 8 * threads
    t = run(npts)
    while t < 0.5:
        npts *= 4
        t = run(npts)
    npts = max(npts, int(npts * seconds / t))
    t = run(npts)
    return {"value": round(2.0 * R * npts / t / 1e12, 6), "unit": "TFLOPS", "cores": O.get_threads(),
            "kind": "oracle",
            "sample": f"{npts} random output elements of {wl.note} (each a {R}-term fp64 dot product), "
                      f"{t:.1f} s; extrapolated linearly to the whole output",
            "affinity_cores": affinity, "cpu_model": cpu_model(), "full": full}


def copy_rates(steps, torch):
    """Device-to-device copy rate of 1 GiB on this GPU (GB/s, bytes read + written): the ceiling a kernel that
    reads and writes every byte once reaches here, next to the 8 TB/s HBM peak."""
    src = torch.empty(1 << 29, dtype=torch.int16, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    nbytes = src.numel() * 2
    st = {}
    time_launches(lambda: dst.copy_(src), steps, 3, torch, st)
    copy = 2 * nbytes / (st["median"] * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"d2d_copy_gbs": round(copy, 1), "bytes": nbytes,
            "note": "1 GiB tensor copied with torch copy_ (hipMemcpy device to device); median of the event times"}


def traffic_bytes():
    """HBM bytes per launch of the conv kernel from committed counter runs, if taken on this kernel source."""
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_hash") != kernel_hash():
        return None
    return rec.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true")
    ap.add_argument("--only", default=None,
                    help="comma list of extra workloads (copy,c1,c2,c4,c4t,c5,pw,c3ex,c2grad,c3s,c5s)")
    ap.add_argument("--profile", action="store_true",
                    help="counter-collection run: the headline conv `steps` times, then one 1 GiB device copy "
                         "(the reference for scaling FETCH_SIZE / WRITE_SIZE); prints nothing else")
    ap.add_argument("--profile-group-m", type=int, default=0,
                    help="with --profile: grouped-raster height in tiles (0 = the planner's choice)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on exactly one GPU: this library has no multi-GPU path (one process, one device).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from implicit_gemm_convolution_conv_amd import binding as B
    from implicit_gemm_convolution_conv_amd import inputs as I
    from implicit_gemm_convolution_conv_amd import pipeline as PL

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    B.load()
    torch.cuda.set_device(0)

    if args.profile:
        wl = I.WORKLOADS["c3"]
        x, w = I.make(wl, "cuda")
        wp = PL.packed_weight(w, "bf16", "NDHWC")
        y = PL.output(wl.x_shape, wl.w_shape, wl.stride, wl.pad, wl.dil, "cuda")
        args5 = (wl.x_shape, wl.w_shape, wl.stride, wl.pad, wl.dil, B.IGC_BF16, B.IGC_NDHWC)
        nws = B.conv_fwd_workspace_bytes(*args5)
        wsb = torch.empty(max(nws, 16) // 4, dtype=torch.float32, device="cuda")
        if args.profile_group_m > 0:  # a raster-height sweep: same tiles and arithmetic, another tile order
            B.conv_debug_force(B.IGC_PATH_AUTO, -1, args.profile_group_m)
        log(f"[bench] profile plan: {B.conv_plan_ws(*args5, max(nws, 0))}")
        for _ in range(args.steps):  # the bench's step: conv_fwd_ws with its workspace
            B.conv_fwd_ws(x, wp, y, *args5, workspace=wsb if nws > 0 else None)
        src = torch.empty(1 << 29, dtype=torch.int16, device="cuda").fill_(1)  # 1 GiB
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] profile run done: {args.steps} conv launches, one {src.numel() * 2} byte copy")
        return

    log(f"[bench] headline c3 bf16, {args.steps} steps after {args.warmup} warm-up")
    head = bench_workload("c3", args.steps, args.warmup, torch, B, I, PL)
    log(f"[bench] c3: {head['ms']:.3f} ms/step, {head['tflops']:.1f} TFLOPS ({head['plan']})")

    extra = {}
    if not args.no_extra:
        names = args.only.split(",") if args.only else ["copy", "c1", "c2", "c4", "c4t", "c5", "pw", "c3ex", "c2grad",
                                                         "c3s", "c5s"]
        for name in names:
            log(f"[bench] extra workload {name}")
            if name == "copy":
                extra[name] = copy_rates(max(20, args.steps), torch)
            elif name == "c3ex":
                extra[name] = bench_epilogue(max(20, args.steps), args.warmup, torch, B, I, PL)
            elif name == "c2grad":
                extra[name] = bench_grad(max(20, args.steps), args.warmup, torch, B, I, PL)
            else:
                extra[name] = bench_workload(name, max(20, args.steps), args.warmup, torch, B, I, PL)
            log(f"[bench] {name}: {json.dumps(extra[name])}")
        ceiling = extra.get("copy", {}).get("d2d_copy_gbs")
        if ceiling:  # data-movement kernels against the measured copy rate as well as the 8 TB/s peak
            for rec in extra.values():
                for key in ("pack_gbs", "transpose_gbs", "amax_gbs", "kernel_gbs", "amax_pass_gbs"):
                    if key in rec:
                        rec[key.replace("_gbs", "_vs_copy")] = round(rec[key] / ceiling, 4)

    cpu = None
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline (oracle), ~{args.cpu_seconds:.0f} s")
        cpu = cpu_baseline(args.cpu_seconds, I)
        log(f"[bench] cpu: {cpu}")

    achieved = head["kernel_tflops"]
    out = {
        "metric": "conv fwd TFLOPS + % of MFMA peak (bf16/fp8), c2048 3x3x3 D60xH80xW45",
        "value": round(head["tflops"], 2),
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; x ~ N(0,1), w ~ N(0, 1/sqrt(C*27)), bf16)",
        "config": {"workload": "conv3d fwd bf16 NDHWC N=1 C=2048 D=60 H=80 W=45 K=2048 3x3x3 stride 1 pad 1",
                   "gemm_m": 216000, "gemm_n": 2048, "reduction": 55296, "flop_per_step": head["flop"],
                   "plan": head["plan"], "kernel_ms_mean": round(head["kernel_ms"], 4),
                   "kernel_ms_median": round(head["kernel_ms_median"], 4),
                   "kernel_ms_min": round(head["kernel_ms_min"], 4)},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_TFLOPS["bf16"],
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_TFLOPS["bf16"], 4),
                     "traffic": traffic_bytes()},
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
