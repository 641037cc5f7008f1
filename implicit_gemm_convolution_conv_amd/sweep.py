"""Offline tile sweep for the im2col paths, and the generated table the planner reads.

FlyDSL PR #860 (first commit: tile parameterisation, per-shape autotune) picks a tile per shape by timing the
candidates. Here the timing is done once, offline, on one GPU: every tile that can run each shape below is
timed through ``conv_fwd_ws`` (with the workspace that tile's plan asks for) and the winners are written to
``csrc/tile_table.h``. ``make_plan`` then takes, for a shape it has not seen, the winner of the nearest swept
shape of the same dtype and path, and falls back to its size rule when that tile cannot run the shape.

    python -m implicit_gemm_convolution_conv_amd.sweep --json tile_sweep.json   (on a GPU)
    python -m implicit_gemm_convolution_conv_amd.sweep --from-json tile_sweep.json --header \\
        implicit_gemm_convolution_conv_amd/csrc/tile_table.h                               (anywhere)
"""

import argparse
import json
import math
import os
import statistics
import sys
import time

HERE = os.path.dirname(os.path.abspath(__file__))

PATH_GENERIC, PATH_TEMPORAL = 1, 2  # IGC_PATH_* of include/igconv.h
BF16, FP8 = 0, 1                    # IGC_BF16, IGC_FP8_E4M3FN

# name, dtype, x (N, C, D, H, W), w (K, C, T, R, S), pad; stride and dilation 1. Grids from under one tile per
# CU to 211 rounds, reductions from 12 to 864 steps of 128 bytes, both filter kinds, both dtypes.
SHAPES = [
    ("c3 3x3x3 C2048 60x80x45 K2048", BF16, (1, 2048, 60, 80, 45), (2048, 2048, 3, 3, 3), (1, 1, 1)),
    ("c3 share K256", BF16, (1, 2048, 60, 80, 45), (256, 2048, 3, 3, 3), (1, 1, 1)),
    ("3x3x3 C1024 8x32x32 K1024", BF16, (1, 1024, 8, 32, 32), (1024, 1024, 3, 3, 3), (1, 1, 1)),
    ("3x3x3 C512 16x32x32 K512", BF16, (1, 512, 16, 32, 32), (512, 512, 3, 3, 3), (1, 1, 1)),
    ("3x3x3 C256 16x48x48 N2 K512", BF16, (2, 256, 16, 48, 48), (512, 256, 3, 3, 3), (1, 1, 1)),
    ("3x3x3 C128 16x64x64 K256", BF16, (1, 128, 16, 64, 64), (256, 128, 3, 3, 3), (1, 1, 1)),
    ("3x3x3 C256 8x16x16 K256", BF16, (1, 256, 8, 16, 16), (256, 256, 3, 3, 3), (1, 1, 1)),
    ("3x3x3 C64 16x64x64 K256", BF16, (1, 64, 16, 64, 64), (256, 64, 3, 3, 3), (1, 1, 1)),
    ("3x3x3 C64 8x32x32 K128", BF16, (1, 64, 8, 32, 32), (128, 64, 3, 3, 3), (1, 1, 1)),
    ("c1 3x3x3 C64 4x16x16 K64", BF16, (1, 64, 4, 16, 16), (64, 64, 3, 3, 3), (1, 1, 1)),
    ("3x3x3 C512 4x16x16 K512", BF16, (1, 512, 4, 16, 16), (512, 512, 3, 3, 3), (1, 1, 1)),
    ("c5 3x1x1 C1024 240x160x90 K1024", BF16, (1, 1024, 240, 160, 90), (1024, 1024, 3, 1, 1), (1, 0, 0)),
    ("c5 share 32 planes", BF16, (1, 1024, 32, 160, 90), (1024, 1024, 3, 1, 1), (0, 0, 0)),
    ("3x1x1 C2048 30x40x48 K1024", BF16, (1, 2048, 30, 40, 48), (1024, 2048, 3, 1, 1), (1, 0, 0)),
    ("3x1x1 C512 16x64x64 K512", BF16, (1, 512, 16, 64, 64), (512, 512, 3, 1, 1), (1, 0, 0)),
    ("3x1x1 C256 8x32x32 K256", BF16, (1, 256, 8, 32, 32), (256, 256, 3, 1, 1), (1, 0, 0)),
    ("3x1x1 C128 4x32x32 K128", BF16, (1, 128, 4, 32, 32), (128, 128, 3, 1, 1), (1, 0, 0)),
    ("c4 3x3x3 C2048 60x80x45 K2048", FP8, (1, 2048, 60, 80, 45), (2048, 2048, 3, 3, 3), (1, 1, 1)),
    ("3x3x3 C1024 8x32x32 K1024", FP8, (1, 1024, 8, 32, 32), (1024, 1024, 3, 3, 3), (1, 1, 1)),
    ("3x3x3 C512 16x32x32 K512", FP8, (1, 512, 16, 32, 32), (512, 512, 3, 3, 3), (1, 1, 1)),
    ("3x3x3 C256 16x64x64 K512", FP8, (1, 256, 16, 64, 64), (512, 256, 3, 3, 3), (1, 1, 1)),
    ("3x3x3 C128 4x16x16 K128", FP8, (1, 128, 4, 16, 16), (128, 128, 3, 3, 3), (1, 1, 1)),
    ("3x3x3 C1024 4x16x16 K512", FP8, (1, 1024, 4, 16, 16), (512, 1024, 3, 3, 3), (1, 1, 1)),
    ("c4t 3x1x1 C2048 60x80x45 K2048", FP8, (1, 2048, 60, 80, 45), (2048, 2048, 3, 1, 1), (1, 0, 0)),
    ("3x1x1 C1024 30x40x48 K1024", FP8, (1, 1024, 30, 40, 48), (1024, 1024, 3, 1, 1), (1, 0, 0)),
    ("3x1x1 C2048 8x32x64 K2048", FP8, (1, 2048, 8, 32, 64), (2048, 2048, 3, 1, 1), (1, 0, 0)),
    ("3x1x1 C256 8x32x32 K256", FP8, (1, 256, 8, 32, 32), (256, 256, 3, 1, 1), (1, 0, 0)),
]

def candidates(dtype, tiles_per_cu, big):
    """Tile ids (include/igconv.h) timed on a shape: the 256-wide tiles everywhere, the 128x128 (global-address
    and buffer-addressed) and 64x64 tiles on grids of under two 256x256 tiles per CU (where they can fill the
    GPU), the bf16-only 256x192 tile where offsets stay 32-bit."""
    c = [0, 4, 5, 6]
    if dtype == BF16 and not big:
        c.append(3)
    if tiles_per_cu < 2:
        c += [1, 2, 8]
    return sorted(c)


def features(xs, ws, pad, dtype, cus=256):
    """(256x256 tiles per CU, 128-byte reduction steps, filter taps) of a shape, as the planner computes them."""
    n, c, d, h, w = xs
    k, _, t, r, s = ws
    do, ho, wo = d + 2 * pad[0] - t + 1, h + 2 * pad[1] - r + 1, w + 2 * pad[2] - s + 1
    m = n * do * ho * wo
    tiles = math.ceil(m / 256) * math.ceil(k / 256)
    esz = 1 if dtype == FP8 else 2
    steps = math.ceil(c * t * r * s * esz / 128)
    return tiles / cus, steps, t * r * s


def randn_bf16(torch, shape, scale, g):
    """N(0, scale^2) values rounded to bf16, drawn in chunks of 2^27 elements."""
    t = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
    flat = t.view(-1)
    for i in range(0, flat.numel(), 1 << 27):
        n = min(1 << 27, flat.numel() - i)
        flat[i:i + n] = (torch.randn(n, generator=g, device="cuda") * scale).to(torch.bfloat16)
    return t


def run(args):
    import torch

    from implicit_gemm_convolution_conv_amd import binding as B

    B.load()
    torch.cuda.set_device(0)
    g = torch.Generator(device="cuda")
    g.manual_seed(2024)
    out = []
    for name, dtype, xs, ws, pad in SHAPES:
        n, c, d, h, w = xs
        lay = B.IGC_NDHWC
        st, dl = (1, 1, 1), (1, 1, 1)
        x = randn_bf16(torch, xs, 1.0, g)
        wt = randn_bf16(torch, ws, 1.0 / math.sqrt(c * ws[2] * ws[3] * ws[4]), g)
        scales = None
        if dtype == FP8:
            amax = torch.empty(2, device="cuda")
            scales = torch.empty(4, device="cuda")
            B.conv_amax(x, x.numel(), amax[0:1]); B.conv_fp8_scales(amax[0:1], scales[0:2])
            B.conv_amax(wt, wt.numel(), amax[1:2]); B.conv_fp8_scales(amax[1:2], scales[2:4])
            xk = torch.empty((n, d, h, w, c), dtype=torch.uint8, device="cuda")
            B.conv_pack_x(x, xk, xs, B.IGC_FP8_E4M3FN, scales[0:2])
            wp = torch.empty((ws[0], B.conv_packed_w_cols(ws, B.IGC_FP8_E4M3FN)), dtype=torch.uint8, device="cuda")
            B.conv_pack_w(wt, wp, ws, B.IGC_FP8_E4M3FN, lay, scales[2:4])
            dt = B.IGC_FP8_E4M3FN
        else:
            xk = torch.empty((n, d, h, w, c), dtype=torch.bfloat16, device="cuda")
            B.conv_pack_x(x, xk, xs, B.IGC_BF16)
            wp = torch.empty((ws[0], B.conv_packed_w_cols(ws, B.IGC_BF16)), dtype=torch.bfloat16, device="cuda")
            B.conv_pack_w(wt, wp, ws, B.IGC_BF16, lay)
            dt = B.IGC_BF16
        del x, wt
        y = torch.empty((n, ws[0]) + B.conv_out_dims(xs, ws, st, pad, dl), dtype=torch.bfloat16, device="cuda")
        a5 = (xs, ws, st, pad, dl, dt, lay)
        default_plan = B.conv_plan(*a5)
        big = " big=1 " in f" {default_plan} "
        tpc, steps, taps = features(xs, ws, pad, dtype)
        times = {}
        plans = {}
        for tile in candidates(dtype, tpc, big):
            B.conv_debug_force(B.IGC_PATH_AUTO, tile, 0)
            try:
                nws = B.conv_fwd_workspace_bytes(*a5)
                plans[tile] = B.conv_plan_ws(*a5, max(nws, 0))
            except B.IgcError:
                continue  # the tile cannot run this shape
            times[tile] = []
        B.conv_debug_force(B.IGC_PATH_AUTO, -1, 0)
        # alternate the tiles over rounds so that no tile always runs first on a power-limited chip
        for rnd in range(args.rounds):
            order = list(times) if rnd % 2 == 0 else list(times)[::-1]
            for tile in order:
                B.conv_debug_force(B.IGC_PATH_AUTO, tile, 0)
                nws = B.conv_fwd_workspace_bytes(*a5)
                wsb = torch.empty(max(nws, 16) // 4, dtype=torch.float32, device="cuda") if nws > 0 else None
                fn = lambda: B.conv_fwd_ws(xk, wp, y, *a5, scales, workspace=wsb)
                for _ in range(2):
                    fn()
                torch.cuda.synchronize()
                ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                      for _ in range(args.calls)]
                for a, b in ev:
                    a.record(); fn(); b.record()
                torch.cuda.synchronize()
                times[tile].append(statistics.median(a.elapsed_time(b) for a, b in ev))
                del wsb
            B.conv_debug_force(B.IGC_PATH_AUTO, -1, 0)
        med = {t: statistics.median(v) for t, v in times.items()}
        order = sorted(med, key=med.get)
        rec = {"name": name, "dtype": dtype, "x": xs, "w": ws, "pad": pad,
               "path": PATH_TEMPORAL if ws[3] == 1 and ws[4] == 1 else PATH_GENERIC,
               "tiles_per_cu": tpc, "steps": steps, "taps": taps, "ms": {str(t): round(v, 5) for t, v in med.items()},
               "best": order[0], "second": order[1] if len(order) > 1 else -1, "default_plan": default_plan,
               "plans": {str(t): p for t, p in plans.items()}}
        out.append(rec)
        print(json.dumps({k: rec[k] for k in ("name", "dtype", "ms", "best", "second")}), flush=True)
        del xk, wp, y
        torch.cuda.empty_cache()
    return out


def emit_header(records, path, command):
    lines = [
        "// Generated by implicit_gemm_convolution_conv_amd/sweep.py; do not edit. Measured winners of the",
        "// im2col tiles on one MI355X (256 CUs): every tile that can run a shape timed through conv_fwd_ws with",
        "// the workspace its plan asks for, in alternating rounds, median of the rounds' per-call medians.",
        f"// {command}",
        "// The planner takes the winner of the nearest entry of the same dtype and path (distance: |log2| of",
        "// the ratio of 256x256 tiles per CU plus |log2| of the ratio of 128-byte reduction steps, at most",
        "// kSweptReach) when that tile can run the shape, and its size rule otherwise.",
        "#pragma once",
        "",
        "namespace igc {",
        "",
        "struct SweptShape {",
        "    int esz;             // bytes per element: 2 bf16, 1 fp8",
        "    int path;            // IGC_PATH_GENERIC or IGC_PATH_TEMPORAL",
        "    double tiles_per_cu; // 256x256 output tiles per CU",
        "    int steps;           // 128-byte reduction steps",
        "    int taps;            // T * R * S",
        "    int tile;            // fastest tile id",
        "    float ms;            // its time",
        "    int second;          // next fastest tile id (-1: none)",
        "    float ms_second;     // its time",
        "};",
        "",
        "constexpr SweptShape kSwept[] = {",
    ]
    for r in records:
        ms = r["ms"]
        sec = r["second"]
        lines.append(f"    {{{2 if r['dtype'] == BF16 else 1}, {r['path']}, {r['tiles_per_cu']:.6f}, {r['steps']}, "
                     f"{r['taps']}, {r['best']}, {ms[str(r['best'])]:.4f}f, {sec}, "
                     f"{ms[str(sec)] if sec >= 0 else 0.0:.4f}f}},  // {'fp8' if r['dtype'] == FP8 else 'bf16'} "
                     f"{r['name']}: x {tuple(r['x'])} w {tuple(r['w'])} pad {tuple(r['pad'])}")
    lines += ["};", "constexpr int kNumSwept = sizeof(kSwept) / sizeof(kSwept[0]);",
              "constexpr double kSweptReach = 2.0;  // beyond this distance no entry speaks for a shape", "",
              "}  // namespace igc", ""]
    with open(path, "w") as fh:
        fh.write("\n".join(lines))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--json", help="write the sweep's records here (GPU run)")
    ap.add_argument("--from-json", help="read records written by an earlier GPU run instead of timing")
    ap.add_argument("--header", help="write the planner's table here")
    ap.add_argument("--rounds", type=int, default=4)
    ap.add_argument("--calls", type=int, default=7)
    args = ap.parse_args()
    if args.from_json:
        with open(args.from_json) as fh:
            doc = json.load(fh)
        records, command = doc["records"], doc["command"]
    else:
        t0 = time.time()
        records = run(args)
        command = ("python -m implicit_gemm_convolution_conv_amd.sweep --json <file> "
                   f"--rounds {args.rounds} --calls {args.calls}  ({time.time() - t0:.0f} s)")
        if args.json:
            with open(args.json, "w") as fh:
                json.dump({"command": command, "records": records}, fh, indent=1)
    if args.header:
        emit_header(records, args.header, command)


if __name__ == "__main__":
    sys.exit(main())
