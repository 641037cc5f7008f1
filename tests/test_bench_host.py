"""Host-side pieces of bench.py (no GPU)."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_flop_convention_matches_the_pages_figures():
    with open(os.path.join(ROOT, "tests", "golden", "page_throughput_figures.txt")) as fh:
        rows = [l.split() for l in fh if l.strip() and not l.startswith("#")]
    assert rows
    for r in rows:
        n, c, d, h, w, k, t, rr, s, sd, sh, sw, pd, ph, pw = map(int, r[:15])
        ms, tf = float(r[15]), float(r[16])
        flops = bench.conv_flops((n, c, d, h, w), (k, c, t, rr, s), (sd, sh, sw), (pd, ph, pw), (1, 1, 1))
        assert abs(flops / (ms * 1e-3) / 1e12 - tf) / tf < 0.01


def test_headline_flops():
    assert bench.conv_flops((1, 2048, 60, 80, 45), (2048, 2048, 3, 3, 3), (1, 1, 1), (1, 1, 1), (1, 1, 1)) \
        == 2 * 216000 * 2048 * 55296


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
