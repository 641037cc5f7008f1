"""The oracle's pins (tests/test_oracle.py) rerun against a build of the oracle with AddressSanitizer and
UndefinedBehaviorSanitizer: any out-of-bounds access, use of freed memory, signed overflow, misaligned access or
other undefined behaviour in conv_oracle.c aborts the run. Host code only; the child process preloads the ASan
runtime because the Python interpreter itself is not instrumented."""

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _runtime(name):
    path = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True).stdout.strip()
    return path if os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc's ASan runtime is not installed")
def test_oracle_pins_under_asan_and_ubsan():
    sys.path.insert(0, ROOT)
    from oracle import oracle as O
    O.build(force=True, sanitized=True)
    env = dict(os.environ, ORACLE_SANITIZED="1", LD_PRELOAD=_runtime("libasan.so"),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               OMP_NUM_THREADS="4", PYTHONPATH=ROOT)
    # the child loads the instrumented build, and that build carries the sanitizer runtimes
    probe = subprocess.run([sys.executable, "-c", "from oracle import oracle as O; O._load(); print(O._SO)"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=120)
    assert probe.returncode == 0 and probe.stdout.strip().endswith("liboracle_san.so"), probe.stderr[-2000:]
    deps = subprocess.run(["ldd", probe.stdout.strip()], capture_output=True, text=True).stdout
    assert "libasan" in deps and "libubsan" in deps, deps
    res = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                          os.path.join(ROOT, "tests", "test_oracle.py")], cwd=ROOT, env=env, capture_output=True,
                         text=True, timeout=900)
    tail = "\n".join((res.stdout + res.stderr).splitlines()[-30:])
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "ERROR: AddressSanitizer" not in res.stderr, tail
    assert "runtime error" not in res.stderr, tail
