"""The library's host-only tests (tests/test_abi.py: validation, plans, the swept tile table, workspace sizes,
error codes, per-thread hooks) rerun against a build whose host code carries AddressSanitizer and
UndefinedBehaviorSanitizer: an out-of-bounds access, use of freed memory, signed overflow or other undefined
behaviour in the planner aborts the run. Device code is not instrumented (no GPU is used); the child process
preloads clang's ASan runtime because the Python interpreter itself is not instrumented."""

import os
import subprocess
import sys

import pytest

from implicit_gemm_convolution_conv_amd import build as BLD

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(BLD.asan_runtime() is None, reason="clang's ASan runtime is not installed")
def test_host_abi_tests_under_asan_and_ubsan(tmp_path):
    lib = BLD.build_host_sanitized(str(tmp_path))
    deps = subprocess.run(["nm", "-D", lib], capture_output=True, text=True).stdout
    assert "__asan_report" in deps and "__ubsan_handle" in deps, "the planner is not instrumented"
    env = dict(os.environ, LD_PRELOAD=BLD.asan_runtime(), ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", PYTHONPATH=ROOT)
    runner = ("import sys; sys.path.insert(0, 'tests')\n"
              "from implicit_gemm_convolution_conv_amd import binding as B\n"
              f"B.load({lib!r})\n"
              "import pytest\n"
              "sys.exit(pytest.main(['-q', '-x', '-p', 'no:cacheprovider', '-m', 'not gpu', 'tests/test_abi.py']))\n")
    res = subprocess.run([sys.executable, "-c", runner], cwd=ROOT, env=env, capture_output=True, text=True,
                         timeout=600)
    tail = "\n".join((res.stdout + res.stderr).splitlines()[-30:])
    assert res.returncode == 0, tail
    assert "passed" in res.stdout and "ERROR: AddressSanitizer" not in res.stderr, tail
    assert "runtime error" not in res.stderr, tail
