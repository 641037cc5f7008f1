"""Build libigconv.so (HIP for gfx950) in the package directory.

``python -m implicit_gemm_convolution_conv_amd.build`` compiles every source
under ``csrc/`` with hipcc (one process per file, in parallel) and links the
shared library next to this file. Always recompiles.
"""

from __future__ import annotations

import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libigconv.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC",
    # packed fp32 VALU forms stay off: only scalar/vector fp32 code is generated
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fvisibility=hidden",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


# No kernel may use private (scratch) memory: scratch means a register spill or a
# kernel argument copied to private memory, which slows a kernel several times
# over, so the build fails on it.
def _scratch_kernels(remarks: str) -> list[str]:
    bad = []
    for blk in re.split(r"Function Name: ", remarks)[1:]:
        name = blk.split()[0]
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", blk)
        if m and int(m.group(1)) > 0:
            bad.append(f"{name} ({m.group(1)} bytes/lane)")
    return bad


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *CFLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the gfx target feature above; that warning is expected
    err = "\n".join(l for l in res.stderr.splitlines() if "packed-fp32-ops" not in l and "remark:" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    bad = _scratch_kernels(res.stderr)
    if bad:
        raise RuntimeError(f"kernels in {src} use scratch memory:\n" + "\n".join(bad))
    return obj


def build(jobs: int | None = None, verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    for f in os.listdir(BUILD):  # objects of sources that no longer exist
        if f.endswith(".o") and not os.path.exists(os.path.join(CSRC, f[:-2] + ".hip")):
            os.remove(os.path.join(BUILD, f))
    # the kernel-instantiation units take minutes each, the rest seconds: start those first
    srcs = sorted(sources(), key=lambda s: not os.path.basename(s).startswith(("conv_dma_", "conv_buf_")))
    jobs = jobs or min(len(srcs), max(1, os.cpu_count() or 2), 8)
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    # a kernel whose host-side instantiation failed leaves an undefined launch stub behind
    nm = subprocess.run(["nm", "-C", tmp], capture_output=True, text=True)
    missing = [l for l in nm.stdout.splitlines() if " U " in l and "__device_stub__" in l]
    if missing:
        raise RuntimeError("kernels without a host launch stub:\n" + "\n".join(missing))
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# Host code of the planner (api.hip: validation, plans, workspace sizes, error paths) built with
# AddressSanitizer and UndefinedBehaviorSanitizer, linked with the kernel objects of the last
# build() (their device code is untouched: every sanitizer flag goes to the host pass only). The
# result needs clang's ASan runtime preloaded, since the Python interpreter is not instrumented.
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def asan_runtime() -> str | None:
    res = subprocess.run([HIPCC, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = res.stdout.strip().splitlines()[-1] if res.stdout.strip() else ""
    if not os.path.isabs(path) or not os.path.exists(path):
        import glob
        found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
        path = found[-1] if found else ""
    return path or None


def build_host_sanitized(out_dir: str) -> str:
    objs = [os.path.join(BUILD, os.path.basename(s)[:-4] + ".o") for s in sources() if not s.endswith("api.hip")]
    missing = [o for o in objs if not os.path.exists(o)]
    if missing:
        raise RuntimeError("run build() first; missing objects: " + ", ".join(missing))
    os.makedirs(out_dir, exist_ok=True)
    api = os.path.join(out_dir, "api_san.o")
    flags = [f if f != "-O3" else "-O1" for f in CFLAGS] + ["-g"]
    res = subprocess.run([HIPCC, *flags, *HOST_SANITIZE, "-c", os.path.join(CSRC, "api.hip"), "-o", api],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"sanitized compile of api.hip failed:\n{res.stderr}")
    lib = os.path.join(out_dir, "libigconv_san.so")
    res = subprocess.run([HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-Xarch_host", "-fsanitize=address",
                          "-Xarch_host", "-fsanitize=undefined", "-shared-libsan", "-o", lib, api, *objs],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{res.stderr}")
    return lib


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
