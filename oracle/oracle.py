"""CPU oracle for forward convolution -- test infrastructure only.

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this module. The product library never imports,
links or runs it, and it imports nothing from the product package.

It is a ctypes wrapper over ``conv_oracle.c`` (plain C, fp64): the seven-loop
definition of 3D cross-correlation with zero padding that FlyDSL PR #860
checks its implicit-GEMM conv kernels against (torch ``conv3d``, commit adding
the large_shape regression test), its two gradients (with respect to x and to
w, the backward-data and backward-weights problems that MIOpen PR #10912 maps
to one GEMM each for point-output shapes), the bf16 and OCP E4M3FN encodings,
and the per-tensor ``amax / 448`` fp8 scaling. Operands are numpy arrays:

* ``float64``  -- plain values,
* ``uint16``   -- bf16 bit patterns,
* ``uint8``    -- E4M3FN codes (with their fp32 scale).

x is NCDHW (or NDHWC with ``x_layout="NDHWC"``), w is KCTRS, y is NCDHW fp64.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "conv_oracle.c")
# ORACLE_SANITIZED=1 loads a build with AddressSanitizer and UndefinedBehaviorSanitizer (the process must preload
# the ASan runtime, see tests/test_oracle_sanitized.py)
_SANITIZED = os.environ.get("ORACLE_SANITIZED") == "1"
_SO = os.path.join(_HERE, "liboracle_san.so" if _SANITIZED else "liboracle.so")

F64, BF16, E4M3 = 0, 1, 2
_LAYOUTS = {"NCDHW": 0, "NDHWC": 1}

_lib = None


def build(force: bool = True, sanitized: bool | None = None) -> str:
    """Compile conv_oracle.c into liboracle.so next to it (gcc, OpenMP, no FMA contraction); with sanitized, into
    liboracle_san.so with AddressSanitizer and UndefinedBehaviorSanitizer (host code, every error fatal)."""
    sanitized = _SANITIZED if sanitized is None else sanitized
    so = os.path.join(_HERE, "liboracle_san.so" if sanitized else "liboracle.so")
    if force or not os.path.exists(so):
        tmp = so + ".tmp"
        san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g"]
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
               "-fno-fast-math", "-Wall", *(san if sanitized else []), "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, so)
    return so


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_SO)
        p, i64, i32, f32, f64 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float, ctypes.c_double
        lib.oracle_f32_to_bf16_array.argtypes = [p, i64, p]
        lib.oracle_e4m3_encode_array.argtypes = [p, i64, p]
        lib.oracle_e4m3_decode_array.argtypes = [p, i64, p]
        lib.oracle_amax_bf16.argtypes = [p, i64]
        lib.oracle_amax_bf16.restype = f32
        lib.oracle_fp8_scales.argtypes = [f32, p, p]
        lib.oracle_quantize_e4m3.argtypes = [p, i64, f32, p]
        lib.oracle_out_dims.argtypes = [p, p, p, p, p, p]
        lib.oracle_conv3d.argtypes = [i32, p, i32, f64, i32, p, f64, p, p, p, p, p, p]
        lib.oracle_conv3d_points.argtypes = [i32, p, i32, f64, i32, p, f64, p, p, p, p, p, p, i64, p]
        lib.oracle_conv3d_bwd_data.argtypes = [i32, p, i32, p, i32, p, p, p, p, p, p]
        lib.oracle_conv3d_bwd_weight.argtypes = [i32, p, i32, i32, p, p, p, p, p, p, p]
        lib.oracle_set_threads.argtypes = [i32]
        lib.oracle_get_threads.restype = i32
        _lib = lib
    return _lib


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


# ---------------------------------------------------------------- encodings

def bf16_round(f) -> np.ndarray:
    """binary32 values -> bf16 bit patterns (round to nearest even)."""
    f = _c(f, np.float32)
    out = np.empty(f.shape, np.uint16)
    _load().oracle_f32_to_bf16_array(_ptr(f), f.size, _ptr(out))
    return out


def bf16_value(bits) -> np.ndarray:
    """bf16 bit patterns -> exact float64 values."""
    bits = _c(bits, np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def e4m3_encode(f) -> np.ndarray:
    """binary32 values -> E4M3FN codes (nearest, ties to even, saturating)."""
    f = _c(f, np.float32)
    out = np.empty(f.shape, np.uint8)
    _load().oracle_e4m3_encode_array(_ptr(f), f.size, _ptr(out))
    return out


def e4m3_decode(q) -> np.ndarray:
    """E4M3FN codes -> float64 values (NaN for S.1111.111)."""
    q = _c(q, np.uint8)
    out = np.empty(q.shape, np.float64)
    _load().oracle_e4m3_decode_array(_ptr(q), q.size, _ptr(out))
    return out


def amax_bf16(bits) -> float:
    bits = _c(bits, np.uint16)
    return float(_load().oracle_amax_bf16(_ptr(bits), bits.size))


def fp8_scales(amax: float) -> tuple[np.float32, np.float32]:
    """(s, inv) = (amax/448, 448/amax) in binary32; (1, 1) for amax == 0."""
    s = np.zeros(1, np.float32)
    inv = np.zeros(1, np.float32)
    _load().oracle_fp8_scales(ctypes.c_float(amax), _ptr(s), _ptr(inv))
    return s[0], inv[0]


def quantize_e4m3(bits, inv: float) -> np.ndarray:
    """bf16 bit patterns -> E4M3FN codes of fp32(v * inv)."""
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.uint8)
    _load().oracle_quantize_e4m3(_ptr(bits), bits.size, ctypes.c_float(inv), _ptr(out))
    return out


def quantize_tensor_e4m3(bits) -> tuple[np.ndarray, np.float32, np.float32]:
    """Per-tensor fp8: amax -> (s, inv) -> codes. Returns (codes, s, inv)."""
    s, inv = fp8_scales(amax_bf16(bits))
    return quantize_e4m3(bits, inv), s, inv


# ---------------------------------------------------------------- convolution

def _kind(a: np.ndarray) -> int:
    if a.dtype == np.float64:
        return F64
    if a.dtype == np.uint16:
        return BF16
    if a.dtype == np.uint8:
        return E4M3
    raise TypeError(f"oracle operand dtype {a.dtype} (want float64, uint16 bf16 bits or uint8 e4m3 codes)")


def _geom(x_shape, w_shape, stride, pad, dil, x_layout):
    if x_layout == "NDHWC":
        n, d, h, w, c = x_shape
        xs = np.array([n, c, d, h, w], np.int64)
    else:
        xs = np.array(x_shape, np.int64)
    ws = np.array(w_shape, np.int64)
    return (xs, ws, np.array(stride, np.int32), np.array(pad, np.int32), np.array(dil, np.int32))


def out_dims(x_shape, w_shape, stride=(1, 1, 1), pad=(0, 0, 0), dil=(1, 1, 1), x_layout="NCDHW"):
    xs, ws, st, pd, dl = _geom(x_shape, w_shape, stride, pad, dil, x_layout)
    out = np.zeros(3, np.int64)
    if _load().oracle_out_dims(_ptr(xs), _ptr(ws), _ptr(st), _ptr(pd), _ptr(dl), _ptr(out)):
        raise ValueError("filter does not fit the padded input")
    return tuple(int(v) for v in out)


def _bias64(bias, k):
    """Per-output-channel bias as float64 (fp32 values widen exactly), or None."""
    if bias is None:
        return None
    b = np.asarray(bias)
    assert b.shape == (k,), (b.shape, k)
    return b.astype(np.float64)


def conv3d(x, w, stride=(1, 1, 1), pad=(0, 0, 0), dil=(1, 1, 1), x_layout="NCDHW", sx=1.0, sw=1.0, bias=None):
    """Full output y (N, K, Do, Ho, Wo) in float64. With ``bias`` (K values) each
    output channel k gets bias[k] added, the bias term of a convolution layer
    (FlyDSL PR #860 tests its fp8 conv with one, gemm8w test cases)."""
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w)
    assert x.ndim == 5 and w.ndim == 5
    xs, ws, st, pd, dl = _geom(x.shape, w.shape, stride, pad, dil, x_layout)
    do, ho, wo = out_dims(x.shape, w.shape, stride, pad, dil, x_layout)
    y = np.empty((int(xs[0]), int(ws[0]), do, ho, wo), np.float64)
    rc = _load().oracle_conv3d(_kind(x), _ptr(x), _LAYOUTS[x_layout], float(sx), _kind(w), _ptr(w), float(sw),
                               _ptr(xs), _ptr(ws), _ptr(st), _ptr(pd), _ptr(dl), _ptr(y))
    if rc:
        raise ValueError(f"oracle_conv3d failed ({rc})")
    b = _bias64(bias, int(ws[0]))
    if b is not None:
        y += b[None, :, None, None, None]
    return y


def conv3d_points(x, w, points, stride=(1, 1, 1), pad=(0, 0, 0), dil=(1, 1, 1), x_layout="NCDHW",
                  sx=1.0, sw=1.0, bias=None):
    """y at sampled positions: points is (P, 5) of (n, k, od, oh, ow); returns (P,) float64
    (plus bias[k] with a bias, as conv3d)."""
    x = np.ascontiguousarray(x)
    w = np.ascontiguousarray(w)
    pts = _c(points, np.int64).reshape(-1, 5)
    xs, ws, st, pd, dl = _geom(x.shape, w.shape, stride, pad, dil, x_layout)
    y = np.empty(pts.shape[0], np.float64)
    rc = _load().oracle_conv3d_points(_kind(x), _ptr(x), _LAYOUTS[x_layout], float(sx), _kind(w), _ptr(w),
                                      float(sw), _ptr(xs), _ptr(ws), _ptr(st), _ptr(pd), _ptr(dl), _ptr(pts),
                                      pts.shape[0], _ptr(y))
    if rc:
        raise ValueError(f"oracle_conv3d_points failed ({rc})")
    b = _bias64(bias, int(ws[0]))
    if b is not None:
        y += b[pts[:, 1]]
    return y


def conv3d_bwd_data(dy, w, x_shape, stride=(1, 1, 1), pad=(0, 0, 0), dil=(1, 1, 1), x_layout="NCDHW"):
    """Gradient of conv3d with respect to x for the incoming gradient dy (N, K, Do, Ho, Wo):
    dx of logical shape x_shape = (N, C, D, H, W), returned in x_layout, float64. MIOpen
    PR #10912 computes it as one GEMM for point-output shapes (backward data)."""
    dy = np.ascontiguousarray(dy)
    w = np.ascontiguousarray(w)
    xs, ws, st, pd, dl = _geom(x_shape, w.shape, stride, pad, dil, "NCDHW")
    assert dy.shape == (int(xs[0]), int(ws[0])) + out_dims(x_shape, w.shape, stride, pad, dil), dy.shape
    n, c, d, h, wd = (int(v) for v in xs)
    dx = np.empty((n, c, d, h, wd) if x_layout == "NCDHW" else (n, d, h, wd, c), np.float64)
    rc = _load().oracle_conv3d_bwd_data(_kind(dy), _ptr(dy), _kind(w), _ptr(w), _LAYOUTS[x_layout], _ptr(xs),
                                        _ptr(ws), _ptr(st), _ptr(pd), _ptr(dl), _ptr(dx))
    if rc:
        raise ValueError(f"oracle_conv3d_bwd_data failed ({rc})")
    return dx


def conv3d_bwd_weight(x, dy, w_shape, stride=(1, 1, 1), pad=(0, 0, 0), dil=(1, 1, 1), x_layout="NCDHW"):
    """Gradient of conv3d with respect to w for the incoming gradient dy: dw (K, C, T, R, S)
    float64. MIOpen PR #10912 computes it as one GEMM for point-output shapes (backward
    weights)."""
    x = np.ascontiguousarray(x)
    dy = np.ascontiguousarray(dy)
    xs, ws, st, pd, dl = _geom(x.shape, w_shape, stride, pad, dil, x_layout)
    x_logical = tuple(int(v) for v in xs)
    assert dy.shape == (x_logical[0], int(ws[0])) + out_dims(x_logical, w_shape, stride, pad, dil), dy.shape
    dw = np.empty(tuple(int(v) for v in ws), np.float64)
    rc = _load().oracle_conv3d_bwd_weight(_kind(x), _ptr(x), _LAYOUTS[x_layout], _kind(dy), _ptr(dy), _ptr(xs),
                                          _ptr(ws), _ptr(st), _ptr(pd), _ptr(dl), _ptr(dw))
    if rc:
        raise ValueError(f"oracle_conv3d_bwd_weight failed ({rc})")
    return dw


def set_threads(n: int) -> None:
    _load().oracle_set_threads(int(n))


def get_threads() -> int:
    return int(_load().oracle_get_threads())
