"""ctypes binding over libigconv.so -- argument marshalling only.

Every function has the name and the arguments of the C entry point it wraps
(include/igconv.h). Tensors are torch tensors on the GPU (their data pointer
is passed); shapes, strides, pads and dilations are Python sequences; stream
defaults to torch's current stream on the tensor's device. A non-zero status
raises IgcError with the library's message. Nothing here computes: all work
runs in the library's HIP kernels.

The library must have been built (``python -m implicit_gemm_convolution_conv_amd.build``);
there is no other implementation to fall back to.
"""

from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libigconv.so")

IGC_OK = 0
IGC_ERR_INVALID, IGC_ERR_UNSUPPORTED, IGC_ERR_ALIGN, IGC_ERR_HIP = -1, -2, -3, -4
IGC_BF16, IGC_FP8_E4M3FN = 0, 1
IGC_NCDHW, IGC_NDHWC = 0, 1
IGC_PATH_AUTO, IGC_PATH_GENERIC, IGC_PATH_TEMPORAL, IGC_PATH_POINT, IGC_PATH_POINTWISE = 0, 1, 2, 3, 4
IGC_TILE_AUTO = -1
IGC_TILE_DMA_256, IGC_TILE_DMA_128, IGC_TILE_DMA_64, IGC_TILE_DMA_256x192 = 0, 1, 2, 3
IGC_TILE_BUF, IGC_TILE_BUF_AHEAD, IGC_TILE_BUF_PINGPONG, IGC_TILE_PW = 4, 5, 6, 7
IGC_TILE_BUF_128 = 8

EXPORTS = ("conv_out_dims", "conv_packed_w_cols", "conv_amax", "conv_fp8_scales", "conv_pack_x", "conv_pack_w",
           "conv_fwd", "conv_fwd_ws", "conv_fwd_ex", "conv_fwd_noalloc", "conv_fwd_workspace_bytes", "conv_plan", "conv_plan_ws", "conv_debug_force",
           "conv_debug_force_splits", "conv_debug_force_grid", "conv_debug_force_tap_raster", "conv_packed_w_t_cols", "conv_pack_w_t", "conv_bwd_data",
           "conv_bwd_weight_workspace_bytes", "conv_bwd_weight", "conv_last_error")


class IgcError(RuntimeError):
    def __init__(self, func: str, status: int, msg: str):
        super().__init__(f"{func} failed with status {status}: {msg}")
        self.status = status


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library once (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is missing: build it with `python -m implicit_gemm_convolution_conv_amd.build`")
        lib = ctypes.CDLL(path)
        P, I64, I32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int
        lib.conv_out_dims.argtypes = [P, P, P, P, P, P]
        lib.conv_packed_w_cols.argtypes = [P, I32]
        lib.conv_packed_w_cols.restype = I64
        lib.conv_amax.argtypes = [P, I64, P, P]
        lib.conv_fp8_scales.argtypes = [P, P, P]
        lib.conv_pack_x.argtypes = [P, P, P, I32, P, P]
        lib.conv_pack_w.argtypes = [P, P, P, I32, I32, P, P]
        lib.conv_fwd.argtypes = [P, P, P, P, P, P, P, P, I32, I32, P, P]
        lib.conv_plan.argtypes = [P, P, P, P, P, I32, I32, ctypes.c_char_p, ctypes.c_size_t]
        lib.conv_fwd_ws.argtypes = [P, P, P, P, P, P, P, P, I32, I32, P, P, ctypes.c_size_t, P]
        lib.conv_fwd_ex.argtypes = [P, P, P, P, P, P, P, P, I32, I32, P, P, P, P, ctypes.c_size_t, P]
        lib.conv_fwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, I32, I32, P, P, P, P]
        lib.conv_fwd_workspace_bytes.argtypes = [P, P, P, P, P, I32, I32]
        lib.conv_fwd_workspace_bytes.restype = I64
        lib.conv_plan_ws.argtypes = [P, P, P, P, P, I32, I32, ctypes.c_size_t, ctypes.c_char_p, ctypes.c_size_t]
        lib.conv_packed_w_t_cols.argtypes = [P]
        lib.conv_packed_w_t_cols.restype = I64
        lib.conv_pack_w_t.argtypes = [P, P, P, I32, P]
        lib.conv_bwd_data.argtypes = [P, P, P, P, P, P, P, P, I32, I32, P]
        lib.conv_bwd_weight_workspace_bytes.argtypes = [P, P, P, P, P, I32, I32]
        lib.conv_bwd_weight_workspace_bytes.restype = I64
        lib.conv_bwd_weight.argtypes = [P, P, P, P, P, P, P, P, I32, I32, P, ctypes.c_size_t, P]
        lib.conv_debug_force.argtypes = [I32, I32, I32]
        lib.conv_debug_force_splits.argtypes = [I32]
        lib.conv_debug_force_grid.argtypes = [I32]
        lib.conv_debug_force_tap_raster.argtypes = [I32]
        lib.conv_last_error.restype = ctypes.c_char_p
        for name in EXPORTS:
            if name not in ("conv_packed_w_cols", "conv_fwd_workspace_bytes", "conv_packed_w_t_cols",
                            "conv_bwd_weight_workspace_bytes", "conv_last_error"):
                getattr(lib, name).restype = I32
        _lib = lib
    return _lib


def _check(func: str, status: int) -> None:
    if status != IGC_OK:
        raise IgcError(func, status, conv_last_error())


_ARRAY_TYPES = {(ctypes.c_int64, 5): ctypes.c_int64 * 5, (ctypes.c_int32, 3): ctypes.c_int32 * 3}
_ARRAYS: dict = {}  # marshalled shape / stride / pad arrays by value: the C side only reads them


def _array(ctype, v, n):
    key = (ctype, tuple(v))
    arr = _ARRAYS.get(key)
    if arr is None:
        vals = tuple(int(a) for a in v)
        if len(vals) != n:
            raise ValueError(f"expected {n} values, got {vals}")
        if len(_ARRAYS) > 4096:
            _ARRAYS.clear()
        arr = _ARRAYS[key] = _ARRAY_TYPES[(ctype, n)](*vals)
    return arr


def _i64(v, n):
    return _array(ctypes.c_int64, v, n)


def _i32(v):
    return _array(ctypes.c_int32, v, 3)


def _dev(t) -> int:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch tensor")
    if not t.is_cuda:
        raise ValueError("tensor must live in GPU memory")
    return t.data_ptr()


# torch's current stream of a device as a raw pointer; the public torch.cuda.current_stream builds a Stream
# object on every call, which costs more host time than a small launch takes on the GPU
_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, t) -> int:
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(t.device.index if t.device.index is not None else torch.cuda.current_device())
        return torch.cuda.current_stream(t.device).cuda_stream
    return stream.cuda_stream if isinstance(stream, torch.cuda.Stream) else int(stream)


def conv_out_dims(xshape, wshape, stride, pad, dilation):
    out = (ctypes.c_int64 * 3)()
    _check("conv_out_dims", load().conv_out_dims(_i64(xshape, 5), _i64(wshape, 5), _i32(stride), _i32(pad),
                                                 _i32(dilation), out))
    return tuple(out)


def conv_packed_w_cols(wshape, dtype) -> int:
    v = load().conv_packed_w_cols(_i64(wshape, 5), int(dtype))
    if v <= 0:
        raise IgcError("conv_packed_w_cols", int(v), "bad filter shape or dtype")
    return int(v)


def conv_amax(t_bf16, numel, amax_dev, stream=None):
    _check("conv_amax", load().conv_amax(_dev(t_bf16), int(numel), _dev(amax_dev), _stream(stream, t_bf16)))


def conv_fp8_scales(amax_dev, scale_pair_dev, stream=None):
    _check("conv_fp8_scales", load().conv_fp8_scales(_dev(amax_dev), _dev(scale_pair_dev),
                                                     _stream(stream, amax_dev)))


def conv_pack_x(x_ncdhw_bf16, x_out, xshape, dtype, scale_pair_dev=None, stream=None):
    _check("conv_pack_x", load().conv_pack_x(_dev(x_ncdhw_bf16), _dev(x_out), _i64(xshape, 5), int(dtype),
                                             _dev(scale_pair_dev), _stream(stream, x_out)))


def conv_pack_w(w_kctrs_bf16, w_packed, wshape, dtype, x_layout, scale_pair_dev=None, stream=None):
    _check("conv_pack_w", load().conv_pack_w(_dev(w_kctrs_bf16), _dev(w_packed), _i64(wshape, 5), int(dtype),
                                             int(x_layout), _dev(scale_pair_dev), _stream(stream, w_packed)))


def conv_fwd(x, w_packed, y, xshape, wshape, stride, pad, dilation, dtype, x_layout, scales_dev=None, stream=None):
    _check("conv_fwd", load().conv_fwd(_dev(x), _dev(w_packed), _dev(y), _i64(xshape, 5), _i64(wshape, 5),
                                       _i32(stride), _i32(pad), _i32(dilation), int(dtype), int(x_layout),
                                       _dev(scales_dev), _stream(stream, y)))


def conv_fwd_ws(x, w_packed, y, xshape, wshape, stride, pad, dilation, dtype, x_layout, scales_dev=None,
                workspace=None, workspace_bytes=None, stream=None):
    """conv_fwd with a device workspace (a torch tensor; its whole size unless workspace_bytes says less)."""
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if workspace_bytes is not None:
        if int(workspace_bytes) > nbytes:
            raise ValueError(f"workspace_bytes {workspace_bytes} exceeds the workspace tensor ({nbytes} bytes)")
        nbytes = int(workspace_bytes)
    _check("conv_fwd_ws", load().conv_fwd_ws(_dev(x), _dev(w_packed), _dev(y), _i64(xshape, 5), _i64(wshape, 5),
                                             _i32(stride), _i32(pad), _i32(dilation), int(dtype), int(x_layout),
                                             _dev(scales_dev), _dev(workspace), nbytes, _stream(stream, y)))


def conv_fwd_ex(x, w_packed, y, xshape, wshape, stride, pad, dilation, dtype, x_layout, scales_dev=None,
                bias=None, y_amax=None, workspace=None, workspace_bytes=None, stream=None):
    """conv_fwd with fused extras: fp32 bias[K] before rounding, max |y| into y_amax (fp32[1])."""
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if workspace_bytes is not None:
        if int(workspace_bytes) > nbytes:
            raise ValueError(f"workspace_bytes {workspace_bytes} exceeds the workspace tensor ({nbytes} bytes)")
        nbytes = int(workspace_bytes)
    _check("conv_fwd_ex", load().conv_fwd_ex(_dev(x), _dev(w_packed), _dev(y), _i64(xshape, 5), _i64(wshape, 5),
                                             _i32(stride), _i32(pad), _i32(dilation), int(dtype), int(x_layout),
                                             _dev(scales_dev), _dev(bias), _dev(y_amax), _dev(workspace), nbytes,
                                             _stream(stream, y)))


def conv_fwd_noalloc(x, w_packed, y, xshape, wshape, stride, pad, dilation, dtype, x_layout, scales_dev=None,
                     bias=None, y_amax=None, stream=None):
    """conv_fwd_ex with its workspace in the library's static device scratch (allocates nothing)."""
    _check("conv_fwd_noalloc", load().conv_fwd_noalloc(_dev(x), _dev(w_packed), _dev(y), _i64(xshape, 5),
                                                       _i64(wshape, 5), _i32(stride), _i32(pad), _i32(dilation),
                                                       int(dtype), int(x_layout), _dev(scales_dev), _dev(bias),
                                                       _dev(y_amax), _stream(stream, y)))


def conv_fwd_workspace_bytes(xshape, wshape, stride, pad, dilation, dtype, x_layout) -> int:
    n = load().conv_fwd_workspace_bytes(_i64(xshape, 5), _i64(wshape, 5), _i32(stride), _i32(pad), _i32(dilation),
                                        int(dtype), int(x_layout))
    if n < 0:
        raise IgcError("conv_fwd_workspace_bytes", int(n), conv_last_error())
    return int(n)


def conv_plan(xshape, wshape, stride, pad, dilation, dtype, x_layout) -> str:
    buf = ctypes.create_string_buffer(512)
    _check("conv_plan", load().conv_plan(_i64(xshape, 5), _i64(wshape, 5), _i32(stride), _i32(pad),
                                         _i32(dilation), int(dtype), int(x_layout), buf, 512))
    return buf.value.decode()


def conv_plan_ws(xshape, wshape, stride, pad, dilation, dtype, x_layout, workspace_bytes) -> str:
    buf = ctypes.create_string_buffer(512)
    _check("conv_plan_ws", load().conv_plan_ws(_i64(xshape, 5), _i64(wshape, 5), _i32(stride), _i32(pad),
                                               _i32(dilation), int(dtype), int(x_layout), int(workspace_bytes),
                                               buf, 512))
    return buf.value.decode()


def conv_debug_force(path, tile, group_m=0):
    _check("conv_debug_force", load().conv_debug_force(int(path), int(tile), int(group_m)))


def conv_packed_w_t_cols(wshape) -> int:
    n = load().conv_packed_w_t_cols(_i64(wshape, 5))
    if n < 0:
        raise IgcError("conv_packed_w_t_cols", int(n), "bad wshape")
    return int(n)


def conv_pack_w_t(w_kctrs_bf16, w_t, wshape, x_layout, stream=None):
    _check("conv_pack_w_t", load().conv_pack_w_t(_dev(w_kctrs_bf16), _dev(w_t), _i64(wshape, 5), int(x_layout),
                                                 _stream(stream, w_t)))


def conv_bwd_data(dy, w_t, dx, xshape, wshape, stride, pad, dilation, dtype, x_layout, stream=None):
    _check("conv_bwd_data", load().conv_bwd_data(_dev(dy), _dev(w_t), _dev(dx), _i64(xshape, 5), _i64(wshape, 5),
                                                 _i32(stride), _i32(pad), _i32(dilation), int(dtype), int(x_layout),
                                                 _stream(stream, dx)))


def conv_bwd_weight_workspace_bytes(xshape, wshape, stride, pad, dilation, dtype, x_layout) -> int:
    n = load().conv_bwd_weight_workspace_bytes(_i64(xshape, 5), _i64(wshape, 5), _i32(stride), _i32(pad),
                                               _i32(dilation), int(dtype), int(x_layout))
    if n < 0:
        raise IgcError("conv_bwd_weight_workspace_bytes", int(n), conv_last_error())
    return int(n)


def conv_bwd_weight(x, dy, dw, xshape, wshape, stride, pad, dilation, dtype, x_layout, workspace,
                    workspace_bytes=None, stream=None):
    nbytes = workspace.numel() * workspace.element_size()
    if workspace_bytes is not None:
        if int(workspace_bytes) > nbytes:
            raise ValueError(f"workspace_bytes {workspace_bytes} exceeds the workspace tensor ({nbytes} bytes)")
        nbytes = int(workspace_bytes)
    _check("conv_bwd_weight", load().conv_bwd_weight(_dev(x), _dev(dy), _dev(dw), _i64(xshape, 5), _i64(wshape, 5),
                                                     _i32(stride), _i32(pad), _i32(dilation), int(dtype),
                                                     int(x_layout), _dev(workspace), nbytes, _stream(stream, dw)))


def conv_debug_force_splits(splits):
    _check("conv_debug_force_splits", load().conv_debug_force_splits(int(splits)))


def conv_debug_force_grid(cus):
    _check("conv_debug_force_grid", load().conv_debug_force_grid(int(cus)))


def conv_debug_force_tap_raster(mode):
    _check("conv_debug_force_tap_raster", load().conv_debug_force_tap_raster(int(mode)))


def conv_last_error() -> str:
    return load().conv_last_error().decode()
