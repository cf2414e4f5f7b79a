"""Python binding of the MI355X NVFP4 library (libnvfp4.so, C ABI in include/nvfp4.h).

Argument marshalling only: every step runs in the library's HIP kernels.
PyTorch supplies device memory and the current HIP stream.  The library
must be built (``python nvfp4_bit_microscaled_amd/build.py``); importing
this package without it raises ImportError -- there is no fallback.

NVFP4 (guiahardware.es "NVFP4: cos'e e come supera FP8 e BF16", section
"Cos'e NVFP4"): E2M1 codes, an E4M3 scale per 16 elements and an FP32 tensor
scale.  Recipe (readjensen.com NVFP4 training-recipe page, recipe paragraph):
1x16 blocks for activations and gradients, 16x16 for weights, RHT on wgrad
inputs, stochastic rounding of gradients, NVFP4 GEMMs with BF16 output.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

# enums (include/nvfp4.h)
OK = 0
STATUS_NAMES = {0: "NVFP4_OK", 1: "NVFP4_ERR_INVALID_ARG", 2: "NVFP4_ERR_SHAPE",
                3: "NVFP4_ERR_ALIGN", 4: "NVFP4_ERR_LAYOUT", 5: "NVFP4_ERR_UNSUPPORTED",
                6: "NVFP4_ERR_WORKSPACE", 7: "NVFP4_ERR_HIP", 8: "NVFP4_ERR_NONFINITE"}
DTYPE_BF16, DTYPE_FP32 = 0, 1
BLOCK_1D, BLOCK_2D = 0, 1
ROUND_RNE, ROUND_SR = 0, 1
LAYOUT = {"NT": 0, "NN": 1, "TN": 2}

EXPORTS = ("nvfp4_version", "nvfp4_status_string", "nvfp4_quantize_workspace_size",
           "nvfp4_quantize", "nvfp4_amax_workspace_size", "nvfp4_amax",
           "nvfp4_swiglu_amax", "nvfp4_rht16",
           "nvfp4_dequantize", "nvfp4_gemm", "nvfp4_mx_quantize", "nvfp4_mx_dequantize",
           "nvfp4_mx_gemm", "nvfp4_gemm_w4a16", "nvfp4_kv_cache_write",
           "nvfp4_kv_cache_read", "nvfp4_gemm_swiglu_workspace_size", "nvfp4_gemm_swiglu",
           "nvfp4_transpose", "nvfp4_quantize_noalloc", "nvfp4_gemm_workspace_size",
           "nvfp4_gemm_native_workspace_size", "nvfp4_gemm_native")


class NVFP4Error(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s returned %s" % (fn, STATUS_NAMES.get(status, status)))
        self.status = status


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libnvfp4.so is not built: run `python nvfp4_bit_microscaled_amd/build.py`"
                          " (expected at %s)" % LIB_PATH)
    L = ctypes.CDLL(LIB_PATH)
    i64, u64, u32, vp, ci = ctypes.c_int64, ctypes.c_uint64, ctypes.c_uint32, ctypes.c_void_p, ctypes.c_int
    L.nvfp4_version.restype = ci
    L.nvfp4_version.argtypes = []
    L.nvfp4_status_string.restype = ctypes.c_char_p
    L.nvfp4_status_string.argtypes = [ci]
    L.nvfp4_quantize_workspace_size.restype = ctypes.c_size_t
    L.nvfp4_quantize_workspace_size.argtypes = [i64, i64]
    L.nvfp4_quantize.restype = ci
    L.nvfp4_quantize.argtypes = [vp, ci, i64, i64, i64, ci, ci, ci, ci, u64, u32, ci, u32, vp, vp,
                                 vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.nvfp4_quantize_noalloc.restype = ci
    L.nvfp4_quantize_noalloc.argtypes = [vp, ci, i64, i64, i64, ci, ci, ci, ci, u64, u32, ci, u32,
                                         vp, vp, vp, vp, vp, vp]
    L.nvfp4_transpose.restype = ci
    L.nvfp4_transpose.argtypes = [vp, vp, i64, i64, ci, ci, vp, vp, vp]
    L.nvfp4_amax_workspace_size.restype = ctypes.c_size_t
    L.nvfp4_amax_workspace_size.argtypes = [i64, i64]
    L.nvfp4_amax.restype = ci
    L.nvfp4_amax.argtypes = [vp, ci, i64, i64, i64, u32, vp, vp, vp, ctypes.c_size_t, vp]
    L.nvfp4_swiglu_amax.restype = ci
    L.nvfp4_swiglu_amax.argtypes = [vp, i64, i64, i64, vp, i64, u32, vp, vp, vp, ctypes.c_size_t,
                                    vp]
    L.nvfp4_rht16.restype = ci
    L.nvfp4_rht16.argtypes = [vp, ci, i64, i64, i64, ci, u32, vp, i64, vp]
    L.nvfp4_dequantize.restype = ci
    L.nvfp4_dequantize.argtypes = [vp, vp, vp, i64, i64, ci, ci, ci, vp, i64, vp]
    L.nvfp4_gemm.restype = ci
    L.nvfp4_gemm.argtypes = [ci, i64, i64, i64, vp, vp, vp, ci, vp, vp, vp, ci, ci, vp, i64, vp,
                             ctypes.c_size_t, vp]
    L.nvfp4_gemm_workspace_size.restype = ctypes.c_size_t
    L.nvfp4_gemm_workspace_size.argtypes = [ci, i64, i64, i64]
    L.nvfp4_gemm_native_workspace_size.restype = ctypes.c_size_t
    L.nvfp4_gemm_native_workspace_size.argtypes = [i64, i64, i64]
    L.nvfp4_gemm_native.restype = ci
    L.nvfp4_gemm_native.argtypes = [i64, i64, i64, vp, vp, vp, ci, vp, vp, vp, ci, ci, vp, i64, vp,
                                    vp, ctypes.c_size_t, vp]
    L.nvfp4_gemm_w4a16.restype = ci
    L.nvfp4_gemm_w4a16.argtypes = [i64, i64, i64, vp, i64, vp, vp, vp, ci, ci, vp, i64, vp]
    L.nvfp4_mx_quantize.restype = ci
    L.nvfp4_mx_quantize.argtypes = [vp, ci, i64, i64, i64, vp, vp, vp]
    L.nvfp4_mx_dequantize.restype = ci
    L.nvfp4_mx_dequantize.argtypes = [vp, vp, i64, i64, ci, vp, i64, vp]
    L.nvfp4_mx_gemm.restype = ci
    L.nvfp4_mx_gemm.argtypes = [i64, i64, i64, vp, vp, vp, vp, ci, vp, i64, vp]
    L.nvfp4_kv_cache_write.restype = ci
    L.nvfp4_kv_cache_write.argtypes = [vp, ci, i64, i64, i64, vp, vp, i64, vp, vp, vp]
    L.nvfp4_kv_cache_read.restype = ci
    L.nvfp4_kv_cache_read.argtypes = [vp, vp, vp, i64, i64, vp, i64, ci, vp, i64, vp]
    L.nvfp4_gemm_swiglu_workspace_size.restype = ctypes.c_size_t
    L.nvfp4_gemm_swiglu_workspace_size.argtypes = [i64, i64]
    L.nvfp4_gemm_swiglu.restype = ci
    L.nvfp4_gemm_swiglu.argtypes = [i64, i64, i64, vp, vp, vp, ci, vp, vp, vp, ci, vp, i64, vp, i64,
                                    u32, vp, vp, vp, ctypes.c_size_t, vp]
    return L


lib = _load()


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, status: int):
    if status != OK:
        raise NVFP4Error(fn, status)


def version() -> int:
    return lib.nvfp4_version()


def status_string(status: int) -> str:
    return lib.nvfp4_status_string(status).decode()


# ---------------------------------------------------------------- raw ABI calls
# Same names and argument order as include/nvfp4.h; tensors stand for device
# pointers, None for NULL.  They return the status code unchanged.

def nvfp4_quantize_workspace_size(rows: int, cols: int) -> int:
    return lib.nvfp4_quantize_workspace_size(rows, cols)


def nvfp4_quantize(x, x_dtype, rows, cols, ld_x, block, axis, transpose_out, rounding, seed,
                   stream_id, rht, rht_sign_mask, amax_in, amax_out, codes, scales, tensor_scale,
                   workspace, workspace_bytes, stream=None) -> int:
    return lib.nvfp4_quantize(_p(x), x_dtype, rows, cols, ld_x, block, axis, transpose_out,
                              rounding, seed, stream_id, rht, rht_sign_mask, _p(amax_in), _p(amax_out),
                              _p(codes), _p(scales), _p(tensor_scale), _p(workspace),
                              workspace_bytes, _stream(stream))


def nvfp4_quantize_noalloc(x, x_dtype, rows, cols, ld_x, block, axis, transpose_out, rounding,
                           seed, stream_id, rht, rht_sign_mask, amax_in, amax_out, codes, scales,
                           tensor_scale, stream=None) -> int:
    return lib.nvfp4_quantize_noalloc(_p(x), x_dtype, rows, cols, ld_x, block, axis,
                                      transpose_out, rounding, seed, stream_id, rht,
                                      rht_sign_mask, _p(amax_in), _p(amax_out), _p(codes),
                                      _p(scales), _p(tensor_scale), _stream(stream))


def nvfp4_transpose(codes, scales, rows, cols, block, axis, codes_t, scales_t, stream=None) -> int:
    return lib.nvfp4_transpose(_p(codes), _p(scales), rows, cols, block, axis, _p(codes_t),
                               _p(scales_t), _stream(stream))


def nvfp4_amax_workspace_size(rows: int, cols: int) -> int:
    return lib.nvfp4_amax_workspace_size(rows, cols)


def nvfp4_amax(x, x_dtype, rows, cols, ld_x, rht_sign_mask, amax, amax_rht, workspace,
               workspace_bytes, stream=None) -> int:
    return lib.nvfp4_amax(_p(x), x_dtype, rows, cols, ld_x, rht_sign_mask, _p(amax),
                          _p(amax_rht), _p(workspace), workspace_bytes, _stream(stream))


def nvfp4_swiglu_amax(h, rows, F, ld_h, act, ld_act, rht_sign_mask, amax, amax_rht, workspace,
                      workspace_bytes, stream=None) -> int:
    return lib.nvfp4_swiglu_amax(_p(h), rows, F, ld_h, _p(act), ld_act, rht_sign_mask, _p(amax),
                                 _p(amax_rht), _p(workspace), workspace_bytes, _stream(stream))


def nvfp4_rht16(x, x_dtype, rows, cols, ld_x, axis, sign_mask, y, ld_y, stream=None) -> int:
    return lib.nvfp4_rht16(_p(x), x_dtype, rows, cols, ld_x, axis, sign_mask, _p(y), ld_y,
                           _stream(stream))


def nvfp4_dequantize(codes, scales, tensor_scale, rows, cols, block, axis, out_dtype, out, ld_out,
                     stream=None) -> int:
    return lib.nvfp4_dequantize(_p(codes), _p(scales), _p(tensor_scale), rows, cols, block, axis,
                                out_dtype, _p(out), ld_out, _stream(stream))


def nvfp4_gemm_workspace_size(layout: int, M: int, N: int, K: int) -> int:
    return lib.nvfp4_gemm_workspace_size(layout, M, N, K)


def nvfp4_gemm(layout, M, N, K, a_codes, a_scales, a_tensor_scale, a_block, b_codes, b_scales,
               b_tensor_scale, b_block, out_dtype, c, ldc, workspace=None, workspace_bytes=0,
               stream=None) -> int:
    return lib.nvfp4_gemm(layout, M, N, K, _p(a_codes), _p(a_scales), _p(a_tensor_scale), a_block,
                          _p(b_codes), _p(b_scales), _p(b_tensor_scale), b_block, out_dtype,
                          _p(c), ldc, _p(workspace), workspace_bytes, _stream(stream))


def nvfp4_gemm_native_workspace_size(M, N, K) -> int:
    return lib.nvfp4_gemm_native_workspace_size(M, N, K)


def nvfp4_gemm_native(M, N, K, a_codes, a_scales, a_tensor_scale, a_block, b_codes, b_scales,
                      b_tensor_scale, b_block, out_dtype, c, ldc, used_native, workspace=None,
                      workspace_bytes=0, stream=None) -> int:
    return lib.nvfp4_gemm_native(M, N, K, _p(a_codes), _p(a_scales), _p(a_tensor_scale), a_block,
                                 _p(b_codes), _p(b_scales), _p(b_tensor_scale), b_block,
                                 out_dtype, _p(c), ldc, _p(used_native), _p(workspace),
                                 workspace_bytes, _stream(stream))


def nvfp4_gemm_w4a16(M, N, K, a, lda, b_codes, b_scales, b_tensor_scale, b_block, out_dtype, c,
                     ldc, stream=None) -> int:
    return lib.nvfp4_gemm_w4a16(M, N, K, _p(a), lda, _p(b_codes), _p(b_scales),
                                _p(b_tensor_scale), b_block, out_dtype, _p(c), ldc,
                                _stream(stream))


def nvfp4_mx_quantize(x, x_dtype, rows, cols, ld_x, codes, scales, stream=None) -> int:
    return lib.nvfp4_mx_quantize(_p(x), x_dtype, rows, cols, ld_x, _p(codes), _p(scales),
                                 _stream(stream))


def nvfp4_mx_dequantize(codes, scales, rows, cols, out_dtype, out, ld_out, stream=None) -> int:
    return lib.nvfp4_mx_dequantize(_p(codes), _p(scales), rows, cols, out_dtype, _p(out), ld_out,
                                   _stream(stream))


def nvfp4_mx_gemm(M, N, K, a_codes, a_scales, b_codes, b_scales, out_dtype, c, ldc,
                  stream=None) -> int:
    return lib.nvfp4_mx_gemm(M, N, K, _p(a_codes), _p(a_scales), _p(b_codes), _p(b_scales),
                             out_dtype, _p(c), ldc, _stream(stream))


def nvfp4_kv_cache_write(x, x_dtype, tokens, cols, ld_x, slots, amax, num_slots, cache_codes,
                         cache_scales, stream=None) -> int:
    return lib.nvfp4_kv_cache_write(_p(x), x_dtype, tokens, cols, ld_x, _p(slots), _p(amax),
                                    num_slots, _p(cache_codes), _p(cache_scales), _stream(stream))


def nvfp4_kv_cache_read(cache_codes, cache_scales, amax, num_slots, cols, slots, n, out_dtype, out,
                        ld_out, stream=None) -> int:
    return lib.nvfp4_kv_cache_read(_p(cache_codes), _p(cache_scales), _p(amax), num_slots, cols,
                                   _p(slots), n, out_dtype, _p(out), ld_out, _stream(stream))


def nvfp4_gemm_swiglu_workspace_size(M: int, N: int) -> int:
    return lib.nvfp4_gemm_swiglu_workspace_size(M, N)


def nvfp4_gemm_swiglu(M, N, K, a_codes, a_scales, a_tensor_scale, a_block, b_codes, b_scales,
                      b_tensor_scale, b_block, h, ldh, act, ld_act, rht_sign_mask, amax, amax_rht,
                      workspace, workspace_bytes, stream=None) -> int:
    return lib.nvfp4_gemm_swiglu(M, N, K, _p(a_codes), _p(a_scales), _p(a_tensor_scale), a_block,
                                 _p(b_codes), _p(b_scales), _p(b_tensor_scale), b_block, _p(h),
                                 ldh, _p(act), ld_act, rht_sign_mask, _p(amax), _p(amax_rht),
                                 _p(workspace), workspace_bytes, _stream(stream))


# ---------------------------------------------------------------- tensor-level helpers

@dataclass
class NVFP4Tensor:
    """codes uint8 [R, C/2], scales uint8 (layout by block/axis), tensor_scale float32 [1]."""
    codes: torch.Tensor
    scales: torch.Tensor
    tensor_scale: torch.Tensor
    amax: torch.Tensor
    rows: int
    cols: int
    block2d: bool
    axis: int


def scale_shape(rows: int, cols: int, block2d: bool, axis: int):
    if block2d:
        return (rows // 16, cols // 16)
    return (rows, cols // 16) if axis == 1 else (rows // 16, cols)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return DTYPE_BF16
    if t.dtype == torch.float32:
        return DTYPE_FP32
    raise TypeError("NVFP4 input must be bfloat16 or float32, got %s" % t.dtype)


_workspaces = {}


def _workspace(device, rows, cols):
    n = max(nvfp4_quantize_workspace_size(rows, cols), nvfp4_amax_workspace_size(rows, cols))
    key = (str(device), torch.cuda.current_stream(device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < n:
        ws = torch.empty(n, dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def quantize(x: torch.Tensor, block2d: bool = False, axis: int = 1, sr: bool = False,
             seed: int = 0, stream_id: int = 0, rht: bool = False, mask: int = 0,
             amax_in: torch.Tensor | None = None, out: NVFP4Tensor | None = None,
             transpose: bool = False) -> NVFP4Tensor:
    """Quantize a 2-D BF16/FP32 CUDA tensor (row stride may exceed its width).

    transpose=True (blocks down the columns: axis 0 or 2D) returns the same
    quantization stored as that of x^T: an NVFP4Tensor of shape [cols, rows]
    with blocks along its rows (axis 1), the K-major operand of a GEMM that
    contracts over the rows of x.
    """
    assert x.dim() == 2 and x.is_cuda and x.stride(1) == 1
    rows, cols = x.shape
    dev = x.device
    o_rows, o_cols, o_axis = (cols, rows, 1) if transpose else (rows, cols, axis)
    if out is None:
        out = NVFP4Tensor(
            codes=torch.empty(o_rows, o_cols // 2, dtype=torch.uint8, device=dev),
            scales=torch.empty(scale_shape(o_rows, o_cols, block2d, o_axis), dtype=torch.uint8,
                               device=dev),
            tensor_scale=torch.empty(1, dtype=torch.float32, device=dev),
            amax=torch.empty(1, dtype=torch.float32, device=dev),
            rows=o_rows, cols=o_cols, block2d=block2d, axis=o_axis)
    ws = None if amax_in is not None else _workspace(dev, rows, cols)
    st = nvfp4_quantize(x, _dtype_code(x), rows, cols, x.stride(0),
                        BLOCK_2D if block2d else BLOCK_1D, axis, int(transpose),
                        ROUND_SR if sr else ROUND_RNE,
                        seed, stream_id, int(rht), mask, amax_in, out.amax, out.codes, out.scales,
                        out.tensor_scale, ws, 0 if ws is None else ws.numel())
    _check("nvfp4_quantize", st)
    return out


def transpose(t: NVFP4Tensor, out: NVFP4Tensor | None = None) -> NVFP4Tensor:
    """The same NVFP4 tensor stored as its transpose [cols, rows]: codes and
    scales transposed, the tensor scale (and amax) shared with `t`.  A 2D
    tensor stays 2D; 1D blocks along rows become blocks down the columns and
    vice versa."""
    o_axis = t.axis if t.block2d else 1 - t.axis
    if out is None:
        dev = t.codes.device
        out = NVFP4Tensor(
            codes=torch.empty(t.cols, t.rows // 2, dtype=torch.uint8, device=dev),
            scales=torch.empty(scale_shape(t.cols, t.rows, t.block2d, o_axis), dtype=torch.uint8,
                               device=dev),
            tensor_scale=t.tensor_scale, amax=t.amax, rows=t.cols, cols=t.rows,
            block2d=t.block2d, axis=o_axis)
    assert out.rows == t.cols and out.cols == t.rows and out.block2d == t.block2d
    assert tuple(out.codes.shape) == (t.cols, t.rows // 2) and out.codes.is_contiguous()
    assert tuple(out.scales.shape) == scale_shape(t.cols, t.rows, t.block2d, o_axis)
    assert out.scales.is_contiguous() and t.codes.is_contiguous() and t.scales.is_contiguous()
    _check("nvfp4_transpose", nvfp4_transpose(
        t.codes, t.scales, t.rows, t.cols, BLOCK_2D if t.block2d else BLOCK_1D, t.axis,
        out.codes, out.scales))
    return out


def amax(x: torch.Tensor, rht_mask: int | None = None):
    """max |x| and, when rht_mask is given, max |RHT16 down the columns of x|,
    in one read; returns (amax, amax_rht or None) as float32 [1] tensors."""
    assert x.dim() == 2 and x.is_cuda and x.stride(1) == 1
    rows, cols = x.shape
    a = torch.empty(1, dtype=torch.float32, device=x.device)
    ar = None if rht_mask is None else torch.empty(1, dtype=torch.float32, device=x.device)
    ws = _workspace(x.device, rows, cols)
    _check("nvfp4_amax", nvfp4_amax(x, _dtype_code(x), rows, cols, x.stride(0),
                                    0 if rht_mask is None else rht_mask, a, ar, ws, ws.numel()))
    return a, ar


def swiglu_amax(h: torch.Tensor, rht_mask: int, out: torch.Tensor | None = None):
    """act = silu(gate) * up over h = [gate | up] (BF16 [rows, 2F]), with
    max |act| and max |RHT16 down the columns of act|; returns (act, amax,
    amax_rht)."""
    assert h.dim() == 2 and h.is_cuda and h.stride(1) == 1 and h.dtype == torch.bfloat16
    rows, F = h.shape[0], h.shape[1] // 2
    if out is None:
        out = torch.empty(rows, F, dtype=torch.bfloat16, device=h.device)
    a = torch.empty(1, dtype=torch.float32, device=h.device)
    ar = torch.empty(1, dtype=torch.float32, device=h.device)
    ws = _workspace(h.device, rows, F)
    _check("nvfp4_swiglu_amax", nvfp4_swiglu_amax(h, rows, F, h.stride(0), out, out.stride(0),
                                                  rht_mask, a, ar, ws, ws.numel()))
    return out, a, ar


def rht16(x: torch.Tensor, axis: int, mask: int) -> torch.Tensor:
    assert x.dim() == 2 and x.is_cuda and x.stride(1) == 1
    rows, cols = x.shape
    y = torch.empty(rows, cols, dtype=torch.float32, device=x.device)
    _check("nvfp4_rht16", nvfp4_rht16(x, _dtype_code(x), rows, cols, x.stride(0), axis, mask, y,
                                      cols))
    return y


def dequantize(t: NVFP4Tensor, out_dtype=torch.bfloat16) -> torch.Tensor:
    out = torch.empty(t.rows, t.cols, dtype=out_dtype, device=t.codes.device)
    _check("nvfp4_dequantize", nvfp4_dequantize(
        t.codes, t.scales, t.tensor_scale, t.rows, t.cols, BLOCK_2D if t.block2d else BLOCK_1D,
        t.axis, _dtype_code(out), out, t.cols))
    return out


def gemm(layout: str, a: NVFP4Tensor, b: NVFP4Tensor, out_dtype=torch.bfloat16,
         out: torch.Tensor | None = None) -> torch.Tensor:
    """NT: a [M,K], b [N,K]; NN: a [M,K], b [K,N]; TN: a [K,M], b [K,N].

    Each operand's blocks must run along K: a 1D operand stored with K along
    its columns has axis 1, one stored with K along its rows axis 0."""
    if layout == "NT":
        M, K = a.rows, a.cols
        N, Kb = b.rows, b.cols
        a_axis, b_axis = 1, 1
    elif layout == "NN":
        M, K = a.rows, a.cols
        Kb, N = b.rows, b.cols
        a_axis, b_axis = 1, 0
    elif layout == "TN":
        K, M = a.rows, a.cols
        Kb, N = b.rows, b.cols
        a_axis, b_axis = 0, 0
    else:
        raise ValueError(layout)
    if Kb != K:
        raise ValueError("gemm %s: A has K = %d but B has K = %d" % (layout, K, Kb))
    for name, op, ax in (("A", a, a_axis), ("B", b, b_axis)):
        if not op.block2d and op.axis != ax:
            raise ValueError("gemm %s: operand %s has 1D blocks along axis %d, not along K "
                             "(axis %d)" % (layout, name, op.axis, ax))
        if tuple(op.codes.shape) != (op.rows, op.cols // 2) or not op.codes.is_contiguous():
            raise ValueError("gemm %s: operand %s codes are not a dense [%d, %d] plane"
                             % (layout, name, op.rows, op.cols // 2))
        if tuple(op.scales.shape) != scale_shape(op.rows, op.cols, op.block2d, op.axis) \
                or not op.scales.is_contiguous():
            raise ValueError("gemm %s: operand %s scales do not match its block layout"
                             % (layout, name))
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype, device=a.codes.device)
    if tuple(out.shape) != (M, N) or out.stride(1) != 1:
        raise ValueError("gemm %s: out must be [%d, %d] with unit column stride" % (layout, M, N))
    nws = nvfp4_gemm_workspace_size(LAYOUT[layout], M, N, K)
    ws = None
    if nws > 0:
        # K longer than one accumulation chain: FP32 planes of the K slices
        key = ("gemm", str(out.device), torch.cuda.current_stream(out.device).cuda_stream)
        ws = _workspaces.get(key)
        if ws is None or ws.numel() < nws:
            ws = torch.empty(nws, dtype=torch.uint8, device=out.device)
            _workspaces[key] = ws
    _check("nvfp4_gemm", nvfp4_gemm(
        LAYOUT[layout], M, N, K, a.codes, a.scales, a.tensor_scale,
        BLOCK_2D if a.block2d else BLOCK_1D, b.codes, b.scales, b.tensor_scale,
        BLOCK_2D if b.block2d else BLOCK_1D, _dtype_code(out), out, out.stride(0), ws,
        0 if ws is None else ws.numel()))
    return out


def gemm_native(a: NVFP4Tensor, b: NVFP4Tensor, out_dtype=torch.bfloat16,
                out: torch.Tensor | None = None, used_native: torch.Tensor | None = None):
    """NT GEMM (a [M, K], b [N, K], blocks along K) on the native scaled FP4
    instruction when every 32-K block of both operands maps onto one
    power-of-two scale exactly, else on the FP16 path.  Returns (out,
    used_native): an int32 device tensor holding 1 or 0 for the path taken."""
    M, K = a.rows, a.cols
    N, Kb = b.rows, b.cols
    if Kb != K:
        raise ValueError("gemm_native: A has K = %d but B has K = %d" % (K, Kb))
    for name, op in (("A", a), ("B", b)):
        if not op.block2d and op.axis != 1:
            raise ValueError("gemm_native: operand %s has 1D blocks along rows, not along K" % name)
        if tuple(op.codes.shape) != (op.rows, op.cols // 2) or not op.codes.is_contiguous():
            raise ValueError("gemm_native: operand %s codes are not a dense plane" % name)
        if tuple(op.scales.shape) != scale_shape(op.rows, op.cols, op.block2d, op.axis) \
                or not op.scales.is_contiguous():
            raise ValueError("gemm_native: operand %s scales do not match its block layout" % name)
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype, device=a.codes.device)
    if tuple(out.shape) != (M, N) or out.stride(1) != 1:
        raise ValueError("gemm_native: out must be [%d, %d] with unit column stride" % (M, N))
    if used_native is None:
        used_native = torch.zeros(1, dtype=torch.int32, device=out.device)
    nws = nvfp4_gemm_native_workspace_size(M, N, K)
    key = ("gemm_native", str(out.device), torch.cuda.current_stream(out.device).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < max(nws, 16):
        ws = torch.empty(max(nws, 16), dtype=torch.uint8, device=out.device)
        _workspaces[key] = ws
    _check("nvfp4_gemm_native", nvfp4_gemm_native(
        M, N, K, a.codes, a.scales, a.tensor_scale, BLOCK_2D if a.block2d else BLOCK_1D,
        b.codes, b.scales, b.tensor_scale, BLOCK_2D if b.block2d else BLOCK_1D,
        _dtype_code(out), out, out.stride(0), used_native, ws, ws.numel()))
    return out, used_native


def interleave_gate_up(w: torch.Tensor) -> torch.Tensor:
    """W_gu [2F, K] as [gate | up] rows -> the row order nvfp4_gemm_swiglu takes:
    gate and up rows interleaved in blocks of 64 (F % 64 == 0).  A plain row
    permutation (a storage-order choice for the weight)."""
    F2, K = w.shape
    F = F2 // 2
    assert F2 % 128 == 0
    return w.reshape(2, F // 64, 64, K).transpose(0, 1).reshape(F2, K).contiguous()


def deinterleave_gate_up_columns(h: torch.Tensor) -> torch.Tensor:
    """The inverse permutation on the columns of H = A W^T: [gate | up]."""
    rows, F2 = h.shape
    F = F2 // 2
    return h.reshape(rows, F // 64, 2, 64).transpose(1, 2).reshape(rows, F2)


def gemm_swiglu(a: NVFP4Tensor, b: NVFP4Tensor, rht_mask: int, store_h: bool = False,
                act_out: torch.Tensor | None = None, h_out: torch.Tensor | None = None):
    """GEMM 1 of the MLP with SwiGLU and both amaxes of its output in the
    epilogue: a [M, K], b [N, K] with gate/up rows interleaved in blocks of 64
    (interleave_gate_up).  Returns (act [M, N/2], amax, amax_rht, H or None)."""
    M, K, N = a.rows, a.cols, b.rows
    assert b.cols == K and not a.axis == 0 and not b.axis == 0
    dev = a.codes.device
    act = act_out if act_out is not None else torch.empty(M, N // 2, dtype=torch.bfloat16,
                                                          device=dev)
    h = h_out
    if h is None and store_h:
        h = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
    am = torch.empty(1, dtype=torch.float32, device=dev)
    amr = torch.empty(1, dtype=torch.float32, device=dev)
    nws = nvfp4_gemm_swiglu_workspace_size(M, N)
    key = ("swiglu", str(dev), torch.cuda.current_stream(dev).cuda_stream)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nws:
        ws = torch.empty(nws, dtype=torch.uint8, device=dev)
        _workspaces[key] = ws
    _check("nvfp4_gemm_swiglu", nvfp4_gemm_swiglu(
        M, N, K, a.codes, a.scales, a.tensor_scale, BLOCK_2D if a.block2d else BLOCK_1D,
        b.codes, b.scales, b.tensor_scale, BLOCK_2D if b.block2d else BLOCK_1D,
        h, h.stride(0) if h is not None else 0, act, act.stride(0), rht_mask, am, amr, ws,
        ws.numel()))
    return act, am, amr, h


def gemm_w4a16(a: torch.Tensor, b: NVFP4Tensor, out_dtype=torch.bfloat16,
               out: torch.Tensor | None = None) -> torch.Tensor:
    """Weight-only decode GEMM, NT: a BF16 [M, K] (M <= 64), b NVFP4 [N, K]."""
    assert a.dim() == 2 and a.is_cuda and a.dtype == torch.bfloat16 and a.stride(1) == 1
    M, K = a.shape
    N = b.rows
    assert b.cols == K and b.axis == 1
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype, device=a.device)
    _check("nvfp4_gemm_w4a16", nvfp4_gemm_w4a16(
        M, N, K, a, a.stride(0), b.codes, b.scales, b.tensor_scale,
        BLOCK_2D if b.block2d else BLOCK_1D, _dtype_code(out), out, out.stride(0)))
    return out


# ---------------------------------------------------------------- MXFP4
# The power-of-two-scaled format the pages compare NVFP4 with (E2M1 codes,
# one E8M0 scale per 32 along the row, no tensor scale; block and scale rule
# of the OCP MX v1.0 standard).

@dataclass
class MXFP4Tensor:
    """codes uint8 [R, C/2], scales uint8 [R, C/32] (E8M0)."""
    codes: torch.Tensor
    scales: torch.Tensor
    rows: int
    cols: int


def mx_quantize(x: torch.Tensor, out: MXFP4Tensor | None = None) -> MXFP4Tensor:
    assert x.dim() == 2 and x.is_cuda and x.stride(1) == 1
    rows, cols = x.shape
    if out is None:
        out = MXFP4Tensor(codes=torch.empty(rows, cols // 2, dtype=torch.uint8, device=x.device),
                          scales=torch.empty(rows, cols // 32, dtype=torch.uint8, device=x.device),
                          rows=rows, cols=cols)
    _check("nvfp4_mx_quantize", nvfp4_mx_quantize(x, _dtype_code(x), rows, cols, x.stride(0),
                                                  out.codes, out.scales))
    return out


def mx_dequantize(t: MXFP4Tensor, out_dtype=torch.bfloat16) -> torch.Tensor:
    out = torch.empty(t.rows, t.cols, dtype=out_dtype, device=t.codes.device)
    _check("nvfp4_mx_dequantize", nvfp4_mx_dequantize(t.codes, t.scales, t.rows, t.cols,
                                                      _dtype_code(out), out, t.cols))
    return out


def mx_gemm(a: MXFP4Tensor, b: MXFP4Tensor, out_dtype=torch.bfloat16,
            out: torch.Tensor | None = None) -> torch.Tensor:
    """NT: a [M, K], b [N, K] -> C [M, N] = a b^T."""
    M, K, N = a.rows, a.cols, b.rows
    assert b.cols == K
    if out is None:
        out = torch.empty(M, N, dtype=out_dtype, device=a.codes.device)
    _check("nvfp4_mx_gemm", nvfp4_mx_gemm(M, N, K, a.codes, a.scales, b.codes, b.scales,
                                          _dtype_code(out), out, out.stride(0)))
    return out


# ---------------------------------------------------------------- KV cache
# NVFP4 KV cache: token rows in 1x16 blocks (RNE) under a fixed tensor scale
# from a calibration amax, written to and gathered from slot-indexed rows.

@dataclass
class NVFP4KVCache:
    """codes uint8 [S, C/2], scales uint8 [S, C/16], amax float32 [1] (the
    calibration amax; s_g = amax / 2688)."""
    codes: torch.Tensor
    scales: torch.Tensor
    amax: torch.Tensor
    num_slots: int
    cols: int


def kv_cache_create(num_slots: int, cols: int, amax, device="cuda") -> NVFP4KVCache:
    """An empty (all-zero) cache; `amax` is a float or a device FP32 tensor [1]."""
    if not torch.is_tensor(amax):
        amax = torch.tensor([float(amax)], dtype=torch.float32, device=device)
    return NVFP4KVCache(codes=torch.zeros(num_slots, cols // 2, dtype=torch.uint8, device=device),
                        scales=torch.zeros(num_slots, cols // 16, dtype=torch.uint8, device=device),
                        amax=amax, num_slots=num_slots, cols=cols)


def kv_cache_write(cache: NVFP4KVCache, x: torch.Tensor, slots: torch.Tensor) -> None:
    """Quantize token rows x [T, C] (BF16/FP32) into cache rows slots[t] (int64
    [T]); slots outside [0, S) are skipped."""
    assert x.dim() == 2 and x.is_cuda and x.stride(1) == 1 and x.shape[1] == cache.cols
    assert slots.dtype == torch.int64 and slots.is_cuda and slots.is_contiguous()
    assert slots.numel() == x.shape[0]
    _check("nvfp4_kv_cache_write", nvfp4_kv_cache_write(
        x, _dtype_code(x), x.shape[0], x.shape[1], x.stride(0), slots, cache.amax,
        cache.num_slots, cache.codes, cache.scales))


def kv_cache_read(cache: NVFP4KVCache, slots: torch.Tensor, out_dtype=torch.bfloat16,
                  out: torch.Tensor | None = None) -> torch.Tensor:
    """Dequantized cache rows slots[j] -> [n, C]; zero rows for slots outside [0, S)."""
    assert slots.dtype == torch.int64 and slots.is_cuda and slots.is_contiguous()
    n = slots.numel()
    if out is None:
        out = torch.empty(n, cache.cols, dtype=out_dtype, device=slots.device)
    assert out.shape == (n, cache.cols) and out.stride(1) == 1
    _check("nvfp4_kv_cache_read", nvfp4_kv_cache_read(
        cache.codes, cache.scales, cache.amax, cache.num_slots, cache.cols, slots, n,
        _dtype_code(out), out, out.stride(0)))
    return out
