"""CPU oracle for NVFP4 quantization, RHT16, dequantization and GEMM, and for
the MXFP4 format the pages compare NVFP4 with.

TEST INFRASTRUCTURE ONLY.  The product library never imports, links or calls
this package; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` do.  It shares no code with the HIP path.

The arithmetic lives in ``nvfp4_oracle.c`` (plain C, IEEE FP32 rounding, FP64
for the GEMM reference); this module only builds it and marshals numpy
arrays.  The format and recipe it follows are described on the pages
"NVFP4: cos'e e come supera FP8 e BF16" (section "Cos'e NVFP4"), "FP4"
(section on the mathematical structure of FP4), the readjensen.com NVFP4
training-recipe news page (recipe paragraph) and "Mastering Low-Precision
AI" (first and third paragraphs).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB = os.path.join(_HERE, "libnvfp4_oracle.so")

DT_BF16 = 0
DT_FP32 = 1
LAYOUTS = {"NT": 0, "NN": 1, "TN": 2}


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (no fast-math, no FP contraction)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
               "-fPIC", "-shared", "-Wall", "-Wextra", "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build(force=False)
        L = ctypes.CDLL(_LIB)
        c_i64, c_u8p, c_vp = ctypes.c_int64, ctypes.POINTER(ctypes.c_uint8), ctypes.c_void_p
        L.oracle_e2m1_value.restype = ctypes.c_double
        L.oracle_e2m1_value.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_value.restype = ctypes.c_float
        L.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e2m1_encode_rne.restype = ctypes.c_uint8
        L.oracle_e2m1_encode_rne.argtypes = [ctypes.c_float]
        L.oracle_e2m1_encode_sr.restype = ctypes.c_uint8
        L.oracle_e2m1_encode_sr.argtypes = [ctypes.c_float, ctypes.c_uint32]
        L.oracle_philox4x32_10.restype = None
        L.oracle_philox4x32_10.argtypes = [c_vp, c_vp, c_vp]
        L.oracle_sr_word.restype = ctypes.c_uint32
        L.oracle_sr_word.argtypes = [ctypes.c_uint64, ctypes.c_uint32, ctypes.c_uint64]
        L.oracle_rht16.restype = ctypes.c_int
        L.oracle_rht16.argtypes = [c_vp, ctypes.c_int, c_i64, c_i64, c_i64, ctypes.c_int,
                                   ctypes.c_uint32, c_vp, c_i64]
        L.oracle_amax.restype = ctypes.c_float
        L.oracle_amax.argtypes = [c_vp, ctypes.c_int, c_i64, c_i64, c_i64, ctypes.c_int,
                                  ctypes.c_int, ctypes.c_uint32]
        L.oracle_quantize.restype = ctypes.c_int
        L.oracle_quantize.argtypes = [c_vp, ctypes.c_int, c_i64, c_i64, c_i64, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint32,
                                      ctypes.c_int, ctypes.c_uint32, c_i64, c_vp, c_vp, c_vp, c_vp,
                                      c_vp]
        L.oracle_f32_to_bf16.restype = ctypes.c_uint16
        L.oracle_f32_to_bf16.argtypes = [ctypes.c_float]
        L.oracle_dequantize.restype = ctypes.c_int
        L.oracle_dequantize.argtypes = [c_vp, c_vp, ctypes.c_float, c_i64, c_i64, ctypes.c_int,
                                        ctypes.c_int, c_vp, c_vp]
        L.oracle_transpose.restype = ctypes.c_int
        L.oracle_transpose.argtypes = [c_vp, c_vp, c_i64, c_i64, ctypes.c_int, ctypes.c_int, c_vp,
                                       c_vp]
        L.oracle_gemm_pairs.restype = ctypes.c_int
        L.oracle_gemm_pairs.argtypes = [ctypes.c_int, c_i64, c_i64, c_i64, c_vp, c_vp,
                                        ctypes.c_float, ctypes.c_int, c_vp, c_vp, ctypes.c_float,
                                        ctypes.c_int, c_i64, c_vp, c_vp, c_vp, c_vp]
        L.oracle_gemm_w4a16_pairs.restype = ctypes.c_int
        L.oracle_gemm_w4a16_pairs.argtypes = [c_i64, c_i64, c_i64, c_vp, c_i64, c_vp, c_vp,
                                              ctypes.c_float, ctypes.c_int, c_i64, c_vp, c_vp,
                                              c_vp, c_vp]
        L.oracle_e8m0_value.restype = ctypes.c_double
        L.oracle_e8m0_value.argtypes = [ctypes.c_uint8]
        L.oracle_mx_scale_code.restype = ctypes.c_uint8
        L.oracle_mx_scale_code.argtypes = [ctypes.c_float]
        L.oracle_mx_quantize.restype = ctypes.c_int
        L.oracle_mx_quantize.argtypes = [c_vp, ctypes.c_int, c_i64, c_i64, c_i64, c_vp, c_vp]
        L.oracle_mx_dequantize.restype = ctypes.c_int
        L.oracle_mx_dequantize.argtypes = [c_vp, c_vp, c_i64, c_i64, c_vp, c_vp]
        L.oracle_mx_gemm_pairs.restype = ctypes.c_int
        L.oracle_mx_gemm_pairs.argtypes = [c_i64, c_i64, c_i64, c_vp, c_vp, c_vp, c_vp, c_i64,
                                           c_vp, c_vp, c_vp, c_vp]
        L.oracle_kv_cache_write.restype = ctypes.c_int
        L.oracle_kv_cache_write.argtypes = [c_vp, ctypes.c_int, c_i64, c_i64, c_i64, c_vp,
                                            ctypes.c_float, c_i64, c_vp, c_vp]
        L.oracle_kv_cache_read.restype = ctypes.c_int
        L.oracle_kv_cache_read.argtypes = [c_vp, c_vp, ctypes.c_float, c_i64, c_i64, c_vp, c_i64,
                                           c_vp, c_vp]
        L.oracle_silu_f32.restype = ctypes.c_float
        L.oracle_silu_f32.argtypes = [ctypes.c_float]
        L.oracle_swiglu_one.restype = ctypes.c_uint16
        L.oracle_swiglu_one.argtypes = [ctypes.c_uint16, ctypes.c_uint16]
        L.oracle_swiglu.restype = ctypes.c_int
        L.oracle_swiglu.argtypes = [c_vp, c_i64, c_i64, c_i64, c_vp, c_vp]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_num_threads.argtypes = []
        L.oracle_set_num_threads.restype = None
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        del c_u8p
        _lib = L
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _as_input(x: np.ndarray):
    """(contiguous array, dtype code).  BF16 data arrives as uint16 bit patterns."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return x, DT_BF16
    if x.dtype == np.float32:
        return x, DT_FP32
    raise TypeError("oracle input must be uint16 (bf16 bits) or float32, got %s" % x.dtype)


# ---------------------------------------------------------------- scalars

def e2m1_value(code: int) -> float:
    return lib().oracle_e2m1_value(code)


def e4m3_value(code: int) -> float:
    return lib().oracle_e4m3_value(code)


def e4m3_encode(t: float) -> int:
    return lib().oracle_e4m3_encode(t)


def e2m1_encode_rne(y: float) -> int:
    return lib().oracle_e2m1_encode_rne(y)


def e2m1_encode_sr(y: float, r: int) -> int:
    return lib().oracle_e2m1_encode_sr(y, r)


def f32_to_bf16(f: float) -> int:
    return lib().oracle_f32_to_bf16(f)


def philox4x32_10(counter, key) -> np.ndarray:
    c = np.ascontiguousarray(np.asarray(counter, dtype=np.uint32))
    k = np.ascontiguousarray(np.asarray(key, dtype=np.uint32))
    out = np.zeros(4, dtype=np.uint32)
    lib().oracle_philox4x32_10(_ptr(c), _ptr(k), _ptr(out))
    return out


def sr_word(seed: int, stream_id: int, idx: int) -> int:
    return lib().oracle_sr_word(seed, stream_id, idx)


# ---------------------------------------------------------------- tensors

def rht16(x: np.ndarray, axis: int, mask: int) -> np.ndarray:
    x, dt = _as_input(x)
    rows, cols = x.shape
    y = np.zeros((rows, cols), dtype=np.float32)
    rc = lib().oracle_rht16(_ptr(x), dt, rows, cols, cols, axis, mask, _ptr(y), cols)
    if rc:
        raise ValueError("oracle_rht16: bad shape")
    return y


def amax(x: np.ndarray, rht: bool = False, axis: int = 1, mask: int = 0) -> float:
    x, dt = _as_input(x)
    rows, cols = x.shape
    return lib().oracle_amax(_ptr(x), dt, rows, cols, cols, int(rht), axis, mask)


def quantize(x: np.ndarray, block2d: bool = False, axis: int = 1, sr: bool = False,
             seed: int = 0, stream_id: int = 0, rht: bool = False, mask: int = 0,
             row0: int = 0, amax_in: float | None = None):
    """Returns (codes uint8 [R, C/2], scales uint8, s_g float, amax float)."""
    x, dt = _as_input(x)
    rows, cols = x.shape
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    if block2d:
        scales = np.zeros((rows // 16, cols // 16), dtype=np.uint8)
    elif axis == 1:
        scales = np.zeros((rows, cols // 16), dtype=np.uint8)
    else:
        scales = np.zeros((rows // 16, cols), dtype=np.uint8)
    ts = np.zeros(1, dtype=np.float32)
    am = np.zeros(1, dtype=np.float32)
    ain = None if amax_in is None else np.array([amax_in], dtype=np.float32)
    rc = lib().oracle_quantize(_ptr(x), dt, rows, cols, cols, int(block2d), axis, int(sr), seed,
                               stream_id, int(rht), mask, row0,
                               None if ain is None else _ptr(ain), _ptr(codes), _ptr(scales),
                               _ptr(ts), _ptr(am))
    if rc:
        raise ValueError("oracle_quantize: bad shape or allocation failure (%d)" % rc)
    return codes, scales, float(ts[0]), float(am[0])


def dequantize(codes: np.ndarray, scales: np.ndarray, s_g: float, rows: int, cols: int,
               block2d: bool = False, axis: int = 1):
    """Returns (fp32 [R, C], bf16 bits uint16 [R, C])."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    f = np.zeros((rows, cols), dtype=np.float32)
    b = np.zeros((rows, cols), dtype=np.uint16)
    lib().oracle_dequantize(_ptr(codes), _ptr(scales), s_g, rows, cols, int(block2d), axis,
                            _ptr(f), _ptr(b))
    return f, b


def transpose(codes: np.ndarray, scales: np.ndarray, rows: int, cols: int,
              block2d: bool = False, axis: int = 1):
    """The NVFP4 tensor [rows, cols] stored as its transpose [cols, rows]:
    returns (codes uint8 [cols, rows/2], scales uint8 in the transposed
    tensor's layout: 2D [cols/16, rows/16]; from axis 1 -> axis 0
    [cols/16, rows]; from axis 0 -> axis 1 [cols, rows/16])."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    ct = np.zeros((cols, rows // 2), dtype=np.uint8)
    if block2d:
        st = np.zeros((cols // 16, rows // 16), dtype=np.uint8)
    elif axis == 1:
        st = np.zeros((cols // 16, rows), dtype=np.uint8)
    else:
        st = np.zeros((cols, rows // 16), dtype=np.uint8)
    if lib().oracle_transpose(_ptr(codes), _ptr(scales), rows, cols, int(block2d), axis, _ptr(ct),
                              _ptr(st)):
        raise ValueError("oracle_transpose: bad shape")
    return ct, st


def gemm_pairs(layout: str, M: int, N: int, K: int, a, b, ms, ns):
    """a, b = (codes, scales, s_g, block2d).  Returns (ref fp64, abs fp64) at (ms, ns)."""
    ac, asc, ats, a2d = a
    bc, bsc, bts, b2d = b
    ac = np.ascontiguousarray(ac, dtype=np.uint8)
    asc = np.ascontiguousarray(asc, dtype=np.uint8)
    bc = np.ascontiguousarray(bc, dtype=np.uint8)
    bsc = np.ascontiguousarray(bsc, dtype=np.uint8)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    ref = np.zeros(len(ms), dtype=np.float64)
    ab = np.zeros(len(ms), dtype=np.float64)
    rc = lib().oracle_gemm_pairs(LAYOUTS[layout], M, N, K, _ptr(ac), _ptr(asc), ats, int(a2d),
                                 _ptr(bc), _ptr(bsc), bts, int(b2d), len(ms), _ptr(ms), _ptr(ns),
                                 _ptr(ref), _ptr(ab))
    if rc:
        raise ValueError("oracle_gemm_pairs: bad layout")
    return ref, ab


def gemm_full(layout: str, M: int, N: int, K: int, a, b):
    """Full M x N reference (small sizes only)."""
    mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ref, ab = gemm_pairs(layout, M, N, K, a, b, mm.ravel(), nn.ravel())
    return ref.reshape(M, N), ab.reshape(M, N)


def gemm_w4a16_pairs(M: int, N: int, K: int, a_bf16: np.ndarray, b, ms, ns):
    """NT with BF16 activations a [M, K] (uint16 bit patterns) and an NVFP4
    weight b = (codes, scales, s_g, block2d) stored [N, K].  Returns (ref fp64,
    abs fp64) at (ms, ns)."""
    bc, bsc, bts, b2d = b
    a = np.ascontiguousarray(a_bf16, dtype=np.uint16)
    bc = np.ascontiguousarray(bc, dtype=np.uint8)
    bsc = np.ascontiguousarray(bsc, dtype=np.uint8)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    ref = np.zeros(len(ms), dtype=np.float64)
    ab = np.zeros(len(ms), dtype=np.float64)
    if lib().oracle_gemm_w4a16_pairs(M, N, K, _ptr(a), K, _ptr(bc), _ptr(bsc), bts, int(b2d),
                                     len(ms), _ptr(ms), _ptr(ns), _ptr(ref), _ptr(ab)):
        raise ValueError("oracle_gemm_w4a16_pairs: bad shape")
    return ref, ab


def gemm_w4a16_full(M: int, N: int, K: int, a_bf16: np.ndarray, b):
    mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ref, ab = gemm_w4a16_pairs(M, N, K, a_bf16, b, mm.ravel(), nn.ravel())
    return ref.reshape(M, N), ab.reshape(M, N)


# ---------------------------------------------------------------- MXFP4
# The power-of-two format the pages compare NVFP4 with ("NVFP4: cos'e e come
# supera FP8 e BF16", section "Cos'e NVFP4"; "FP4", the section comparing
# NVFP4 with the open standard), with the block size (32) and scale rule of
# the OCP Microscaling (MX) v1.0 specification, which the pages do not give.

def e8m0_value(code: int) -> float:
    return lib().oracle_e8m0_value(code)


def mx_scale_code(amax: float) -> int:
    return lib().oracle_mx_scale_code(amax)


def mx_quantize(x: np.ndarray):
    """Blocks of 32 along the columns.  Returns (codes uint8 [R, C/2], scales uint8 [R, C/32])."""
    x, dt = _as_input(x)
    rows, cols = x.shape
    codes = np.zeros((rows, cols // 2), dtype=np.uint8)
    scales = np.zeros((rows, cols // 32), dtype=np.uint8)
    if lib().oracle_mx_quantize(_ptr(x), dt, rows, cols, cols, _ptr(codes), _ptr(scales)):
        raise ValueError("oracle_mx_quantize: bad shape")
    return codes, scales


def mx_dequantize(codes: np.ndarray, scales: np.ndarray, rows: int, cols: int):
    """Returns (fp32 [R, C], bf16 bits uint16 [R, C])."""
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    f = np.zeros((rows, cols), dtype=np.float32)
    b = np.zeros((rows, cols), dtype=np.uint16)
    if lib().oracle_mx_dequantize(_ptr(codes), _ptr(scales), rows, cols, _ptr(f), _ptr(b)):
        raise ValueError("oracle_mx_dequantize: bad shape")
    return f, b


def mx_gemm_pairs(M: int, N: int, K: int, a, b, ms, ns):
    """NT: a = (codes [M, K/2], scales [M, K/32]), b likewise [N, ...].
    Returns (ref fp64, abs fp64) at (ms, ns)."""
    ac, asc = (np.ascontiguousarray(t, dtype=np.uint8) for t in a)
    bc, bsc = (np.ascontiguousarray(t, dtype=np.uint8) for t in b)
    ms = np.ascontiguousarray(ms, dtype=np.int64)
    ns = np.ascontiguousarray(ns, dtype=np.int64)
    ref = np.zeros(len(ms), dtype=np.float64)
    ab = np.zeros(len(ms), dtype=np.float64)
    if lib().oracle_mx_gemm_pairs(M, N, K, _ptr(ac), _ptr(asc), _ptr(bc), _ptr(bsc), len(ms),
                                  _ptr(ms), _ptr(ns), _ptr(ref), _ptr(ab)):
        raise ValueError("oracle_mx_gemm_pairs: bad shape")
    return ref, ab


def mx_gemm_full(M: int, N: int, K: int, a, b):
    mm, nn = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ref, ab = mx_gemm_pairs(M, N, K, a, b, mm.ravel(), nn.ravel())
    return ref.reshape(M, N), ab.reshape(M, N)


def silu_f32(g: float) -> float:
    return lib().oracle_silu_f32(g)


def swiglu(h_bf16: np.ndarray):
    """act = BF16(BF16(silu(gate)) * up) for h = [gate | up] (uint16 BF16 bits,
    [rows, 2F]); returns (act, BF16(silu(gate))) as uint16 BF16 bits [rows, F]."""
    h = np.ascontiguousarray(h_bf16, dtype=np.uint16)
    rows, F2 = h.shape
    act = np.zeros((rows, F2 // 2), dtype=np.uint16)
    sb = np.zeros((rows, F2 // 2), dtype=np.uint16)
    rc = lib().oracle_swiglu(_ptr(h), rows, F2 // 2, F2, _ptr(act), _ptr(sb))
    if rc:
        raise ValueError("oracle_swiglu: bad shape")
    return act, sb


def kv_cache_write(x: np.ndarray, slots, amax: float, cache_codes: np.ndarray,
                   cache_scales: np.ndarray) -> None:
    """Quantize token rows of x (BF16 bits or FP32, [T, C]) into cache rows
    slots[t] of (cache_codes [S, C/2], cache_scales [S, C/16]) in place; slots
    outside [0, S) are skipped.  s_g = RN(amax / 2688)."""
    x, dt = _as_input(x)
    tokens, cols = x.shape
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    assert slots.shape == (tokens,)
    assert cache_codes.dtype == np.uint8 and cache_codes.flags.c_contiguous
    assert cache_scales.dtype == np.uint8 and cache_scales.flags.c_contiguous
    num_slots = cache_codes.shape[0]
    assert cache_codes.shape == (num_slots, cols // 2)
    assert cache_scales.shape == (num_slots, cols // 16)
    rc = lib().oracle_kv_cache_write(_ptr(x), dt, tokens, cols, cols, _ptr(slots), amax,
                                     num_slots, _ptr(cache_codes), _ptr(cache_scales))
    if rc:
        raise ValueError("oracle_kv_cache_write: bad shape (%d)" % rc)


def kv_cache_read(cache_codes: np.ndarray, cache_scales: np.ndarray, amax: float, slots):
    """Returns (fp32 [n, C], bf16 bits uint16 [n, C]) of cache rows slots[j],
    zero rows for slots outside [0, S)."""
    cache_codes = np.ascontiguousarray(cache_codes, dtype=np.uint8)
    cache_scales = np.ascontiguousarray(cache_scales, dtype=np.uint8)
    slots = np.ascontiguousarray(slots, dtype=np.int64)
    num_slots, half = cache_codes.shape
    cols = 2 * half
    n = slots.shape[0]
    f = np.zeros((n, cols), dtype=np.float32)
    b = np.zeros((n, cols), dtype=np.uint16)
    rc = lib().oracle_kv_cache_read(_ptr(cache_codes), _ptr(cache_scales), amax, num_slots, cols,
                                    _ptr(slots), n, _ptr(f), _ptr(b))
    if rc:
        raise ValueError("oracle_kv_cache_read: bad shape (%d)" % rc)
    return f, b


def num_threads() -> int:
    return lib().oracle_num_threads()


def set_num_threads(n: int) -> None:
    lib().oracle_set_num_threads(n)
