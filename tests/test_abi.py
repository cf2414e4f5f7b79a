"""Host-side checks of the C ABI (CPU only: no call here reaches the GPU).

The library must load and export every entry point include/nvfp4.h declares;
argument validation must reject bad calls before anything is enqueued (these
calls return before touching HIP, so they run without a GPU).
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    import nvfp4_bit_microscaled_amd as m
    return m.lib


def test_header_declares_the_abi():
    names = declared_functions()
    assert names == sorted(["nvfp4_version", "nvfp4_status_string",
                            "nvfp4_quantize_workspace_size", "nvfp4_quantize",
                            "nvfp4_amax_workspace_size", "nvfp4_amax", "nvfp4_swiglu_amax",
                            "nvfp4_rht16",
                            "nvfp4_dequantize", "nvfp4_gemm", "nvfp4_mx_quantize",
                            "nvfp4_mx_dequantize", "nvfp4_mx_gemm", "nvfp4_gemm_w4a16",
                            "nvfp4_kv_cache_write", "nvfp4_kv_cache_read",
                            "nvfp4_gemm_swiglu_workspace_size", "nvfp4_gemm_swiglu",
                            "nvfp4_transpose", "nvfp4_quantize_noalloc",
                            "nvfp4_gemm_workspace_size", "nvfp4_gemm_native_workspace_size",
                            "nvfp4_gemm_native"])


def test_library_exports_every_declared_symbol(lib):
    import nvfp4_bit_microscaled_amd as m
    for name in declared_functions():
        assert hasattr(lib, name), name
        assert name in m.EXPORTS


def test_version_and_status_strings(lib):
    import nvfp4_bit_microscaled_amd as m
    assert m.version() >= 100
    for code, name in m.STATUS_NAMES.items():
        assert m.status_string(code) == name
    assert m.status_string(99) == "NVFP4_ERR_UNKNOWN"
    assert m.nvfp4_quantize_workspace_size(1 << 15, 1 << 12) >= 4


FAKE = ctypes.c_void_p(0x10000)        # aligned, never dereferenced: validation fails first
MISALIGNED = ctypes.c_void_p(0x10008)
ODD = ctypes.c_void_p(0x10001)


def q(lib, **kw):
    args = dict(x=FAKE, dt=0, rows=32, cols=64, ld=64, block=0, axis=1, tr=0, rnd=0, seed=0, sid=0,
                rht=0, mask=0, amax_in=FAKE, amax_out=None, codes=FAKE, scales=FAKE, ts=FAKE,
                ws=None, wsb=0, stream=None)
    args.update(kw)
    return lib.nvfp4_quantize(*args.values())


def test_quantize_validation(lib):
    assert q(lib, dt=5) == 1
    assert q(lib, block=3) == 1
    assert q(lib, rnd=2) == 1
    assert q(lib, axis=2) == 1
    assert q(lib, rht=2) == 1
    assert q(lib, rows=-1) == 1
    assert q(lib, ts=None) == 1
    assert q(lib, cols=40, ld=40) == 2              # cols % 16
    assert q(lib, rows=24, axis=0) == 2             # rows % 16 for axis 0
    assert q(lib, rows=24, block=1) == 2            # rows % 16 for 2D
    assert q(lib, ld=32) == 2                       # ld < cols
    assert q(lib, block=1, rht=1) == 5              # RHT needs 1D
    assert q(lib, tr=2) == 1
    assert q(lib, tr=1) == 5                        # transposed output needs blocks down columns
    assert q(lib, tr=1, axis=0, rows=24) == 2
    assert q(lib, x=MISALIGNED) == 3
    assert q(lib, ld=68, dt=0) == 3                 # 136-byte BF16 rows are not 16-byte multiples
    assert q(lib, codes=MISALIGNED) == 3
    assert q(lib, amax_in=None, ws=None) == 6       # amax pass needs the workspace
    assert q(lib, amax_in=None, ws=FAKE, wsb=8) == 6
    assert q(lib, x=None) == 1


def a(lib, **kw):
    args = dict(x=FAKE, dt=0, rows=32, cols=64, ld=64, mask=0, amax=FAKE, amax_rht=FAKE, ws=FAKE,
                wsb=1 << 20, stream=None)
    args.update(kw)
    return lib.nvfp4_amax(*args.values())


def test_amax_validation(lib):
    assert a(lib, dt=5) == 1
    assert a(lib, amax=None) == 1
    assert a(lib, rows=-1) == 1
    assert a(lib, cols=40, ld=40) == 2              # cols % 16
    assert a(lib, rows=24) == 2                     # rows % 16 with the RHT amax
    assert a(lib, ld=32) == 2
    assert a(lib, x=MISALIGNED) == 3
    assert a(lib, ws=None) == 6
    assert a(lib, wsb=8) == 6
    assert a(lib, x=None) == 1
    assert lib.nvfp4_amax_workspace_size(1 << 15, 1 << 12) >= 8


def sw(lib, **kw):
    args = dict(h=FAKE, rows=32, F=64, ldh=128, act=FAKE, lda=64, mask=0, amax=FAKE,
                amax_rht=FAKE, ws=FAKE, wsb=1 << 20, stream=None)
    args.update(kw)
    return lib.nvfp4_swiglu_amax(*args.values())


def test_swiglu_amax_validation(lib):
    assert sw(lib, amax=None) == 1
    assert sw(lib, amax_rht=None) == 1
    assert sw(lib, rows=-16) == 1
    assert sw(lib, rows=24) == 2                    # rows % 16
    assert sw(lib, F=40, ldh=80, lda=40) == 2       # F % 16
    assert sw(lib, ldh=100) == 2                    # ld_h < 2F
    assert sw(lib, lda=32) == 2                     # ld_act < F
    assert sw(lib, h=MISALIGNED) == 3
    assert sw(lib, ldh=132) == 3                    # 264-byte rows are not 16-byte multiples
    assert sw(lib, ws=None) == 6
    assert sw(lib, h=None) == 1


def g(lib, **kw):
    args = dict(layout=0, M=64, N=64, K=64, ac=FAKE, asc=FAKE, ats=FAKE, ab=0, bc=FAKE, bsc=FAKE,
                bts=FAKE, bb=1, odt=0, c=FAKE, ldc=64, ws=None, wsb=0, stream=None)
    args.update(kw)
    return lib.nvfp4_gemm(*args.values())


def test_gemm_validation(lib):
    assert g(lib, layout=3) == 1
    assert g(lib, odt=7) == 1
    assert g(lib, M=-1) == 1
    assert g(lib, K=40) == 2                        # K % 16
    assert g(lib, ldc=32) == 2
    assert g(lib, layout=1, N=40, ldc=40) == 2      # NN: B packed along N
    assert g(lib, layout=2, M=40) == 2              # TN: A packed along M
    assert g(lib, bb=1, N=40, ldc=40) == 4          # 2D operand with N % 16
    assert g(lib, c=ODD) == 3
    assert g(lib, ac=MISALIGNED) == 3
    assert g(lib, ac=None) == 1
    assert g(lib, M=0) == 0                         # empty output: nothing to do
    assert g(lib, N=0) == 0
    # K above one accumulation chain (32768): K slices need a workspace of one
    # FP32 M x N plane per slice (slices of at most 32768, multiples of 512)
    import nvfp4_bit_microscaled_amd as m
    assert m.nvfp4_gemm_workspace_size(0, 64, 64, 32768) == 0
    assert m.nvfp4_gemm_workspace_size(1, 64, 64, 32784) == 2 * 64 * 64 * 4
    assert m.nvfp4_gemm_workspace_size(0, 8192, 16384, 106496) == 4 * 8192 * 16384 * 4
    assert m.nvfp4_gemm_workspace_size(2, 0, 64, 106496) == 0
    assert m.nvfp4_gemm_workspace_size(1, 4096, 14336, 32768) == 0   # no last-round split for NN
    assert g(lib, K=106496) == 6                    # workspace missing
    assert g(lib, K=106496, ws=FAKE, wsb=4 * 64 * 64 * 4 - 1) == 6
    assert g(lib, K=106496, ws=MISALIGNED, wsb=4 * 64 * 64 * 4) == 3


def test_rht_and_dequant_validation(lib):
    assert lib.nvfp4_rht16(FAKE, 0, 32, 40, 40, 1, 0, FAKE, 40, None) == 2
    assert lib.nvfp4_rht16(FAKE, 0, 24, 64, 64, 0, 0, FAKE, 64, None) == 2
    assert lib.nvfp4_rht16(FAKE, 0, 32, 64, 64, 3, 0, FAKE, 64, None) == 1
    assert lib.nvfp4_rht16(FAKE, 0, 0, 64, 64, 1, 0, FAKE, 64, None) == 0
    assert lib.nvfp4_dequantize(FAKE, FAKE, FAKE, 32, 40, 0, 1, 0, FAKE, 40, None) == 2
    assert lib.nvfp4_dequantize(FAKE, FAKE, FAKE, 24, 64, 1, 1, 0, FAKE, 64, None) == 2
    assert lib.nvfp4_dequantize(FAKE, FAKE, FAKE, 32, 64, 0, 1, 9, FAKE, 64, None) == 1
    assert lib.nvfp4_dequantize(MISALIGNED, FAKE, FAKE, 32, 64, 0, 1, 0, FAKE, 64, None) == 3


def mxg(lib, **kw):
    args = dict(M=64, N=64, K=256, ac=FAKE, asc=FAKE, bc=FAKE, bsc=FAKE, odt=0, c=FAKE, ldc=64,
                stream=None)
    args.update(kw)
    return lib.nvfp4_mx_gemm(*args.values())


def test_mx_validation(lib):
    # quantize: x, dtype, rows, cols, ld, codes, scales, stream
    assert lib.nvfp4_mx_quantize(FAKE, 2, 4, 64, 64, FAKE, FAKE, None) == 1
    assert lib.nvfp4_mx_quantize(FAKE, 0, 4, 48, 48, FAKE, FAKE, None) == 2   # cols % 32
    assert lib.nvfp4_mx_quantize(FAKE, 0, 4, 64, 32, FAKE, FAKE, None) == 2   # ld < cols
    assert lib.nvfp4_mx_quantize(MISALIGNED, 0, 4, 64, 64, FAKE, FAKE, None) == 3
    assert lib.nvfp4_mx_quantize(FAKE, 0, 4, 64, 68, FAKE, FAKE, None) == 3   # 136-byte rows
    assert lib.nvfp4_mx_quantize(FAKE, 0, 4, 64, 64, None, FAKE, None) == 1
    assert lib.nvfp4_mx_quantize(FAKE, 0, 0, 64, 64, None, None, None) == 0
    assert lib.nvfp4_mx_dequantize(FAKE, FAKE, 4, 48, 0, FAKE, 48, None) == 2
    assert lib.nvfp4_mx_dequantize(FAKE, FAKE, 4, 64, 5, FAKE, 64, None) == 1
    assert lib.nvfp4_mx_dequantize(MISALIGNED, FAKE, 4, 64, 0, FAKE, 64, None) == 3
    assert mxg(lib, K=192) == 2                      # K % 128
    assert mxg(lib, ldc=32) == 2
    assert mxg(lib, odt=3) == 1
    assert mxg(lib, M=-1) == 1
    assert mxg(lib, c=ODD) == 3
    assert mxg(lib, ac=MISALIGNED) == 3
    assert mxg(lib, bsc=None) == 1
    assert mxg(lib, K=1 << 24) == 5                  # 256 rows of codes past 2^31 bytes
    assert mxg(lib, K=32896) == 5                    # longer than one accumulation chain
    assert mxg(lib, M=0) == 0


def ng(lib, **kw):
    args = dict(M=64, N=64, K=256, ac=FAKE, asc=FAKE, ats=FAKE, ab=0, bc=FAKE, bsc=FAKE, bts=FAKE,
                bb=0, odt=0, c=FAKE, ldc=64, used=FAKE, ws=FAKE, wsb=1 << 20, stream=None)
    args.update(kw)
    return lib.nvfp4_gemm_native(*args.values())


def test_gemm_native_validation(lib):
    import nvfp4_bit_microscaled_amd as m
    # E8M0 planes: M x K/32 (rounded up to 16 bytes) + N x K/32
    assert m.nvfp4_gemm_native_workspace_size(64, 64, 256) == 64 * 8 + 64 * 8
    assert m.nvfp4_gemm_native_workspace_size(5, 7, 128) == 32 + 28
    assert m.nvfp4_gemm_native_workspace_size(5, 7, 100) == 0
    assert ng(lib, ab=2) == 1
    assert ng(lib, odt=5) == 1
    assert ng(lib, N=-1) == 1
    assert ng(lib, K=192) == 2                       # K % 128
    assert ng(lib, ldc=32) == 2
    assert ng(lib, ab=1, M=40) == 4                  # 2D operand with M % 16
    assert ng(lib, K=32896) == 5                     # longer than one accumulation chain
    assert ng(lib, c=ODD) == 3
    assert ng(lib, used=None) == 1
    assert ng(lib, ats=None) == 1
    assert ng(lib, bsc=MISALIGNED) == 3
    assert ng(lib, used=ODD) == 3
    assert ng(lib, ws=None) == 6
    assert ng(lib, wsb=64 * 8 + 64 * 8 - 1) == 6
    assert ng(lib, ws=MISALIGNED) == 3
    assert ng(lib, M=0) == 0


def w4(lib, **kw):
    args = dict(M=1, N=64, K=512, a=FAKE, lda=512, bc=FAKE, bsc=FAKE, bts=FAKE, bb=0, odt=0,
                c=FAKE, ldc=64, stream=None)
    args.update(kw)
    return lib.nvfp4_gemm_w4a16(*args.values())


def test_w4a16_validation(lib):
    assert w4(lib, bb=2) == 1
    assert w4(lib, odt=9) == 1
    assert w4(lib, M=-1) == 1
    assert w4(lib, K=256, lda=256) == 2             # K % 512
    assert w4(lib, lda=100) == 2                    # lda < K
    assert w4(lib, ldc=32) == 2
    assert w4(lib, bb=1, N=40, ldc=40) == 4         # 2D weight with N % 16
    assert w4(lib, M=65) == 5                       # decode shapes only
    assert w4(lib, a=MISALIGNED) == 3
    assert w4(lib, lda=516) == 3                    # 1032-byte rows
    assert w4(lib, c=ODD) == 3
    assert w4(lib, bts=None) == 1
    assert w4(lib, M=0) == 0
    assert w4(lib, K=33280, lda=33280) == 5         # longer than one accumulation chain


def kvw(lib, **kw):
    args = dict(x=FAKE, dt=0, tokens=4, cols=128, ld=128, slots=FAKE, amax=FAKE, S=16, cc=FAKE,
                cs=FAKE, stream=None)
    args.update(kw)
    return lib.nvfp4_kv_cache_write(*args.values())


def kvr(lib, **kw):
    args = dict(cc=FAKE, cs=FAKE, amax=FAKE, S=16, cols=128, slots=FAKE, n=4, odt=0, out=FAKE,
                ld=128, stream=None)
    args.update(kw)
    return lib.nvfp4_kv_cache_read(*args.values())


def test_kv_cache_validation(lib):
    assert kvw(lib, dt=2) == 1
    assert kvw(lib, tokens=-1) == 1
    assert kvw(lib, S=-1) == 1
    assert kvw(lib, cols=40, ld=40) == 2          # cols % 16
    assert kvw(lib, ld=64) == 2                   # ld < cols
    assert kvw(lib, tokens=1 << 30, cols=1 << 10, ld=1 << 10) == 5   # > 2^32 blocks
    assert kvw(lib, x=MISALIGNED) == 3
    assert kvw(lib, ld=132) == 3                  # 264-byte rows
    assert kvw(lib, slots=ctypes.c_void_p(0x10004)) == 3
    assert kvw(lib, cc=MISALIGNED) == 3
    assert kvw(lib, amax=None) == 1
    assert kvw(lib, slots=None) == 1
    assert kvw(lib, tokens=0, x=None, slots=None) == 0
    assert kvw(lib, S=0, cc=None, cs=None) == 0
    assert kvr(lib, odt=7) == 1
    assert kvr(lib, n=-2) == 1
    assert kvr(lib, cols=24, ld=24) == 2
    assert kvr(lib, ld=100) == 2
    assert kvr(lib, out=MISALIGNED) == 3
    assert kvr(lib, ld=132) == 3                  # 264-byte BF16 rows
    assert kvr(lib, slots=ctypes.c_void_p(0x10002)) == 3
    assert kvr(lib, out=None) == 1
    assert kvr(lib, cc=None) == 1
    assert kvr(lib, n=0, out=None) == 0
    assert kvr(lib, S=0, cc=None, cs=None, out=MISALIGNED) == 3   # checked before the zero fill


def test_transpose_validation(lib):
    def tr(**kw):
        args = dict(codes=FAKE, scales=FAKE, rows=32, cols=64, block=1, axis=1, codes_t=FAKE,
                    scales_t=FAKE, stream=None)
        args.update(kw)
        return lib.nvfp4_transpose(*args.values())
    assert tr(block=2) == 1
    assert tr(block=0, axis=3) == 1
    assert tr(rows=-16) == 1
    assert tr(rows=24) == 2                       # rows % 16
    assert tr(cols=40) == 2                       # cols % 16
    assert tr(rows=1 << 31, cols=1 << 7) == 5     # more than 2^32 code words
    assert tr(codes_t=None) == 1
    assert tr(scales=None) == 1
    assert tr(codes=MISALIGNED) == 3
    assert tr(codes_t=MISALIGNED) == 3
    assert tr(rows=0, codes=None, scales=None, codes_t=None, scales_t=None) == 0


def test_gemm_binding_checks_operands():
    """The Python gemm() rejects operands whose K, block axis or planes do not
    fit the layout, and a wrong out tensor, before any library call."""
    import torch

    import nvfp4_bit_microscaled_amd as m

    def op(rows, cols, block2d=False, axis=1):
        return m.NVFP4Tensor(torch.zeros(rows, cols // 2, dtype=torch.uint8),
                             torch.zeros(m.scale_shape(rows, cols, block2d, axis), dtype=torch.uint8),
                             torch.ones(1), torch.zeros(1), rows, cols, block2d, axis)
    with pytest.raises(ValueError, match="K"):
        m.gemm("NT", op(32, 64), op(48, 128))                # K 64 vs 128
    with pytest.raises(ValueError, match="K"):
        m.gemm("NN", op(32, 64), op(32, 48, axis=0))         # B has 32 rows, K = 64
    with pytest.raises(ValueError, match="K"):
        m.gemm("TN", op(64, 32, axis=0), op(48, 16, axis=0))
    with pytest.raises(ValueError, match="axis"):
        m.gemm("NT", op(32, 64), op(48, 64, axis=0))         # NT needs axis 1 on B
    with pytest.raises(ValueError, match="axis"):
        m.gemm("NN", op(32, 64), op(64, 48, axis=1))         # NN needs axis 0 on B
    with pytest.raises(ValueError, match="axis"):
        m.gemm("TN", op(64, 32, axis=1), op(64, 48, axis=0))
    bad = op(32, 64)
    bad.scales = torch.zeros(32, 2, dtype=torch.uint8)
    with pytest.raises(ValueError, match="scales"):
        m.gemm("NT", bad, op(48, 64))
    with pytest.raises(ValueError, match="out"):
        m.gemm("NT", op(32, 64), op(48, 64), out=torch.empty(32, 40))
    with pytest.raises(ValueError, match="out"):
        m.gemm("NT", op(32, 64), op(48, 64), out=torch.empty(48, 32).t())


def gsw(lib, **kw):
    args = dict(M=256, N=256, K=256, ac=FAKE, asc=FAKE, ats=FAKE, ab=0, bc=FAKE, bsc=FAKE, bts=FAKE,
                bb=1, h=None, ldh=0, act=FAKE, ld_act=128, mask=0, amax=FAKE, amax_rht=FAKE,
                ws=FAKE, wsb=1 << 20, stream=None)
    args.update(kw)
    return lib.nvfp4_gemm_swiglu(*args.values())


def test_gemm_swiglu_validation(lib):
    import nvfp4_bit_microscaled_amd as m
    assert m.nvfp4_gemm_swiglu_workspace_size(256, 256) == 8
    assert m.nvfp4_gemm_swiglu_workspace_size(32768, 28672) == 2 * 128 * 112 * 4
    assert gsw(lib, ab=3) == 1
    assert gsw(lib, M=-16) == 1
    assert gsw(lib, amax=None) == 1
    assert gsw(lib, N=192) == 2                 # N % 128
    assert gsw(lib, M=40) == 2                  # M % 16
    assert gsw(lib, K=0) == 2
    assert gsw(lib, K=96) == 2                  # K % 128
    assert gsw(lib, ld_act=120) == 2            # ld_act < N / 2
    assert gsw(lib, h=FAKE, ldh=200) == 2       # ldh < N
    assert gsw(lib, K=1 << 24) == 5             # 256-row records past 2^31 bytes
    assert gsw(lib, K=32896) == 5               # longer than one accumulation chain
    assert gsw(lib, act=None) == 1
    assert gsw(lib, bc=MISALIGNED) == 3
    assert gsw(lib, act=ctypes.c_void_p(0x10004)) == 3
    assert gsw(lib, ld_act=130) == 3            # rows not a multiple of 8 bytes
    assert gsw(lib, h=ODD, ldh=256) == 3
    assert gsw(lib, wsb=4) == 6
    assert gsw(lib, ws=None) == 6
