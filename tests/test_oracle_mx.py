"""Pins for the oracle's MXFP4 functions (CPU only).

"NVFP4: cos'e e come supera FP8 e BF16" (section "Cos'e NVFP4") compares
NVFP4's E4M3-per-16 scaling with power-of-two scaling such as MXFP4; "FP4"
(chaitex.ru, the section comparing NVFP4 with the open standard) says MXFP4
has larger blocks and coarser scales.  The oracle takes the OCP MX v1.0 block
of 32 and scale X = 2^(floor(log2 amax) - 2).  Pinned here by torch's E8M0
dtype, constructed blocks whose quantization is known exactly, the clipping
the scale rule implies, the E2M1 ties, and a brute-force GEMM.
"""
import numpy as np
import pytest
import torch

import oracle

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def test_e8m0_decode_matches_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).double().numpy()
    got = np.array([oracle.e8m0_value(u) for u in range(256)])
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])


def test_scale_puts_block_amax_in_4_to_8():
    # amax / X lies in [4, 8): the block maximum quantizes to 4 or 6 (codes 6
    # or 7), never lower and never all-saturated below 4.  A scale off by one
    # exponent either way breaks this.
    rng = np.random.default_rng(1)
    for j in range(-120, 120, 7):
        for f in rng.uniform(1.0, 2.0, 5):
            amax = np.float32(np.ldexp(f, j))
            X = oracle.e8m0_value(oracle.mx_scale_code(float(amax)))
            assert 4.0 <= amax / X < 8.0, (j, f)


def test_scale_clamps_and_zero():
    assert oracle.mx_scale_code(0.0) == 0
    assert oracle.mx_scale_code(float(np.float32(2.0 ** -149))) == 0   # below 2^-125: clamped
    assert oracle.mx_scale_code(float(np.finfo(np.float32).max)) == 127 + 125


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_exact_round_trip_of_representable_blocks(dtype):
    # blocks 2^j * v with v from the E2M1 set and one |v| in {4, 6}: the
    # scale is 2^j and every element is represented exactly
    rng = np.random.default_rng(2)
    R, C = 6, 128
    vals = rng.choice(E2M1, size=(R, C)) * rng.choice([-1.0, 1.0], size=(R, C))
    js = rng.integers(-20, 20, size=(R, C // 32))
    for r in range(R):
        for b in range(C // 32):
            vals[r, 32 * b + rng.integers(0, 32)] = rng.choice([4.0, 6.0, -4.0, -6.0])
    x = vals * np.ldexp(1.0, np.repeat(js, 32, axis=1))
    xin = x.astype(np.float32)
    if dtype == "bf16":
        xin = torch.from_numpy(xin).to(torch.bfloat16).view(torch.uint16).numpy()
    codes, scales = oracle.mx_quantize(xin)
    assert np.array_equal(scales.astype(np.int64), js + 127)
    f, _ = oracle.mx_dequantize(codes, scales, R, C)
    assert np.array_equal(f.astype(np.float64), x)


def test_block_above_6_clips():
    x = np.zeros((1, 32), dtype=np.float32)
    x[0, 0] = 7.5 * 2.0 ** 3
    x[0, 1] = -7.0 * 2.0 ** 3
    x[0, 2] = 5.0 * 2.0 ** 3       # tie between 4 and 6: even code (4)
    codes, scales = oracle.mx_quantize(x)
    assert scales[0, 0] == 127 + 3
    f, _ = oracle.mx_dequantize(codes, scales, 1, 32)
    assert f[0, 0] == 6.0 * 8 and f[0, 1] == -6.0 * 8 and f[0, 2] == 4.0 * 8


def test_midpoints_round_to_even_codes():
    mids = [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]
    expect = [0.0, 1.0, 1.0, 2.0, 2.0, 4.0, 4.0]
    x = np.zeros((2, 32), dtype=np.float32)
    x[:, 0] = 6.0                  # fixes X = 1
    x[0, 1:8] = mids
    x[1, 0] = -6.0
    x[1, 1:8] = [-m for m in mids]
    codes, scales = oracle.mx_quantize(x)
    assert list(scales[:, 0]) == [127, 127]
    f, _ = oracle.mx_dequantize(codes, scales, 2, 32)
    assert list(f[0, 1:8]) == expect
    assert list(f[1, 1:8]) == [-e for e in expect]
    # signed zeros keep the sign bit (code 8) like the NVFP4 path
    assert (codes[1, 0] >> 4) & 0xF == 0x8


def test_gemm_brute_force():
    rng = np.random.default_rng(3)
    M, N, K = 5, 7, 96
    a = (rng.standard_normal((M, K)) * np.exp(rng.standard_normal((M, 1)))).astype(np.float32)
    b = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    qa, qb = oracle.mx_quantize(a), oracle.mx_quantize(b)
    fa, _ = oracle.mx_dequantize(*qa, M, K)
    fb, _ = oracle.mx_dequantize(*qb, N, K)
    ref = torch.from_numpy(fa.astype(np.float64)) @ torch.from_numpy(fb.astype(np.float64)).T
    got, ab = oracle.mx_gemm_full(M, N, K, qa, qb)
    assert np.allclose(got, ref.numpy(), rtol=0, atol=1e-12 * np.abs(ab).max())
    assert np.all(ab >= np.abs(got))


def test_gemm_all_ones_gives_k():
    M, N, K = 3, 4, 64
    ones = (np.full((M, K // 2), 0x22, dtype=np.uint8), np.full((M, K // 32), 127, dtype=np.uint8))
    onesb = (np.full((N, K // 2), 0x22, dtype=np.uint8), np.full((N, K // 32), 127, dtype=np.uint8))
    got, _ = oracle.mx_gemm_full(M, N, K, ones, onesb)
    assert np.array_equal(got, np.full((M, N), float(K)))


def test_nvfp4_error_below_mxfp4_on_gaussian_blocks():
    # Not a pin of either quantizer: the comparison the pages draw, on data
    # where both are well defined (standard normal, no outliers).  NVFP4's
    # per-16 E4M3 scales must give a smaller mean squared error.
    rng = np.random.default_rng(4)
    x = rng.standard_normal((64, 1024)).astype(np.float32)
    cm, sm = oracle.mx_quantize(x)
    fm, _ = oracle.mx_dequantize(cm, sm, 64, 1024)
    cn, sn, sg, _ = oracle.quantize(x)
    fn, _ = oracle.dequantize(cn, sn, sg, 64, 1024)
    mse_mx = np.mean((fm.astype(np.float64) - x) ** 2)
    mse_nv = np.mean((fn.astype(np.float64) - x) ** 2)
    assert mse_nv < mse_mx
