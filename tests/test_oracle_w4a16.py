"""Pins for the oracle's weight-only (BF16 activation x NVFP4 weight) GEMM
reference (CPU only), by brute force and a closed form.

The juejin.cn page on NVFP4 (item 3) has models trained at higher precision
quantized to NVFP4 for inference; chaitex.ru "FP4" (item 1 of the scaling
scheme) quantizes the weight matrix in 16-element blocks.
"""
import numpy as np
import pytest
import torch

import oracle


def bf16_bits(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("b2d", [False, True])
def test_brute_force_against_float64_matmul(b2d):
    rng = np.random.default_rng(11 + b2d)
    M, N, K = 5, 32, 96
    a = bf16_bits(rng.standard_normal((M, K)) * 3)
    w = (rng.standard_normal((N, K)) * 0.02).astype(np.float32)
    codes, scales, sg, _ = oracle.quantize(w, block2d=b2d)
    # val * e exactly (s_g = 1 in the oracle's own dequantization), then s_g
    ve, _ = oracle.dequantize(codes, scales, 1.0, N, K, block2d=b2d)
    af = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).double()
    ref = sg * (af @ torch.from_numpy(ve.astype(np.float64)).T).numpy()
    got, ab = oracle.gemm_w4a16_full(M, N, K, a, (codes, scales, sg, b2d))
    assert np.allclose(got, ref, rtol=0, atol=1e-12 * np.abs(ab).max())
    assert np.all(ab >= np.abs(got) * (1 - 1e-15))


def test_all_ones_gives_k_times_scale():
    M, N, K = 2, 16, 64
    a = bf16_bits(np.ones((M, K)))
    codes = np.full((N, K // 2), 0x22, dtype=np.uint8)        # E2M1 1.0 everywhere
    scales = np.full((N, K // 16), 0x38, dtype=np.uint8)      # E4M3 1.0
    got, _ = oracle.gemm_w4a16_full(M, N, K, a, (codes, scales, 0.5, False))
    assert np.array_equal(got, np.full((M, N), 0.5 * K))


def test_matches_nvfp4_gemm_when_activations_are_representable():
    # activations that are exactly NVFP4 (s_A = 1, e = 1, codes random) give
    # the NVFP4 GEMM's reference value
    rng = np.random.default_rng(3)
    M, N, K = 3, 16, 64
    acodes = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    ascales = np.full((M, K // 16), 0x38, dtype=np.uint8)
    af, ab16 = oracle.dequantize(acodes, ascales, 1.0, M, K)
    w = (rng.standard_normal((N, K)) * 0.1).astype(np.float32)
    bq = oracle.quantize(w, block2d=True)
    b = (bq[0], bq[1], bq[2], True)
    ref_nv, _ = oracle.gemm_full("NT", M, N, K, (acodes, ascales, 1.0, False), b)
    got, _ = oracle.gemm_w4a16_full(M, N, K, ab16, b)
    assert np.array_equal(got, ref_nv)
