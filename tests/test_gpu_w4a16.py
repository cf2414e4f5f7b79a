"""GPU parity of the weight-only decode GEMM (BF16 activations x NVFP4
weights, nvfp4_gemm_w4a16) against the oracle, through the C ABI.

The juejin.cn page on NVFP4 (item 3) has models quantized to NVFP4 for
inference; chaitex.ru "FP4" (item 1) quantizes the weight matrix in
16-element blocks.  Tolerance as for the NVFP4 GEMM: FP32 within 1e-5 of
sum |a b|, BF16 within one BF16 step of the rounded reference.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import check_gemm, to_oracle_input

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import nvfp4_bit_microscaled_amd as m
    return m


# M <= 16, 17..32, 33..64 (the three kernel instances); ragged N (partial
# last workgroup of 64 columns); one, an odd and an even number of 512-K chunks
SHAPES = [(1, 64, 512, False), (5, 100, 1536, True), (16, 1000, 2048, False),
          (17, 200, 1024, True), (32, 77, 2560, False), (33, 130, 512, False),
          (64, 96, 4096, True), (24, 64, 512, False), (40, 64, 1536, True),
          (63, 200, 2560, False)]


@pytest.mark.parametrize("M,N,K,b2d", SHAPES)
def test_w4a16_random(nv, M, N, K, b2d):
    rng = np.random.default_rng(M * 100 + N + K)
    if b2d:
        N = (N + 15) // 16 * 16
    a = torch.from_numpy((rng.standard_normal((M, K)) * np.exp(rng.standard_normal((M, 1))))
                         .astype(np.float32)).to(torch.bfloat16)
    w = workloads.weights(N, K, 7 + M)
    print("w4a16", M, N, K, b2d, flush=True)
    wq = nv.quantize(w.cuda(), block2d=b2d)
    yf = nv.gemm_w4a16(a.cuda(), wq, torch.float32).cpu().numpy()
    yb = nv.gemm_w4a16(a.cuda(), wq, torch.bfloat16).float().cpu().numpy()
    b = (wq.codes.cpu().numpy(), wq.scales.cpu().numpy(), float(wq.tensor_scale.item()), b2d)
    ref, ab = oracle.gemm_w4a16_full(M, N, K, to_oracle_input(a), b)
    check_gemm(yf, yb, ref, ab, "w4a16 %dx%dx%d" % (M, N, K))


def test_w4a16_strided_activations_and_output(nv):
    rng = np.random.default_rng(4)
    M, N, K = 9, 256, 1024
    abig = torch.from_numpy(rng.standard_normal((M, K + 64)).astype(np.float32)).to(torch.bfloat16)
    a = abig.cuda()[:, 32:32 + K]
    wq = nv.quantize(workloads.weights(N, K, 3).cuda(), block2d=True)
    buf = torch.full((M, N + 8), -3.0, dtype=torch.float32, device="cuda")
    out = buf[:, 8:]
    nv.gemm_w4a16(a, wq, torch.float32, out=out)
    b = (wq.codes.cpu().numpy(), wq.scales.cpu().numpy(), float(wq.tensor_scale.item()), True)
    ref, ab = oracle.gemm_w4a16_full(M, N, K, to_oracle_input(abig[:, 32:32 + K]), b)
    check_gemm(out.cpu().numpy(), None, ref, ab, "w4a16 strided")
    assert torch.all(buf[:, :8] == -3.0)


@pytest.mark.parametrize("M", [1, 16, 64])
def test_w4a16_decode_fullsize_sampled(nv, M):
    """Decode shape: activations [M, 8192] BF16, weights [28672, 8192] 1x16."""
    K, N = workloads.DECODE["k"], workloads.DECODE["n"]
    a = workloads.activations(M, K, workloads.DECODE["act_seed"])
    wq = nv.quantize(workloads.weights(N, K, workloads.DECODE["w_seed"], device="cuda"))
    y = nv.gemm_w4a16(a.cuda(), wq, torch.float32).cpu().numpy()
    rng = np.random.default_rng(M)
    ns = np.concatenate([[0, N - 1], rng.integers(0, N, 2000)])
    ms = rng.integers(0, M, len(ns))
    b = (wq.codes.cpu().numpy(), wq.scales.cpu().numpy(), float(wq.tensor_scale.item()), False)
    ref, ab = oracle.gemm_w4a16_pairs(M, N, K, to_oracle_input(a), b, ms, ns)
    check_gemm(y[ms, ns], None, ref, ab, "w4a16 decode M=%d" % M)
