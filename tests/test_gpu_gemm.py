"""GPU parity: nvfp4_gemm (NT fprop, NN dgrad, TN wgrad) against the CPU oracle.

Operands are quantized by the oracle (or drawn as random codes) on the CPU and
copied to the GPU, so no expected value depends on the HIP path.  Tolerance
(FP32 accumulation order is not fixed by the method): |C - ref| <= 1e-5 S with
S = s_A s_B sum_k |a_k b_k|, then BF16 within one ulp of RNE_bf16(ref).
Source: the three MLP GEMMs on NVFP4 inputs with BF16 outputs, readjensen.com
NVFP4 training-recipe page, recipe paragraph.
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
    torch.cuda.set_device(0)
    return m


def to_gpu_tensor(nv, codes, scales, ts, rows, cols, block2d, axis):
    return nv.NVFP4Tensor(torch.from_numpy(np.ascontiguousarray(codes)).cuda(),
                          torch.from_numpy(np.ascontiguousarray(scales)).cuda(),
                          torch.tensor([ts], dtype=torch.float32, device="cuda"),
                          torch.zeros(1, device="cuda"), rows, cols, block2d, axis)


def oracle_operand(nv, x, block2d, axis, **kw):
    rows, cols = x.shape
    c, s, ts, _ = oracle.quantize(to_oracle_input(x), block2d=block2d, axis=axis, **kw)
    return (c, s, ts, block2d), to_gpu_tensor(nv, c, s, ts, rows, cols, block2d, axis)


def random_operand(nv, rng, rows, cols, block2d, axis, ts, scale_lo=0x00):
    c = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    shape = nv.scale_shape(rows, cols, block2d, axis)
    s = rng.integers(scale_lo, 0x7F, size=shape, dtype=np.uint8)   # finite E4M3 codes
    return (c, s, ts, block2d), to_gpu_tensor(nv, c, s, ts, rows, cols, block2d, axis)


def run_and_check(nv, layout, M, N, K, a_or, a_gpu, b_or, b_gpu, pairs=None):
    yf = nv.gemm(layout, a_gpu, b_gpu, out_dtype=torch.float32)
    yb = nv.gemm(layout, a_gpu, b_gpu, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    # same accumulators and scale: the BF16 output is the FP32 one rounded to
    # nearest even (torch's CPU float -> bfloat16 conversion is RNE)
    assert torch.equal(yb.cpu(), yf.cpu().to(torch.bfloat16))
    if pairs is None:
        ref, ab = oracle.gemm_full(layout, M, N, K, a_or, b_or)
        check_gemm(yf.cpu().numpy(), yb.float().cpu().numpy(), ref, ab, layout)
    else:
        ms, ns = pairs
        ref, ab = oracle.gemm_pairs(layout, M, N, K, a_or, b_or, ms, ns)
        mt, nt = torch.from_numpy(ms).cuda(), torch.from_numpy(ns).cuda()
        check_gemm(yf[mt, nt].cpu().numpy(), yb[mt, nt].float().cpu().numpy(), ref, ab, layout)
    return yf


def test_tiny_config_fprop(nv):
    cfg = workloads.TINY
    M, N, K = cfg["gemm"]
    x = workloads.activations(*cfg["act"], seed=cfg["act_seed"])[:M]
    w = workloads.weights(*cfg["w"], seed=cfg["w_seed"])
    a_or, a_g = oracle_operand(nv, x, False, 1)
    b_or, b_g = oracle_operand(nv, w, True, 1)
    run_and_check(nv, "NT", M, N, K, a_or, a_g, b_or, b_g)


# (layout, M, N, K): ragged M/N tails and a K tail that is not a multiple of 64
SHAPES = [("NT", 200, 136, 272), ("NT", 256, 384, 512), ("NT", 1, 64, 16), ("NT", 33, 17, 48),
          ("NN", 200, 144, 272), ("NN", 256, 384, 512), ("NN", 7, 16, 32),
          ("TN", 208, 144, 272), ("TN", 256, 384, 512), ("TN", 16, 16, 16)]


@pytest.mark.parametrize("layout,M,N,K", SHAPES)
def test_quantized_operands(nv, layout, M, N, K):
    # fprop: X [M,K] 1D x W [N,K] 2D; dgrad: dY [M,K] 1D SR x W [K,N] 2D;
    # wgrad: dY [K,M] colwise RHT+SR x X [K,N] colwise RHT (same mask)
    mask = workloads.sign_mask(1)
    if layout == "NT":
        a_or, a_g = oracle_operand(nv, workloads.activations(M, K, seed=1), False, 1)
        b2d = N % 16 == 0
        b_or, b_g = oracle_operand(nv, workloads.weights(N, K, seed=2), b2d, 1)
    elif layout == "NN":
        a_or, a_g = oracle_operand(nv, workloads.gradients(M, K, seed=3), False, 1, sr=True, seed=1)
        b_or, b_g = oracle_operand(nv, workloads.weights(K, N, seed=4), True, 1)
    else:
        a_or, a_g = oracle_operand(nv, workloads.gradients(K, M, seed=5), False, 0, sr=True,
                                   seed=1, stream_id=1, rht=True, mask=mask)
        b_or, b_g = oracle_operand(nv, workloads.activations(K, N, seed=6), False, 0, rht=True,
                                   mask=mask)
    run_and_check(nv, layout, M, N, K, a_or, a_g, b_or, b_g)


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
@pytest.mark.parametrize("a2d,b2d", [(False, False), (True, True), (False, True), (True, False)])
def test_random_codes_all_block_modes(nv, layout, a2d, b2d):
    rng = np.random.default_rng(hash((layout, a2d, b2d)) & 0xFFFF)
    M, N, K = 160, 96, 320
    a_shape = (M, K) if layout != "TN" else (K, M)
    b_shape = (N, K) if layout == "NT" else (K, N)
    a_axis = 1 if layout != "TN" else 0
    b_axis = 1 if layout == "NT" else 0
    a_or, a_g = random_operand(nv, rng, *a_shape, a2d, a_axis, 0.75)
    b_or, b_g = random_operand(nv, rng, *b_shape, b2d, b_axis, 1.5)
    run_and_check(nv, layout, M, N, K, a_or, a_g, b_or, b_g)


def test_layouts_agree_on_transposed_operands(nv):
    rng = np.random.default_rng(3)
    M, N, K = 128, 64, 256
    a_or, a_g = random_operand(nv, rng, M, K, False, 1, 1.0, scale_lo=0x30)
    b_or, b_g = random_operand(nv, rng, N, K, False, 1, 1.0, scale_lo=0x30)
    y_nt = nv.gemm("NT", a_g, b_g, out_dtype=torch.float32)
    # the same values stored [K, N] with blocks along K (axis 0)
    def transpose(codes, scales, rows, cols):
        q = np.empty((rows, cols), dtype=np.uint8)
        q[:, 0::2] = codes & 0xF
        q[:, 1::2] = codes >> 4
        qt = np.ascontiguousarray(q.T)
        return (qt[:, 0::2] | (qt[:, 1::2] << 4)).astype(np.uint8), np.ascontiguousarray(scales.T)
    bc, bs = transpose(b_or[0], b_or[1], N, K)
    ac, as_ = transpose(a_or[0], a_or[1], M, K)
    bT = to_gpu_tensor(nv, bc, bs, 1.0, K, N, False, 0)
    aT = to_gpu_tensor(nv, ac, as_, 1.0, K, M, False, 0)
    y_nn = nv.gemm("NN", a_g, bT, out_dtype=torch.float32)
    y_tn = nv.gemm("TN", aT, bT, out_dtype=torch.float32)
    torch.cuda.synchronize()
    ref, ab = oracle.gemm_full("NT", M, N, K, a_or, b_or)
    for y in (y_nt, y_nn, y_tn):
        check_gemm(y.cpu().numpy(), None, ref, ab, "transposed storage")


def test_k_zero_and_ones(nv):
    a = nv.NVFP4Tensor(torch.empty(32, 0, dtype=torch.uint8, device="cuda"),
                       torch.empty(32, 0, dtype=torch.uint8, device="cuda"),
                       torch.ones(1, device="cuda"), torch.zeros(1, device="cuda"), 32, 0, False, 1)
    b = nv.NVFP4Tensor(torch.empty(48, 0, dtype=torch.uint8, device="cuda"),
                       torch.empty(48, 0, dtype=torch.uint8, device="cuda"),
                       torch.ones(1, device="cuda"), torch.zeros(1, device="cuda"), 48, 0, False, 1)
    y = torch.full((32, 48), 7.0, device="cuda")
    nv.gemm("NT", a, b, out=y)
    torch.cuda.synchronize()
    assert torch.count_nonzero(y).item() == 0
    # all codes 1.0, all scales 1.0, s = 1: C = K exactly
    K = 4096
    ones = lambda r, c: nv.NVFP4Tensor(torch.full((r, c // 2), 0x22, dtype=torch.uint8, device="cuda"),
                                       torch.full((r, c // 16), 0x38, dtype=torch.uint8, device="cuda"),
                                       torch.ones(1, device="cuda"), torch.zeros(1, device="cuda"),
                                       r, c, False, 1)
    y = nv.gemm("NT", ones(64, K), ones(80, K), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.all(y == K)


@pytest.mark.parametrize("layout", ["NT", "NN", "TN"])
@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("pad,offset", [(2, 0), (4, 1), (0, 0)])
def test_full_tiles_strided_output(nv, layout, out_dtype, pad, offset):
    """Full 256 x 256 tiles written into a row-padded / offset view of a larger
    buffer: the results match the oracle and nothing outside the view changes
    (with a row stride that is not a multiple of 4, or a start that is not
    4-element aligned, the kernel must fall back to element stores)."""
    rng = np.random.default_rng(11 + pad + 7 * offset)
    M, N, K = 256, 512, 384
    a_shape = (M, K) if layout != "TN" else (K, M)
    b_shape = (N, K) if layout == "NT" else (K, N)
    a_axis = 1 if layout != "TN" else 0
    b_axis = 1 if layout == "NT" else 0
    a_or, a_g = random_operand(nv, rng, *a_shape, False, a_axis, 0.5, scale_lo=0x30)
    b_or, b_g = random_operand(nv, rng, *b_shape, layout == "NT", b_axis, 0.25, scale_lo=0x30)
    buf = torch.full((M, N + pad + offset), -3.0, dtype=out_dtype, device="cuda")
    view = buf[:, offset:offset + N]
    nv.gemm(layout, a_g, b_g, out=view)
    torch.cuda.synchronize()
    ref, ab = oracle.gemm_full(layout, M, N, K, a_or, b_or)
    got = view.float().cpu().numpy()
    if out_dtype == torch.float32:
        check_gemm(got, None, ref, ab, "strided fp32")
    else:
        yf = nv.gemm(layout, a_g, b_g, out_dtype=torch.float32)
        torch.cuda.synchronize()
        check_gemm(yf.cpu().numpy(), got, ref, ab, "strided bf16")
        assert torch.equal(view.cpu(), yf.cpu().to(torch.bfloat16))
    outside = torch.cat([buf[:, :offset], buf[:, offset + N:]], dim=1)
    assert torch.all(outside == -3.0)


# K-major x K-major with K % 128 == 0: the direct-to-LDS three-stage kernel.
# One, two, three and many k-tiles (prologue-only, ring start, ring wrap),
# ragged M and N on both sides of the 256 tile, every block-mode pair.
KK_SHAPES = [(256, 256, 128), (272, 208, 256), (80, 528, 384), (512, 256, 1152), (784, 96, 640)]


@pytest.mark.parametrize("M,N,K", KK_SHAPES)
@pytest.mark.parametrize("a2d,b2d", [(False, False), (False, True), (True, True), (True, False)])
def test_nt_kmajor_kernel(nv, M, N, K, a2d, b2d):
    rng = np.random.default_rng(M * 7 + N * 3 + K + 2 * a2d + b2d)
    a_or, a_g = random_operand(nv, rng, M, K, a2d, 1, 0.375)
    b_or, b_g = random_operand(nv, rng, N, K, b2d, 1, 1.25)
    run_and_check(nv, "NT", M, N, K, a_or, a_g, b_or, b_g)


def test_nt_kmajor_odd_rows(nv):
    """M and N not multiples of 16 (1D blocks only): clamped row loads."""
    rng = np.random.default_rng(5)
    M, N, K = 301, 77, 256
    a_or, a_g = random_operand(nv, rng, M, K, False, 1, 0.5)
    b_or, b_g = random_operand(nv, rng, N, K, False, 1, 0.5)
    run_and_check(nv, "NT", M, N, K, a_or, a_g, b_or, b_g)


# decode-style NT shapes (M <= 64, K a multiple of the kernel's 512 K chunk):
# the skinny kernel, with M and N ragged and one, an odd number and an even
# number of chunks (its chunk loop runs in pairs)
SKINNY = [(1, 64, 2048, False), (5, 100, 4096, True), (16, 1000, 2048, False),
          (17, 200, 1024, True), (32, 77, 3072, False), (33, 130, 1536, False),
          (64, 96, 512, True), (64, 64, 8192, False), (1, 300, 2560, False),
          (7, 48, 512, True), (12, 4200, 1536, False)]


@pytest.mark.parametrize("M,N,K,b2d", SKINNY)
def test_skinny_decode_kernel(nv, M, N, K, b2d):
    rng = np.random.default_rng(M * 1000 + N + K)
    if b2d:
        N = (N + 15) // 16 * 16
    a_or, a_g = random_operand(nv, rng, M, K, False, 1, 0.5)
    b_or, b_g = random_operand(nv, rng, N, K, b2d, 1, 0.75)
    run_and_check(nv, "NT", M, N, K, a_or, a_g, b_or, b_g)
