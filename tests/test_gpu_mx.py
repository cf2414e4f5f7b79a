"""GPU parity of the MXFP4 path (quantize, dequantize, NT GEMM on the native
scaled FP4 MFMA) against the oracle, through the C ABI.

MXFP4 is the power-of-two-scaled format the pages set NVFP4 against
("NVFP4: cos'e e come supera FP8 e BF16", section "Cos'e NVFP4"; "FP4",
the comparison with the open standard); block of 32 and E8M0 scale rule of
the OCP MX v1.0 standard.  Quantize and dequantize are bit-exact; the GEMM
is within the FP32-accumulation tolerance of the NVFP4 GEMM tests.
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


def special_blocks(rows, cols, seed):
    """Random blocks plus blocks that hit every branch of the scale rule: zero,
    subnormal amax, huge amax, E2M1 midpoints, tiny negatives (signed zeros),
    amax just below / at powers of two."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((rows, cols)) * np.exp(2 * rng.standard_normal((rows, 1)))).astype(np.float32)
    nb = cols // 32
    for r in range(rows):
        kind = r % 8
        b = rng.integers(0, nb)
        blk = x[r, 32 * b:32 * b + 32]
        if kind == 0:
            blk[:] = 0.0
        elif kind == 1:
            blk[:] = rng.standard_normal(32).astype(np.float32) * np.float32(1e-39)
        elif kind == 2:
            blk[:] = rng.standard_normal(32).astype(np.float32) * np.float32(1e37)
        elif kind == 3:
            blk[:] = np.array([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0] * 4, dtype=np.float32)
            blk[8:16] *= -1
        elif kind == 4:
            blk[:] = -np.abs(rng.standard_normal(32).astype(np.float32)) * np.float32(1e-30)
            blk[0] = 1e3
        elif kind == 5:
            blk[:] = rng.uniform(-1, 1, 32).astype(np.float32)
            blk[3] = np.nextafter(np.float32(8.0), np.float32(0))
        elif kind == 6:
            blk[:] = rng.uniform(-1, 1, 32).astype(np.float32)
            blk[5] = -8.0
    return x


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("rows,cols,pad", [(1, 32, 0), (7, 96, 32), (130, 4096, 0), (64, 1024, 64)])
def test_mx_quantize_bit_exact(nv, dtype, rows, cols, pad):
    x = torch.from_numpy(special_blocks(rows, cols + pad, rows * 31 + cols)).to(dtype)
    xg = x.cuda()[:, :cols]
    print("mx quantize", dtype, rows, cols, pad, flush=True)
    t = nv.mx_quantize(xg)
    torch.cuda.synchronize()
    codes, scales = oracle.mx_quantize(to_oracle_input(x[:, :cols]))
    assert np.array_equal(t.scales.cpu().numpy(), scales)
    assert np.array_equal(t.codes.cpu().numpy(), codes)


def test_mx_quantize_workload_activations(nv):
    x = workloads.activations(512, 4096, 0)
    t = nv.mx_quantize(x.cuda())
    torch.cuda.synchronize()
    codes, scales = oracle.mx_quantize(to_oracle_input(x))
    assert np.array_equal(t.scales.cpu().numpy(), scales)
    assert np.array_equal(t.codes.cpu().numpy(), codes)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_mx_dequantize_bit_exact(nv, out_dtype):
    rng = np.random.default_rng(5)
    rows, cols = 37, 512
    codes = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(0, 255, (rows, cols // 32), dtype=np.uint8)   # all but NaN
    t = nv.MXFP4Tensor(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), rows, cols)
    out = nv.mx_dequantize(t, out_dtype).cpu()
    f, b = oracle.mx_dequantize(codes, scales, rows, cols)
    if out_dtype == torch.float32:
        assert np.array_equal(out.numpy().view(np.uint32), f.view(np.uint32))
    else:
        assert np.array_equal(out.view(torch.int16).numpy().view(np.uint16), b)


def random_mx(rng, rows, cols, lo=118, hi=136):
    codes = rng.integers(0, 256, (rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(lo, hi, (rows, cols // 32), dtype=np.uint8)
    return codes, scales


def to_gpu(nv, codes, scales, rows, cols):
    return nv.MXFP4Tensor(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), rows, cols)


# one, two, three and many k-tiles; ragged M and N on both sides of the 256 tile
MX_SHAPES = [(256, 256, 128), (300, 200, 256), (64, 96, 384), (520, 1000, 1024), (17, 1, 128),
             (256, 512, 2048)]


@pytest.mark.parametrize("M,N,K", MX_SHAPES)
def test_mx_gemm_random_operands(nv, M, N, K):
    rng = np.random.default_rng(M * 3 + N * 7 + K)
    a = random_mx(rng, M, K)
    b = random_mx(rng, N, K)
    print("mx gemm", M, N, K, flush=True)
    ag, bg = to_gpu(nv, *a, M, K), to_gpu(nv, *b, N, K)
    yf_t = nv.mx_gemm(ag, bg, torch.float32).cpu()
    yb_t = nv.mx_gemm(ag, bg, torch.bfloat16).cpu()
    # same accumulators: the BF16 output is the FP32 one rounded to nearest
    # even (torch's CPU float -> bfloat16 conversion is RNE)
    assert torch.equal(yb_t, yf_t.to(torch.bfloat16))
    yf, yb = yf_t.numpy(), yb_t.float().numpy()
    if M * N <= 300 * 300:
        ref, ab = oracle.mx_gemm_full(M, N, K, a, b)
        check_gemm(yf, yb, ref, ab, "mx %dx%dx%d" % (M, N, K))
    else:
        ms = rng.integers(0, M, 3000)
        ns = rng.integers(0, N, 3000)
        ms[:4] = [0, 0, M - 1, M - 1]
        ns[:4] = [0, N - 1, 0, N - 1]
        ref, ab = oracle.mx_gemm_pairs(M, N, K, a, b, ms, ns)
        check_gemm(yf[ms, ns], yb[ms, ns], ref, ab, "mx %dx%dx%d sampled" % (M, N, K))


def test_mx_gemm_quantized_workload(nv):
    """Activations x weights quantized on the GPU, against the oracle on the
    same codes."""
    M, N, K = 384, 640, 1024
    x = workloads.activations(M, K, 0)
    w = workloads.weights(N, K, 2)
    a, b = nv.mx_quantize(x.cuda()), nv.mx_quantize(w.cuda())
    y = nv.mx_gemm(a, b, torch.float32).cpu().numpy()
    ao = (a.codes.cpu().numpy(), a.scales.cpu().numpy())
    bo = (b.codes.cpu().numpy(), b.scales.cpu().numpy())
    assert np.array_equal(ao[1], oracle.mx_quantize(to_oracle_input(x))[1])
    ref, ab = oracle.mx_gemm_full(M, N, K, ao, bo)
    check_gemm(y, None, ref, ab, "mx quantized workload")


def test_mx_gemm_strided_output_and_k_zero(nv):
    rng = np.random.default_rng(9)
    M, N, K = 256, 256, 256
    a, b = random_mx(rng, M, K), random_mx(rng, N, K)
    ag, bg = to_gpu(nv, *a, M, K), to_gpu(nv, *b, N, K)
    buf = torch.full((M, N + 40), -3.0, dtype=torch.float32, device="cuda")
    view = buf[:, 8:8 + N]
    nv.mx_gemm(ag, bg, torch.float32, out=view)
    ref, ab = oracle.mx_gemm_full(M, N, K, a, b)
    check_gemm(view.cpu().numpy(), None, ref, ab, "mx strided")
    outside = torch.cat([buf[:, :8], buf[:, 8 + N:]], dim=1)
    assert torch.all(outside == -3.0)
    z = nv.MXFP4Tensor(torch.empty(M, 0, dtype=torch.uint8, device="cuda"),
                       torch.empty(M, 0, dtype=torch.uint8, device="cuda"), M, 0)
    zb = nv.MXFP4Tensor(torch.empty(N, 0, dtype=torch.uint8, device="cuda"),
                        torch.empty(N, 0, dtype=torch.uint8, device="cuda"), N, 0)
    y = nv.mx_gemm(z, zb, torch.float32)
    assert torch.all(y == 0)


def test_mx_error_larger_than_nvfp4_on_activations(nv):
    """The pages' comparison, measured (not a parity check): the same synthetic
    activations through both quantizers on the GPU; NVFP4's mean squared
    error must be the smaller."""
    x = workloads.activations(1024, 4096, 0).cuda()
    xm = nv.mx_dequantize(nv.mx_quantize(x), torch.float32)
    xn = nv.dequantize(nv.quantize(x), torch.float32)
    xf = x.float()
    mse_mx = ((xm - xf) ** 2).mean().item()
    mse_nv = ((xn - xf) ** 2).mean().item()
    print("mse mx %.4g nvfp4 %.4g ratio %.3f" % (mse_mx, mse_nv, mse_nv / mse_mx))
    assert mse_nv < mse_mx


def _finite_bf16():
    bits = np.arange(1 << 16, dtype=np.uint32)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    return torch.from_numpy(bits[finite].astype(np.int32).astype(np.int16)).view(torch.bfloat16)


@pytest.mark.parametrize("layout", ["maxima", "elements"])
def test_mx_quantize_every_bf16_value(nv, layout):
    """Every finite BF16 value as the maximum of a 32-block of its own
    ("maxima": the block is v and v times 31 fractions in [-1, 1], rounded to
    BF16, so every E8M0 scale the rule can give, zero blocks and denormal
    maxima included), or as an element beside block maxima 2^-126, 1 and
    2^127 ("elements"): codes and scales bit-exact against the oracle."""
    vals = _finite_bf16()
    if layout == "maxima":
        frac = torch.linspace(-1.0, 1.0, 31, dtype=torch.float32)
        x = torch.empty(vals.numel(), 32, dtype=torch.bfloat16)
        x[:, 0] = vals
        x[:, 1:] = (vals.float()[:, None] * frac[None, :]).to(torch.bfloat16)
    else:
        parts = []
        for m in (2.0 ** -126, 1.0, 2.0 ** 127):
            v = vals[vals.float().abs() <= m]
            nb = (v.numel() + 30) // 31
            blk = torch.zeros(nb, 32, dtype=torch.bfloat16)
            blk[:, 0] = m
            body = torch.zeros(nb * 31, dtype=torch.bfloat16)
            body[:v.numel()] = v
            blk[:, 1:] = body.reshape(nb, 31)
            parts.append(blk)
        x = torch.cat(parts)
    rows = (x.shape[0] + 3) // 4
    xx = torch.zeros(rows * 4, 32, dtype=torch.bfloat16)
    xx[:x.shape[0]] = x
    xx = xx.reshape(rows, 128)                 # four blocks per row
    t = nv.mx_quantize(xx.cuda())
    torch.cuda.synchronize()
    codes, scales = oracle.mx_quantize(to_oracle_input(xx))
    assert np.array_equal(t.scales.cpu().numpy(), scales)
    assert np.array_equal(t.codes.cpu().numpy(), codes)
