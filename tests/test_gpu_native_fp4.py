"""GPU parity: nvfp4_gemm_native, the NVFP4 GEMM on the native scaled FP4
matrix instruction where that is exact, against the CPU oracle.

The pages note that CDNA 4's matrix cores run FP4 natively (guiahardware.es,
"NVFP4: cos'e e come supera FP8 e BF16", section "Roadmap e disponibilita").
That instruction scales 32 K-consecutive codes by one power of two, so an
NVFP4 operand maps onto it exactly only when, in every 32-K block of a row,
each 16-element E4M3 scale is a power of two (or zero over all-zero codes)
and the non-zero ones are equal.  Operands built that way must take the
native path (used_native = 1) and match the oracle within the GEMM tolerance;
any block that breaks the rule must send the call to the FP16 path
(used_native = 0), whose output is nvfp4_gemm's bit for bit.  The expected
path comes from a host-side reading of the scale bytes, not from the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import check_gemm

pytestmark = pytest.mark.gpu

# E4M3 bytes that are powers of two: normals E << 3 (E = 1..15, 2^(E-7)) and
# the subnormals 1, 2, 4 (2^-9, 2^-8, 2^-7)
POW2 = np.array([e << 3 for e in range(1, 16)] + [1, 2, 4], dtype=np.uint8)


@pytest.fixture(scope="module")
def nv():
    import nvfp4_bit_microscaled_amd as m
    torch.cuda.set_device(0)
    return m


def gpu_tensor(nv, codes, scales, ts, rows, cols, block2d):
    return nv.NVFP4Tensor(torch.from_numpy(np.ascontiguousarray(codes)).cuda(),
                          torch.from_numpy(np.ascontiguousarray(scales)).cuda(),
                          torch.tensor([ts], dtype=torch.float32, device="cuda"),
                          torch.zeros(1, device="cuda"), rows, cols, block2d, 1)


def native_operand(rng, rows, K, block2d, lo=5, hi=12):
    """Random codes; per (scale row, 32-K block) one power-of-two E4M3 byte
    (from POW2[lo:hi], a spread of 2^-2 .. 2^4 by default) for both 16-blocks;
    some blocks zero-scaled with their codes cleared (one half or both)."""
    codes = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    srows = rows // 16 if block2d else rows
    pair = rng.choice(POW2[lo:hi], size=(srows, K // 32))
    scales = np.repeat(pair, 2, axis=1).astype(np.uint8)
    zero = rng.random((srows, K // 16)) < 0.08
    scales[zero] = 0
    # clear the codes of zero-scaled blocks (every row a 2D scale row covers)
    zrows = np.repeat(zero, 16, axis=0) if block2d else zero
    codes.reshape(rows, K // 16, 8)[zrows] = 0
    return codes, scales


def expect_native(codes, scales, block2d):
    """The rule, read on the host from the bytes."""
    rows = codes.shape[0]
    srows, nb16 = scales.shape
    pow2 = np.isin(scales, POW2)
    zero = scales == 0
    # zero-scaled 16-blocks must have all-zero codes in every row they cover
    blk_codes = codes.reshape(rows, nb16, 8)
    nz = (blk_codes != 0).any(axis=2)
    if block2d:
        nz = nz.reshape(srows, 16, nb16).any(axis=1)
    ok16 = pow2 | (zero & ~nz)
    s0, s1 = scales[:, 0::2], scales[:, 1::2]
    same = (s0 == s1) | (s0 == 0) | (s1 == 0)
    return bool(ok16.all() and same.all())


def run(nv, M, N, K, a, b, a2d, b2d, out_dtype):
    ts_a, ts_b = 0.75, 1.25
    ag = gpu_tensor(nv, a[0], a[1], ts_a, M, K, a2d)
    bg = gpu_tensor(nv, b[0], b[1], ts_b, N, K, b2d)
    out, used = nv.gemm_native(ag, bg, out_dtype=out_dtype)
    ref_path = nv.gemm("NT", ag, bg, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return ag, bg, out, int(used.item()), ref_path, (a[0], a[1], ts_a, a2d), (b[0], b[1], ts_b, b2d)


@pytest.mark.parametrize("M,N,K,a2d,b2d", [
    (256, 256, 256, False, False), (200, 144, 384, False, True), (64, 512, 1024, False, True),
    (300, 260, 128, False, False), (512, 256, 4096, True, True), (17, 33, 640, False, False)])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_native_path_on_pow2_scales(nv, M, N, K, a2d, b2d, out_dtype):
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    a = native_operand(rng, M, K, a2d)
    b = native_operand(rng, N, K, b2d)
    assert expect_native(*a, a2d) and expect_native(*b, b2d)
    print("native", M, N, K, a2d, b2d, out_dtype, flush=True)
    _, _, out, used, fp16_out, a_or, b_or = run(nv, M, N, K, a, b, a2d, b2d, out_dtype)
    assert used == 1
    ref, ab = oracle.gemm_full("NT", M, N, K, a_or, b_or)
    got = out.float().cpu().numpy()
    if out_dtype == torch.float32:
        check_gemm(got, None, ref, ab, "native fp4")
    else:
        check_gemm(None, got, ref, ab, "native fp4")
    # and the FP16 path agrees with it to the same tolerance
    got16 = fp16_out.float().cpu().numpy()
    if out_dtype == torch.float32:
        check_gemm(got16, None, ref, ab, "fp16 path")


def break_one_block(rng, a, kind):
    codes, scales = a[0].copy(), a[1].copy()
    r = rng.integers(0, scales.shape[0])
    j = 2 * rng.integers(0, scales.shape[1] // 2)
    if kind == "not_pow2":
        scales[r, j] = 0x39                       # 1.125 * 2^0
    elif kind == "pair_differs":
        scales[r, j], scales[r, j + 1] = POW2[5], POW2[6]
    elif kind == "zero_scale_nonzero_codes":
        scales[r, j] = 0
        codes[r, 8 * j] = 0x21                    # a non-zero code under a zero scale
    return codes, scales


@pytest.mark.parametrize("kind", ["not_pow2", "pair_differs", "zero_scale_nonzero_codes"])
@pytest.mark.parametrize("operand", ["A", "B"])
def test_fp16_path_when_a_block_breaks_the_rule(nv, kind, operand):
    M, N, K = 192, 320, 512
    rng = np.random.default_rng(hash((kind, operand)) % 1000)
    a = native_operand(rng, M, K, False)
    b = native_operand(rng, N, K, False)
    if operand == "A":
        a = break_one_block(rng, a, kind)
        assert not expect_native(*a, False)
    else:
        b = break_one_block(rng, b, kind)
        assert not expect_native(*b, False)
    print("fallback", kind, operand, flush=True)
    _, _, out, used, fp16_out, a_or, b_or = run(nv, M, N, K, a, b, False, False, torch.float32)
    assert used == 0
    assert torch.equal(out, fp16_out)            # the same FP16 kernel
    ref, ab = oracle.gemm_full("NT", M, N, K, a_or, b_or)
    check_gemm(out.cpu().numpy(), None, ref, ab, "fallback")


def test_random_e4m3_scales_take_the_fp16_path(nv):
    """Quantizer output (E4M3 scales with mantissas) is the common case."""
    rng = np.random.default_rng(3)
    M, N, K = 256, 256, 1024
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy(0.02 * rng.standard_normal((N, K)).astype(np.float32)).to(torch.bfloat16)
    a = nv.quantize(x.cuda())
    b = nv.quantize(w.cuda(), block2d=True)
    out, used = nv.gemm_native(a, b)
    ref = nv.gemm("NT", a, b)
    torch.cuda.synchronize()
    assert int(used.item()) == 0
    assert torch.equal(out, ref)


def test_two_calls_reuse_the_flag(nv):
    """A native call after a fallback call on the same flag (and the reverse)."""
    rng = np.random.default_rng(11)
    M, N, K = 256, 256, 256
    a = native_operand(rng, M, K, False)
    b = native_operand(rng, N, K, False)
    bad = break_one_block(rng, a, "not_pow2")
    flag = torch.zeros(1, dtype=torch.int32, device="cuda")
    bg = gpu_tensor(nv, b[0], b[1], 1.0, N, K, False)
    for codes, scales, want in ((bad[0], bad[1], 0), (a[0], a[1], 1), (bad[0], bad[1], 0)):
        ag = gpu_tensor(nv, codes, scales, 1.0, M, K, False)
        out, used = nv.gemm_native(ag, bg, out_dtype=torch.float32, used_native=flag)
        torch.cuda.synchronize()
        assert int(used.item()) == want
        ref, ab = oracle.gemm_full("NT", M, N, K, (codes, scales, 1.0, False), (b[0], b[1], 1.0, False))
        check_gemm(out.cpu().numpy(), None, ref, ab, "flag reuse")


def test_full_size_sampled(nv):
    """The step's first GEMM shape (32768 x 28672 x 4096) on power-of-two-scaled
    operands (2D weight), sampled outputs against the oracle."""
    M, N, K = 32768, 28672, 4096
    rng = np.random.default_rng(21)
    a = native_operand(rng, M, K, False)
    b = native_operand(rng, N, K, True)
    ag = gpu_tensor(nv, a[0], a[1], 0.5, M, K, False)
    bg = gpu_tensor(nv, b[0], b[1], 0.25, N, K, True)
    out, used = nv.gemm_native(ag, bg)
    torch.cuda.synchronize()
    assert int(used.item()) == 1
    ms = np.concatenate([rng.integers(0, M, 1500), [0, M - 1]]).astype(np.int64)
    ns = np.concatenate([rng.integers(0, N, 1500), [N - 1, 0]]).astype(np.int64)
    ref, ab = oracle.gemm_pairs("NT", M, N, K, (a[0], a[1], 0.5, False), (b[0], b[1], 0.25, True),
                                ms, ns)
    got = out[torch.from_numpy(ms).cuda(), torch.from_numpy(ns).cuda()].float().cpu().numpy()
    check_gemm(None, got, ref, ab, "native fp4 full size")
