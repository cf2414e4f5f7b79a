"""Pins for the oracle's 16-point random Hadamard transform and NVFP4 GEMM (CPU only).

The recipe paragraph of the readjensen.com NVFP4 training-recipe page puts a
random Hadamard transform on the wgrad inputs and runs the three MLP GEMMs
(fprop, dgrad, wgrad) on NVFP4 inputs with BF16 outputs; "Mastering
Low-Precision AI" (third paragraph) lists Hadamard transforms among the
stabilisers.  The transform is pinned by its closed form
H16[i][j] = (-1)^popcount(i & j); the GEMM by brute force on small inputs.
"""
import numpy as np
import pytest
import torch

import oracle


def hadamard16_closed_form():
    i = np.arange(16)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0)


def signs(mask):
    return np.array([-1.0 if (mask >> i) & 1 else 1.0 for i in range(16)])


@pytest.mark.parametrize("mask", [0x0000, 0xFFFF, 0xA5C3, 0x0001, 0x8000])
def test_rht_one_hot_columns_match_closed_form(mask):
    H = hadamard16_closed_form()
    D = signs(mask)
    eye = np.eye(16, dtype=np.float32)          # row j = unit vector e_j along 16 columns
    T = oracle.rht16(eye, axis=1, mask=mask)    # row j = transform of e_j
    expect = 0.25 * (H * D[None, :]).T          # row j = column j of H D / 4
    assert np.array_equal(T.astype(np.float64), expect)


def test_hadamard_is_orthogonal():
    H = hadamard16_closed_form()
    assert np.array_equal(H @ H.T, 16 * np.eye(16))
    T = oracle.rht16(np.eye(16, dtype=np.float32), axis=1, mask=0x3C5A).astype(np.float64)
    assert np.allclose(T @ T.T, np.eye(16), atol=0, rtol=0)


def test_rht_exact_on_integer_inputs_both_axes():
    rng = np.random.default_rng(0)
    H = hadamard16_closed_form()
    mask = 0x5AA5
    Q = 0.25 * H @ np.diag(signs(mask))
    x = rng.integers(-1000, 1000, size=(48, 64)).astype(np.float32)
    y1 = oracle.rht16(x, axis=1, mask=mask).astype(np.float64)
    ref1 = (x.astype(np.float64).reshape(48, 4, 16) @ Q.T).reshape(48, 64)
    assert np.array_equal(y1, ref1)
    y0 = oracle.rht16(x, axis=0, mask=mask).astype(np.float64)
    ref0 = (Q @ x.astype(np.float64).reshape(3, 16, 64)).reshape(48, 64)
    assert np.array_equal(y0, ref0)
    assert np.array_equal(oracle.rht16(np.ascontiguousarray(x.T), axis=1, mask=mask), y0.T)


def test_rht_preserves_wgrad_products():
    import workloads
    a = workloads.gradients(256, 32, seed=1)   # [tokens, out]
    b = workloads.activations(256, 48, seed=2)  # [tokens, in]
    mask = workloads.sign_mask(1)
    qa = oracle.rht16(workloads.bf16_bits(a), axis=0, mask=mask).astype(np.float64)
    qb = oracle.rht16(workloads.bf16_bits(b), axis=0, mask=mask).astype(np.float64)
    ref = a.double().numpy().T @ b.double().numpy()
    got = qa.T @ qb
    scale = np.abs(a.double().numpy()).T @ np.abs(b.double().numpy())
    assert np.all(np.abs(got - ref) <= 1e-6 * scale)
    # the transform round-trips: Q^T Q x = x (within FP32 rounding)
    H = hadamard16_closed_form()
    Q = 0.25 * H @ np.diag(signs(mask))
    back = (Q.T @ qa.reshape(16, 16, 32)).reshape(256, 32)
    assert np.allclose(back, a.double().numpy(), rtol=0, atol=1e-6 * np.abs(a.double().numpy()).max())


def test_fused_rht_quantize_equals_rht_then_quantize():
    import workloads
    g = workloads.gradients(64, 96, seed=4)
    gb = workloads.bf16_bits(g)
    mask = 0x1234
    y = oracle.rht16(gb, axis=0, mask=mask)
    for sr in (False, True):
        c1, s1, t1, a1 = oracle.quantize(gb, axis=0, rht=True, mask=mask, sr=sr, seed=1,
                                         stream_id=1)
        c2, s2, t2, a2 = oracle.quantize(y, axis=0, sr=sr, seed=1, stream_id=1)
        assert (t1, a1) == (t2, a2)
        assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
        assert a1 == oracle.amax(gb, rht=True, axis=0, mask=mask)


# ------------------------------------------------------------------ GEMM

def _rand_operand(rng, rows, cols, block2d, axis, ts):
    codes = rng.integers(0, 256, size=(rows, cols // 2)).astype(np.uint8)
    if block2d:
        shape = (rows // 16, cols // 16)
    elif axis == 1:
        shape = (rows, cols // 16)
    else:
        shape = (rows // 16, cols)
    scales = rng.integers(0, 0x7F, size=shape).astype(np.uint8)  # finite E4M3 codes
    return codes, scales, ts, block2d, axis


def _dequant64(op, rows, cols):
    codes, scales, ts, block2d, axis = op
    f, _ = oracle.dequantize(codes, scales, ts, rows, cols, block2d=block2d, axis=axis)
    return f.astype(np.float64)


CASES = [  # layout, A block2d, B block2d
    ("NT", False, True), ("NT", False, False), ("NT", True, True),
    ("NN", False, True), ("NN", False, False),
    ("TN", False, False), ("TN", True, False),
]


@pytest.mark.parametrize("layout,a2d,b2d", CASES)
def test_gemm_brute_force_16x16x32(layout, a2d, b2d):
    rng = np.random.default_rng(hash((layout, a2d, b2d)) & 0xFFFF)
    M, N, K = 16, 16, 32
    a_shape = (M, K) if layout in ("NT", "NN") else (K, M)
    b_shape = (N, K) if layout == "NT" else (K, N)
    a_axis = 1 if layout in ("NT", "NN") else 0
    b_axis = 1 if layout == "NT" else 0
    A = _rand_operand(rng, *a_shape, a2d, a_axis, 0.25)   # power-of-two tensor scales
    B = _rand_operand(rng, *b_shape, b2d, b_axis, 2.0)
    ref, ab = oracle.gemm_full(layout, M, N, K, A[:4], B[:4])
    Ad = torch.from_numpy(_dequant64(A, *a_shape))
    Bd = torch.from_numpy(_dequant64(B, *b_shape))
    if layout == "TN":
        Ad = Ad.T
    if layout == "NT":
        Bd = Bd.T
    expect = torch.matmul(Ad.contiguous(), Bd.contiguous()).numpy()
    expect_abs = torch.matmul(Ad.abs().contiguous(), Bd.abs().contiguous()).numpy()
    assert np.allclose(ref, expect, rtol=1e-14, atol=1e-14 * np.abs(expect_abs).max())
    assert np.allclose(ab, expect_abs, rtol=1e-14, atol=0)


def test_gemm_all_ones_gives_k():
    M, N, K = 8, 24, 160
    ones = np.full((M, K // 2), 0x22, dtype=np.uint8)          # code 2 = 1.0
    e_one = 0x38                                               # E4M3 1.0
    A = (ones, np.full((M, K // 16), e_one, np.uint8), 1.0, False)
    B = (np.full((K, N // 2), 0x22, np.uint8), np.full((K // 16, N), e_one, np.uint8), 1.0, False)
    ref, ab = oracle.gemm_full("NN", M, N, K, A, B)
    assert np.all(ref == K) and np.all(ab == K)
    # negative codes flip the sign exactly
    A2 = (np.full((M, K // 2), 0xAA, np.uint8), A[1], 1.0, False)  # code 10 = -1.0
    ref2, _ = oracle.gemm_full("NN", M, N, K, A2, B)
    assert np.all(ref2 == -K)


def _transpose_nvfp4(codes, scales, rows, cols, axis_from):
    """Storage transpose of a 1D NVFP4 tensor: [rows, cols] axis a -> [cols, rows] axis 1-a."""
    q = np.empty((rows, cols), dtype=np.uint8)
    q[:, 0::2] = codes & 0xF
    q[:, 1::2] = codes >> 4
    qt = np.ascontiguousarray(q.T)
    ct = (qt[:, 0::2] | (qt[:, 1::2] << 4)).astype(np.uint8)
    return ct, np.ascontiguousarray(scales.T)


def test_gemm_layouts_agree_on_transposed_storage():
    rng = np.random.default_rng(5)
    M, N, K = 32, 48, 64
    a_codes, a_scales, *_ = _rand_operand(rng, M, K, False, 1, 1.0)
    b_codes, b_scales, *_ = _rand_operand(rng, N, K, False, 1, 0.5)
    nt, _ = oracle.gemm_full("NT", M, N, K, (a_codes, a_scales, 1.0, False),
                             (b_codes, b_scales, 0.5, False))
    bT = _transpose_nvfp4(b_codes, b_scales, N, K, 1)   # [K, N], blocks along K (axis 0)
    nn, _ = oracle.gemm_full("NN", M, N, K, (a_codes, a_scales, 1.0, False), (*bT, 0.5, False))
    aT = _transpose_nvfp4(a_codes, a_scales, M, K, 1)   # [K, M]
    tn, _ = oracle.gemm_full("TN", M, N, K, (*aT, 1.0, False), (*bT, 0.5, False))
    assert np.array_equal(nt, nn) and np.array_equal(nt, tn)
    # a transposed operand is a different GEMM: the check above is not vacuous
    sq = oracle.gemm_full("NT", M, M, K, (a_codes, a_scales, 1.0, False),
                          (a_codes, a_scales, 1.0, False))[0]
    assert np.array_equal(sq, sq.T) and not np.array_equal(nt[:, :M], sq)


def test_gemm_sampled_equals_full():
    rng = np.random.default_rng(6)
    M, N, K = 40, 24, 96
    A = _rand_operand(rng, M, K, False, 1, 0.125)[:4]
    B = _rand_operand(rng, N, K, False, 1, 4.0)[:4]
    full, fab = oracle.gemm_full("NT", M, N, K, A, B)
    ms = rng.integers(0, M, 50)
    ns = rng.integers(0, N, 50)
    ref, ab = oracle.gemm_pairs("NT", M, N, K, A, B, ms, ns)
    assert np.array_equal(ref, full[ms, ns]) and np.array_equal(ab, fab[ms, ns])
