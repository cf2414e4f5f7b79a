"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

The oracle cannot redo a whole 32768 x 28672 tensor quickly, so these tests
compare: the tensor amax and scale (full pass), and codes/scales on sampled
row slices (first, middle and last rows) quantized by the oracle with the
same amax and global row offset; GEMMs on the four corner 128 x 128 output
tiles plus 4096 seeded random outputs, each a full-K FP64 dot product.

Workloads: Llama-3-8B MLP at 32768 tokens (fprop and backward, in the NN/TN
storage layouts and in the all-K-major configuration the training step
times), decode-style
GEMMs (M in {1, 16, 32, 64}, K 8192, N 28672) and one GPU's token share of
a Llama-3.1-405B MLP (8192 tokens, hidden 16384, intermediate 53248).  The
token count follows the benchmark paragraph of the readjensen.com NVFP4
training-recipe page; the recipe (2D weights, RHT + SR on wgrad inputs, SR on
gradients) follows its recipe paragraph.
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
    oracle.set_num_threads(16)
    return m


def gen(kind, rows, cols, seed):
    f = {"act": workloads.activations, "w": workloads.weights, "grad": workloads.gradients}[kind]
    return f(rows, cols, seed=seed, device="cuda")


def sample_slices(rows, step=16):
    mid = (rows // 2) // step * step
    return [(0, 64), (mid, mid + 64), (rows - 64, rows)]


def transpose_codes(codes):
    q = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    q[:, 0::2] = codes & 0xF
    q[:, 1::2] = codes >> 4
    qt = np.ascontiguousarray(q.T)
    return (qt[:, 0::2] | (qt[:, 1::2] << 4)).astype(np.uint8)


def check_quantize_sampled(nv, x, block2d=False, axis=1, sr=False, seed=0, stream_id=0,
                           rht=False, mask=0, transpose=False, via_transpose=False):
    """via_transpose: quantize in x's own storage, then nvfp4_transpose (the
    training step's path for the 16x16 dgrad weight); the result is checked
    as the transposed-storage quantization."""
    rows, cols = x.shape
    print("quantize %dx%d 2d=%d axis=%d sr=%d rht=%d transpose=%d via=%d" % (
        rows, cols, block2d, axis, sr, rht, transpose, via_transpose), flush=True)
    q = nv.quantize(x, block2d=block2d, axis=axis, sr=sr, seed=seed, stream_id=stream_id,
                    rht=rht, mask=mask, transpose=transpose and not via_transpose)
    if via_transpose:
        q = nv.transpose(q)
        transpose = True
    torch.cuda.synchronize()
    xc = x.cpu()
    xo = to_oracle_input(xc)
    am = oracle.amax(xo, rht=rht, axis=axis, mask=mask)
    assert q.amax.item() == am
    assert q.tensor_scale.item() == np.float32(am) / np.float32(2688.0)
    gc = q.codes.cpu().numpy()
    gs = q.scales.cpu().numpy()
    for r0, r1 in sample_slices(rows):
        c, s, ts, _ = oracle.quantize(np.ascontiguousarray(xo[r0:r1]), block2d=block2d, axis=axis,
                                      sr=sr, seed=seed, stream_id=stream_id, rht=rht, mask=mask,
                                      row0=r0, amax_in=am)
        assert ts == q.tensor_scale.item()
        if transpose:  # the stored tensor is x^T: rows r0..r1 of x are its columns
            assert np.array_equal(transpose_codes(c), gc[:, r0 // 2:r1 // 2]), \
                "transposed codes differ for rows %d..%d" % (r0, r1)
            assert np.array_equal(np.ascontiguousarray(s.T), gs[:, r0 // 16:r1 // 16])
            continue
        assert np.array_equal(c, gc[r0:r1]), "codes differ in rows %d..%d" % (r0, r1)
        if block2d or axis == 0:
            assert np.array_equal(s, gs[r0 // 16:r1 // 16])
        else:
            assert np.array_equal(s, gs[r0:r1])
    del q


L8 = workloads.LLAMA8B


def test_llama8b_fprop_quantize(nv):
    T, D, F = L8["tokens"], L8["hidden"], L8["ffn"]
    check_quantize_sampled(nv, gen("act", T, D, L8["x_seed"]))                    # X, 1x16 RNE
    check_quantize_sampled(nv, gen("w", 2 * F, D, L8["wgu_seed"]), block2d=True)  # W_gu 16x16
    check_quantize_sampled(nv, gen("w", D, F, L8["wdown_seed"]), block2d=True)    # W_down 16x16
    check_quantize_sampled(nv, gen("act", T, F, 13))                              # Act shape


def test_llama8b_backward_quantize(nv):
    T, D, F = L8["tokens"], L8["hidden"], L8["ffn"]
    mask = workloads.sign_mask(L8["mask_seed"])
    sr = L8["sr_seed"]
    dY = gen("grad", T, D, L8["dy_seed"])
    check_quantize_sampled(nv, dY, sr=True, seed=sr, stream_id=0)
    check_quantize_sampled(nv, dY, axis=0, rht=True, mask=mask, sr=True, seed=sr, stream_id=1)
    del dY
    X = gen("act", T, D, L8["x_seed"])
    check_quantize_sampled(nv, X, axis=0, rht=True, mask=mask)
    del X


def test_llama8b_transposed_quantize(nv):
    """The K-major operands of dgrad (W^T, 16x16) and wgrad (dY^T with RHT + SR,
    X^T with RHT) as the training step quantizes them."""
    T, D, F = L8["tokens"], L8["hidden"], L8["ffn"]
    mask = workloads.sign_mask(L8["mask_seed"])
    check_quantize_sampled(nv, gen("w", 2 * F, D, L8["wgu_seed"]), block2d=True, transpose=True)
    check_quantize_sampled(nv, gen("w", D, F, L8["wdown_seed"]), block2d=True, transpose=True)
    dY = gen("grad", T, D, L8["dy_seed"])
    check_quantize_sampled(nv, dY, axis=0, rht=True, mask=mask, sr=True, seed=L8["sr_seed"],
                           stream_id=1, transpose=True)
    del dY
    check_quantize_sampled(nv, gen("act", T, D, L8["x_seed"]), axis=0, rht=True, mask=mask,
                           transpose=True)


def test_llama8b_dh_quantize(nv):
    T, F = L8["tokens"], L8["ffn"]
    mask = workloads.sign_mask(L8["mask_seed"])
    dH = gen("grad", T, 2 * F, L8["dh_seed"])
    check_quantize_sampled(nv, dH, sr=True, seed=L8["sr_seed"], stream_id=0)
    check_quantize_sampled(nv, dH, axis=0, rht=True, mask=mask, sr=True, seed=L8["sr_seed"],
                           stream_id=1)


# ----------------------------------------------------------------- GEMMs

def random_nvfp4(nv, rng, rows, cols, block2d, axis, ts):
    """Valid NVFP4 operand with random codes and scale codes in [2^-3, 448]."""
    c = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    s = rng.integers(0x30, 0x7F, size=nv.scale_shape(rows, cols, block2d, axis), dtype=np.uint8)
    g = nv.NVFP4Tensor(torch.from_numpy(c).cuda(), torch.from_numpy(s).cuda(),
                       torch.tensor([ts], dtype=torch.float32, device="cuda"),
                       torch.zeros(1, device="cuda"), rows, cols, block2d, axis)
    return (c, s, ts, block2d), g


def sampled_pairs(M, N, seed, t=128):
    rng = np.random.default_rng(seed)
    ms, ns = [], []
    for (r0, c0) in [(0, 0), (0, N - t), (M - t, 0), (M - t, N - t)]:
        r0, c0 = max(r0, 0), max(c0, 0)
        mm, nn = np.meshgrid(np.arange(r0, min(r0 + t, M)), np.arange(c0, min(c0 + t, N)),
                             indexing="ij")
        ms.append(mm.ravel()); ns.append(nn.ravel())
    ms.append(rng.integers(0, M, 4096)); ns.append(rng.integers(0, N, 4096))
    return np.concatenate(ms).astype(np.int64), np.concatenate(ns).astype(np.int64)


def run_gemm_sampled(nv, layout, M, N, K, seed, a2d=False, b2d=False):
    rng = np.random.default_rng(seed)
    a_shape = (M, K) if layout != "TN" else (K, M)
    b_shape = (N, K) if layout == "NT" else (K, N)
    a_axis = 1 if layout != "TN" else 0
    b_axis = 1 if layout == "NT" else 0
    a_or, a_g = random_nvfp4(nv, rng, *a_shape, a2d, a_axis, 2.0 ** -6)
    b_or, b_g = random_nvfp4(nv, rng, *b_shape, b2d, b_axis, 2.0 ** -7)
    # corner tiles shrink for the longest K so the FP64 reference stays quick
    ms, ns = sampled_pairs(M, N, seed, t=128 if K <= 32768 else 64)
    mt, nt = torch.from_numpy(ms).cuda(), torch.from_numpy(ns).cuda()
    yb = nv.gemm(layout, a_g, b_g, out_dtype=torch.bfloat16)
    gb = yb[mt, nt].float().cpu().numpy()
    del yb
    yf = nv.gemm(layout, a_g, b_g, out_dtype=torch.float32)
    gf = yf[mt, nt].cpu().numpy()
    del yf, a_g, b_g
    torch.cuda.synchronize()
    ref, ab = oracle.gemm_pairs(layout, M, N, K, a_or, b_or, ms, ns)
    check_gemm(gf, gb, ref, ab, "%s %dx%dx%d" % (layout, M, N, K))


T8, D8, F8 = L8["tokens"], L8["hidden"], L8["ffn"]
LLAMA8B_GEMMS = [
    ("NT", T8, 2 * F8, D8, False, True),    # fprop gate+up
    ("NT", T8, D8, F8, False, True),        # fprop down
    ("NN", T8, F8, D8, False, True),        # dgrad down
    ("NN", T8, D8, 2 * F8, False, True),    # dgrad gate+up
    ("TN", D8, F8, T8, False, False),       # wgrad down
    ("TN", 2 * F8, D8, T8, False, False),   # wgrad gate+up
]


# the launch configuration of the training step: every GEMM K-major x K-major,
# the dgrad weights 16x16 blocks stored transposed
LLAMA8B_GEMMS += [
    ("NT", T8, F8, D8, False, True),        # dgrad down, W_down^T
    ("NT", T8, D8, 2 * F8, False, True),    # dgrad gate+up, W_gu^T
    ("NT", D8, F8, T8, False, False),       # wgrad down, dY^T x Act^T
    ("NT", 2 * F8, D8, T8, False, False),   # wgrad gate+up, dH^T x X^T
]


@pytest.mark.parametrize("layout,M,N,K,a2d,b2d", LLAMA8B_GEMMS)
def test_llama8b_gemms_sampled(nv, layout, M, N, K, a2d, b2d):
    run_gemm_sampled(nv, layout, M, N, K, seed=M ^ N ^ K, a2d=a2d, b2d=b2d)


L405 = workloads.LLAMA405B
T4, D4, F4 = L405["tokens"], L405["hidden"], L405["ffn"]
LLAMA405B_GEMMS = [
    ("NT", T4, 2 * F4, D4, False, True),
    ("NT", T4, D4, F4, False, True),
    ("NN", T4, F4, D4, False, True),
    ("NN", T4, D4, 2 * F4, False, True),
    ("TN", D4, F4, T4, False, False),
    ("TN", 2 * F4, D4, T4, False, False),
]


# the K-major launches of the 405B-share step: dgrad against the transposed
# 16x16 weights, wgrad on the transposed 1D (RHT) gradient and input
LLAMA405B_GEMMS += [
    ("NT", T4, F4, D4, False, True),        # dgrad down, W_down^T  (K = 16384)
    ("NT", T4, D4, 2 * F4, False, True),    # dgrad gate+up, W_gu^T (K = 106496)
    ("NT", D4, F4, T4, False, False),       # wgrad down, dY^T x Act^T (K = 8192)
    ("NT", 2 * F4, D4, T4, False, False),   # wgrad gate+up, dH^T x X^T (K = 8192)
]


@pytest.mark.parametrize("layout,M,N,K,a2d,b2d", LLAMA405B_GEMMS)
def test_llama405b_gemms_sampled(nv, layout, M, N, K, a2d, b2d):
    run_gemm_sampled(nv, layout, M, N, K, seed=(M ^ N ^ K) + 1, a2d=a2d, b2d=b2d)


def test_llama405b_quantize(nv):
    T, D, F = T4, D4, F4
    mask = workloads.sign_mask(L405["mask_seed"])
    X = gen("act", T, D, L405["x_seed"])
    check_quantize_sampled(nv, X)
    check_quantize_sampled(nv, X, axis=0, rht=True, mask=mask, transpose=True)        # X^T
    del X
    dY = gen("grad", T, D, L405["dy_seed"])
    check_quantize_sampled(nv, dY, sr=True, seed=L405["sr_seed"])
    check_quantize_sampled(nv, dY, axis=0, rht=True, mask=mask, sr=True, seed=L405["sr_seed"],
                           stream_id=1)
    check_quantize_sampled(nv, dY, axis=0, rht=True, mask=mask, sr=True, seed=L405["sr_seed"],
                           stream_id=1, transpose=True)                              # dY^T


def test_llama405b_weights(nv):
    """W_down and W_gu (106496 x 16384, the largest tensor of any workload) in
    16x16 blocks, and their K-major dgrad copies W^T from nvfp4_transpose."""
    D, F = D4, F4
    W = gen("w", D, F, L405["wdown_seed"])
    check_quantize_sampled(nv, W, block2d=True)
    check_quantize_sampled(nv, W, block2d=True, via_transpose=True)
    del W
    W = gen("w", 2 * F, D, L405["wgu_seed"])
    check_quantize_sampled(nv, W, block2d=True)
    check_quantize_sampled(nv, W, block2d=True, via_transpose=True)
    del W


def test_llama405b_dh_and_act(nv):
    """dH [8192, 106496]: rows with SR (dgrad) and RHT + SR down the columns in
    transposed storage (wgrad); Act [8192, 53248] (activation-distributed
    stand-in): rows RNE (fprop) and RHT down the columns, transposed (wgrad)."""
    T, F = T4, F4
    mask = workloads.sign_mask(L405["mask_seed"])
    dH = gen("grad", T, 2 * F, L405["dh_seed"])
    check_quantize_sampled(nv, dH, sr=True, seed=L405["sr_seed"], stream_id=0)
    check_quantize_sampled(nv, dH, axis=0, rht=True, mask=mask, sr=True, seed=L405["sr_seed"],
                           stream_id=1, transpose=True)
    del dH
    Act = gen("act", T, F, 14)
    check_quantize_sampled(nv, Act)
    check_quantize_sampled(nv, Act, axis=0, rht=True, mask=mask, transpose=True)
    del Act


def positive_nvfp4(nv, rng, rows, cols, ts, scale_lo, scale_hi):
    """Operand whose every element is positive (codes 1..7: 0.5 .. 6) with
    scales drawn from [scale_lo, scale_hi]: a constant-sign dot product, where
    FP32 accumulation errors do not cancel."""
    c = (rng.integers(1, 8, size=(rows, cols // 2), dtype=np.uint8)
         | (rng.integers(1, 8, size=(rows, cols // 2), dtype=np.uint8) << 4)).astype(np.uint8)
    s = rng.integers(scale_lo, scale_hi + 1, size=(rows, cols // 16), dtype=np.uint8)
    g = nv.NVFP4Tensor(torch.from_numpy(c).cuda(), torch.from_numpy(s).cuda(),
                       torch.tensor([ts], dtype=torch.float32, device="cuda"),
                       torch.zeros(1, device="cuda"), rows, cols, False, 1)
    return (c, s, ts, False), g


# the step's longest K (405B dgrad gate+up) and the 8B wgrad K; a narrow scale
# band (E4M3 1.0 .. 2.0: similar-sized terms) and the full normal range
@pytest.mark.parametrize("M,N,K", [(160, 96, 106496), (128, 96, 53248), (256, 256, 32768)])
@pytest.mark.parametrize("band", [(0x38, 0x40), (0x08, 0x7E)])
def test_constant_sign_long_k(nv, M, N, K, band):
    rng = np.random.default_rng(K + band[0])
    a_or, a_g = positive_nvfp4(nv, rng, M, K, 2.0 ** -6, *band)
    b_or, b_g = positive_nvfp4(nv, rng, N, K, 2.0 ** -5, *band)
    print("constant sign %dx%dx%d band %s" % (M, N, K, band), flush=True)
    yf = nv.gemm("NT", a_g, b_g, out_dtype=torch.float32)
    yb = nv.gemm("NT", a_g, b_g, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    ref, ab = oracle.gemm_full("NT", M, N, K, a_or, b_or)
    assert np.all(ref > 0) and np.array_equal(ref, ab)
    check_gemm(yf.cpu().numpy(), yb.float().cpu().numpy(), ref, ab, "constant sign K=%d" % K)


DEC = workloads.DECODE


@pytest.mark.parametrize("M", list(DEC["ms"]))
def test_decode_gemm(nv, M):
    """Activations [M, 8192] and weights [28672, 8192], both 1x16 RNE along K."""
    K, N = DEC["k"], DEC["n"]
    x = workloads.activations(64, K, seed=DEC["act_seed"])[:M]
    w = workloads.weights(N, K, seed=DEC["w_seed"], device="cuda").cpu()
    xc, xs, xts, _ = oracle.quantize(workloads.bf16_bits(x))
    wc, wsc, wts, _ = oracle.quantize(workloads.bf16_bits(w))
    a = nv.NVFP4Tensor(torch.from_numpy(xc).cuda(), torch.from_numpy(xs).cuda(),
                       torch.tensor([xts], device="cuda"), torch.zeros(1, device="cuda"), M, K,
                       False, 1)
    b = nv.NVFP4Tensor(torch.from_numpy(wc).cuda(), torch.from_numpy(wsc).cuda(),
                       torch.tensor([wts], device="cuda"), torch.zeros(1, device="cuda"), N, K,
                       False, 1)
    yf = nv.gemm("NT", a, b, out_dtype=torch.float32)
    yb = nv.gemm("NT", a, b, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    rng = np.random.default_rng(M)
    cols = np.concatenate([np.arange(256), rng.integers(256, N, 768)])
    mm, nn = np.meshgrid(np.arange(M), cols, indexing="ij")
    ms, ns = mm.ravel().astype(np.int64), nn.ravel().astype(np.int64)
    ref, ab = oracle.gemm_pairs("NT", M, N, K, (xc, xs, xts, False), (wc, wsc, wts, False), ms, ns)
    mt, nt = torch.from_numpy(ms).cuda(), torch.from_numpy(ns).cuda()
    check_gemm(yf[mt, nt].cpu().numpy(), yb[mt, nt].float().cpu().numpy(), ref, ab, "decode")
