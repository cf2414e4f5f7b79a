"""GPU parity: nvfp4_quantize with transpose_out = 1 against the CPU oracle.

The transposed output is, by definition, the untransposed quantization (blocks
down the columns: 1x16 along rows, or 16x16) stored as that of x^T, so the
expected codes and scales are the oracle's, transposed here element by element
(codes unpacked to nibbles, transposed, repacked).  Bit-exact, including SR
and the RHT.  Sources: 1x16 / 16x16 blocks, RHT on wgrad inputs, stochastic
rounding of gradients -- readjensen.com NVFP4 recipe paragraph.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import every_bf16_below, to_oracle_input

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import nvfp4_bit_microscaled_amd as m
    torch.cuda.set_device(0)
    return m


def transpose_codes(codes: np.ndarray) -> np.ndarray:
    """[R, C/2] packed (low nibble first) -> [C, R/2] packed codes of the transpose."""
    q = np.empty((codes.shape[0], codes.shape[1] * 2), dtype=np.uint8)
    q[:, 0::2] = codes & 0xF
    q[:, 1::2] = codes >> 4
    qt = np.ascontiguousarray(q.T)
    return (qt[:, 0::2] | (qt[:, 1::2] << 4)).astype(np.uint8)


def check(nv, x_cpu, block2d, sr=False, rht=False, mask=0, seed=0, stream_id=0, ld_pad=0):
    rows, cols = x_cpu.shape
    if ld_pad:
        wide = torch.zeros(rows, cols + ld_pad, dtype=x_cpu.dtype)
        wide[:, :cols] = x_cpu
        xg = wide.cuda()[:, :cols]
    else:
        xg = x_cpu.cuda()
    kw = dict(block2d=block2d, axis=0, sr=sr, rht=rht, mask=mask, seed=seed, stream_id=stream_id)
    qt = nv.quantize(xg, transpose=True, **kw)
    q = nv.quantize(xg, **kw)
    torch.cuda.synchronize()
    assert (qt.rows, qt.cols, qt.axis, qt.block2d) == (cols, rows, 1, block2d)
    oc, osc, ots, oam = oracle.quantize(to_oracle_input(x_cpu), **kw)
    assert qt.tensor_scale.item() == ots and qt.amax.item() == oam
    exp_c = transpose_codes(oc)
    exp_s = np.ascontiguousarray(osc.T)
    gc, gs = qt.codes.cpu().numpy(), qt.scales.cpu().numpy()
    assert gs.shape == exp_s.shape and gc.shape == exp_c.shape
    nbad_s, nbad_c = int((gs != exp_s).sum()), int((gc != exp_c).sum())
    assert nbad_s == 0 and nbad_c == 0, "%d scale bytes and %d code bytes differ" % (nbad_s, nbad_c)
    # and the untransposed GPU result, transposed, is the same tensor
    assert np.array_equal(transpose_codes(q.codes.cpu().numpy()), gc)
    assert np.array_equal(np.ascontiguousarray(q.scales.cpu().numpy().T), gs)
    return qt


# whole tiles, ragged row and column tails, a single block, several tiles
SHAPES = [(256, 256), (16, 16), (272, 48), (528, 304), (48, 1040), (784, 528)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("block2d", [False, True])
def test_rne(nv, shape, block2d):
    kind = workloads.weights if block2d else workloads.activations
    check(nv, kind(*shape, seed=shape[0] ^ shape[1]), block2d)


@pytest.mark.parametrize("shape", [(256, 256), (272, 48), (784, 528)])
@pytest.mark.parametrize("block2d", [False, True])
def test_sr(nv, shape, block2d):
    x = workloads.gradients(*shape, seed=9)
    check(nv, x, block2d, sr=True, seed=1, stream_id=1)
    check(nv, x, block2d, sr=True, seed=0xDEADBEEF12345, stream_id=3)


@pytest.mark.parametrize("shape", [(256, 256), (528, 304), (48, 1040)])
@pytest.mark.parametrize("sr", [False, True])
def test_rht(nv, shape, sr):
    mask = workloads.sign_mask(1)
    check(nv, workloads.gradients(*shape, seed=4), False, sr=sr, rht=True, mask=mask, seed=1,
          stream_id=1)


@pytest.mark.parametrize("block2d", [False, True])
def test_fp32_strided_input(nv, block2d):
    x = workloads.activations(272, 304, seed=5).to(torch.float32)
    check(nv, x, block2d, ld_pad=16)


def test_zero_blocks_and_saturation(nv):
    x = workloads.activations(64, 80, seed=3)
    x[16:32, :] = 0            # zero row blocks
    x[:, 32:48] = 0            # zero column blocks
    x[40, 5] = 1.0e30          # one huge value: most blocks underflow to scale 0
    for block2d in (False, True):
        check(nv, x, block2d)


def test_transposed_operands_give_the_nt_gemm(nv):
    """wgrad from transposed storage: dW = dY^T X as an NT GEMM of the two
    K-major transposed tensors equals the TN GEMM of the untransposed ones."""
    T, M, N = 512, 256, 272
    mask = workloads.sign_mask(2)
    dy = workloads.gradients(T, M, seed=1).cuda()
    x = workloads.activations(T, N, seed=2).cuda()
    kw_a = dict(axis=0, sr=True, seed=5, stream_id=1, rht=True, mask=mask)
    kw_b = dict(axis=0, rht=True, mask=mask)
    a, b = nv.quantize(dy, **kw_a), nv.quantize(x, **kw_b)
    at, bt = nv.quantize(dy, transpose=True, **kw_a), nv.quantize(x, transpose=True, **kw_b)
    y_tn = nv.gemm("TN", a, b, out_dtype=torch.float32)
    y_nt = nv.gemm("NT", at, bt, out_dtype=torch.float32)
    torch.cuda.synchronize()
    # the same products summed in a different K order: equal within FP32 accumulation
    ref = y_tn.double()
    assert torch.allclose(y_nt.double(), ref, rtol=0, atol=1e-5 * float(ref.abs().max()))


@pytest.mark.parametrize("exp2", [0, -37, -38, 127])
def test_every_bf16_element_value_transposed(nv, exp2):
    """The transposed-storage kernel on every finite BF16 value up to
    M = 2^exp2 in blocks (down the columns) whose maximum is M: round to
    nearest and stochastic rounding, bit-exact against the oracle."""
    x = every_bf16_below(exp2).t().contiguous()
    check(nv, x, block2d=False)
    check(nv, x, block2d=False, sr=True, seed=4, stream_id=1)
