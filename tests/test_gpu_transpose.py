"""GPU parity: nvfp4_transpose, the storage transpose of an NVFP4 tensor.

Bit-exact against the oracle's transpose of the oracle's quantization, in all
three block layouts, at ragged sizes (tiles of 256 x 256 with partial edge
tiles in both directions and odd numbers of 16-row blocks, so half-filled
128-byte output segments occur) and at the Llama-3-8B weight sizes the
training step transposes.  For 16x16 weight blocks the result also equals the
quantization written in transposed storage directly (nvfp4_quantize with
transpose_out), which is the recipe's transpose consistency (readjensen.com
NVFP4 training-recipe page, recipe paragraph).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import to_oracle_input

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import nvfp4_bit_microscaled_amd as m
    torch.cuda.set_device(0)
    return m


MODES = [(True, 1), (False, 1), (False, 0)]
SHAPES = [(16, 16), (16, 528), (272, 48), (528, 784), (256, 256), (1040, 240)]


@pytest.mark.parametrize("block2d,axis", MODES)
@pytest.mark.parametrize("rows,cols", SHAPES)
def test_transpose_matches_oracle(nv, block2d, axis, rows, cols):
    x = workloads.activations(rows, cols, seed=rows * 31 + cols)
    c, s, ts, _ = oracle.quantize(to_oracle_input(x), block2d=block2d, axis=axis)
    t = nv.NVFP4Tensor(torch.from_numpy(c).cuda(), torch.from_numpy(s).cuda(),
                       torch.tensor([ts], device="cuda"), torch.zeros(1, device="cuda"),
                       rows, cols, block2d, axis)
    print("transpose", rows, cols, block2d, axis, flush=True)
    tt = nv.transpose(t)
    torch.cuda.synchronize()
    ct, st = oracle.transpose(c, s, rows, cols, block2d, axis)
    assert tt.rows == cols and tt.cols == rows
    assert tt.axis == (axis if block2d else 1 - axis)
    assert np.array_equal(tt.codes.cpu().numpy(), ct)
    assert np.array_equal(tt.scales.cpu().numpy(), st)
    assert tt.tensor_scale.data_ptr() == t.tensor_scale.data_ptr()


def test_transpose_leaves_padding_alone(nv):
    """Output planes written through the caller's buffers: bytes past the
    planes stay untouched (a 16-row-block count that is odd leaves the last
    8-byte chunk of each output row as the only one of its pair)."""
    rows, cols = 48, 272
    x = workloads.weights(rows, cols, seed=4)
    q = nv.quantize(x.cuda(), block2d=True)
    codes = torch.full((cols * rows // 2 + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    scales = torch.full(((cols // 16) * (rows // 16) + 64,), 0x5A, dtype=torch.uint8, device="cuda")
    out = nv.NVFP4Tensor(codes[:cols * rows // 2].view(cols, rows // 2),
                         scales[:(cols // 16) * (rows // 16)].view(cols // 16, rows // 16),
                         q.tensor_scale, q.amax, cols, rows, True, 1)
    nv.transpose(q, out=out)
    torch.cuda.synchronize()
    assert torch.all(codes[cols * rows // 2:] == 0xA5)
    assert torch.all(scales[(cols // 16) * (rows // 16):] == 0x5A)
    ref = nv.quantize(x.cuda(), block2d=True, transpose=True)
    torch.cuda.synchronize()
    assert torch.equal(out.codes, ref.codes) and torch.equal(out.scales, ref.scales)


L8 = workloads.LLAMA8B


@pytest.mark.parametrize("name", ["W_gu", "W_down"])
def test_llama8b_weights(nv, name):
    """The step's dgrad weights: W^T from W's own 16x16 quantization equals the
    oracle's transpose of the oracle's quantization of W (whole tensor) and the
    transposed-storage quantization of W."""
    D, F = L8["hidden"], L8["ffn"]
    rows, cols, seed = (2 * F, D, L8["wgu_seed"]) if name == "W_gu" else (D, F, L8["wdown_seed"])
    w = workloads.weights(rows, cols, seed, device="cuda")
    q = nv.quantize(w, block2d=True)
    qt = nv.transpose(q)
    direct = nv.quantize(w, block2d=True, transpose=True)
    torch.cuda.synchronize()
    assert torch.equal(qt.codes, direct.codes) and torch.equal(qt.scales, direct.scales)
    assert direct.tensor_scale.item() == q.tensor_scale.item()
    del direct
    oracle.set_num_threads(16)
    c, s, ts, _ = oracle.quantize(to_oracle_input(w.cpu()), block2d=True)
    assert ts == q.tensor_scale.item()
    ct, st = oracle.transpose(c, s, rows, cols, True, 1)
    assert np.array_equal(qt.codes.cpu().numpy(), ct)
    assert np.array_equal(qt.scales.cpu().numpy(), st)


def test_empty(nv):
    t = nv.NVFP4Tensor(torch.empty(0, 8, dtype=torch.uint8, device="cuda"),
                       torch.empty(0, 1, dtype=torch.uint8, device="cuda"),
                       torch.ones(1, device="cuda"), torch.zeros(1, device="cuda"), 0, 16, True, 1)
    tt = nv.transpose(t)
    torch.cuda.synchronize()
    assert tt.codes.shape == (16, 0) and tt.scales.shape == (1, 0)
