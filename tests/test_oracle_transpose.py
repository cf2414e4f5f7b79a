"""Pins of the oracle's storage transpose (CPU).

The transposed tensor holds element (c, r) = element (r, c) of the input with
its code and its block scale.  Pinned against independent facts:
  - dequantizing the transposed tensor (its own block layout) gives the
    transpose of the dequantized input, bit for bit (the dequantization is
    pinned by its own tests);
  - 16x16 weight blocks are transpose-consistent (readjensen.com NVFP4
    training-recipe page, recipe paragraph): the transpose of quantize(W) is
    bit for bit quantize(W^T), computed from W^T's own values;
  - a 1x16 RNE quantization along rows, transposed, is the 1x16 RNE
    quantization of x^T down its columns (same blocks, same amax);
  - transposing twice gives the input back.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads

MODES = [(True, 1), (False, 1), (False, 0)]


def bits(x):
    return workloads.bf16_bits(x)


@pytest.mark.parametrize("block2d,axis", MODES)
@pytest.mark.parametrize("rows,cols", [(16, 16), (48, 80), (256, 32), (32, 272)])
def test_dequantize_commutes_with_transpose(block2d, axis, rows, cols):
    x = workloads.activations(rows, cols, seed=rows + cols)
    c, s, ts, _ = oracle.quantize(bits(x), block2d=block2d, axis=axis)
    ct, st = oracle.transpose(c, s, rows, cols, block2d, axis)
    axis_t = axis if block2d else 1 - axis
    f, b = oracle.dequantize(c, s, ts, rows, cols, block2d, axis)
    ft, bt = oracle.dequantize(ct, st, ts, cols, rows, block2d, axis_t)
    assert np.array_equal(ft, f.T) and np.array_equal(bt, b.T)
    c2, s2 = oracle.transpose(ct, st, cols, rows, block2d, axis_t)
    assert np.array_equal(c2, c) and np.array_equal(s2, s)


@pytest.mark.parametrize("rows,cols", [(32, 64), (128, 48), (256, 256)])
def test_2d_blocks_are_transpose_consistent(rows, cols):
    w = workloads.weights(rows, cols, seed=7 + rows)
    c, s, ts, am = oracle.quantize(bits(w), block2d=True)
    ct, st, tst, amt = oracle.quantize(bits(w.t().contiguous()), block2d=True)
    assert am == amt and ts == tst
    xc, xs = oracle.transpose(c, s, rows, cols, True, 1)
    assert np.array_equal(xc, ct) and np.array_equal(xs, st)


def test_1d_rne_blocks_along_rows_transpose_to_blocks_down_columns():
    x = workloads.activations(64, 96, seed=3)
    c, s, ts, _ = oracle.quantize(bits(x), axis=1)
    ct, st, tst, _ = oracle.quantize(bits(x.t().contiguous()), axis=0)
    assert ts == tst
    xc, xs = oracle.transpose(c, s, 64, 96, False, 1)
    assert np.array_equal(xc, ct) and np.array_equal(xs, st)


def test_single_element_lands_transposed():
    """One non-zero code at (r, c) moves to (c, r); its block scale moves with it."""
    rows, cols = 32, 48
    for (r, cc) in [(0, 1), (5, 17), (31, 47), (16, 0)]:
        codes = np.zeros((rows, cols // 2), dtype=np.uint8)
        codes[r, cc // 2] = 0x7 << (4 * (cc & 1))
        scales = np.arange((rows // 16) * (cols // 16), dtype=np.uint8).reshape(rows // 16, cols // 16)
        ct, st = oracle.transpose(codes, scales, rows, cols, True, 1)
        q = np.zeros((cols, rows), dtype=np.uint8)
        q[:, 0::2] = ct & 0xF
        q[:, 1::2] = ct >> 4
        assert q[cc, r] == 7 and np.count_nonzero(q) == 1
        assert st[cc // 16, r // 16] == scales[r // 16, cc // 16]
        assert np.array_equal(st, scales.T)


def test_shape_errors():
    with pytest.raises(ValueError):
        oracle.transpose(np.zeros((8, 8), np.uint8), np.zeros((8, 1), np.uint8), 8, 16)
