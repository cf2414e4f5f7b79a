"""GPU check of nvfp4_quantize_noalloc, the allocation-free variant of
nvfp4_quantize (its amax pass uses the library's own per-GPU scratch instead
of a caller workspace).

Through the C ABI, on two calls in a row (the second on a smaller tensor, so
stale partial maxima of the first call sit in the scratch), in every block
layout and rounding mode: codes, scales, tensor scale and amax equal
nvfp4_quantize's with a caller workspace, bit for bit.  The inputs follow
the activation recipe (1x16 RNE rows), the weight recipe (16x16) and the
gradient recipe (SR; RHT + SR down the columns, transposed storage) of the
readjensen.com NVFP4 training-recipe page.
"""
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import nvfp4_bit_microscaled_amd as m
    torch.cuda.set_device(0)
    return m


def outputs(nv, rows, cols, block2d, axis, transpose):
    o_rows, o_cols, o_axis = (cols, rows, 1) if transpose else (rows, cols, axis)
    dev = "cuda"
    return dict(codes=torch.full((o_rows, o_cols // 2), 0xEE, dtype=torch.uint8, device=dev),
                scales=torch.full(nv.scale_shape(o_rows, o_cols, block2d, o_axis), 0xEE,
                                  dtype=torch.uint8, device=dev),
                ts=torch.full((1,), -1.0, device=dev), amax=torch.full((1,), -1.0, device=dev))


CASES = [  # (kind, block2d, axis, sr, rht, transpose)
    ("act", False, 1, False, False, False),
    ("w", True, 1, False, False, False),
    ("grad", False, 1, True, False, False),
    ("grad", False, 0, True, True, True),
    ("act", False, 0, False, True, False),
]


@pytest.mark.parametrize("kind,block2d,axis,sr,rht,transpose", CASES)
def test_noalloc_equals_workspace_call(nv, kind, block2d, axis, sr, rht, transpose):
    gen = {"act": workloads.activations, "w": workloads.weights, "grad": workloads.gradients}[kind]
    mask = workloads.sign_mask(3)
    # the first call leaves its partial maxima in the scratch; the second,
    # smaller tensor (fewer workgroups in its amax pass) must not see them
    for rows, cols, seed in ((4096, 2048, 1), (272, 528, 2)):
        x = gen(rows, cols, seed=seed + 10 * block2d, device="cuda")
        ref = outputs(nv, rows, cols, block2d, axis, transpose)
        got = outputs(nv, rows, cols, block2d, axis, transpose)
        ws = torch.empty(nv.nvfp4_quantize_workspace_size(rows, cols), dtype=torch.uint8,
                         device="cuda")
        common = (x, nv.DTYPE_BF16, rows, cols, cols, int(block2d), axis, int(transpose),
                  int(sr), 5, 1, int(rht), mask, None)
        print("noalloc", kind, rows, cols, block2d, axis, sr, rht, transpose, flush=True)
        st = nv.nvfp4_quantize(*common, ref["amax"], ref["codes"], ref["scales"], ref["ts"],
                               ws, ws.numel())
        assert st == 0
        st = nv.nvfp4_quantize_noalloc(*common, got["amax"], got["codes"], got["scales"],
                                       got["ts"])
        assert st == 0
        torch.cuda.synchronize()
        for k in ("codes", "scales"):
            assert torch.equal(ref[k], got[k]), (k, rows, cols)
        assert ref["ts"].item() == got["ts"].item() and ref["amax"].item() == got["amax"].item()
        if not rht:
            assert got["amax"].item() == x.float().abs().max().item()


def test_noalloc_with_amax_in_and_errors(nv):
    """With amax_in the scratch is not used; argument errors come back as
    from nvfp4_quantize, before anything is enqueued."""
    x = workloads.activations(64, 256, seed=4, device="cuda")
    a = x.float().abs().max().reshape(1)
    got = outputs(nv, 64, 256, False, 1, False)
    ref = outputs(nv, 64, 256, False, 1, False)
    common = (x, nv.DTYPE_BF16, 64, 256, 256, 0, 1, 0, 0, 0, 0, 0, 0, a)
    assert nv.nvfp4_quantize_noalloc(*common, got["amax"], got["codes"], got["scales"],
                                     got["ts"]) == 0
    assert nv.nvfp4_quantize(*common, ref["amax"], ref["codes"], ref["scales"], ref["ts"], None,
                             0) == 0
    torch.cuda.synchronize()
    assert torch.equal(got["codes"], ref["codes"]) and torch.equal(got["scales"], ref["scales"])
    assert nv.nvfp4_quantize_noalloc(x, nv.DTYPE_BF16, 64, 40, 256, 0, 1, 0, 0, 0, 0, 0, 0,
                                     None, None, got["codes"], got["scales"], got["ts"]) == 2
    assert nv.nvfp4_quantize_noalloc(x, nv.DTYPE_BF16, 64, 256, 256, 0, 1, 0, 0, 0, 0, 0, 0,
                                     None, None, got["codes"], got["scales"], None) == 1
