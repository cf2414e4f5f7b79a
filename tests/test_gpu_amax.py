"""GPU parity: nvfp4_amax (max |x| and max |RHT16 down the columns of x| in one
read) against the CPU oracle, bit-exact, and its use as amax_in.

The tensor amax is the first step of the two-level scaling (s_g = amax /
2688; guiahardware.es "Cos'e NVFP4"); the RHT amax is that of the wgrad
operands (readjensen.com recipe paragraph).
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


def strided(x_cpu, pad):
    rows, cols = x_cpu.shape
    if not pad:
        return x_cpu.cuda()
    wide = torch.zeros(rows, cols + pad, dtype=x_cpu.dtype)
    wide[:, :cols] = x_cpu
    return wide.cuda()[:, :cols]


@pytest.mark.parametrize("shape", [(16, 16), (48, 272), (528, 1040), (256, 4112)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("pad", [0, 16])
def test_both_amaxes_match_oracle(nv, shape, dtype, pad):
    x = workloads.gradients(*shape, seed=shape[0] + shape[1]).to(dtype)
    mask = workloads.sign_mask(shape[1])
    a, ar = nv.amax(strided(x, pad), rht_mask=mask)
    torch.cuda.synchronize()
    xo = to_oracle_input(x)
    assert a.item() == oracle.amax(xo)
    assert ar.item() == oracle.amax(xo, rht=True, axis=0, mask=mask)


def test_plain_amax_any_rows(nv):
    x = workloads.activations(37, 64, seed=2)
    a, ar = nv.amax(x.cuda())
    torch.cuda.synchronize()
    assert ar is None
    assert a.item() == oracle.amax(to_oracle_input(x))


def test_empty_tensor(nv):
    a, ar = nv.amax(torch.empty(0, 64, dtype=torch.bfloat16, device="cuda"), rht_mask=3)
    torch.cuda.synchronize()
    assert a.item() == 0.0 and ar.item() == 0.0


def test_amax_in_gives_the_same_quantization(nv):
    """Passing the one-read maxima as amax_in reproduces the self-computed
    quantizations bit for bit (row-wise SR and transposed column RHT + SR)."""
    x = workloads.gradients(528, 1040, seed=8).cuda()
    mask = workloads.sign_mask(4)
    a, ar = nv.amax(x, rht_mask=mask)
    kw_r = dict(sr=True, seed=3, stream_id=0)
    kw_c = dict(axis=0, rht=True, mask=mask, sr=True, seed=3, stream_id=1, transpose=True)
    q1, q2 = nv.quantize(x, **kw_r), nv.quantize(x, amax_in=a, **kw_r)
    t1, t2 = nv.quantize(x, **kw_c), nv.quantize(x, amax_in=ar, **kw_c)
    torch.cuda.synchronize()
    for u, v in ((q1, q2), (t1, t2)):
        assert torch.equal(u.codes, v.codes) and torch.equal(u.scales, v.scales)
        assert u.tensor_scale.item() == v.tensor_scale.item()
