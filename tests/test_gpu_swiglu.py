"""GPU parity: nvfp4_swiglu_amax, the MLP activation between the two fprop
GEMMs fused with both tensor amaxes of its output.

act is compared with the oracle's SwiGLU and with a plain PyTorch FP32
computation, both taking the same rounding points (silu in FP32 rounded to
BF16, product rounded to BF16).  The kernel's FP32 silu may differ from a
reference's by an ulp or two (exponential and reciprocal implementations),
which can move silu's BF16 rounding by one step: act must equal the rounded
product of up with the reference silu's BF16 value or one of its two BF16
neighbours, the latter only near a BF16 rounding boundary.  The two amaxes
must equal the oracle's on the act the kernel produced, bit for bit.
Source: the MLP GEMMs with BF16 outputs (readjensen.com recipe paragraph);
Llama 3's SwiGLU MLP (benchmark paragraph models).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import bf16_neighbours, check_act_against_oracle, to_oracle_input

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import nvfp4_bit_microscaled_amd as m
    torch.cuda.set_device(0)
    return m


def candidates(h):
    """act from the reference silu rounded to BF16, and from its two BF16
    neighbours (a one-ulp difference in the FP32 silu can move its BF16
    rounding by one step, which the product with up carries to act)."""
    F = h.shape[1] // 2
    g, u = h[:, :F].float(), h[:, F:].float()
    sg = (g / (1.0 + torch.exp(-g))).to(torch.bfloat16).float()
    lo, hi = bf16_neighbours(sg)
    return [(v * u).to(torch.bfloat16) for v in (sg, lo, hi)]


def make_h(rows, F, seed):
    h = 3.0 * workloads.activations(rows, 2 * F, seed=seed).float()
    h[0, :4] = torch.tensor([-100.0, 100.0, -1000.0, 88.0])   # exp overflow / underflow
    return h.to(torch.bfloat16)


@pytest.mark.parametrize("rows,F", [(16, 16), (48, 272), (256, 1040), (528, 64)])
@pytest.mark.parametrize("pad", [0, 16])
def test_swiglu_and_amaxes(nv, rows, F, pad):
    h = make_h(rows, F, seed=rows + F)
    mask = workloads.sign_mask(F)
    if pad:
        hw = torch.zeros(rows, 2 * F + pad, dtype=torch.bfloat16)
        hw[:, :2 * F] = h
        hg = hw.cuda()[:, :2 * F]
        out = torch.zeros(rows, F + pad, dtype=torch.bfloat16, device="cuda")[:, :F]
    else:
        hg, out = h.cuda(), None
    act, a, ar = nv.swiglu_amax(hg, mask, out=out)
    torch.cuda.synchronize()
    got = act.cpu().view(torch.int16)
    ref, lo, hi = (c.view(torch.int16) for c in candidates(h))
    same = got == ref
    ok = same | (got == lo) | (got == hi)
    assert bool(ok.all()), "%d outputs match no BF16 silu candidate" % int((~ok).sum())
    assert float((~same).float().mean()) < 1e-3
    xo = to_oracle_input(act.cpu())
    assert a.item() == oracle.amax(xo)
    assert ar.item() == oracle.amax(xo, rht=True, axis=0, mask=mask)


def test_feeds_the_same_quantizations(nv):
    """Quantizing act with the fused amaxes as amax_in equals quantizing it
    with self-computed ones (row-wise RNE and transposed column RHT)."""
    h = make_h(256, 528, seed=3).cuda()
    mask = workloads.sign_mask(9)
    act, a, ar = nv.swiglu_amax(h, mask)
    q1, q2 = nv.quantize(act), nv.quantize(act, amax_in=a)
    kw = dict(axis=0, rht=True, mask=mask, transpose=True)
    t1, t2 = nv.quantize(act, **kw), nv.quantize(act, amax_in=ar, **kw)
    torch.cuda.synchronize()
    for u, v in ((q1, q2), (t1, t2)):
        assert torch.equal(u.codes, v.codes) and torch.equal(u.scales, v.scales)


@pytest.mark.parametrize("rows,F", [(48, 272), (528, 64), (4096, 1024)])
def test_act_against_the_oracle(nv, rows, F):
    """act against the oracle's SwiGLU (FP32 silu with the C library's expf and
    an IEEE division, BF16 rounding points): equal, or the product of up with
    one of the two BF16 neighbours of the oracle's BF16 silu, and the latter
    only where the oracle's FP32 silu lies within 4 FP32 ulps of the BF16
    rounding boundary between the two (the kernel's exp and reciprocal are
    within an ulp or two, so they may round silu to the other side)."""
    h = make_h(rows, F, seed=rows * 3 + F)
    mask = workloads.sign_mask(F + 1)
    act, a, ar = nv.swiglu_amax(h.cuda(), mask)
    torch.cuda.synchronize()
    check_act_against_oracle(h, act.cpu(), "swiglu %dx%d" % (rows, F))


@pytest.mark.parametrize("up", ["one", "mixed"])
def test_every_bf16_gate(nv, up):
    """Every finite BF16 gate value once (65280 of them, [16, 4080]): the
    reciprocal path, the division where 1 + exp(-g) reaches 2^126 (g below
    -87.3), exp(-g) overflowing (g <= -89) and underflowing (g >= 104), signed
    zeros and denormal gates, against the oracle's SwiGLU under the same flip
    rule; up is 1, or a mix of signs and magnitudes up to 1 (products that
    underflow BF16 included; larger ones would overflow act or its column
    transform for the largest gates).  The amaxes equal the oracle's on act."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    g = torch.from_numpy(bits[finite].astype(np.int32).astype(np.int16)).view(torch.bfloat16)
    assert g.numel() == 16 * 4080
    g = g.reshape(16, 4080)
    if up == "one":
        u = torch.ones_like(g)
    else:
        rng = np.random.default_rng(5)
        pool = np.array([1.0, -1.0, 0.375, -7.0e-3, 1.0e-30, -0.75, 2.0 ** -100, -0.9921875],
                        dtype=np.float32)
        u = torch.from_numpy(pool[rng.integers(0, len(pool), size=g.shape)]).to(torch.bfloat16)
    h = torch.cat([g, u], dim=1)
    mask = workloads.sign_mask(77)
    act, a, ar = nv.swiglu_amax(h.cuda(), mask)
    torch.cuda.synchronize()
    check_act_against_oracle(h, act.cpu(), "every BF16 gate, up=%s" % up)
    xo = to_oracle_input(act.cpu())
    assert a.item() == oracle.amax(xo)
    assert ar.item() == oracle.amax(xo, rht=True, axis=0, mask=mask)
