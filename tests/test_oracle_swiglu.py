"""Pins for the oracle's SwiGLU (CPU only): act = BF16(BF16(silu(g)) * u),
silu(g) = g / (1 + exp(-g)) in FP32, on h = [gate | up].

The MLP's activation between its GEMMs (readjensen.com recipe paragraph: the
MLP GEMMs emit BF16; the Llama 3 models of its benchmark paragraph use
SwiGLU).  Pinned by silu in FP64, its closed-form limits, torch's bfloat16
rounding of the product, and the gate/up column layout.
"""
import numpy as np
import torch

import oracle


def bf16(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)


def bits(t):
    return t.view(torch.int16).numpy().view(np.uint16)


def test_silu_matches_float64_within_two_ulp():
    rng = np.random.default_rng(1)
    g = bf16(rng.uniform(-80, 80, 4000)).float().numpy()
    got = np.array([oracle.silu_f32(float(v)) for v in g], dtype=np.float32)
    ref = g.astype(np.float64) / (1.0 + np.exp(-g.astype(np.float64)))
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got - ref) <= 2 * ulp + 1e-45)


def test_silu_limits():
    assert oracle.silu_f32(0.0) == 0.0
    for g in (104.0, 200.0, 3.0e38):            # exp(-g) underflows: silu(g) = g
        assert oracle.silu_f32(g) == np.float32(g)
    for g in (-89.0, -1000.0):                  # exp(-g) overflows: silu(g) = -0
        v = oracle.silu_f32(g)
        assert v == 0.0 and np.signbit(v)
    assert abs(oracle.silu_f32(1.0) - 1.0 / (1.0 + np.exp(-1.0))) < 1e-7


def test_act_is_the_bf16_product_of_bf16_silu_and_up():
    rng = np.random.default_rng(2)
    rows, F = 16, 96
    h = bf16(rng.standard_normal((rows, 2 * F)) * 4)
    act, sb = oracle.swiglu(bits(h))
    g, u = h[:, :F].float(), h[:, F:].float()
    # the BF16 silu is torch's bfloat16 rounding of the oracle's FP32 silu
    s32 = torch.tensor([[oracle.silu_f32(float(v)) for v in row] for row in g.numpy()],
                       dtype=torch.float32)
    assert np.array_equal(sb, bits(s32.to(torch.bfloat16)))
    # act = bfloat16(bf16 silu * up), products exact in FP32 (8 x 8 bits)
    sbf = torch.from_numpy(sb.view(np.int16)).view(torch.bfloat16).float()
    assert np.array_equal(act, bits((sbf * u).to(torch.bfloat16)))


def test_gate_and_up_columns_pair_by_offset_f():
    # gate column c pairs with up column F + c: one up column of 2s, the rest
    # 0 -> act is zero except in that column, where it is 2 * BF16(silu(g))
    rows, F = 4, 32
    h = torch.zeros(rows, 2 * F)
    h[:, :F] = torch.linspace(-3, 3, rows * F).reshape(rows, F)
    h[:, F + 5] = 2.0
    hb = h.to(torch.bfloat16)
    act, sb = oracle.swiglu(bits(hb))
    a = torch.from_numpy(act.view(np.int16)).view(torch.bfloat16).float()
    s = torch.from_numpy(sb.view(np.int16)).view(torch.bfloat16).float()
    assert torch.all(a[:, [c for c in range(F) if c != 5]] == 0)
    assert torch.equal(a[:, 5], 2 * s[:, 5])
