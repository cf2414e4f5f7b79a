"""GPU parity of nvfp4_gemm_swiglu: the first fprop GEMM of the MLP with the
SwiGLU activation and both amaxes of its output in the GEMM's epilogue.

- H (stored when asked) is the NT GEMM with BF16 output: within the GEMM
  tolerance of the oracle's FP64 reference, and bit-equal to nvfp4_gemm on
  the same operands (same kernel main loop).
- act against the oracle's SwiGLU of that H (after undoing the gate/up
  column interleave): equal, or one BF16 step of silu away only where the
  oracle's FP32 silu is within 4 FP32 ulps of a BF16 rounding boundary
  (check_act_against_oracle); at full size on sampled row slices.
- act and both amaxes also equal, bit for bit, nvfp4_swiglu_amax run on that
  H (the same arithmetic in the standalone pass).
- Both amaxes equal the oracle's on the act the kernel produced.

Source: the MLP GEMMs on NVFP4 inputs with BF16 outputs (readjensen.com
recipe paragraph); the Llama 3 models of its benchmark paragraph use SwiGLU.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import check_act_against_oracle, check_gemm, to_oracle_input

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import nvfp4_bit_microscaled_amd as m
    torch.cuda.set_device(0)
    return m


def operands(nv, M, F, K, seed):
    x = workloads.activations(M, K, seed)
    w = nv.interleave_gate_up(workloads.weights(2 * F, K, seed + 1))
    a = nv.quantize(x.cuda())
    b = nv.quantize(w.cuda(), block2d=True)
    a_or = (a.codes.cpu().numpy(), a.scales.cpu().numpy(), a.tensor_scale.item(), False)
    b_or = (b.codes.cpu().numpy(), b.scales.cpu().numpy(), b.tensor_scale.item(), True)
    return a, b, a_or, b_or


def check_act_oracle(nv, act, h, rows=None):
    """act vs the oracle's SwiGLU of the kernel's own H (rows: a slice)."""
    sl = slice(None) if rows is None else slice(*rows)
    hd = nv.deinterleave_gate_up_columns(h[sl]).contiguous().cpu()
    check_act_against_oracle(hd, act[sl].cpu(), "fused act")


def check_against_unfused(nv, act, am, amr, h, mask):
    hd = nv.deinterleave_gate_up_columns(h).contiguous()
    act_u, am_u, amr_u = nv.swiglu_amax(hd, mask)
    torch.cuda.synchronize()
    assert torch.equal(act.view(torch.int16), act_u.view(torch.int16))
    assert am.item() == am_u.item() and amr.item() == amr_u.item()


def check_amaxes_oracle(act, am, amr, mask):
    a_np = to_oracle_input(act)
    assert np.float32(am.item()) == np.float32(oracle.amax(a_np))
    assert np.float32(amr.item()) == np.float32(oracle.amax(a_np, rht=True, axis=0, mask=mask))


# one full tile; ragged M (M % 256 = 16) with a half tile in N (N % 256 =
# 128: that tile's second wave column is past N); a short M; several tiles
SHAPES = [(256, 128, 256), (272, 192, 384), (48, 64, 128), (512, 1024, 512)]


@pytest.mark.parametrize("M,F,K", SHAPES)
def test_fused_matches_gemm_then_swiglu(nv, M, F, K):
    mask = workloads.sign_mask(M + F)
    a, b, a_or, b_or = operands(nv, M, F, K, M + K)
    print("gemm_swiglu", M, F, K, flush=True)
    act, am, amr, h = nv.gemm_swiglu(a, b, mask, store_h=True)
    torch.cuda.synchronize()
    # H: the oracle's GEMM within tolerance
    ref, ab = oracle.gemm_full("NT", M, 2 * F, K, a_or, b_or)
    check_gemm(None, h.float().cpu().numpy(), ref, ab, "gemm_swiglu H %dx%dx%d" % (M, 2 * F, K))
    if M > 64:  # nvfp4_gemm takes the same 256 x 256 kernel above the decode sizes
        hb = nv.gemm("NT", a, b, out_dtype=torch.bfloat16)
        torch.cuda.synchronize()
        assert torch.equal(h.view(torch.int16), hb.view(torch.int16))
    check_act_oracle(nv, act, h)
    check_against_unfused(nv, act, am, amr, h, mask)
    check_amaxes_oracle(act, am, amr, mask)
    # without H: the same act and amaxes
    act2, am2, amr2, h2 = nv.gemm_swiglu(a, b, mask)
    torch.cuda.synchronize()
    assert h2 is None
    assert torch.equal(act2.view(torch.int16), act.view(torch.int16))
    assert am2.item() == am.item() and amr2.item() == amr.item()


@pytest.mark.parametrize("pad", [8, 4])
def test_strided_outputs(nv, pad):
    """act and H written into wider buffers: the padding stays untouched.
    pad 4 (rows of 8-byte but not 16-byte multiples) takes the direct
    8-byte act stores instead of the LDS-staged ones."""
    M, F, K = 256, 256, 256
    mask = workloads.sign_mask(7)
    a, b, a_or, b_or = operands(nv, M, F, K, 11)
    abuf = torch.full((M, F + pad), -2.0, dtype=torch.bfloat16, device="cuda")
    hbuf = torch.full((M, 2 * F + 24), -3.0, dtype=torch.bfloat16, device="cuda")
    act, am, amr, h = nv.gemm_swiglu(a, b, mask, act_out=abuf[:, :F], h_out=hbuf[:, 8:8 + 2 * F])
    torch.cuda.synchronize()
    assert torch.all(abuf[:, F:] == -2.0)
    assert torch.all(hbuf[:, :8] == -3.0) and torch.all(hbuf[:, 8 + 2 * F:] == -3.0)
    act_d, am_d, amr_d, h_d = nv.gemm_swiglu(a, b, mask, store_h=True)
    torch.cuda.synchronize()
    assert torch.equal(act.view(torch.int16), act_d.view(torch.int16))
    assert torch.equal(h.view(torch.int16), h_d.view(torch.int16))
    assert am.item() == am_d.item() and amr.item() == amr_d.item()


def test_empty_and_validation(nv):
    a, b, _, _ = operands(nv, 32, 64, 128, 3)
    am = torch.full((1,), 5.0, device="cuda")
    amr = torch.full((1,), 5.0, device="cuda")
    ws = torch.empty(64, dtype=torch.uint8, device="cuda")
    act = torch.empty(32, 64, dtype=torch.bfloat16, device="cuda")
    st = nv.nvfp4_gemm_swiglu(0, 128, 128, None, None, None, 0, None, None, None, 1, None, 0,
                              None, 64, 0, am, amr, None, 0)
    torch.cuda.synchronize()
    assert st == 0 and am.item() == 0.0 and amr.item() == 0.0
    common = (a.codes, a.scales, a.tensor_scale, 0, b.codes, b.scales, b.tensor_scale, 1, None, 0,
              act, 64, 0, am, amr)
    assert nv.nvfp4_gemm_swiglu(32, 128, 128, *common, ws, 0) == 6          # workspace too small
    assert nv.nvfp4_gemm_swiglu(32, 120, 128, *common, ws, 64) == 2         # N % 128
    assert nv.nvfp4_gemm_swiglu(24, 128, 128, *common, ws, 64) == 2         # M % 16
    assert nv.nvfp4_gemm_swiglu(32, 128, 64, *common, ws, 64) == 2          # K % 128


def test_full_size_llama8b_gemm1(nv):
    """The step's first GEMM at full size, 32768 x 28672 x 4096: H on sampled
    outputs against the oracle and bit-equal to nvfp4_gemm; act and both
    amaxes bit-equal to nvfp4_swiglu_amax on that H; amaxes equal to the
    oracle's on act."""
    cfg = workloads.LLAMA8B
    T, D, Fh = cfg["tokens"], cfg["hidden"], cfg["ffn"]
    mask = workloads.sign_mask(cfg["mask_seed"])
    x = workloads.activations(T, D, cfg["x_seed"], device="cuda")
    w = nv.interleave_gate_up(workloads.weights(2 * Fh, D, cfg["wgu_seed"], device="cuda"))
    a = nv.quantize(x)
    b = nv.quantize(w, block2d=True)
    del x, w
    print("gemm_swiglu full size", flush=True)
    act, am, amr, h = nv.gemm_swiglu(a, b, mask, store_h=True)
    hb = nv.gemm("NT", a, b, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    assert torch.equal(h.view(torch.int16), hb.view(torch.int16))
    del hb
    rng = np.random.default_rng(12)
    ms = rng.integers(0, T, 2048)
    ns = rng.integers(0, 2 * Fh, 2048)
    ms[:2], ns[:2] = [0, T - 1], [0, 2 * Fh - 1]
    a_or = (a.codes.cpu().numpy(), a.scales.cpu().numpy(), a.tensor_scale.item(), False)
    b_or = (b.codes.cpu().numpy(), b.scales.cpu().numpy(), b.tensor_scale.item(), True)
    ref, ab = oracle.gemm_pairs("NT", T, 2 * Fh, D, a_or, b_or, ms, ns)
    hs = h[torch.from_numpy(ms).cuda(), torch.from_numpy(ns).cuda()].float().cpu().numpy()
    check_gemm(None, hs, ref, ab, "gemm_swiglu full size H")
    for r0 in (0, T // 2, T - 64):
        check_act_oracle(nv, act, h, rows=(r0, r0 + 64))
    check_against_unfused(nv, act, am, amr, h, mask)
    del h
    check_amaxes_oracle(act, am, amr, mask)


def test_gate_values_below_minus_87_take_the_division(nv):
    """Weights scaled so that many gate values fall below -87, where silu's
    denominator passes 2^126 and the epilogue takes its division path (waves
    without such values take the path without it): still bit-equal to the
    separate pass, which selects per element."""
    M, F, K = 512, 256, 256
    mask = workloads.sign_mask(9)
    x = workloads.activations(M, K, 21)
    w = nv.interleave_gate_up(workloads.weights(2 * F, K, 22).float() * 150.0)
    a = nv.quantize(x.cuda())
    b = nv.quantize(w.to(torch.bfloat16).cuda(), block2d=True)
    act, am, amr, h = nv.gemm_swiglu(a, b, mask, store_h=True)
    torch.cuda.synchronize()
    gate = nv.deinterleave_gate_up_columns(h)[:, :F].float()
    frac = (gate < -87.0).float().mean().item()
    assert 0.001 < frac < 0.5, frac     # some waves take the division path, others not
    check_act_oracle(nv, act, h)
    check_against_unfused(nv, act, am, amr, h, mask)
    check_amaxes_oracle(act, am, amr, mask)
