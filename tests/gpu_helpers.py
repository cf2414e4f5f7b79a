"""Shared helpers for the GPU parity tests (no NVFP4 arithmetic here)."""
from __future__ import annotations

import numpy as np
import torch

import oracle


def to_oracle_input(x: torch.Tensor) -> np.ndarray:
    """CPU numpy view of a BF16 (as uint16 bits) or FP32 tensor, dense."""
    x = x.detach().cpu().contiguous()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16)
    return x.numpy()


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    """Spacing of BF16 numbers at |v| (8 significant bits)."""
    a = np.abs(v.astype(np.float64))
    a = np.where(a == 0, np.finfo(np.float32).tiny, a)
    e = np.floor(np.log2(a))
    return np.exp2(e - 7)


def check_gemm(out_f32: np.ndarray | None, out_bf16: np.ndarray | None, ref: np.ndarray,
               absref: np.ndarray, what: str = ""):
    """FP32: |C - ref| <= 1e-5 * S.  BF16: |C - RNE_bf16(ref)| <= 1 ulp, widened to
    1/2 ulp + 1e-5 S where cancellation makes 1e-5 S exceed half an ulp."""
    tol = 1e-5 * absref
    if out_f32 is not None:
        err = np.abs(out_f32.astype(np.float64) - ref)
        bad = err > tol
        assert not bad.any(), "%s: %d FP32 outputs outside 1e-5*S (max err/S %.3g)" % (
            what, bad.sum(), float((err / np.maximum(absref, 1e-300)).max()))
    if out_bf16 is not None:
        ref_b = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
        ulp = bf16_ulp(ref)
        allowed = np.where(tol > 0.5 * ulp, 0.5 * ulp + tol, ulp)
        err = np.abs(out_bf16.astype(np.float64) - ref_b)
        bad = err > allowed
        assert not bad.any(), "%s: %d BF16 outputs off by more than the bound" % (what, bad.sum())


def bf16_neighbours(x: torch.Tensor):
    """The BF16 values one step below and above each (finite, BF16) x."""
    b = x.to(torch.bfloat16).view(torch.int16).to(torch.int32)
    mag = b & 0x7FFF
    neg = (b & 0x8000) != 0
    up_mag, dn_mag = mag + 1, mag - 1
    # stepping through zero flips the sign
    above = torch.where(neg, torch.where(mag == 0, 1, -dn_mag), up_mag)
    below = torch.where(neg, -up_mag, torch.where(mag == 0, -1, dn_mag))

    def to_f(v):
        bits = torch.where(v < 0, (-v) | 0x8000, v).to(torch.int16)
        return bits.view(torch.bfloat16).float()
    return to_f(below), to_f(above)


def check_act_against_oracle(h: torch.Tensor, act: torch.Tensor, what: str = ""):
    """act (CPU BF16 [rows, F]) against the oracle's SwiGLU of h = [gate | up]
    (CPU BF16 [rows, 2F]): equal, or the product of up with one of the two BF16
    neighbours of the oracle's BF16 silu, the latter only where the oracle's
    FP32 silu lies within 4 FP32 ulps of the BF16 rounding boundary between
    the two (the kernel's exp and reciprocal are within an ulp or two, so they
    may round silu to the other side).  Returns the number of such flips."""
    F = h.shape[1] // 2
    hb = to_oracle_input(h)
    ref, sb = oracle.swiglu(hb)
    sbf = torch.from_numpy(sb.view(np.int16)).view(torch.bfloat16).float()
    lo, hi = bf16_neighbours(sbf)
    u = h[:, F:].float()
    got = act.view(torch.int16).numpy().view(np.uint16)
    cand_lo = (lo * u).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    cand_hi = (hi * u).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    same = got == ref
    ok = same | (got == cand_lo) | (got == cand_hi)
    assert ok.all(), "%s: %d outputs off by more than one BF16 step of silu" % (
        what, int((~ok).sum()))
    g = h[:, :F].float().numpy()
    for r, c in np.argwhere(~same):
        sg = np.float32(oracle.silu_f32(float(g[r, c])))
        other = (lo if got[r, c] == cand_lo[r, c] else hi)[r, c].item()
        mid = (float(sbf[r, c]) + other) / 2.0
        assert abs(float(sg) - mid) <= 4 * float(np.spacing(np.abs(sg))), (what, g[r, c], sg, mid)
    return int((~same).sum())


def every_bf16_below(exp2: int) -> torch.Tensor:
    """Every finite BF16 value of magnitude at most M = 2^exp2 (both signs,
    denormals and zeros included), as BF16 [rows, 16] 1x16 blocks whose first
    element is M: the block maximum and the tensor amax, so every block gets
    the largest E4M3 scale and d = RN(448 * RN(M / 2688)), about M / 6.
    rows is a multiple of 16 (zero-padded)."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    vals = torch.from_numpy(bits[finite].astype(np.int32).astype(np.int16)).view(torch.bfloat16)
    m = float(2.0 ** exp2)
    vals = vals[vals.float().abs() <= m]
    nblk = (vals.numel() + 14) // 15
    rows = (nblk + 15) // 16 * 16
    x = torch.zeros(rows, 16, dtype=torch.bfloat16)
    x[:, 0] = m
    body = torch.zeros(rows * 15, dtype=torch.bfloat16)
    body[:vals.numel()] = vals
    x[:, 1:] = body.reshape(rows, 15)
    return x


def every_bf16_block_max(exp2: int) -> torch.Tensor:
    """One 1x16 block per finite BF16 value v with |v| <= M = 2^exp2 (both
    signs, zeros and denormals included): v first, then v times 15 fractions
    in [-1, 1] rounded to BF16 (never above |v|), so v is the block maximum;
    the first block holds M, the tensor amax.  BF16 [rows, 16], rows a
    multiple of 16 (padding rows are zero blocks)."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    vals = torch.from_numpy(bits[finite].astype(np.int32).astype(np.int16)).view(torch.bfloat16)
    m = float(2.0 ** exp2)
    vals = torch.cat([torch.tensor([m], dtype=torch.bfloat16), vals[vals.float().abs() <= m]])
    rows = (vals.numel() + 15) // 16 * 16
    frac = torch.tensor([-1.0, 0.875, -0.5, 0.3, -0.1, 0.05, -0.01, 1e-3, -1e-5, 1e-9, -0.7,
                         0.99, -0.26, 0.74, 0.0], dtype=torch.float32)
    x = torch.zeros(rows, 16, dtype=torch.bfloat16)
    x[:vals.numel(), 0] = vals
    x[:vals.numel(), 1:] = (vals.float()[:, None] * frac[None, :]).to(torch.bfloat16)
    return x
