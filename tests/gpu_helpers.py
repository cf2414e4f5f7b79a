"""Shared helpers for the GPU parity tests (no NVFP4 arithmetic here)."""
from __future__ import annotations

import numpy as np
import torch


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
