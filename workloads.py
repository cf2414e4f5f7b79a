"""Seeded synthetic inputs and workload shapes shared by the tests, the bench and smoke().

This module holds no NVFP4 arithmetic: it only draws random tensors (with
torch's own generators) and names the shapes of the workloads.  Both the
HIP path and the CPU oracle receive the tensors it returns.

Distributions (the pages name the workloads but publish no data):
  activations  z ~ N(0,1), u ~ U[0,1) drawn after z from the same generator,
               x = 50 z where u < 0.001 else z   (0.1 % outliers x50; the
               recipe page stresses outliers in activations)
  weights      0.02 * N(0,1)
  gradients    1e-3 * Student-t(3), t = g0 / sqrt((g1^2 + g2^2 + g3^2) / 3)
               with g0..g3 ~ N(0,1) drawn in that order
All tensors are produced in FP32 and cast to BF16 (round to nearest even).

The token count of the Llama-shaped workloads (32768 = seq 8192 x batch 4)
follows the benchmark described on the readjensen.com NVFP4 training-recipe
page (benchmark paragraph); model dims are those of Llama 3 8B and of one
GPU's token share of Llama 3.1 405B.
"""
from __future__ import annotations

import torch


def _gen(seed: int, device: str) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def activations(rows: int, cols: int, seed: int, device: str = "cpu") -> torch.Tensor:
    g = _gen(seed, device)
    z = torch.randn(rows, cols, generator=g, device=device, dtype=torch.float32)
    u = torch.rand(rows, cols, generator=g, device=device, dtype=torch.float32)
    x = torch.where(u < 0.001, z * 50.0, z)
    del z, u
    return x.to(torch.bfloat16)


def weights(rows: int, cols: int, seed: int, device: str = "cpu") -> torch.Tensor:
    g = _gen(seed, device)
    return (torch.randn(rows, cols, generator=g, device=device, dtype=torch.float32) * 0.02).to(
        torch.bfloat16)


def gradients(rows: int, cols: int, seed: int, device: str = "cpu") -> torch.Tensor:
    g = _gen(seed, device)
    g0 = torch.randn(rows, cols, generator=g, device=device, dtype=torch.float32)
    den = torch.zeros_like(g0)
    for _ in range(3):
        gi = torch.randn(rows, cols, generator=g, device=device, dtype=torch.float32)
        den.addcmul_(gi, gi)
        del gi
    den.div_(3.0).sqrt_()
    t = g0.div_(den).mul_(1e-3)
    del den
    return t.to(torch.bfloat16)


def sign_mask(seed: int) -> int:
    """16 random sign bits for the Hadamard transform (an input to the method)."""
    g = _gen(seed, "cpu")
    return int(torch.randint(0, 1 << 16, (1,), generator=g).item())


def paged_slots(tokens: int, num_slots: int, seed: int, page: int = 16) -> torch.Tensor:
    """Cache slot of each token for a paged cache: tokens fill pages of `page`
    consecutive slots in order, and the pages are a seeded random choice of
    the cache's num_slots / page pages (int64 [tokens])."""
    g = _gen(seed, "cpu")
    npages = (tokens + page - 1) // page
    assert npages * page <= num_slots
    pages = torch.randperm(num_slots // page, generator=g)[:npages]
    t = torch.arange(tokens)
    return pages[t // page] * page + t % page


def bf16_bits(x: torch.Tensor):
    """BF16 CPU tensor -> numpy uint16 bit patterns (for the oracle)."""
    assert x.dtype == torch.bfloat16
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")


# Workload shapes ----------------------------------------------------------

# Tiny: 256x256 activation tensor, GEMM on its first 128 rows against a
# 128x256 weight (2D blocks).
TINY = dict(act=(256, 256), act_seed=0, w=(128, 256), w_seed=1, gemm=(128, 128, 256))

# Llama-3-8B MLP at 32768 tokens: hidden 4096, intermediate 14336 (gate+up
# fused into one 28672-wide GEMM).
LLAMA8B = dict(tokens=32768, hidden=4096, ffn=14336, x_seed=0, wgu_seed=2, wdown_seed=3,
               dy_seed=4, dh_seed=5, sr_seed=1, mask_seed=1)

# Decode-style skinny GEMM: activations [M, 8192] for M in {1, 16, 32, 64},
# weights [28672, 8192] pre-quantized 1x16 along K.
DECODE = dict(ms=(1, 16, 32, 64), k=8192, n=28672, act_seed=6, w_seed=7)

# One GPU's token share of a Llama-3.1-405B MLP: 8192 tokens, hidden 16384,
# intermediate 53248.
LLAMA405B = dict(tokens=8192, hidden=16384, ffn=53248, x_seed=8, wgu_seed=9, wdown_seed=10,
                 dy_seed=11, dh_seed=12, sr_seed=1, mask_seed=1)

# NVFP4 KV cache of a Llama-3-8B-shaped model: 8 KV heads x head dim 128 =
# 1024 features per token for K (and again for V); 262144 tokens (8 sequences
# of 32768) scattered over a cache of as many slots in pages of 16.
KVCACHE = dict(tokens=262144, cols=1024, num_slots=262144, x_seed=13, slot_seed=14, read_seed=15)
