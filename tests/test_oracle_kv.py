"""Pins for the oracle's NVFP4 KV-cache write and read (CPU only).

The juejin.cn translation of the NVIDIA blog (point 3, the ecosystem) lists
an NVFP4 KV cache among the format's inference uses; "FP4" (chaitex.ru,
mathematical-structure section) gives the layout: 16-element micro-blocks
with an E4M3 scale and an FP32 tensor scale.  Reading taken: 1x16 blocks
along the features, round to nearest-even, a fixed tensor scale
s_g = RN(amax_cal / 2688) from a calibration amax, token t written to cache
row slots[t], out-of-range slots skipped on write and read as zero rows.

Pinned here by constructed rows whose codes and scales are known without
the oracle, torch's float8_e4m3fn decoding for the read, the saturation
closed form, and the untouched rows around every write.
"""
import numpy as np
import pytest
import torch

import oracle

E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def empty_cache(num_slots, cols, fill=0xA5):
    return (np.full((num_slots, cols // 2), fill, dtype=np.uint8),
            np.full((num_slots, cols // 16), fill, dtype=np.uint8))


def e4m3_values():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().numpy()


def constructed_rows(rng, tokens, cols, k):
    """Rows whose quantization is known in closed form under amax_cal =
    2688 * 2^k (so s_g = 2^k exactly): each block is 2^k * e * v with v drawn
    from the E2M1 set, e a random E4M3 value in [2^-6, 448], and one element
    of magnitude 6 * e so that a_B / (6 s_g) = e exactly.  Returns
    (x fp32, codes, scales)."""
    ev = e4m3_values()
    normal_codes = np.array([c for c in range(0x08, 0x7F)])   # 2^-6 .. 448
    x = np.zeros((tokens, cols), dtype=np.float64)
    codes = np.zeros((tokens, cols // 2), dtype=np.uint8)
    scales = np.zeros((tokens, cols // 16), dtype=np.uint8)
    for t in range(tokens):
        for b in range(cols // 16):
            ec = int(rng.choice(normal_codes))
            m = rng.integers(0, 8, 16)
            s = rng.integers(0, 2, 16)
            m[rng.integers(0, 16)] = 7
            q = (s << 3) | m
            vals = np.where(s == 1, -1.0, 1.0) * E2M1[m]
            x[t, 16 * b:16 * b + 16] = vals * float(ev[ec]) * 2.0 ** k
            scales[t, b] = ec
            for j in range(16):
                c = 16 * b + j
                codes[t, c // 2] |= np.uint8(q[j] << (4 * (c & 1)))
    return x.astype(np.float32), codes, scales


@pytest.mark.parametrize("k", [-20, 0, 7])
def test_constructed_rows_land_in_their_slots(k):
    rng = np.random.default_rng(100 + k)
    T, C, S = 12, 64, 40
    x, codes, scales = constructed_rows(rng, T, C, k)
    assert np.array_equal(x.astype(np.float64), x)     # exact in FP32
    slots = rng.permutation(S)[:T]
    cc, cs = empty_cache(S, C)
    oracle.kv_cache_write(x, slots, 2688.0 * 2.0 ** k, cc, cs)
    assert np.array_equal(cc[slots], codes)
    assert np.array_equal(cs[slots], scales)
    others = np.setdiff1d(np.arange(S), slots)
    assert np.all(cc[others] == 0xA5) and np.all(cs[others] == 0xA5)
    # the read gives the constructed values back exactly, in slot order
    f, b = oracle.kv_cache_read(cc, cs, 2688.0 * 2.0 ** k, slots)
    assert np.array_equal(f, x)
    bt = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(b, bt)


def test_read_matches_torch_e4m3_decoding():
    # random cache bytes (scales below the NaN code): v = RN32(val * e * s_g)
    rng = np.random.default_rng(7)
    S, C, n = 30, 96, 50
    cc = rng.integers(0, 256, (S, C // 2), dtype=np.uint8)
    cs = rng.integers(0, 0x7F, (S, C // 16), dtype=np.uint8)
    amax = np.float32(3.7)
    slots = rng.integers(-3, S + 3, n)
    f, _ = oracle.kv_cache_read(cc, cs, float(amax), slots)
    s_g = np.float32(amax / np.float32(2688.0))
    ev = e4m3_values()
    for j, s in enumerate(slots):
        if s < 0 or s >= S:
            assert np.all(f[j] == 0) and not np.any(np.signbit(f[j]))
            continue
        nib = np.stack([cc[s] & 0xF, cc[s] >> 4], axis=1).reshape(-1)
        val = np.where(nib & 8, -1.0, 1.0) * E2M1[nib & 7]
        e = np.repeat(ev[cs[s]], 16)
        want = (val * e).astype(np.float32) * s_g      # val*e exact, one FP32 rounding
        assert np.array_equal(f[j].view(np.uint32), want.astype(np.float32).view(np.uint32))


def test_values_beyond_calibration_saturate():
    k = 3
    amax = 2688.0 * 2.0 ** k
    x = np.zeros((2, 32), dtype=np.float32)
    x[0, 0] = 10 * amax
    x[0, 5] = -3 * amax
    x[1, 17] = -amax                  # exactly at the calibration amax
    cc, cs = empty_cache(4, 32)
    oracle.kv_cache_write(x, np.array([2, 0]), amax, cc, cs)
    assert cs[2, 0] == 0x7E and cs[0, 1] == 0x7E          # E4M3 448
    f, _ = oracle.kv_cache_read(cc, cs, amax, np.array([2, 0]))
    assert f[0, 0] == amax and f[0, 5] == -amax            # 6 * 448 * 2^k
    assert f[1, 17] == -amax
    assert np.count_nonzero(f) == 3


def test_invalid_slots_skip_writes_and_read_zero():
    rng = np.random.default_rng(3)
    T, C, S = 6, 32, 5
    x = rng.standard_normal((T, C)).astype(np.float32)
    slots = np.array([-1, 4, 5, 1, -100, 1 << 40])
    cc, cs = empty_cache(S, C)
    oracle.kv_cache_write(x, slots, 4.0, cc, cs)
    for r in (0, 2, 3):
        assert np.all(cc[r] == 0xA5) and np.all(cs[r] == 0xA5)
    # rows 4 and 1 hold tokens 1 and 3 quantized alone
    for t, s in ((1, 4), (3, 1)):
        c1, s1, _, _ = oracle.quantize(x[t:t + 1], amax_in=4.0)
        assert np.array_equal(cc[s], c1[0]) and np.array_equal(cs[s], s1[0])
    f, b = oracle.kv_cache_read(cc, cs, 4.0, slots)
    for j in (0, 2, 4, 5):
        assert np.all(f[j] == 0) and np.all(b[j] == 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_identity_slots_equal_tensor_quantize(dtype):
    # slots 0..T-1 make the cache the 1x16 RNE quantization of the whole
    # tensor under amax_in = the calibration amax
    rng = np.random.default_rng(5)
    T, C = 33, 128
    x = (rng.standard_normal((T, C)) * np.exp(rng.standard_normal((T, 1)))).astype(np.float32)
    if dtype == "bf16":
        x = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    amax = 2.5
    cc, cs = empty_cache(T, C)
    oracle.kv_cache_write(x, np.arange(T), amax, cc, cs)
    codes, scales, s_g, _ = oracle.quantize(x, amax_in=amax)
    assert np.array_equal(cc, codes) and np.array_equal(cs, scales)
    f, b = oracle.kv_cache_read(cc, cs, amax, np.arange(T))
    f2, b2 = oracle.dequantize(codes, scales, s_g, T, C)
    assert np.array_equal(f, f2) and np.array_equal(b, b2)
