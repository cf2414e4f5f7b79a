"""Pins for the oracle's element/scale formats (CPU only).

E2M1 bit split and the per-16 E4M3 + FP32 two-level scheme: guiahardware.es
"NVFP4: cos'e e come supera FP8 e BF16", section "Cos'e NVFP4"; chaitex.ru
"FP4", section on the mathematical structure of FP4.
"""
import json
import math
import os
import struct

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _facts():
    with open(os.path.join(GOLDEN, "format_facts.json")) as f:
        return json.load(f)


def test_e2m1_decodes_to_the_value_set():
    facts = _facts()
    assert facts["e2m1_field_bits"] == {**facts["e2m1_field_bits"], "sign": 1, "exponent": 2,
                                        "mantissa": 1}
    vals = [oracle.e2m1_value(c) for c in range(16)]
    assert vals[:8] == facts["e2m1_value_set"]
    assert vals[8:] == [-v for v in facts["e2m1_value_set"]]
    # bit 3 is the sign bit: -0.0 for code 8
    assert math.copysign(1.0, vals[8]) == -1.0
    assert max(abs(v) for v in vals) == 6.0


def test_e4m3_decode_matches_torch_for_all_codes():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float32).numpy()
    got = np.array([oracle.e4m3_value(c) for c in range(256)], dtype=np.float32)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert oracle.e4m3_value(0x7E) == _facts()["e4m3_max"]


def _e4m3_sweep():
    """FP32 test points in [0, 470]: every E4M3 value, every midpoint between
    neighbours and the FP32 values one ulp either side, plus random points."""
    vals = sorted({oracle.e4m3_value(c) for c in range(0x7F)})
    pts = []
    for a, b in zip(vals[:-1], vals[1:]):
        m = np.float32((a + b) / 2)
        pts += [a, m, np.nextafter(m, np.float32(0)), np.nextafter(m, np.float32(1e9))]
    pts += [448.0, 455.0, 463.99, 464.0, 470.0, 2.0 ** -10, 2.0 ** -11, 1e-30, 0.0]
    rng = np.random.default_rng(0)
    pts += list(np.exp(rng.uniform(np.log(1e-4), np.log(460), 4000)))
    return np.array(pts, dtype=np.float32)


def test_e4m3_encode_matches_torch_rne_cast():
    t = _e4m3_sweep()
    # torch's cast rounds to nearest even but turns values >= 464 into NaN;
    # the method saturates, so clamp to 448 before the library cast.
    ref = torch.from_numpy(np.minimum(t, 448.0)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.e4m3_encode(float(v)) for v in t], dtype=np.uint8)
    assert np.array_equal(ref, got)


def test_e4m3_encode_saturates():
    for t in [448.0, 464.0, 500.0, 1e30, float("inf")]:
        assert oracle.e4m3_encode(t) == 0x7E


def test_e2m1_rne_worked_ties():
    with open(os.path.join(GOLDEN, "e2m1_rne_ties.json")) as f:
        cases = json.load(f)["cases"]
    for y, code in cases:
        assert oracle.e2m1_encode_rne(y) == code, y
    assert oracle.e2m1_encode_rne(-0.0) == 8
    assert oracle.e2m1_encode_rne(float("inf")) == 7


def _all_finite_bf16_as_f32():
    bits = np.arange(1 << 16, dtype=np.uint32) << 16
    f = bits.view(np.float32)
    return f[np.isfinite(f)]


def test_e2m1_rne_exhaustive_bf16_is_nearest_even():
    y = _all_finite_bf16_as_f32()
    codes = np.array([oracle.e2m1_encode_rne(float(v)) for v in y], dtype=np.int64)
    grid = np.array([0, .5, 1, 1.5, 2, 3, 4, 6], dtype=np.float64)
    a = np.abs(y.astype(np.float64))
    mag = codes & 7
    # saturation: everything at or beyond 6 maps to the largest magnitude
    assert np.all(mag[a >= 6.0] == 7)
    inr = a < 6.0
    a, mag = a[inr], mag[inr]
    dist = np.abs(a[:, None] - grid[None, :])
    best = dist.min(axis=1)
    # chosen magnitude is a nearest grid point
    assert np.array_equal(dist[np.arange(len(a)), mag], best)
    # among ties the even code wins
    ties = (dist == best[:, None]).sum(axis=1) > 1
    assert np.all(mag[ties] % 2 == 0)
    # sign bit follows the IEEE sign
    assert np.array_equal((codes >> 3) & 1, np.signbit(y).astype(np.int64))
    assert ties.sum() == 7 * 2  # the seven midpoints, each with either sign


def test_e2m1_sr_stays_on_neighbours_and_hits_frac():
    grid = [0, .5, 1, 1.5, 2, 3, 4, 6]
    for y in [0.1, 0.3, 0.7, 1.2, 1.9, 2.25, 3.9, 5.5, -0.6, -4.5]:
        y = float(np.float32(y))  # the oracle takes FP32 quotients
        a = abs(y)
        lo = max(g for g in grid if g <= a)
        hi = min(g for g in grid if g > a)
        frac = (a - lo) / (hi - lo)
        # r = 0 always rounds up (frac > 0); r = 2^32-1 never does (frac < 1)
        assert oracle.e2m1_value(oracle.e2m1_encode_sr(y, 0)) == math.copysign(hi, y)
        assert oracle.e2m1_value(oracle.e2m1_encode_sr(y, 0xFFFFFFFF)) == math.copysign(lo, y)
        # threshold: up iff r < frac * 2^32
        thr = frac * 2.0 ** 32
        r_up = int(math.ceil(thr)) - 1
        assert oracle.e2m1_value(oracle.e2m1_encode_sr(y, r_up)) == math.copysign(hi, y)
        assert oracle.e2m1_value(oracle.e2m1_encode_sr(y, r_up + 1)) == math.copysign(lo, y)
    # representable values never move, whatever the word
    for c in range(16):
        v = oracle.e2m1_value(c)
        for r in [0, 1, 12345, 0x80000000, 0xFFFFFFFF]:
            assert oracle.e2m1_encode_sr(v, r) == c
    assert oracle.e2m1_encode_sr(9.0, 0) == 7


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(1)
    f = np.concatenate([
        rng.standard_normal(20000).astype(np.float32) * np.float32(1e3),
        np.array([0.0, -0.0, 1.0, 3.3895314e38, 1e-40, -1e-40, 1.00390625, 1.01171875],
                 dtype=np.float32),
        # exact ties between bf16 neighbours
        (np.arange(1 << 12, dtype=np.uint32) << 15 | 0x3F800000).view(np.float32),
    ])
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = np.array([oracle.f32_to_bf16(float(v)) for v in f], dtype=np.uint16)
    assert np.array_equal(ref, got)


def test_float32_helpers_are_ieee():
    # the oracle relies on IEEE single rounding: 1/3 in FP32
    assert struct.unpack("<f", struct.pack("<f", 1 / 3))[0] == np.float32(1) / np.float32(3)
