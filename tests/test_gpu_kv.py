"""GPU parity of the NVFP4 KV cache (slot-mapped write of token rows, gathered
read) against the oracle, through the C ABI.  Both are bit-exact: the write
is the 1x16 RNE quantization of each token row under the fixed calibration
scale, the read is the exact dequantization of the gathered rows.

The NVIDIA-blog translation on juejin.cn (point 3) names the NVFP4 KV cache;
"FP4" (chaitex.ru, mathematical-structure section) gives the 16-element
blocks with E4M3 scales and the FP32 tensor scale.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import to_oracle_input

pytestmark = pytest.mark.gpu

SENTINEL = 0xA5


@pytest.fixture(scope="module")
def nv():
    import nvfp4_bit_microscaled_amd as m
    return m


def make_caches(nv, S, C, amax):
    cache = nv.kv_cache_create(S, C, amax)
    cache.codes.fill_(SENTINEL)
    cache.scales.fill_(SENTINEL)
    ref = (np.full((S, C // 2), SENTINEL, dtype=np.uint8),
           np.full((S, C // 16), SENTINEL, dtype=np.uint8))
    return cache, ref


def slots_with_padding(rng, T, S):
    # distinct valid slots plus padding entries on both sides of the range
    slots = rng.permutation(S)[:T].astype(np.int64)
    bad = rng.random(T) < 0.1
    slots[bad] = rng.choice([-1, -7, S, S + 3, 1 << 40], bad.sum())
    return slots


def check_cache(cache, ref, what):
    assert np.array_equal(cache.scales.cpu().numpy(), ref[1]), what + ": scales"
    assert np.array_equal(cache.codes.cpu().numpy(), ref[0]), what + ": codes"


# one block, several tiles of 256 threads, ragged thread counts, wide rows
SHAPES = [(1, 16, 1), (37, 1024, 100), (300, 128, 1000), (4096, 1024, 8192), (5, 4112, 9)]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("T,C,S", SHAPES)
def test_kv_write_bit_exact(nv, dtype, T, C, S):
    rng = np.random.default_rng(T * 7 + C + S)
    x = workloads.activations(T, C, T + C).to(dtype)
    if dtype == torch.float32:   # full FP32 mantissas, not only BF16 values
        g = torch.Generator().manual_seed(T + C)
        x = x * (1 + 1e-3 * torch.randn(T, C, generator=g))
    # calibration amax below the data's own: the largest features saturate
    amax = float(x.float().abs().max()) * (0.5 if T % 2 else 1.0)
    slots = slots_with_padding(rng, T, S)
    print("kv write", dtype, T, C, S, flush=True)
    cache, ref = make_caches(nv, S, C, amax)
    nv.kv_cache_write(cache, x.cuda(), torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    oracle.kv_cache_write(to_oracle_input(x), slots, amax, *ref)
    check_cache(cache, ref, "kv write %dx%d" % (T, C))


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_kv_read_bit_exact_with_repeats_and_padding(nv, out_dtype):
    rng = np.random.default_rng(21)
    S, C, n = 700, 512, 2000
    cc = rng.integers(0, 256, (S, C // 2), dtype=np.uint8)
    cs = rng.integers(0, 0x7F, (S, C // 16), dtype=np.uint8)     # every finite E4M3 code
    amax = 5.25
    slots = rng.integers(-5, S + 5, n).astype(np.int64)
    cache = nv.kv_cache_create(S, C, amax)
    cache.codes.copy_(torch.from_numpy(cc))
    cache.scales.copy_(torch.from_numpy(cs))
    print("kv read", out_dtype, flush=True)
    out = nv.kv_cache_read(cache, torch.from_numpy(slots).cuda(), out_dtype).cpu()
    f, b = oracle.kv_cache_read(cc, cs, amax, slots)
    if out_dtype == torch.float32:
        assert np.array_equal(out.numpy().view(np.uint32), f.view(np.uint32))
    else:
        assert np.array_equal(out.view(torch.int16).numpy().view(np.uint16), b)


def test_kv_strided_input_and_output(nv):
    rng = np.random.default_rng(4)
    T, C, S, pad = 64, 256, 128, 48
    xb = workloads.activations(T, C + pad, 3)
    x = xb.cuda()[:, 8:8 + C]                       # row pitch C + pad, 16-byte aligned start
    amax = 7.0
    slots = slots_with_padding(rng, T, S)
    cache, ref = make_caches(nv, S, C, amax)
    nv.kv_cache_write(cache, x, torch.from_numpy(slots).cuda())
    oracle.kv_cache_write(to_oracle_input(xb[:, 8:8 + C]), slots, amax, *ref)
    check_cache(cache, ref, "kv strided write")
    rs = rng.integers(-2, S + 2, 90).astype(np.int64)
    buf = torch.full((90, C + 40), -3.0, dtype=torch.float32, device="cuda")
    view = buf[:, 8:8 + C]
    nv.kv_cache_read(cache, torch.from_numpy(rs).cuda(), torch.float32, out=view)
    f, _ = oracle.kv_cache_read(*ref, amax, rs)
    assert np.array_equal(view.cpu().numpy().view(np.uint32), f.view(np.uint32))
    outside = torch.cat([buf[:, :8], buf[:, 8 + C:]], dim=1)
    assert torch.all(outside == -3.0)


def test_kv_prefill_then_decode_appends(nv):
    """A prefill batch in pages, then single-token appends, then one read of
    every sequence position: the cache and the read match the oracle after
    each step (writes touch only their own rows)."""
    C, S = 1024, 4096
    amax = torch.tensor([9.5], dtype=torch.float32, device="cuda")
    cache = nv.kv_cache_create(S, C, amax)
    ref = (np.zeros((S, C // 2), dtype=np.uint8), np.zeros((S, C // 16), dtype=np.uint8))
    T0 = 1000
    slots = workloads.paged_slots(T0 + 40, S, 5)
    x = workloads.activations(T0, C, 11)
    nv.kv_cache_write(cache, x.cuda(), slots[:T0].cuda())
    oracle.kv_cache_write(to_oracle_input(x), slots[:T0].numpy(), 9.5, *ref)
    for i in range(40):
        xi = workloads.activations(1, C, 100 + i)
        si = slots[T0 + i:T0 + i + 1]
        nv.kv_cache_write(cache, xi.cuda(), si.cuda())
        oracle.kv_cache_write(to_oracle_input(xi), si.numpy(), 9.5, *ref)
    torch.cuda.synchronize()
    check_cache(cache, ref, "kv appends")
    out = nv.kv_cache_read(cache, slots.cuda(), torch.bfloat16).cpu()
    _, b = oracle.kv_cache_read(*ref, 9.5, slots.numpy())
    assert np.array_equal(out.view(torch.int16).numpy().view(np.uint16), b)


def test_kv_empty_calls(nv):
    cache = nv.kv_cache_create(8, 64, 1.0)
    nv.kv_cache_write(cache, torch.empty(0, 64, dtype=torch.bfloat16, device="cuda"),
                      torch.empty(0, dtype=torch.int64, device="cuda"))
    out = nv.kv_cache_read(cache, torch.empty(0, dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    assert out.shape == (0, 64)
    assert torch.all(cache.codes == 0) and torch.all(cache.scales == 0)


@pytest.mark.parametrize("out_dtype", [torch.bfloat16, torch.float32])
def test_kv_read_from_an_empty_cache(nv, out_dtype):
    """A cache of zero slots: every slot is out of range, so every row reads
    as zeros (the library fills the output; no cache memory is touched)."""
    cache = nv.kv_cache_create(0, 64, 1.0)
    slots = torch.tensor([0, 3, -1, 7], dtype=torch.int64, device="cuda")
    out = torch.full((4, 64), 9.0, dtype=out_dtype, device="cuda")
    nv.kv_cache_read(cache, slots, out_dtype, out=out)
    torch.cuda.synchronize()
    assert torch.count_nonzero(out).item() == 0
    ref_f, ref_b = oracle.kv_cache_read(np.zeros((0, 32), np.uint8), np.zeros((0, 4), np.uint8),
                                        1.0, slots.cpu().numpy())
    assert not ref_f.any() and not ref_b.any()


def test_kv_cache_full_size_llama8b_layer(nv):
    """The bench's workload at one tensor's full size: 262144 tokens x 1024
    features written in pages over 262144 slots, then all read back in a
    different page order; writes bit-exact over the whole cache, reads on
    8192 sampled rows."""
    cfg = workloads.KVCACHE
    T, C, S = cfg["tokens"], cfg["cols"], cfg["num_slots"]
    x = workloads.activations(T, C, cfg["x_seed"])
    amax = float(x.float().abs().max())
    slots = workloads.paged_slots(T, S, cfg["slot_seed"])
    print("kv full size write", flush=True)
    cache = nv.kv_cache_create(S, C, amax)
    nv.kv_cache_write(cache, x.cuda(), slots.cuda())
    torch.cuda.synchronize()
    ref = (np.zeros((S, C // 2), dtype=np.uint8), np.zeros((S, C // 16), dtype=np.uint8))
    oracle.kv_cache_write(to_oracle_input(x), slots.numpy(), amax, *ref)
    check_cache(cache, ref, "kv full size")
    del x
    rslots = workloads.paged_slots(S, S, cfg["read_seed"])
    out = nv.kv_cache_read(cache, rslots.cuda(), torch.bfloat16)
    rng = np.random.default_rng(8)
    rows = rng.integers(0, S, 8192)
    rows[:2] = [0, S - 1]
    got = out[torch.from_numpy(rows).cuda()].cpu().view(torch.int16).numpy().view(np.uint16)
    _, b = oracle.kv_cache_read(*ref, amax, rslots.numpy()[rows])
    assert np.array_equal(got, b)


@pytest.mark.parametrize("amax", [1.0, 2.0 ** -100, 3.0e38])
def test_kv_write_every_bf16_value(nv, amax):
    """Every finite BF16 value as a feature of a token row (4080 features per
    row, 16 rows), written under calibration amaxes 1, 2^-100 and 3e38: the
    saturation of values past amax_cal, blocks whose scale underflows, signed
    zeros and denormals; the cache bytes and the read-back (BF16 and FP32)
    bit-exact against the oracle."""
    bits = np.arange(1 << 16, dtype=np.uint32)
    finite = ((bits >> 7) & 0xFF) != 0xFF
    x = torch.from_numpy(bits[finite].astype(np.int32).astype(np.int16)).view(torch.bfloat16)
    x = x.reshape(16, 4080)
    T, C, S = 16, 4080, 40
    slots = np.array([3, 39, 0, 17, 8, 25, 30, 1, 12, 33, 5, 21, 38, 9, 14, 27], dtype=np.int64)
    cache, ref = make_caches(nv, S, C, amax)
    nv.kv_cache_write(cache, x.cuda(), torch.from_numpy(slots).cuda())
    torch.cuda.synchronize()
    oracle.kv_cache_write(to_oracle_input(x), slots, amax, *ref)
    check_cache(cache, ref, "kv write every BF16 value, amax %g" % amax)
    rd = np.concatenate([slots[::-1], [-1, S]]).astype(np.int64)
    f, b = oracle.kv_cache_read(ref[0], ref[1], amax, rd)
    outf = nv.kv_cache_read(cache, torch.from_numpy(rd).cuda(), torch.float32).cpu()
    outb = nv.kv_cache_read(cache, torch.from_numpy(rd).cuda(), torch.bfloat16).cpu()
    assert np.array_equal(outf.numpy().view(np.uint32), f.view(np.uint32))
    assert np.array_equal(outb.view(torch.int16).numpy().view(np.uint16), b)
