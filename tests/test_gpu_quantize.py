"""GPU parity: nvfp4_quantize / nvfp4_rht16 / nvfp4_dequantize against the CPU oracle.

Codes, scales, the tensor scale and amax must be bit-identical (integer
results decided in FP32 on both sides under the documented convention).
Sources: two-level microscaling -- guiahardware.es "NVFP4: cos'e e come supera
FP8 e BF16", section "Cos'e NVFP4"; 2D weight blocks, RHT on wgrad inputs and
stochastic rounding of gradients -- readjensen.com NVFP4 recipe paragraph.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from gpu_helpers import every_bf16_block_max, every_bf16_below, to_oracle_input

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import nvfp4_bit_microscaled_amd as m
    torch.cuda.set_device(0)
    return m


MODES = {"rows": dict(block2d=False, axis=1), "cols": dict(block2d=False, axis=0),
         "2d": dict(block2d=True, axis=1)}


def gen(kind, rows, cols, seed, dtype=torch.bfloat16):
    f = {"act": workloads.activations, "w": workloads.weights, "grad": workloads.gradients}[kind]
    x = f(rows, cols, seed=seed)
    return x if dtype == torch.bfloat16 else x.to(torch.float32)


def compare(nv, x_cpu, mode, sr=False, rht=False, mask=0, seed=0, stream_id=0, ld_pad=0,
            amax_in=None):
    rows, cols = x_cpu.shape
    if ld_pad:
        wide = torch.zeros(rows, cols + ld_pad, dtype=x_cpu.dtype)
        wide[:, :cols] = x_cpu
        xg = wide.cuda()[:, :cols]
    else:
        xg = x_cpu.cuda()
    ain = None if amax_in is None else torch.tensor([amax_in], dtype=torch.float32, device="cuda")
    q = nv.quantize(xg, sr=sr, rht=rht, mask=mask, seed=seed, stream_id=stream_id, amax_in=ain,
                    **MODES[mode])
    torch.cuda.synchronize()
    oc, osc, ots, oam = oracle.quantize(to_oracle_input(x_cpu), sr=sr, rht=rht, mask=mask,
                                        seed=seed, stream_id=stream_id, amax_in=amax_in,
                                        **MODES[mode])
    assert q.tensor_scale.item() == ots
    assert q.amax.item() == oam
    gc, gs = q.codes.cpu().numpy(), q.scales.cpu().numpy()
    nbad_s = int((gs != osc).sum())
    nbad_c = int((gc != oc).sum())
    assert nbad_s == 0 and nbad_c == 0, "%d scale bytes and %d code bytes differ" % (nbad_s, nbad_c)
    return q


SHAPES = [(256, 256), (48, 272), (16, 16), (528, 1040), (96, 4112)]


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("kind", ["act", "w", "grad"])
def test_rne_matches_oracle(nv, mode, shape, kind):
    compare(nv, gen(kind, *shape, seed=hash((mode, shape, kind)) & 0xFFFF), mode)


@pytest.mark.parametrize("mode", list(MODES))
@pytest.mark.parametrize("shape", [(256, 256), (48, 272), (528, 1040)])
def test_sr_matches_oracle(nv, mode, shape):
    x = gen("grad", *shape, seed=7)
    compare(nv, x, mode, sr=True, seed=1, stream_id=0)
    compare(nv, x, mode, sr=True, seed=0xDEADBEEF12345, stream_id=3)


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("sr", [False, True])
@pytest.mark.parametrize("shape", [(256, 256), (48, 272), (528, 1040)])
def test_rht_quantize_matches_oracle(nv, axis, sr, shape):
    x = gen("grad" if sr else "act", *shape, seed=11)
    mode = "rows" if axis == 1 else "cols"
    compare(nv, x, mode, sr=sr, rht=True, mask=workloads.sign_mask(1), seed=1, stream_id=1)


@pytest.mark.parametrize("mode", list(MODES))
def test_fp32_input_strided_and_amax_in(nv, mode):
    x = gen("act", 64, 320, seed=3, dtype=torch.float32)
    compare(nv, x, mode, ld_pad=16)
    compare(nv, x.to(torch.bfloat16), mode, ld_pad=48)
    compare(nv, x, mode, amax_in=123.5)
    compare(nv, x, mode, sr=True, seed=5, amax_in=float(x.abs().max()) * 4)


def test_edge_values(nv):
    rows, cols = 32, 64
    x = torch.zeros(rows, cols, dtype=torch.float32)
    x[0, 0] = 2688.0                      # s_g = 1
    x[1, 16:32] = 1e-4                    # scale underflows: zero block
    x[2, 32:48] = -0.0                    # all-zero block
    x[3, 48] = 6 * 2.0 ** -9 * 1.0001     # smallest subnormal E4M3 scale
    x[3, 49] = -0.0
    x[4, :16] = torch.tensor([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.0, -0.25, -0.75, -1.25,
                              -1.75, -2.5, -3.5, -5.0, -6.0]) * (6.0 / 6.0)  # exact E2M1 midpoints
    x[5, :16] = torch.tensor([1e-40, -1e-40, 3e-39, 1.17e-38, 1e-30, 7.0, 100.0, -1e-45,
                              0.0, 2.0 ** -126, 2.0 ** -149, 5.9, 6.1, -6.1, 0.1, 0.3])
    x[6:8, :] = torch.randn(2, cols) * 1e-38  # subnormal-range values
    for mode in MODES:
        compare(nv, x, mode)
        compare(nv, x, mode, sr=True, seed=2)
    compare(nv, x, "rows", rht=True, mask=0xBEEF)
    compare(nv, x, "cols", rht=True, mask=0xBEEF, sr=True, seed=3)
    # all-zero and tiny tensors
    for mode in MODES:
        compare(nv, torch.zeros(16, 32), mode)
        compare(nv, torch.full((16, 32), 1e-42), mode)


def test_empty_tensor_writes_zero_scale(nv):
    x = torch.empty(0, 64, dtype=torch.bfloat16, device="cuda")
    q = nv.quantize(x)
    torch.cuda.synchronize()
    assert q.tensor_scale.item() == 0.0 and q.amax.item() == 0.0


def test_rht16_standalone_matches_oracle(nv):
    for axis in (0, 1):
        for dtype in (torch.bfloat16, torch.float32):
            x = gen("act", 528, 1040, seed=9, dtype=dtype)
            y = nv.rht16(x.cuda(), axis, 0x5A3C)
            torch.cuda.synchronize()
            ref = oracle.rht16(to_oracle_input(x), axis=axis, mask=0x5A3C)
            assert np.array_equal(y.cpu().numpy().view(np.uint32), ref.view(np.uint32))


def test_fused_rht_equals_rht_then_quantize(nv):
    x = gen("grad", 256, 512, seed=12)
    xg = x.cuda()
    for axis in (0, 1):
        y = nv.rht16(xg, axis, 0x1234)
        q1 = nv.quantize(xg, axis=axis, rht=True, mask=0x1234, sr=True, seed=1, stream_id=1)
        q2 = nv.quantize(y, axis=axis, sr=True, seed=1, stream_id=1)
        torch.cuda.synchronize()
        assert torch.equal(q1.codes, q2.codes) and torch.equal(q1.scales, q2.scales)
        assert q1.tensor_scale.item() == q2.tensor_scale.item()


@pytest.mark.parametrize("mode", list(MODES))
def test_dequantize_matches_oracle(nv, mode):
    x = gen("act", 528, 1040, seed=4)
    oc, osc, ots, _ = oracle.quantize(to_oracle_input(x), **MODES[mode])
    t = nv.NVFP4Tensor(torch.from_numpy(oc).cuda(), torch.from_numpy(osc).cuda(),
                       torch.tensor([ots], dtype=torch.float32, device="cuda"),
                       torch.zeros(1, device="cuda"), 528, 1040, MODES[mode]["block2d"],
                       MODES[mode]["axis"])
    f = nv.dequantize(t, torch.float32)
    b = nv.dequantize(t, torch.bfloat16)
    torch.cuda.synchronize()
    rf, rb = oracle.dequantize(oc, osc, ots, 528, 1040, **MODES[mode])
    assert np.array_equal(f.cpu().numpy().view(np.uint32), rf.view(np.uint32))
    assert np.array_equal(b.cpu().view(torch.int16).numpy().view(np.uint16), rb)


def test_deterministic_and_stream_ordered(nv):
    x = gen("grad", 512, 1024, seed=21).cuda()
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        q1 = nv.quantize(x, axis=0, rht=True, mask=7, sr=True, seed=9)
        q2 = nv.quantize(x, axis=0, rht=True, mask=7, sr=True, seed=9)
    s.synchronize()
    assert torch.equal(q1.codes, q2.codes) and torch.equal(q1.scales, q2.scales)
    q3 = nv.quantize(x, axis=0, rht=True, mask=7, sr=True, seed=10)
    torch.cuda.synchronize()
    assert not torch.equal(q1.codes, q3.codes)


def test_debug_mode_reports_nonfinite_amax(nv, monkeypatch):
    """With NVFP4_DEBUG=1 the quantizer synchronizes once and refuses a tensor
    whose amax is not finite (NVFP4_ERR_NONFINITE), writing no codes; finite
    tensors quantize as without the flag."""
    monkeypatch.setenv("NVFP4_DEBUG", "1")
    x = workloads.activations(32, 64, 3).cuda()
    ok = nv.quantize(x)
    monkeypatch.delenv("NVFP4_DEBUG")
    ref = nv.quantize(x)
    assert torch.equal(ok.codes, ref.codes) and torch.equal(ok.scales, ref.scales)
    monkeypatch.setenv("NVFP4_DEBUG", "1")
    bad = x.clone()
    bad[3, 5] = float("inf")
    codes = torch.full((32, 32), 0x5A, dtype=torch.uint8, device="cuda")
    scales = torch.full((32, 4), 0x5A, dtype=torch.uint8, device="cuda")
    ts = torch.zeros(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(nv.nvfp4_quantize_workspace_size(32, 64), dtype=torch.uint8, device="cuda")
    st = nv.nvfp4_quantize(bad, nv.DTYPE_BF16, 32, 64, 64, nv.BLOCK_1D, 1, 0, nv.ROUND_RNE, 0, 0,
                           0, 0, None, None, codes, scales, ts, ws, ws.numel())
    torch.cuda.synchronize()
    assert st == 8, nv.status_string(st)
    assert torch.all(codes == 0x5A) and torch.all(scales == 0x5A)


def h16():
    i = np.arange(16)
    return np.where(np.bitwise_count((i[:, None] & i[None, :]).astype(np.uint64)) % 2 == 1,
                    -1.0, 1.0)


def inverse_rht16(y, mask, axis):
    """x with RHT16(x) = y up to FP32 rounding: x = D (1/4 H y) per group of 16
    along `axis` (H symmetric, H H = 16 I, D = D^-1)."""
    d = np.array([-1.0 if (mask >> i) & 1 else 1.0 for i in range(16)])
    H = h16()
    y = np.asarray(y, dtype=np.float64)
    if axis == 1:
        g = y.reshape(y.shape[0], -1, 16)
        x = np.einsum("ij,rgj->rgi", H, g) * 0.25 * d
        return x.reshape(y.shape).astype(np.float32)
    g = y.reshape(-1, 16, y.shape[1])
    x = np.einsum("ij,gjc->gic", H, g) * 0.25 * d[None, :, None]
    return x.reshape(y.shape).astype(np.float32)


@pytest.mark.parametrize("s_g", [1.0, 1.37, 2.0 ** -20 * 1.9])
@pytest.mark.parametrize("mode", list(MODES) + ["rows_rht", "cols_rht", "cols_rht_t"])
def test_quotients_around_every_e2m1_boundary(nv, s_g, mode):
    """Elements whose quotient x/d lands on and within 6 FP32 ulps of every
    E2M1 rounding boundary (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5), both signs,
    under every positive normal E4M3 block scale: the round-to-nearest path
    (which multiplies by the block's reciprocal and takes the exact quotient
    only near a boundary) must encode exactly as the oracle's correctly
    rounded quotient.  FP32 input; the tensor amax sits in the first block.
    The *_rht modes feed the inverse transform of these values, so the
    Hadamard-transformed quotients land on or next to the boundaries (exactly
    where the inverse is exact in FP32); cols_rht_t writes transposed
    storage."""
    f32 = np.float32
    amax = f32(2688.0) * f32(s_g)
    sg = f32(amax / f32(2688.0))
    d6 = f32(f32(6.0) * sg)
    probes = []
    for m in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0):
        for j in range(-6, 7):
            probes.append((m, j))
    blocks = []
    for code in range(0x08, 0x7F):              # normal E4M3 scales 2^-6 .. 448
        e = f32(oracle.e4m3_value(code))
        aB = f32(e * d6)                         # block amax giving this scale
        d = f32(e * sg)
        vals = []
        for sign in (1.0, -1.0):
            for m, j in probes:
                x = np.nextafter(f32(f32(m) * d), f32(np.inf) if j > 0 else f32(-np.inf),
                                 dtype=np.float32) if j else f32(f32(m) * d)
                for _ in range(abs(j) - 1):
                    x = np.nextafter(x, f32(np.inf) if j > 0 else f32(-np.inf), dtype=np.float32)
                vals.append(f32(sign) * x)
        for k in range(0, len(vals), 15):
            blk = [aB] + vals[k:k + 15]
            blk += [f32(0.0)] * (16 - len(blk))
            blocks.append(blk)
    nb = len(blocks)
    cols = 256
    rows = (nb * 16 + cols - 1) // cols
    rows = (rows + 15) // 16 * 16
    flat = np.zeros(rows * cols, dtype=np.float32)
    flat[0] = amax
    flat[16:16 + nb * 16] = np.asarray(blocks, dtype=np.float32).ravel()
    x = torch.from_numpy(flat.reshape(rows, cols))
    if mode.startswith("cols"):     # the same blocks down the columns
        x = x.reshape(rows // 16, 16, cols // 16, 16).permute(0, 3, 2, 1).reshape(rows, cols)
        x = x.contiguous()
    if not mode.endswith(("rht", "rht_t")):
        compare(nv, x, mode)
        return
    mask = 0x5A3C
    axis = 1 if mode == "rows_rht" else 0
    x = torch.from_numpy(inverse_rht16(x.numpy(), mask, axis))
    if mode == "cols_rht_t":
        q = nv.quantize(x.cuda(), axis=0, rht=True, mask=mask, transpose=True)
        torch.cuda.synchronize()
        oc, osc, ots, _ = oracle.quantize(to_oracle_input(x), axis=0, rht=True, mask=mask)
        assert q.tensor_scale.item() == ots
        qc = q.codes.cpu().numpy()
        tq = np.empty((qc.shape[0], qc.shape[1] * 2), dtype=np.uint8)
        tq[:, 0::2], tq[:, 1::2] = qc & 0xF, qc >> 4
        oq = np.empty((oc.shape[0], oc.shape[1] * 2), dtype=np.uint8)
        oq[:, 0::2], oq[:, 1::2] = oc & 0xF, oc >> 4
        assert np.array_equal(tq, oq.T) and np.array_equal(q.scales.cpu().numpy(), osc.T)
        return
    compare(nv, x, "rows" if axis == 1 else "cols", rht=True, mask=mask)


@pytest.mark.parametrize("exp2", [0, -30, -37, -38, 60, 100, 127])
def test_every_bf16_element_value(nv, exp2):
    """Every finite BF16 value up to M = 2^exp2 as an element of blocks whose
    maximum is M (d about M / 6): round-to-nearest codes of denormal and tiny
    elements (below 2^-60) where d >= 2^-40 (M up to 2^-37 and 2^60, which
    skip the per-element tiny-operand test), where d is below it (2^-38) or
    beyond Markstein's range (2^100, 2^127), and of every other magnitude;
    rows, columns (the same blocks down the columns) and 16x16 blocks, BF16
    and FP32 input, plus stochastic rounding on the rows, and the same blocks
    through the RHT16 (RNE rows, SR columns).  Bit-exact against the
    oracle."""
    x = every_bf16_below(exp2)
    compare(nv, x, "rows")
    compare(nv, x.float(), "rows")
    compare(nv, x.t().contiguous(), "cols")
    compare(nv, x, "2d")
    compare(nv, x, "rows", sr=True, seed=9)
    # the same blocks through the transform (RNE takes the reciprocal fast path
    # there), where its sums of 16 values stay finite: at M = 2^127 they
    # overflow FP32, an infinite transformed amax, outside the finite-input
    # contract
    if exp2 <= 100:
        compare(nv, x, "rows", rht=True, mask=0x6C1B)
        compare(nv, x.t().contiguous(), "cols", rht=True, mask=0x6C1B, sr=True, seed=10)


@pytest.mark.parametrize("exp2", [0, -100, 127])
def test_every_bf16_block_max(nv, exp2):
    """Every finite BF16 value up to M = 2^exp2 as the maximum of a block of
    its own under the tensor amax M: block scales across the whole E4M3 range,
    its rounding, subnormal scales and the scales that underflow to a zero
    block, with the block's codes; rows, columns, 16x16 blocks (four maxima
    share a 16x16 block there), RNE and SR.  Bit-exact against the oracle."""
    x = every_bf16_block_max(exp2)
    compare(nv, x, "rows")
    compare(nv, x.t().contiguous(), "cols")
    compare(nv, x, "2d")
    compare(nv, x, "rows", sr=True, seed=12)


@pytest.mark.parametrize("s_g", [1.0, 1.7e-5, 2.0 ** -110, 1.2e35])
@pytest.mark.parametrize("mode", list(MODES))
def test_dequantize_every_code_and_scale(nv, s_g, mode):
    """Every code byte (two E2M1 codes) under every finite positive E4M3 scale
    byte (0x00-0x7E, subnormals included), in each block layout, under tensor
    scales 1, an arbitrary 1.7e-5, 2^-110 (products in FP32's denormal range)
    and 1.2e35 (about the largest any tensor amax gives, 3.4e38 / 2688: the
    largest products near FP32's and BF16's top): FP32 and BF16 outputs
    bit-exact against the oracle."""
    from nvfp4_bit_microscaled_amd import scale_shape
    R, C = 256, 4096
    codes = np.tile(np.arange(256, dtype=np.uint8), (R, C // 2 // 256))
    codes = np.roll(codes, 7, axis=1) ^ (np.arange(R, dtype=np.uint8)[:, None] * 37).astype(np.uint8)
    sr, sc = scale_shape(R, C, MODES[mode]["block2d"], MODES[mode]["axis"])
    scales = ((np.arange(sr)[:, None] * 5 + np.arange(sc)[None, :]) % 127).astype(np.uint8)
    ts = np.float32(s_g)
    t = nv.NVFP4Tensor(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                       torch.tensor([ts], dtype=torch.float32, device="cuda"),
                       torch.zeros(1, device="cuda"), R, C, MODES[mode]["block2d"],
                       MODES[mode]["axis"])
    f = nv.dequantize(t, torch.float32)
    b = nv.dequantize(t, torch.bfloat16)
    torch.cuda.synchronize()
    rf, rb = oracle.dequantize(codes, scales, float(ts), R, C, **MODES[mode])
    assert np.array_equal(f.cpu().numpy().view(np.uint32), rf.view(np.uint32))
    assert np.array_equal(b.cpu().view(torch.int16).numpy().view(np.uint16), rb)
