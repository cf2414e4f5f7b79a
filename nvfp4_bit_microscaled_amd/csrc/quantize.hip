// NVFP4 quantization, 16-point RHT and dequantization kernels for gfx950.
//
// Two-level microscaling (guiahardware.es "NVFP4: cos'e e come supera FP8 e
// BF16", section "Cos'e NVFP4"; chaitex.ru "FP4", items 1-2 of the
// mathematical-structure section): per 16-element block an E4M3 scale, per
// tensor an FP32 scale.  Recipe (readjensen.com NVFP4 training-recipe page,
// recipe paragraph): 1x16 blocks for activations/gradients, 16x16 blocks for
// weights, a random Hadamard transform on wgrad inputs, stochastic rounding
// of gradients.
//
// All kernels stream HBM once: 16-byte loads, every value kept in registers
// from load to packed store.  The global amax is a separate pass (the tensor
// scale depends on every element) that writes per-workgroup partial maxima;
// a one-workgroup kernel reduces them.  No atomics, so results do not depend
// on scheduling.
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {

// ------------------------------------------------------------ fast division

// Unsigned 32-bit division by a runtime constant (Granlund & Montgomery,
// "Division by invariant integers using multiplication", PLDI'94): with
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1, n / d equals
// (umulhi(n, m) + n) >> l for every 32-bit n.
struct FastDiv {
    uint32_t d, m, l;
};

static FastDiv make_fastdiv(uint32_t d)
{
    FastDiv f;
    f.d = d;
    uint32_t l = 0;
    while (((uint64_t)1 << l) < d) ++l;
    f.l = l;
    f.m = (uint32_t)((((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1);
    return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f)
{
    uint64_t t = (uint64_t)__umulhi(n, f.m) + n;
    return (uint32_t)(t >> f.l);
}

// ------------------------------------------------------------ block logic

struct QuantParams {
    const uint8_t* x;  // bytes
    int64_t rows, cols, ld;  // ld in elements
    uint8_t* codes;
    uint8_t* scales;
    const float* amax_src;
    float* tensor_scale;
    float* amax_out;
    float* partials;
    uint64_t seed;
    uint32_t stream_id;
    uint32_t mask;
    uint32_t items;  // work items of the kernel's mapping (< 2^32)
    FastDiv div;     // items per row-group, for the item -> (row, col) split
    int write_amax_out;
};

struct TensorScale {
    float s_g;
    BlockDiv d6;  // division by RN(6 * s_g)
};

__device__ __forceinline__ TensorScale make_tensor_scale(float amax)
{
    TensorScale t;
    t.s_g = amax / kGlobalDivisor;
    t.d6 = make_block_div(6.0f * t.s_g);
    return t;
}

// Block scale from the block amax.  Returns the E4M3 code (0 for a zero
// block) and fills bd with d = RN(e * s_g) and its reciprocal.
__device__ __forceinline__ uint32_t block_scale(float aB, const TensorScale& ts, BlockDiv& bd,
                                                bool& zero)
{
    zero = true;
    bd.d = 1.0f;
    bd.r = 1.0f;
    bd.fast = true;
    bd.codes_fast = true;
    if (!(aB > 0.0f)) return 0u;
    float t = quotient(aB, ts.d6);  // RN(a_B / RN(6 s_g))
    uint32_t e = e4m3_encode(t);
    float d = e4m3_decode(e) * ts.s_g;
    if (e == 0u || d == 0.0f) return 0u;
    zero = false;
    bd = make_block_div(d);
    return e;
}

// Codes of 8 quotients y[] = RN(x/d) (sign of x kept), packed low nibble
// first: element 2j in the low nibble of byte j.
__device__ __forceinline__ uint32_t pack8_rne(const float y[8])
{
    uint32_t w = 0u;
    w = fp4_pack2<0>(w, y[0], y[1]);
    w = fp4_pack2<1>(w, y[2], y[3]);
    w = fp4_pack2<2>(w, y[4], y[5]);
    w = fp4_pack2<3>(w, y[6], y[7]);
    return w;
}

// Stochastic rounding: each signed quotient y[i] = RN(x[i]/d) is replaced by
// the E2M1 value its word selects (with its sign), which the RNE conversion
// then encodes exactly.
template <int n>
__device__ __forceinline__ void sr_values(float* y, const uint32_t* r)
{
#pragma unroll
    for (int i = 0; i < n; ++i) {
        float v = e2m1_sr_value(__builtin_fabsf(y[i]), r[i]);
        y[i] = __uint_as_float(__float_as_uint(v) | (__float_as_uint(y[i]) & 0x80000000u));
    }
}

// The same from magnitudes y[i] = RN(|x[i]|/d), with the signs taken from x.
template <int n>
__device__ __forceinline__ void sr_values_mag(float* y, const float* x, const uint32_t* r)
{
#pragma unroll
    for (int i = 0; i < n; ++i) {
        float v = e2m1_sr_value(y[i], r[i]);
        y[i] = __uint_as_float(__float_as_uint(v) | (__float_as_uint(x[i]) & 0x80000000u));
    }
}

// Quantize 8 values sharing one block scale (kRHT: Hadamard-transformed
// values, for which round-to-nearest takes the reciprocal fast path).
template <bool kSR, bool kRHT = false>
__device__ __forceinline__ uint32_t encode8(const float v[8], const BlockDiv& bd, bool zero,
                                            const uint32_t r[8])
{
    if (zero) return 0u;
    float y[8];
    if (kSR) {
        quotient_mags<8>(v, bd, y);
        sr_values_mag<8>(y, v, r);
    } else if (kRHT) {
        quotients_rne<8>(v, bd, y);
    } else {
        quotients_codes<8>(v, bd, y);
    }
    return pack8_rne(y);
}

__device__ __forceinline__ void block_reduce_max_store(float m, float* dst)
{
    __shared__ float red[16];
    m = wave_max(m);
    int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float r = red[0];
        for (int i = 1; i < (int)(blockDim.x >> 6); ++i) r = __builtin_fmaxf(r, red[i]);
        *dst = r;
    }
}

__device__ __forceinline__ void write_scale_outputs(const QuantParams& p, const TensorScale& ts)
{
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        *p.tensor_scale = ts.s_g;
        if (p.write_amax_out) *p.amax_out = *p.amax_src;
    }
}

// ------------------------------------------------------------ 1x16 along rows

// One thread per 16-element block of a row (axis 1).  Work item b is block
// cb = b % (cols/16) of row b / (cols/16); its flat element index is 16 b.
template <bool kBF16, bool kSR, bool kRHT, bool kAmaxOnly, bool kDense>
__global__ __launch_bounds__(256) void k_quant_rows(QuantParams p)
{
    constexpr int esz = kBF16 ? 2 : 4;
    float amax_local = 0.0f;
    TensorScale ts;
    if (!kAmaxOnly) {
        ts = make_tensor_scale(*p.amax_src);
        write_scale_outputs(p, ts);
    }
    const uint32_t stride = gridDim.x * blockDim.x;
    for (uint32_t b = blockIdx.x * blockDim.x + threadIdx.x; b < p.items; b += stride) {
        const uint8_t* src;
        if (kDense) {
            src = p.x + (int64_t)b * 16 * esz;
        } else {
            uint32_t row = fdiv(b, p.div);
            uint32_t cb = b - row * p.div.d;
            src = p.x + ((int64_t)row * p.ld + (int64_t)cb * 16) * esz;
        }
        float v[16];
        load8<kBF16>(src, v);
        load8<kBF16>(src + 8 * esz, v + 8);
        if (kRHT) rht16_inplace(v, p.mask);
        float aB = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) aB = __builtin_fmaxf(aB, __builtin_fabsf(v[i]));
        if (kAmaxOnly) {
            amax_local = __builtin_fmaxf(amax_local, aB);
            continue;
        }
        BlockDiv bd;
        bool zero;
        uint32_t e = block_scale(aB, ts, bd, zero);
        uint32_t r[16];
        if (kSR) {
            uint64_t g = (uint64_t)b * 4;  // flat index 16 b, four words per Philox call
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                u32x4 w = sr_words(p.seed, p.stream_id, g + q);
                r[4 * q] = w[0]; r[4 * q + 1] = w[1]; r[4 * q + 2] = w[2]; r[4 * q + 3] = w[3];
            }
        }
        u32x2 out;
        out[0] = encode8<kSR, kRHT>(v, bd, zero, r);
        out[1] = encode8<kSR, kRHT>(v + 8, bd, zero, r + 8);
        *reinterpret_cast<u32x2*>(p.codes + (int64_t)b * 8) = out;
        p.scales[b] = (uint8_t)e;
    }
    if (kAmaxOnly) block_reduce_max_store(amax_local, p.partials + blockIdx.x);
}

// ------------------------------------------------------------ 1x16 along columns

template <bool kBF16>
__device__ __forceinline__ void load4(const uint8_t* p, float v[4])
{
    if (kBF16) {
        u32x2 w = *reinterpret_cast<const u32x2*>(p);
        v[0] = bf16_lo(w[0]); v[1] = bf16_hi(w[0]);
        v[2] = bf16_lo(w[1]); v[3] = bf16_hi(w[1]);
    } else {
        u32x4 w = *reinterpret_cast<const u32x4*>(p);
        v[0] = __uint_as_float(w[0]); v[1] = __uint_as_float(w[1]);
        v[2] = __uint_as_float(w[2]); v[3] = __uint_as_float(w[3]);
    }
}

// One thread per 16-row x 4-column tile (axis 0): four column blocks.  Work
// item t is column group cg = t % (cols/4) of row block rb = t / (cols/4).
// A wave reads 512 contiguous bytes of each BF16 row.
template <bool kBF16, bool kSR, bool kRHT, bool kAmaxOnly>
__global__ __launch_bounds__(256) void k_quant_cols(QuantParams p)
{
    constexpr int esz = kBF16 ? 2 : 4;
    float amax_local = 0.0f;
    TensorScale ts;
    if (!kAmaxOnly) {
        ts = make_tensor_scale(*p.amax_src);
        write_scale_outputs(p, ts);
    }
    const uint32_t stride = gridDim.x * blockDim.x;
    for (uint32_t t = blockIdx.x * blockDim.x + threadIdx.x; t < p.items; t += stride) {
        uint32_t rb = fdiv(t, p.div);
        uint32_t cg = t - rb * p.div.d;
        int64_t r0 = (int64_t)rb * 16, c0 = (int64_t)cg * 4;
        float v[4][16];  // [column][row]
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float w[4];
            load4<kBF16>(p.x + ((r0 + i) * p.ld + c0) * esz, w);
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j][i] = w[j];
        }
        if (kRHT) {
#pragma unroll
            for (int j = 0; j < 4; ++j) rht16_inplace(v[j], p.mask);
        }
        float aB[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            aB[j] = 0.0f;
#pragma unroll
            for (int i = 0; i < 16; ++i) aB[j] = __builtin_fmaxf(aB[j], __builtin_fabsf(v[j][i]));
        }
        if (kAmaxOnly) {
#pragma unroll
            for (int j = 0; j < 4; ++j) amax_local = __builtin_fmaxf(amax_local, aB[j]);
            continue;
        }
        uint32_t sc = 0u;
        float y[4][16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            BlockDiv bd;
            bool zero;
            uint32_t e = block_scale(aB[j], ts, bd, zero);
            sc |= e << (8 * j);
            if (zero) {
#pragma unroll
                for (int i = 0; i < 16; ++i) y[j][i] = 0.0f;
            } else {
                if (!kSR && kRHT) quotients_rne<16>(v[j], bd, y[j]);
                else if (!kSR) quotients_codes<16>(v[j], bd, y[j]);
                else quotients<16>(v[j], bd, y[j]);
            }
        }
        *reinterpret_cast<uint32_t*>(p.scales + rb * p.cols + c0) = sc;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float q[4] = {y[0][i], y[1][i], y[2][i], y[3][i]};
            if (kSR) {
                uint64_t g = (uint64_t)((r0 + i) * p.cols + c0) >> 2;
                u32x4 w = sr_words(p.seed, p.stream_id, g);
                uint32_t r[4] = {w[0], w[1], w[2], w[3]};
                sr_values<4>(q, r);
            }
            uint32_t code = fp4_pack2<1>(fp4_pack2<0>(0u, q[0], q[1]), q[2], q[3]);
            *reinterpret_cast<uint16_t*>(p.codes + (r0 + i) * (p.cols / 2) + c0 / 2) =
                (uint16_t)code;
        }
    }
    if (kAmaxOnly) block_reduce_max_store(amax_local, p.partials + blockIdx.x);
}

// ------------------------------------------------------------ both amaxes

// The two tensor amaxes a tensor that feeds both a row-wise quantization and
// the column-wise RHT quantization of wgrad needs, in one read: max |x| and
// max |RHT16 down the columns of x| (rows % 16 == 0).  Thread mapping as in
// the column kernel (16 rows x 4 columns); per-workgroup partial maxima go to
// partials[0 .. grid) and partials[kMaxAmaxPartials .. + grid).
template <bool kBF16>
__global__ __launch_bounds__(256) void k_amax_dual(QuantParams p)
{
    constexpr int esz = kBF16 ? 2 : 4;
    float m_plain = 0.0f, m_rht = 0.0f;
    const uint32_t stride = gridDim.x * blockDim.x;
    for (uint32_t t = blockIdx.x * blockDim.x + threadIdx.x; t < p.items; t += stride) {
        uint32_t rb = fdiv(t, p.div);
        uint32_t cg = t - rb * p.div.d;
        int64_t r0 = (int64_t)rb * 16, c0 = (int64_t)cg * 4;
        float v[4][16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float w[4];
            load4<kBF16>(p.x + ((r0 + i) * p.ld + c0) * esz, w);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                v[j][i] = w[j];
                m_plain = __builtin_fmaxf(m_plain, __builtin_fabsf(w[j]));
            }
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            rht16_butterflies(v[j], p.mask);
#pragma unroll
            for (int i = 0; i < 16; ++i) m_rht = __builtin_fmaxf(m_rht, __builtin_fabsf(v[j][i]));
        }
    }
    block_reduce_max_store(m_plain, p.partials + blockIdx.x);
    __syncthreads();  // the reduction's shared slots are reused
    block_reduce_max_store(0.25f * m_rht, p.partials + kMaxAmaxPartials + blockIdx.x);
}

// ------------------------------------------------------------ SwiGLU + amaxes

// The producer of the MLP's second GEMM input, fused with both of its tensor
// amaxes: act = BF16(BF16(silu(gate)) * up) with silu(g) = g / (1 + exp(-g))
// in FP32 (the reciprocal from the hardware unit; the BF16 rounding points of
// a BF16 framework's silu and multiply),
// written as BF16 [rows, F], plus max |act| and max |RHT16 down the columns of
// act| (rows % 16 == 0).  gate = h[:, 0:F], up = h[:, F:2F].  Mapping as the
// column kernel: thread = 16 rows x 4 columns of act.
__global__ __launch_bounds__(256) void k_swiglu_amax(const uint8_t* h, int64_t ld_h,
                                                     uint8_t* act, int64_t ld_a, int64_t F,
                                                     uint32_t items, FastDiv div, uint32_t mask,
                                                     float* partials)
{
    float m_plain = 0.0f, m_rht = 0.0f;
    const uint32_t stride = gridDim.x * blockDim.x;
    for (uint32_t t = blockIdx.x * blockDim.x + threadIdx.x; t < items; t += stride) {
        uint32_t rb = fdiv(t, div);
        uint32_t cg = t - rb * div.d;
        int64_t r0 = (int64_t)rb * 16, c0 = (int64_t)cg * 4;
        // all 32 loads of the tile first: the stores below could alias h as
        // far as the compiler knows, so loads issued between them would wait
        u32x2 graw[16], uraw[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            graw[i] = *reinterpret_cast<const u32x2*>(h + ((r0 + i) * ld_h + c0) * 2);
            uraw[i] = *reinterpret_cast<const u32x2*>(h + ((r0 + i) * ld_h + F + c0) * 2);
        }
        float v[4][16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float g[4] = {bf16_lo(graw[i][0]), bf16_hi(graw[i][0]), bf16_lo(graw[i][1]),
                                bf16_hi(graw[i][1])};
            const float u[4] = {bf16_lo(uraw[i][0]), bf16_hi(uraw[i][0]), bf16_lo(uraw[i][1]),
                                bf16_hi(uraw[i][1])};
            float den[4], sg[4];
            bool need_div = false;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                den[j] = silu_den(g[j]);
                sg[j] = silu_rcp(g[j], den[j]);
                need_div |= silu_needs_division(den[j]);
            }
            // the division only in waves with a gate below -87.3
            if (__builtin_amdgcn_ballot_w64(need_div) != 0) {
#pragma unroll
                for (int j = 0; j < 4; ++j) sg[j] = silu_fix(g[j], den[j], sg[j]);
            }
            u32x2 w;
            w[0] = swiglu_pack(sg[0], u[0], sg[1], u[1]);
            w[1] = swiglu_pack(sg[2], u[2], sg[3], u[3]);
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float a = (j & 1) ? bf16_hi(w[j >> 1]) : bf16_lo(w[j >> 1]);
                v[j][i] = a;
                m_plain = __builtin_fmaxf(m_plain, __builtin_fabsf(a));
            }
            *reinterpret_cast<u32x2*>(act + ((r0 + i) * ld_a + c0) * 2) = w;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            rht16_butterflies(v[j], mask);
#pragma unroll
            for (int i = 0; i < 16; ++i) m_rht = __builtin_fmaxf(m_rht, __builtin_fabsf(v[j][i]));
        }
    }
    block_reduce_max_store(m_plain, partials + blockIdx.x);
    __syncthreads();  // the reduction's shared slots are reused
    // the transform's 1/4 on the maximum (RN(0.25 x) is monotone in x)
    block_reduce_max_store(0.25f * m_rht, partials + kMaxAmaxPartials + blockIdx.x);
}

// fp4_pack2 into byte `sel` of `old` (sel is a constant once loops unroll)
__device__ __forceinline__ uint32_t fp4_pack2_at(uint32_t old, float a, float b, int sel)
{
    switch (sel) {
    case 0: return fp4_pack2<0>(old, a, b);
    case 1: return fp4_pack2<1>(old, a, b);
    case 2: return fp4_pack2<2>(old, a, b);
    default: return fp4_pack2<3>(old, a, b);
    }
}

// ------------------------------------------------------------ transposed output

// Blocks down the columns (1x16 along rows, or 16x16), written as the
// quantization of the transposed tensor: codes [cols, rows/2] and scales
// [cols, rows/16] (1D) or [cols/16, rows/16] (2D), so a GEMM that contracts
// over the rows reads both operands K-major.  Element values, scales, the
// transform and the stochastic-rounding counter are those of the untransposed
// quantization (idx = row * cols + col of x).
//
// One workgroup per 256 x 256 tile.  Thread t quantizes columns 4 (t % 64) ..
// +3 of row blocks w, w + 4, w + 8, w + 12 (w = t / 64), 16 rows x 4 columns
// at a time as in the column kernel; the packed codes (8 bytes per column and
// row block) go to LDS as [column][row block], then leave as 128-byte rows
// of the transposed tensor.  The row-block slot is XOR-swizzled with the
// column group so the 64 lanes of a wave write 64 different banks pairs.
constexpr int kTT = 256;                  // tile rows and columns
constexpr int kTCodeRow = kTT / 2;        // LDS bytes per transposed row (16 slots x 8)
constexpr int kTCodeBytes = kTT * kTCodeRow;
constexpr int kTScaleBytes = kTT * 16;

// Occupancy: the 1D variants fit three waves per SIMD (at most 168 VGPRs)
// without spilling; left alone the compiler took 203 for the SR variant,
// two waves per SIMD, and ran 7% slower.  The 2D variants keep their
// registers (they would spill).
template <bool kBF16, bool kSR, bool kRHT, bool k2D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(k2D ? 1 : 3)))
void k_quant_t(QuantParams p)
{
    constexpr int esz = kBF16 ? 2 : 4;
    __shared__ __attribute__((aligned(16))) uint8_t lds_codes[kTCodeBytes];
    __shared__ __attribute__((aligned(16))) uint8_t lds_scales[kTScaleBytes];
    const TensorScale ts = make_tensor_scale(*p.amax_src);
    write_scale_outputs(p, ts);
    const int t = threadIdx.x, cg = t & 63, w = t >> 6;
    const int64_t rows = p.rows, cols = p.cols;
    const int64_t out_ld = rows / 2;     // bytes per transposed code row
    const int64_t sc_ld = rows / 16;     // bytes per transposed scale row
    // every transposed code row starts 16-byte aligned (tiles start at
    // multiples of 128 bytes of a row)
    const bool codes16 = ((uintptr_t)p.codes & 15) == 0 && (out_ld & 15) == 0;
    for (uint32_t tile = blockIdx.x; tile < p.items; tile += gridDim.x) {
        const uint32_t tr = fdiv(tile, p.div);
        const uint32_t tc = tile - tr * p.div.d;
        const int64_t R0 = (int64_t)tr * kTT, C0 = (int64_t)tc * kTT;
        const int64_t c0 = C0 + 4 * cg;
        const bool col_ok = c0 < cols;   // cols % 16 == 0: a column group is whole
#pragma unroll 1
        for (int it = 0; it < 4; ++it) {
            const int rbl = 4 * it + w;
            const int64_t r0 = R0 + 16 * rbl;
            if (r0 >= rows) break;           // uniform: later row blocks are past the end too
            // a 16x16 block's four lanes share col_ok, so the shuffles below
            // only ever read lanes that took the same path
            if (!col_ok) continue;
            const uint8_t* src = p.x + (r0 * p.ld + c0) * esz;
            float v[4][16];  // [column][row]
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                float x4[4];
                load4<kBF16>(src + (int64_t)i * p.ld * esz, x4);
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j][i] = x4[j];
            }
            if (kRHT) {
#pragma unroll
                for (int j = 0; j < 4; ++j) rht16_inplace(v[j], p.mask);
            }
            float aB[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                aB[j] = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) aB[j] = __builtin_fmaxf(aB[j], __builtin_fabsf(v[j][i]));
            }
            if (k2D) {  // the 16x16 block spans the four lanes cg & ~3 .. +3
                float m = __builtin_fmaxf(__builtin_fmaxf(aB[0], aB[1]), __builtin_fmaxf(aB[2], aB[3]));
                m = __builtin_fmaxf(m, __shfl_xor(m, 1, 64));
                m = __builtin_fmaxf(m, __shfl_xor(m, 2, 64));
#pragma unroll
                for (int j = 0; j < 4; ++j) aB[j] = m;
            }
            uint32_t e[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {  // quotients in place
                BlockDiv bd;
                bool zero;
                e[j] = block_scale(aB[j], ts, bd, zero);
                if (zero) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) v[j][i] = 0.0f;
                } else {
                    float y[16];
                    if (!kSR && kRHT) quotients_rne<16>(v[j], bd, y);
                    else if (!kSR) quotients_codes<16>(v[j], bd, y);
                    else quotients<16>(v[j], bd, y);
#pragma unroll
                    for (int i = 0; i < 16; ++i) v[j][i] = y[i];
                }
            }
            // two rows at a time: SR words of both rows, then one byte
            // (rows i, i+1) per column into that column's 8-byte code word
            u32x2 out[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) out[j] = u32x2{0u, 0u};
#pragma unroll
            for (int i = 0; i < 16; i += 2) {
                float a[4], b[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) { a[j] = v[j][i]; b[j] = v[j][i + 1]; }
                if (kSR) {
                    const uint64_t g = (uint64_t)((r0 + i) * cols + c0) >> 2;
                    const uint64_t gstep = (uint64_t)cols >> 2;
                    u32x4 ra = sr_words(p.seed, p.stream_id, g);
                    u32x4 rb = sr_words(p.seed, p.stream_id, g + gstep);
                    uint32_t wa[4] = {ra[0], ra[1], ra[2], ra[3]};
                    uint32_t wb[4] = {rb[0], rb[1], rb[2], rb[3]};
                    sr_values<4>(a, wa);
                    sr_values<4>(b, wb);
                }
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    out[j][i >> 3] = fp4_pack2_at(out[j][i >> 3], a[j], b[j], (i >> 1) & 3);
            }
            const int slot = rbl ^ (cg & 15);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                *reinterpret_cast<u32x2*>(lds_codes + (4 * cg + j) * kTCodeRow + 8 * slot) = out[j];
            if (k2D) {
                if ((cg & 3) == 0) lds_scales[(cg >> 2) * 16 + rbl] = (uint8_t)e[0];
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) lds_scales[(4 * cg + j) * 16 + rbl] = (uint8_t)e[j];
            }
        }
        __syncthreads();
        // codes: transposed row cl gets its 16 slots (row blocks) in order,
        // two slots per 16-byte store where the rows allow it
        const int nrb = (int)((rows - R0) / 16 < 16 ? (rows - R0) / 16 : 16);
#pragma unroll 1
        for (int pass = 0; pass < 8; ++pass) {
            const int cl = 32 * pass + (t >> 3), ch = t & 7;
            if (C0 + cl >= cols) continue;
            const int s = (cl >> 2) & 15;
            uint8_t* dst = p.codes + (C0 + cl) * out_ld + R0 / 2 + 16 * ch;
            const uint8_t* row = lds_codes + cl * kTCodeRow;
            if (codes16 && 2 * ch + 1 < nrb) {
                const u32x2 lo = *reinterpret_cast<const u32x2*>(row + 8 * ((2 * ch) ^ s));
                const u32x2 hi = *reinterpret_cast<const u32x2*>(row + 8 * ((2 * ch + 1) ^ s));
                *reinterpret_cast<u32x4*>(dst) = u32x4{lo[0], lo[1], hi[0], hi[1]};
                continue;
            }
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int rb = 2 * ch + h;
                if (rb < nrb)
                    *reinterpret_cast<u32x2*>(dst + 8 * h) =
                        *reinterpret_cast<const u32x2*>(row + 8 * (rb ^ s));
            }
        }
        // scales: one 16-byte row per transposed scale row (one store when
        // the row is whole and 16-byte aligned, else byte by byte)
        const int nsr = k2D ? 16 : 256;
        if (t < nsr) {
            const int64_t orow = k2D ? C0 / 16 + t : C0 + t;
            if (orow < (k2D ? cols / 16 : cols)) {
                uint8_t* dst = p.scales + orow * sc_ld + R0 / 16;
                const uint8_t* src = lds_scales + t * 16;
                if (nrb == 16 && ((uintptr_t)dst & 15) == 0)
                    *reinterpret_cast<u32x4*>(dst) = *reinterpret_cast<const u32x4*>(src);
                else
                    for (int b = 0; b < nrb; ++b) dst[b] = src[b];
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------ storage transpose

// The same NVFP4 tensor stored as its transpose: element (r, c) of the
// rows x cols input becomes element (c, r) of the cols x rows output with
// the same code and block scale.  For 16x16 blocks this is the recipe's
// transpose consistency (readjensen.com recipe paragraph: fprop and dgrad
// see the same weight values), so dgrad's K-major weight needs no second
// quantization.  The scale plane is transposed byte for byte: 2D
// [R/16, C/16] -> [C/16, R/16]; blocks along rows [R, C/16] -> blocks down
// the columns of the output [C/16, R]; and the reverse.
struct TransposeParams {
    const uint8_t* codes;
    const uint8_t* scales;
    uint8_t* codes_t;
    uint8_t* scales_t;
    int64_t rows, cols;
    int64_t s_rows, s_cols;  // input scale plane [s_rows, s_cols]
    int s_tr_log, s_tc_log;  // log2 of its sub-block per 256 x 256 tile
    int s_r_div, s_c_div;    // tile origin -> sub-block origin (divide by 1 or 16)
    uint32_t tiles;
    FastDiv div;             // tiles per tile row
};

// Transpose a 16 x 16 matrix of nibbles held as 16 rows of 64 bits (row i
// = lo[i] | hi[i] << 32, element j at bits 4j .. 4j+3).  Block-recursive:
// at each level the top-right and bottom-left sub-blocks of every block
// trade places, which swaps one bit of the row and column indices; the four
// levels together map (i, j) to (j, i).  The 8x8 level swaps whole words;
// the others work within each 32-bit word.
__device__ __forceinline__ void nibble_transpose16(uint32_t lo[16], uint32_t hi[16])
{
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const uint32_t t = hi[i];
        hi[i] = lo[i + 8];
        lo[i + 8] = t;
    }
#pragma unroll
    for (int lvl = 0; lvl < 3; ++lvl) {
        const int dist = 4 >> lvl, sh = 16 >> lvl;
        const uint32_t m = lvl == 0 ? 0x0000FFFFu : (lvl == 1 ? 0x00FF00FFu : 0x0F0F0F0Fu);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i & dist) continue;
            uint32_t t = ((lo[i] >> sh) ^ lo[i + dist]) & m;
            lo[i + dist] ^= t;
            lo[i] ^= t << sh;
            t = ((hi[i] >> sh) ^ hi[i + dist]) & m;
            hi[i + dist] ^= t;
            hi[i] ^= t << sh;
        }
    }
}

// LDS chunk swizzle of the transposed tile: 8-byte chunk c of row R sits at
// c ^ swz(R) (even, so 16-byte pairs stay adjacent).
__device__ __forceinline__ int transpose_swz(int R) { return (R >> 3) & 14; }

// One workgroup per 256 x 256 tile of the input.  Thread (br, bc) = (t / 16,
// t % 16) loads block (br, bc) of the tile as 16 rows of 8 bytes (16 lanes
// cover one 128-byte row segment), transposes it in registers and writes its
// 16 output rows to LDS; the tile then leaves as 128-byte segments of the
// output rows (8 bytes per lane).
__global__ __launch_bounds__(256) void k_transpose(TransposeParams p)
{
    __shared__ __attribute__((aligned(16))) uint8_t lds_c[kTT * kTCodeRow];
    __shared__ uint8_t lds_s[kTT * 16];
    const int t = threadIdx.x, br = t >> 4, bc = t & 15;
    const int64_t rows = p.rows, cols = p.cols;
    const int64_t in_ld = cols / 2, out_ld = rows / 2;
    const int s_tr = 1 << p.s_tr_log, s_n = s_tr << p.s_tc_log;
    for (uint32_t tile = blockIdx.x; tile < p.tiles; tile += gridDim.x) {
        const uint32_t tr = fdiv(tile, p.div);
        const uint32_t tc = tile - tr * p.div.d;
        const int64_t R0 = (int64_t)tr * kTT, C0 = (int64_t)tc * kTT;
        if (R0 + 16 * br < rows && C0 + 16 * bc < cols) {
            const uint8_t* src = p.codes + (R0 + 16 * br) * in_ld + (C0 + 16 * bc) / 2;
            uint32_t lo[16], hi[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const u32x2 w = *reinterpret_cast<const u32x2*>(src + i * in_ld);
                lo[i] = w[0];
                hi[i] = w[1];
            }
            nibble_transpose16(lo, hi);
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                const int R = 16 * bc + j;
                *reinterpret_cast<u32x2*>(lds_c + R * kTCodeRow + 8 * (br ^ transpose_swz(R))) =
                    u32x2{lo[j], hi[j]};
            }
        }
        // scale sub-block [sr0, +s_tr) x [sc0, +s_tc), stored transposed in LDS
        const int64_t sr0 = R0 / p.s_r_div, sc0 = C0 / p.s_c_div;
        for (int i = t; i < s_n; i += 256) {
            const int r = i >> p.s_tc_log, c = i & ((1 << p.s_tc_log) - 1);
            if (sr0 + r < p.s_rows && sc0 + c < p.s_cols)
                lds_s[c * s_tr + r] = p.scales[(sr0 + r) * p.s_cols + sc0 + c];
        }
        __syncthreads();
#pragma unroll 4
        for (int k = 0; k < 16; ++k) {
            const int idx = t + 256 * k, R = idx >> 4, c8 = idx & 15;
            if (C0 + R < cols && R0 + 16 * c8 < rows)
                *reinterpret_cast<u32x2*>(p.codes_t + (C0 + R) * out_ld + R0 / 2 + 8 * c8) =
                    *reinterpret_cast<const u32x2*>(lds_c + R * kTCodeRow +
                                                    8 * (c8 ^ transpose_swz(R)));
        }
        for (int i = t; i < s_n; i += 256) {
            const int c = i >> p.s_tr_log, r = i & (s_tr - 1);
            if (sr0 + r < p.s_rows && sc0 + c < p.s_cols)
                p.scales_t[(sc0 + c) * p.s_rows + sr0 + r] = lds_s[c * s_tr + r];
        }
        __syncthreads();
    }
}

// 16 consecutive inputs as raw words (BF16: two 16-byte loads, FP32: four),
// kept unconverted so that several rows' loads can be in flight at once.
template <bool kBF16>
struct Raw16 {
    u32x4 q[kBF16 ? 2 : 4];
};

template <bool kBF16>
__device__ __forceinline__ Raw16<kBF16> load_raw16(const uint8_t* src)
{
    Raw16<kBF16> r;
#pragma unroll
    for (int i = 0; i < (kBF16 ? 2 : 4); ++i) r.q[i] = reinterpret_cast<const u32x4*>(src)[i];
    return r;
}

template <bool kBF16>
__device__ __forceinline__ void unpack16(const Raw16<kBF16>& r, float v[16])
{
    if (kBF16) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t w = r.q[i / 4][i % 4];
            v[2 * i] = bf16_lo(w);
            v[2 * i + 1] = bf16_hi(w);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) v[i] = __uint_as_float(r.q[i / 4][i % 4]);
    }
}

// ------------------------------------------------------------ 16x16 blocks

// One wave per 16-row x 256-column strip; lane l covers columns
// 16 (l % 16) .. +15 of rows (l / 16) + 4k, k = 0..3, so the four lanes
// holding one 16x16 block combine their maxima with two lane swaps.
// Work item w (a wave) is column strip w % strips of row block w / strips.
template <bool kBF16, bool kSR>
__global__ __launch_bounds__(256) void k_quant_2d(QuantParams p)
{
    constexpr int esz = kBF16 ? 2 : 4;
    TensorScale ts = make_tensor_scale(*p.amax_src);
    write_scale_outputs(p, ts);
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t waves = gridDim.x * (blockDim.x >> 6);
    const uint32_t cg = lane & 15, rq = lane >> 4;
    for (uint32_t w = blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6); w < p.items;
         w += waves) {
        uint32_t rb = fdiv(w, p.div);
        uint32_t strip = w - rb * p.div.d;
        int64_t c0 = (int64_t)strip * 256 + cg * 16;
        bool valid = c0 < p.cols;
        int64_t rbase = (int64_t)rb * 16 + rq;
        // all four rows' loads issue before any use: lanes past the last
        // column load column 0 of their rows instead and drop the values
        const int64_t cl = valid ? c0 : 0;
        Raw16<kBF16> raw[4];
#pragma unroll
        for (int k = 0; k < 4; ++k)
            raw[k] = load_raw16<kBF16>(p.x + ((rbase + 4 * k) * p.ld + cl) * esz);
        float v[4][16];
        float aB = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            unpack16<kBF16>(raw[k], v[k]);
            if (!valid) {
#pragma unroll
                for (int i = 0; i < 16; ++i) v[k][i] = 0.0f;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) aB = __builtin_fmaxf(aB, __builtin_fabsf(v[k][i]));
        }
        aB = __builtin_fmaxf(aB, __shfl_xor(aB, 16, 64));
        aB = __builtin_fmaxf(aB, __shfl_xor(aB, 32, 64));
        if (!valid) continue;
        BlockDiv bd;
        bool zero;
        uint32_t e = block_scale(aB, ts, bd, zero);
        if (rq == 0) p.scales[(int64_t)rb * (p.cols / 16) + c0 / 16] = (uint8_t)e;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            int64_t row = rbase + 4 * k;
            uint32_t r[16];
            if (kSR) {
                uint64_t g = (uint64_t)(row * p.cols + c0) >> 2;
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    u32x4 ww = sr_words(p.seed, p.stream_id, g + q);
                    r[4 * q] = ww[0]; r[4 * q + 1] = ww[1]; r[4 * q + 2] = ww[2]; r[4 * q + 3] = ww[3];
                }
            }
            u32x2 out;
            out[0] = encode8<kSR>(v[k], bd, zero, r);
            out[1] = encode8<kSR>(v[k] + 8, bd, zero, r + 8);
            *reinterpret_cast<u32x2*>(p.codes + row * (p.cols / 2) + c0 / 2) = out;
        }
    }
}

// ------------------------------------------------------------ amax reduce

__global__ __launch_bounds__(256) void k_amax_finalize(const float* partials, int n,
                                                       float* amax_dst, float* amax_out)
{
    float m = 0.0f;
    for (int i = threadIdx.x; i < n; i += blockDim.x) m = __builtin_fmaxf(m, partials[i]);
    __shared__ float red[4];
    m = wave_max(m);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        float r = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
        *amax_dst = r;
        if (amax_out) *amax_out = r;
    }
}

__global__ void k_write_zero_scale(float* ts, float* amax_out)
{
    *ts = 0.0f;
    if (amax_out) *amax_out = 0.0f;
}

// ------------------------------------------------------------ RHT16 standalone

// axis 1: one thread per 16-element group of a row; axis 0: one thread per
// 16-row x 8-column tile.  FP32 output.
template <bool kBF16>
__global__ __launch_bounds__(256) void k_rht16_rows(const uint8_t* x, int64_t ld, uint32_t items,
                                                    FastDiv div, uint32_t mask, float* y,
                                                    int64_t ld_y)
{
    constexpr int esz = kBF16 ? 2 : 4;
    const uint32_t stride = gridDim.x * blockDim.x;
    for (uint32_t b = blockIdx.x * blockDim.x + threadIdx.x; b < items; b += stride) {
        uint32_t row = fdiv(b, div);
        uint32_t cb = b - row * div.d;
        const uint8_t* src = x + ((int64_t)row * ld + (int64_t)cb * 16) * esz;
        float v[16];
        load8<kBF16>(src, v);
        load8<kBF16>(src + 8 * esz, v + 8);
        rht16_inplace(v, mask);
        float* dst = y + (int64_t)row * ld_y + (int64_t)cb * 16;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            u32x4 w;
            w[0] = __float_as_uint(v[4 * i]); w[1] = __float_as_uint(v[4 * i + 1]);
            w[2] = __float_as_uint(v[4 * i + 2]); w[3] = __float_as_uint(v[4 * i + 3]);
            reinterpret_cast<u32x4*>(dst)[i] = w;
        }
    }
}

template <bool kBF16>
__global__ __launch_bounds__(256) void k_rht16_cols(const uint8_t* x, int64_t ld, uint32_t items,
                                                    FastDiv div, uint32_t mask, float* y,
                                                    int64_t ld_y)
{
    constexpr int esz = kBF16 ? 2 : 4;
    const uint32_t stride = gridDim.x * blockDim.x;
    for (uint32_t t = blockIdx.x * blockDim.x + threadIdx.x; t < items; t += stride) {
        uint32_t rb = fdiv(t, div);
        uint32_t cg = t - rb * div.d;
        int64_t r0 = (int64_t)rb * 16, c0 = (int64_t)cg * 8;
        float v[16][8];
#pragma unroll
        for (int i = 0; i < 16; ++i) load8<kBF16>(x + ((r0 + i) * ld + c0) * esz, v[i]);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float col[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) col[i] = v[i][j];
            rht16_inplace(col, mask);
#pragma unroll
            for (int i = 0; i < 16; ++i) v[i][j] = col[i];
        }
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float* dst = y + (r0 + i) * ld_y + c0;
            u32x4 a, b;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                a[j] = __float_as_uint(v[i][j]);
                b[j] = __float_as_uint(v[i][4 + j]);
            }
            reinterpret_cast<u32x4*>(dst)[0] = a;
            reinterpret_cast<u32x4*>(dst)[1] = b;
        }
    }
}

// ------------------------------------------------------------ dequantize

// Eight elements of one 32-bit code word (element 2j in the low nibble of
// byte j) with their scales e[]: v = RN32((val * e) * s_g), val * e exact in
// FP32; stored as FP32 or BF16 (round to nearest even) at dst, 16-byte
// aligned.
template <bool kOutBF16>
__device__ __forceinline__ void dequant8_store(uint32_t w, const float e[8], float s_g, uint8_t* dst)
{
    float v[8];
    float2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    float2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    float2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    float2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    v[0] = p0[0]; v[1] = p0[1]; v[2] = p1[0]; v[3] = p1[1];
    v[4] = p2[0]; v[5] = p2[1]; v[6] = p3[0]; v[7] = p3[1];
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = (v[j] * e[j]) * s_g;
    if (kOutBF16) {
        u32x4 o;
#pragma unroll
        for (int j = 0; j < 4; ++j) o[j] = bf16_pair(v[2 * j], v[2 * j + 1]);
        // a wave's 64 stores are 1 KB of consecutive bytes: streaming stores,
        // which skip the caches (the output is written once per call)
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(dst));
    } else {
        u32x4 a, b;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            a[j] = __float_as_uint(v[j]);
            b[j] = __float_as_uint(v[4 + j]);
        }
        // two 16-byte halves per lane: plain stores, which L2 merges into whole
        // lines (streaming stores of half lines measured 40% slower)
        u32x4* d = reinterpret_cast<u32x4*>(dst);
        d[0] = a;
        d[1] = b;
    }
}

// One thread per 8 consecutive elements of a row (one 32-bit code word).
// v = RN32((val * e) * s_g); val * e is exact in FP32.  kMode 3 is MXFP4:
// e = 2^(u - 127) from an E8M0 byte per 32 along the row and no tensor scale
// (val * e is exact: the smallest product 0.5 * 2^-127 is an FP32 subnormal).
template <bool kOutBF16, int kMode>  // kMode: 0 = 1D axis 1, 1 = 1D axis 0, 2 = 2D, 3 = MX
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* codes, const uint8_t* scales,
                                                 const float* ts, int64_t cols, uint32_t items,
                                                 FastDiv div, uint8_t* out, int64_t ld_out)
{
    const float s_g = kMode == 3 ? 1.0f : *ts;
    const uint32_t stride = gridDim.x * blockDim.x;
    // kU items per trip, all their loads issued before any store, so each
    // lane keeps kU code words in flight
    constexpr int kU = 4;
    for (uint32_t t0 = blockIdx.x * blockDim.x + threadIdx.x; t0 < items; t0 += kU * stride) {
        uint32_t w[kU], row[kU];
        int64_t c0[kU];
        uint32_t sraw[kU][2];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            const uint32_t t = t0 + u * stride;
            const bool ok = t < items;
            const uint32_t tc = ok ? t : t0;  // a valid item, stored only when ok
            row[u] = fdiv(tc, div);
            c0[u] = (int64_t)(tc - row[u] * div.d) * 8;
            w[u] = *reinterpret_cast<const uint32_t*>(codes + (int64_t)row[u] * (cols / 2) +
                                                      c0[u] / 2);
            if (kMode == 3) {
                sraw[u][0] = scales[(int64_t)row[u] * (cols / 32) + c0[u] / 32];
            } else if (kMode == 1) {
                const u32x2 sv = *reinterpret_cast<const u32x2*>(
                    scales + (int64_t)(row[u] / 16) * cols + c0[u]);
                sraw[u][0] = sv[0];
                sraw[u][1] = sv[1];
            } else {
                const int64_t si = (kMode == 0) ? (int64_t)row[u] * (cols / 16) + c0[u] / 16
                                                : (int64_t)(row[u] / 16) * (cols / 16) + c0[u] / 16;
                sraw[u][0] = scales[si];
            }
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            if (t0 + u * stride >= items) break;
            float e[8];
            if (kMode == 3) {
                const uint32_t v = sraw[u][0];
                const float ev = __uint_as_float(v == 0 ? 0x00400000u
                                                        : (v == 255 ? 0x7FC00000u : v << 23));
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) e[jj] = ev;
            } else if (kMode == 1) {
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    e[jj] = e4m3_decode(sraw[u][0] >> (8 * jj));
                    e[4 + jj] = e4m3_decode(sraw[u][1] >> (8 * jj));
                }
            } else {
                const float ev = e4m3_decode(sraw[u][0]);
#pragma unroll
                for (int jj = 0; jj < 8; ++jj) e[jj] = ev;
            }
            dequant8_store<kOutBF16>(w[u], e, s_g,
                                     out + ((int64_t)row[u] * ld_out + c0[u]) * (kOutBF16 ? 2 : 4));
        }
    }
}

// ------------------------------------------------------------ KV cache
// NVFP4 KV cache (NVIDIA-blog translation on juejin.cn, point 3: an NVFP4
// KV cache for long contexts and large batches; "FP4", chaitex.ru,
// mathematical-structure section: 16-element micro-blocks with an E4M3
// scale and an FP32 tensor scale).  A cache is num_slots rows of `cols`
// features in 1x16 blocks, rounded to nearest-even, under one tensor scale
// s_g = RN(amax / 2688) from a calibration amax that stays fixed while rows
// arrive.  Writes scatter token rows to cache rows slots[t]; reads gather
// cache rows slots[j] and dequantize them.  Slots outside [0, num_slots) are
// skipped on write and read as zero rows.
struct KvParams {
    const uint8_t* x;       // write: token rows (BF16 / FP32 bytes)
    int64_t ld;             // write: row pitch of x in elements; read: of out
    const int64_t* slots;
    int64_t num_slots;
    int64_t cols;
    const float* amax;      // calibration amax (device scalar)
    uint8_t* codes;         // [num_slots, cols/2]
    uint8_t* scales;        // [num_slots, cols/16]
    uint8_t* out;           // read: [n, cols] rows of pitch ld
    uint32_t units;         // (row, chunk) pairs, one per wave iteration
    FastDiv div;            // chunks per row
};

// Work is split into units of one row chunk; each wave takes units
// wave, wave + waves, ...  The unit's slot is wave-uniform (a scalar load),
// and the next unit's slot is loaded one iteration ahead so that its latency
// overlaps the current unit's memory traffic.
// (64-bit counters: u + step must not wrap below the unit count.)
struct KvWalk {
    uint64_t u, step;
};

__device__ __forceinline__ KvWalk kv_walk()
{
    KvWalk w;
    w.u = __builtin_amdgcn_readfirstlane(blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6));
    w.step = gridDim.x * (blockDim.x >> 6);
    return w;
}

__device__ __forceinline__ int64_t kv_slot_of(const KvParams& p, uint64_t u)
{
    if (u >= p.units) return -1;
    const uint32_t row = __builtin_amdgcn_readfirstlane(fdiv((uint32_t)u, p.div));
    // the slot table is read-only here: the constant address space lets the
    // uniform load go through the scalar unit
    typedef const __attribute__((address_space(4))) int64_t* slot_ptr;
    return ((slot_ptr)p.slots)[row];
}

// Write: a chunk is 64 blocks of 16 features of one token row, one block per
// lane, with the arithmetic of the 1x16 row quantization under amax_in.  Each
// iteration takes two units (u and u + step) and issues both rows' loads
// before either is encoded, doubling the bytes in flight per wave.
template <bool kBF16>
__device__ __forceinline__ void kv_write_block(const KvParams& p, const TensorScale& ts,
                                               int64_t slot, uint32_t cb, const float v[16])
{
    float aB = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) aB = __builtin_fmaxf(aB, __builtin_fabsf(v[i]));
    BlockDiv bd;
    bool zero;
    const uint32_t e = block_scale(aB, ts, bd, zero);
    u32x2 out;
    out[0] = encode8<false>(v, bd, zero, nullptr);
    out[1] = encode8<false>(v + 8, bd, zero, nullptr);
    *reinterpret_cast<u32x2*>(p.codes + slot * (p.cols / 2) + (int64_t)cb * 8) = out;
    p.scales[slot * (p.cols / 16) + cb] = (uint8_t)e;
}

template <bool kBF16>
__global__ __launch_bounds__(256) void k_kv_write(KvParams p)
{
    constexpr int esz = kBF16 ? 2 : 4;
    const TensorScale ts = make_tensor_scale(*p.amax);
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t nbc = (uint32_t)(p.cols / 16);
    KvWalk w = kv_walk();
    int64_t next0 = kv_slot_of(p, w.u);
    int64_t next1 = kv_slot_of(p, w.u + w.step);
    for (; w.u < p.units; w.u += 2 * w.step) {
        const int64_t slot0 = next0, slot1 = next1;
        next0 = kv_slot_of(p, w.u + 2 * w.step);
        next1 = kv_slot_of(p, w.u + 3 * w.step);
        // the second unit exists only while u + step < units; otherwise it
        // repeats the first unit's addresses (loads in bounds, no stores)
        const bool has1 = w.u + w.step < p.units;
        const uint32_t u0 = (uint32_t)w.u;
        const uint32_t u1 = has1 ? (uint32_t)(w.u + w.step) : u0;
        const uint32_t t0 = __builtin_amdgcn_readfirstlane(fdiv(u0, p.div));
        const uint32_t t1 = __builtin_amdgcn_readfirstlane(fdiv(u1, p.div));
        const uint32_t cb0 = (u0 - t0 * p.div.d) * 64u + lane;
        const uint32_t cb1 = (u1 - t1 * p.div.d) * 64u + lane;
        // lanes past the row's last block load that block and store nothing
        const uint32_t lb0 = cb0 < nbc ? cb0 : nbc - 1u;
        const uint32_t lb1 = cb1 < nbc ? cb1 : nbc - 1u;
        const Raw16<kBF16> r0 = load_raw16<kBF16>(p.x + ((int64_t)t0 * p.ld + (int64_t)lb0 * 16) * esz);
        const Raw16<kBF16> r1 = load_raw16<kBF16>(p.x + ((int64_t)t1 * p.ld + (int64_t)lb1 * 16) * esz);
        float v[16];
        if (slot0 >= 0 && slot0 < p.num_slots && cb0 < nbc) {
            unpack16<kBF16>(r0, v);
            kv_write_block<kBF16>(p, ts, slot0, cb0, v);
        }
        if (has1 && slot1 >= 0 && slot1 < p.num_slots && cb1 < nbc) {
            unpack16<kBF16>(r1, v);
            kv_write_block<kBF16>(p, ts, slot1, cb1, v);
        }
    }
}

// Read: a chunk is 512 features of one gathered row, 8 per lane (one code
// word), so each lane's 16-byte BF16 store (or two FP32 stores) sits next to
// its neighbours'.  Out-of-range slots give zero rows.  Two units per
// iteration, loads first, as in the write.
template <bool kOutBF16>
__global__ __launch_bounds__(256) void k_kv_read(KvParams p)
{
    const float s_g = *p.amax / kGlobalDivisor;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t nq = (uint32_t)(p.cols / 8);
    KvWalk w = kv_walk();
    int64_t next0 = kv_slot_of(p, w.u);
    int64_t next1 = kv_slot_of(p, w.u + w.step);
    for (; w.u < p.units; w.u += 2 * w.step) {
        const int64_t slot0 = next0, slot1 = next1;
        next0 = kv_slot_of(p, w.u + 2 * w.step);
        next1 = kv_slot_of(p, w.u + 3 * w.step);
        const bool has1 = w.u + w.step < p.units;
        const uint32_t u0 = (uint32_t)w.u;
        const uint32_t u1 = has1 ? (uint32_t)(w.u + w.step) : u0;
        const uint32_t r0 = __builtin_amdgcn_readfirstlane(fdiv(u0, p.div));
        const uint32_t r1 = __builtin_amdgcn_readfirstlane(fdiv(u1, p.div));
        const uint32_t cq0 = (u0 - r0 * p.div.d) * 64u + lane;
        const uint32_t cq1 = (u1 - r1 * p.div.d) * 64u + lane;
        const bool v0 = slot0 >= 0 && slot0 < p.num_slots;
        const bool v1 = slot1 >= 0 && slot1 < p.num_slots;
        // loads from clamped addresses (slot 0, the row's last word) so that
        // both units' loads issue unconditionally; invalid ones are discarded
        const int64_t s0 = v0 ? slot0 : 0, s1 = v1 ? slot1 : 0;
        const int64_t l0 = (int64_t)(cq0 < nq ? cq0 : nq - 1u) * 8;
        const int64_t l1 = (int64_t)(cq1 < nq ? cq1 : nq - 1u) * 8;
        uint32_t w0 = *reinterpret_cast<const uint32_t*>(p.codes + s0 * (p.cols / 2) + l0 / 2);
        uint32_t w1 = *reinterpret_cast<const uint32_t*>(p.codes + s1 * (p.cols / 2) + l1 / 2);
        const uint32_t b0 = p.scales[s0 * (p.cols / 16) + l0 / 16];
        const uint32_t b1 = p.scales[s1 * (p.cols / 16) + l1 / 16];
        float e[8];
        if (cq0 < nq) {
            const float ev = v0 ? e4m3_decode(b0) : 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) e[j] = ev;
            dequant8_store<kOutBF16>(v0 ? w0 : 0u, e, s_g,
                                     p.out + ((int64_t)r0 * p.ld + l0) * (kOutBF16 ? 2 : 4));
        }
        if (has1 && cq1 < nq) {
            const float ev = v1 ? e4m3_decode(b1) : 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) e[j] = ev;
            dequant8_store<kOutBF16>(v1 ? w1 : 0u, e, s_g,
                                     p.out + ((int64_t)r1 * p.ld + l1) * (kOutBF16 ? 2 : 4));
        }
    }
}

// ------------------------------------------------------------ launchers

// ------------------------------------------------------------ MXFP4
// The power-of-two format the pages set NVFP4 against (guiahardware.es
// "NVFP4: cos'e e come supera FP8 e BF16", section "Cos'e NVFP4"; chaitex.ru
// "FP4", the comparison with the open standard), with the OCP MX v1.0 block
// and scale rule: 32 consecutive elements of a row share the E8M0 scale
// X = 2^(floor(log2 amax) - 2) (exponent clamped to -127 from below), and
// each element is E2M1_RNE_sat(x / X) with its sign.  floor(log2 amax) is
// the biased exponent field of amax minus 127 (0 for zero and subnormal
// amax, which the clamp sends to X = 2^-127), so the scale byte is
// max(field - 2, 0), and x / X = x * 2^(127 - u) exactly (a power of two).
struct MxQuantParams {
    const uint8_t* x;
    int64_t ld;       // elements
    uint32_t items;   // blocks of 32
    FastDiv div;      // blocks per row
    uint8_t* codes;   // [rows, cols/2]
    uint8_t* scales;  // [rows, cols/32]
};

template <bool kBF16>
__global__ __launch_bounds__(256) void k_mx_quant(MxQuantParams p)
{
    constexpr int esz = kBF16 ? 2 : 4;
    const uint32_t stride = gridDim.x * blockDim.x;
    for (uint32_t b = blockIdx.x * blockDim.x + threadIdx.x; b < p.items; b += stride) {
        const uint32_t row = fdiv(b, p.div);
        const uint32_t cb = b - row * p.div.d;
        const uint8_t* src = p.x + ((int64_t)row * p.ld + (int64_t)cb * 32) * esz;
        float v[32];
#pragma unroll
        for (int q = 0; q < 4; ++q) load8<kBF16>(src + 8 * q * esz, v + 8 * q);
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < 32; ++i) amax = __builtin_fmaxf(amax, __builtin_fabsf(v[i]));
        const uint32_t field = __float_as_uint(amax) >> 23;
        const uint32_t u = field > 2u ? field - 2u : 0u;
        const float inv = __uint_as_float((254u - u) << 23);  // 2^(127 - u) = 1 / X
        float y[32];
#pragma unroll
        for (int i = 0; i < 32; ++i)
            y[i] = __uint_as_float(__float_as_uint(__builtin_fabsf(v[i]) * inv) |
                                   (__float_as_uint(v[i]) & 0x80000000u));
        u32x4 out;
#pragma unroll
        for (int w = 0; w < 4; ++w) out[w] = pack8_rne(y + 8 * w);
        *reinterpret_cast<u32x4*>(p.codes + (int64_t)b * 16) = out;
        p.scales[b] = (uint8_t)u;
    }
}

static int grid_for(uint64_t work_threads, int cap)
{
    uint64_t g = (work_threads + 255) / 256;
    if (g < 1) g = 1;
    if (g > (uint64_t)cap) g = cap;
    return (int)g;
}

constexpr int kGridCap = 8192;  // >= 32 workgroups per CU on 256 CUs

static QuantParams make_params(const QuantArgs& a)
{
    QuantParams p{};
    p.x = static_cast<const uint8_t*>(a.x);
    p.rows = a.rows;
    p.cols = a.cols;
    p.ld = a.ld;
    p.codes = a.codes;
    p.scales = a.scales;
    p.tensor_scale = a.tensor_scale;
    p.amax_out = a.amax_out;
    p.seed = a.seed;
    p.stream_id = a.stream_id;
    p.mask = a.mask;
    return p;
}

// Which kernel family a quantize call maps to, with its work items.
enum Family { kRows, kCols, k2D };

static Family family_of(const QuantArgs& a)
{
    if (a.block2d) return k2D;
    return a.axis == 1 ? kRows : kCols;
}

static void set_items(const QuantArgs& a, Family f, QuantParams& p)
{
    if (f == kRows) {
        p.items = (uint32_t)(a.rows * (a.cols / 16));
        p.div = make_fastdiv((uint32_t)(a.cols / 16));
    } else if (f == kCols) {
        p.items = (uint32_t)((a.rows / 16) * (a.cols / 4));
        p.div = make_fastdiv((uint32_t)(a.cols / 4));
    } else {
        uint32_t strips = (uint32_t)((a.cols + 255) / 256);
        p.items = (uint32_t)((a.rows / 16) * strips);
        p.div = make_fastdiv(strips);
    }
}

#define NVFP4_DISPATCH_BOOL(cond, NAME, ...) \
    do {                                     \
        if (cond) {                          \
            constexpr bool NAME = true;      \
            __VA_ARGS__;                     \
        } else {                             \
            constexpr bool NAME = false;     \
            __VA_ARGS__;                     \
        }                                    \
    } while (0)

hipError_t launch_amax(const QuantArgs& a, float* partials, float* amax_dst, hipStream_t s)
{
    QuantParams p = make_params(a);
    p.partials = partials;
    // amax without the transform is layout independent: use the row kernel
    Family f = (a.rht && !a.block2d && a.axis == 0) ? kCols : kRows;
    QuantArgs aa = a;
    set_items(aa, f, p);
    int grid = grid_for(p.items, kMaxAmaxPartials);
    bool dense = (a.ld == a.cols);
    bool rht = a.rht && !a.block2d;
    if (f == kRows) {
        NVFP4_DISPATCH_BOOL(a.bf16, BF, NVFP4_DISPATCH_BOOL(rht, RH, NVFP4_DISPATCH_BOOL(dense, DE,
            hipLaunchKernelGGL((k_quant_rows<BF, false, RH, true, DE>), dim3(grid), dim3(256), 0, s,
                               p))));
    } else {
        NVFP4_DISPATCH_BOOL(a.bf16, BF,
            hipLaunchKernelGGL((k_quant_cols<BF, false, true, true>), dim3(grid), dim3(256), 0, s,
                               p));
    }
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_amax_finalize, dim3(1), dim3(256), 0, s, partials, grid, amax_dst,
                       a.amax_out);
    return hipGetLastError();
}

hipError_t launch_amax_dual(const QuantArgs& a, float* partials, float* amax_dst,
                            float* amax_rht_dst, hipStream_t s)
{
    QuantParams p = make_params(a);
    p.partials = partials;
    set_items(a, kCols, p);
    int grid = grid_for(p.items, kMaxAmaxPartials);
    NVFP4_DISPATCH_BOOL(a.bf16, BF,
        hipLaunchKernelGGL((k_amax_dual<BF>), dim3(grid), dim3(256), 0, s, p));
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_amax_finalize, dim3(1), dim3(256), 0, s, partials, grid, amax_dst,
                       (float*)nullptr);
    hipLaunchKernelGGL(k_amax_finalize, dim3(1), dim3(256), 0, s, partials + kMaxAmaxPartials,
                       grid, amax_rht_dst, (float*)nullptr);
    return hipGetLastError();
}

hipError_t launch_amax_finalize(const float* partials, int n, float* amax, hipStream_t s)
{
    hipLaunchKernelGGL(k_amax_finalize, dim3(1), dim3(256), 0, s, partials, n, amax,
                       (float*)nullptr);
    return hipGetLastError();
}

hipError_t launch_swiglu_amax(const void* h, int64_t rows, int64_t F, int64_t ld_h, void* act,
                              int64_t ld_a, uint32_t mask, float* partials, float* amax,
                              float* amax_rht, hipStream_t s)
{
    const uint32_t items = (uint32_t)((rows / 16) * (F / 4));
    const FastDiv div = make_fastdiv((uint32_t)(F / 4));
    int grid = grid_for(items, kMaxAmaxPartials);
    hipLaunchKernelGGL(k_swiglu_amax, dim3(grid), dim3(256), 0, s, static_cast<const uint8_t*>(h),
                       ld_h, static_cast<uint8_t*>(act), ld_a, F, items, div, mask & 0xFFFFu,
                       partials);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(k_amax_finalize, dim3(1), dim3(256), 0, s, partials, grid, amax,
                       (float*)nullptr);
    hipLaunchKernelGGL(k_amax_finalize, dim3(1), dim3(256), 0, s, partials + kMaxAmaxPartials,
                       grid, amax_rht, (float*)nullptr);
    return hipGetLastError();
}

hipError_t launch_quantize(const QuantArgs& a, const float* amax_src, bool write_amax_out,
                           hipStream_t s)
{
    QuantParams p = make_params(a);
    p.amax_src = amax_src;
    p.write_amax_out = write_amax_out && a.amax_out != nullptr;
    Family f = family_of(a);
    set_items(a, f, p);
    bool dense = (a.ld == a.cols);
    if (f == kRows) {
        int grid = grid_for(p.items, kGridCap);
        NVFP4_DISPATCH_BOOL(a.bf16, BF, NVFP4_DISPATCH_BOOL(a.sr, SR,
            NVFP4_DISPATCH_BOOL(a.rht, RH, NVFP4_DISPATCH_BOOL(dense, DE,
                hipLaunchKernelGGL((k_quant_rows<BF, SR, RH, false, DE>), dim3(grid), dim3(256), 0,
                                   s, p)))));
    } else if (f == kCols) {
        int grid = grid_for(p.items, kGridCap);
        NVFP4_DISPATCH_BOOL(a.bf16, BF, NVFP4_DISPATCH_BOOL(a.sr, SR,
            NVFP4_DISPATCH_BOOL(a.rht, RH,
                hipLaunchKernelGGL((k_quant_cols<BF, SR, RH, false>), dim3(grid), dim3(256), 0, s,
                                   p))));
    } else {
        int grid = grid_for((uint64_t)p.items * 64, kGridCap);
        NVFP4_DISPATCH_BOOL(a.bf16, BF, NVFP4_DISPATCH_BOOL(a.sr, SR,
            hipLaunchKernelGGL((k_quant_2d<BF, SR>), dim3(grid), dim3(256), 0, s, p)));
    }
    return hipGetLastError();
}

hipError_t launch_quantize_transposed(const QuantArgs& a, const float* amax_src,
                                      bool write_amax_out, hipStream_t s)
{
    QuantParams p = make_params(a);
    p.amax_src = amax_src;
    p.write_amax_out = write_amax_out && a.amax_out != nullptr;
    const uint32_t tiles_c = (uint32_t)((a.cols + kTT - 1) / kTT);
    p.items = (uint32_t)((a.rows + kTT - 1) / kTT) * tiles_c;
    p.div = make_fastdiv(tiles_c);
    int grid = (int)(p.items < (uint32_t)kGridCap ? p.items : (uint32_t)kGridCap);
    if (a.block2d) {
        NVFP4_DISPATCH_BOOL(a.bf16, BF, NVFP4_DISPATCH_BOOL(a.sr, SR,
            hipLaunchKernelGGL((k_quant_t<BF, SR, false, true>), dim3(grid), dim3(256), 0, s, p)));
    } else {
        NVFP4_DISPATCH_BOOL(a.bf16, BF, NVFP4_DISPATCH_BOOL(a.sr, SR,
            NVFP4_DISPATCH_BOOL(a.rht, RH,
                hipLaunchKernelGGL((k_quant_t<BF, SR, RH, false>), dim3(grid), dim3(256), 0, s,
                                   p))));
    }
    return hipGetLastError();
}

hipError_t launch_transpose(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                            int64_t cols, int block2d, int axis, uint8_t* codes_t,
                            uint8_t* scales_t, hipStream_t s)
{
    TransposeParams p{};
    p.codes = codes;
    p.scales = scales;
    p.codes_t = codes_t;
    p.scales_t = scales_t;
    p.rows = rows;
    p.cols = cols;
    if (block2d) {
        p.s_rows = rows / 16; p.s_cols = cols / 16;
        p.s_tr_log = 4; p.s_tc_log = 4; p.s_r_div = 16; p.s_c_div = 16;
    } else if (axis == 1) {
        p.s_rows = rows; p.s_cols = cols / 16;
        p.s_tr_log = 8; p.s_tc_log = 4; p.s_r_div = 1; p.s_c_div = 16;
    } else {
        p.s_rows = rows / 16; p.s_cols = cols;
        p.s_tr_log = 4; p.s_tc_log = 8; p.s_r_div = 16; p.s_c_div = 1;
    }
    const uint32_t tiles_c = (uint32_t)((cols + kTT - 1) / kTT);
    p.tiles = (uint32_t)((rows + kTT - 1) / kTT) * tiles_c;
    p.div = make_fastdiv(tiles_c);
    const int grid = (int)(p.tiles < (uint32_t)kGridCap ? p.tiles : (uint32_t)kGridCap);
    hipLaunchKernelGGL(k_transpose, dim3(grid), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_write_zero_scale(float* tensor_scale, float* amax_out, hipStream_t s)
{
    hipLaunchKernelGGL(k_write_zero_scale, dim3(1), dim3(1), 0, s, tensor_scale, amax_out);
    return hipGetLastError();
}

hipError_t launch_rht16(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld_x,
                        int axis, uint32_t mask, float* y, int64_t ld_y, hipStream_t s)
{
    const uint8_t* xb = static_cast<const uint8_t*>(x);
    if (axis == 1) {
        uint32_t items = (uint32_t)(rows * (cols / 16));
        FastDiv div = make_fastdiv((uint32_t)(cols / 16));
        int grid = grid_for(items, kGridCap);
        NVFP4_DISPATCH_BOOL(bf16, BF,
            hipLaunchKernelGGL((k_rht16_rows<BF>), dim3(grid), dim3(256), 0, s, xb, ld_x, items,
                               div, mask, y, ld_y));
    } else {
        uint32_t items = (uint32_t)((rows / 16) * (cols / 8));
        FastDiv div = make_fastdiv((uint32_t)(cols / 8));
        int grid = grid_for(items, kGridCap);
        NVFP4_DISPATCH_BOOL(bf16, BF,
            hipLaunchKernelGGL((k_rht16_cols<BF>), dim3(grid), dim3(256), 0, s, xb, ld_x, items,
                               div, mask, y, ld_y));
    }
    return hipGetLastError();
}

hipError_t launch_mx_quantize(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld,
                              uint8_t* codes, uint8_t* scales, hipStream_t s)
{
    MxQuantParams p;
    p.x = static_cast<const uint8_t*>(x);
    p.ld = ld;
    p.items = (uint32_t)(rows * (cols / 32));
    p.div = make_fastdiv((uint32_t)(cols / 32));
    p.codes = codes;
    p.scales = scales;
    const int grid = grid_for(p.items, kGridCap);
    NVFP4_DISPATCH_BOOL(bf16, BF, hipLaunchKernelGGL((k_mx_quant<BF>), dim3(grid), dim3(256), 0, s, p));
    return hipGetLastError();
}

hipError_t launch_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                int64_t cols, bool out_bf16, void* out, int64_t ld_out,
                                hipStream_t s)
{
    uint32_t items = (uint32_t)(rows * (cols / 8));
    FastDiv div = make_fastdiv((uint32_t)(cols / 8));
    int grid = grid_for(items, kGridCap);
    NVFP4_DISPATCH_BOOL(out_bf16, OB,
        hipLaunchKernelGGL((k_dequant<OB, 3>), dim3(grid), dim3(256), 0, s, codes, scales,
                           (const float*)nullptr, cols, items, div, static_cast<uint8_t*>(out),
                           ld_out));
    return hipGetLastError();
}

hipError_t launch_kv_cache_write(const void* x, bool bf16, int64_t tokens, int64_t cols,
                                 int64_t ld, const int64_t* slots, int64_t num_slots,
                                 const float* amax, uint8_t* codes, uint8_t* scales,
                                 hipStream_t s)
{
    KvParams p{};
    p.x = static_cast<const uint8_t*>(x);
    p.ld = ld;
    p.slots = slots;
    p.num_slots = num_slots;
    p.cols = cols;
    p.amax = amax;
    p.codes = codes;
    p.scales = scales;
    const uint32_t chunks = (uint32_t)((cols / 16 + 63) / 64);  // 64 blocks per chunk
    p.units = (uint32_t)(tokens * chunks);
    p.div = make_fastdiv(chunks);
    const int grid = grid_for((uint64_t)p.units * 64, kGridCap);
    NVFP4_DISPATCH_BOOL(bf16, BF, hipLaunchKernelGGL((k_kv_write<BF>), dim3(grid), dim3(256), 0, s, p));
    return hipGetLastError();
}

hipError_t launch_kv_cache_read(const uint8_t* codes, const uint8_t* scales, const float* amax,
                                int64_t num_slots, int64_t cols, const int64_t* slots, int64_t n,
                                bool out_bf16, void* out, int64_t ld_out, hipStream_t s)
{
    KvParams p{};
    p.ld = ld_out;
    p.slots = slots;
    p.num_slots = num_slots;
    p.cols = cols;
    p.amax = amax;
    p.codes = const_cast<uint8_t*>(codes);
    p.scales = const_cast<uint8_t*>(scales);
    p.out = static_cast<uint8_t*>(out);
    const uint32_t chunks = (uint32_t)((cols / 8 + 63) / 64);   // 512 features per chunk
    p.units = (uint32_t)(n * chunks);
    p.div = make_fastdiv(chunks);
    const int grid = grid_for((uint64_t)p.units * 64, kGridCap);
    NVFP4_DISPATCH_BOOL(out_bf16, OB, hipLaunchKernelGGL((k_kv_read<OB>), dim3(grid), dim3(256), 0, s, p));
    return hipGetLastError();
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* ts,
                             int64_t rows, int64_t cols, int block2d, int axis, bool out_bf16,
                             void* out, int64_t ld_out, hipStream_t s)
{
    uint32_t items = (uint32_t)(rows * (cols / 8));
    FastDiv div = make_fastdiv((uint32_t)(cols / 8));
    int grid = grid_for(items, kGridCap);
    uint8_t* o = static_cast<uint8_t*>(out);
    int mode = block2d ? 2 : (axis == 1 ? 0 : 1);
#define NVFP4_DQ(M)                                                                              \
    NVFP4_DISPATCH_BOOL(out_bf16, OB,                                                            \
        hipLaunchKernelGGL((k_dequant<OB, M>), dim3(grid), dim3(256), 0, s, codes, scales, ts,   \
                           cols, items, div, o, ld_out))
    if (mode == 0) NVFP4_DQ(0);
    else if (mode == 1) NVFP4_DQ(1);
    else NVFP4_DQ(2);
#undef NVFP4_DQ
    return hipGetLastError();
}

}  // namespace nvfp4
