// Device helpers shared by the NVFP4 kernels (gfx950 / CDNA4).
//
// Format (guiahardware.es "NVFP4: cos'e e come supera FP8 e BF16", section
// "Cos'e NVFP4"; chaitex.ru "FP4", mathematical-structure section): E2M1
// elements, one E4M3 scale per 16 elements, one FP32 tensor scale.
//
// Every helper here is exact with respect to the IEEE FP32 convention the
// C ABI documents (include/nvfp4.h): each step is one FP32 operation rounded
// to nearest-even.  The hardware conversions used were checked to round to
// nearest-even: FP32->E2M1 (v_cvt_scalef32_pk_fp4_f32, saturating, sign
// kept) and FP32->E4M3 (v_cvt_pk_fp8_f32, which gives NaN from 464 on, so
// inputs are clamped to 448 first).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace nvfp4 {

typedef float float2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// 6 * 448: largest E2M1 magnitude times largest E4M3 magnitude.
constexpr float kGlobalDivisor = 2688.0f;

// ---------------------------------------------------------------- loads

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Eight consecutive input values (BF16 or FP32) starting at p (16-byte aligned).
template <bool kBF16>
__device__ __forceinline__ void load8(const void* p, float v[8])
{
    if (kBF16) {
        u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf16_lo(w[i]);
            v[2 * i + 1] = bf16_hi(w[i]);
        }
    } else {
        u32x4 a = reinterpret_cast<const u32x4*>(p)[0];
        u32x4 b = reinterpret_cast<const u32x4*>(p)[1];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[i] = __uint_as_float(a[i]);
            v[4 + i] = __uint_as_float(b[i]);
        }
    }
}

// ---------------------------------------------------------------- E4M3

// E4M3 code of t >= 0 (RNE, saturating at 448; +inf also gives 448).
__device__ __forceinline__ uint32_t e4m3_encode(float t)
{
    float c = __builtin_fminf(t, 448.0f);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, c, 0, false) & 0xFFu;
}

// FP32 value of the E4M3 code held in the low byte of `code`.
__device__ __forceinline__ float e4m3_decode(uint32_t code)
{
    return __builtin_amdgcn_cvt_f32_fp8((int)code, 0);
}

// ---------------------------------------------------------------- division

// Correctly rounded |x| / d for a block: r = RN(1/d) comes from one IEEE
// division per block; two FMA refinement steps (Markstein) then give
// RN(|x|/d) per element.  The first step turns q0 = RN(|x| r) into an
// approximation within one ulp; the second is Markstein's theorem
// (correct rounding from a faithful quotient and a correctly rounded
// reciprocal, with exact FMA remainders).  Valid when no intermediate
// underflows or overflows; callers route the rest through IEEE division.
__device__ __forceinline__ float div_markstein(float ax, float d, float r)
{
    float q0 = ax * r;
    float e0 = __builtin_fmaf(-q0, d, ax);
    float q1 = __builtin_fmaf(e0, r, q0);
    float e1 = __builtin_fmaf(-q1, d, ax);
    return __builtin_fmaf(e1, r, q1);
}

// Per-block quotient context: d = RN(e * s_g) and r = RN(1/d).
struct BlockDiv {
    float d, r;
    bool fast;        // d far from the FP32 range ends, so Markstein applies to non-tiny |x|
    bool codes_fast;  // d >= 2^-40 as well: codes need no per-element test (quotients_codes)
};

__device__ __forceinline__ BlockDiv make_block_div(float d)
{
    BlockDiv b;
    b.d = d;
    b.r = 1.0f / d;
    b.fast = (d >= 0x1p-60f) && (d <= 0x1p60f);
    b.codes_fast = (d >= 0x1p-40f) && (d <= 0x1p60f);
    return b;
}

// 0 < a < 2^-60 (a >= 0): operands whose Markstein intermediates could underflow.
__device__ __forceinline__ bool tiny_nonzero(float a)
{
    return (__float_as_uint(a) - 1u) < 0x217FFFFFu;
}

// y[i] = RN(|x[i]| / d) for n values of one block.  Markstein everywhere; a
// wave-uniform branch redoes the rare tiny or extreme operands with IEEE
// division.
template <int n>
__device__ __forceinline__ void quotient_mags(const float* x, const BlockDiv& b, float* y)
{
    bool slow = !b.fast;
#pragma unroll
    for (int i = 0; i < n; ++i) {
        float ax = __builtin_fabsf(x[i]);
        y[i] = div_markstein(ax, b.d, b.r);
        slow |= tiny_nonzero(ax);
    }
    if (slow) {
#pragma unroll
        for (int i = 0; i < n; ++i) {
            float ax = __builtin_fabsf(x[i]);
            if (!b.fast || tiny_nonzero(ax)) y[i] = ax / b.d;
        }
    }
}

// y[i] = RN(x[i] / d) with the sign of x[i] (so -0 stays -0).
template <int n>
__device__ __forceinline__ void quotients(const float* x, const BlockDiv& b, float* y)
{
    quotient_mags<n>(x, b, y);
#pragma unroll
    for (int i = 0; i < n; ++i)
        y[i] = __uint_as_float(__float_as_uint(y[i]) | (__float_as_uint(x[i]) & 0x80000000u));
}

// The same where only the E2M1 codes (round to nearest) of the quotients
// matter.  In a block with d >= 2^-40 an element below 2^-60 has |x| / d <
// 2^-20, far under the first rounding boundary 0.25, and Markstein's
// intermediates on it, denormal or not, stay that small, so its code is the
// signed zero either way; every other element meets Markstein's conditions.
// Such blocks skip the per-element test; the rest take quotients().
template <int n>
__device__ __forceinline__ void quotients_codes(const float* x, const BlockDiv& b, float* y)
{
    if (b.codes_fast) {
#pragma unroll
        for (int i = 0; i < n; ++i) {
            const float q = div_markstein(__builtin_fabsf(x[i]), b.d, b.r);
            y[i] = __uint_as_float(__float_as_uint(q) | (__float_as_uint(x[i]) & 0x80000000u));
        }
    } else {
        quotients<n>(x, b, y);
    }
}

// True when y (FP32 bits u, either sign) lies within 8 units in the last
// place of a number whose significand has at most 3 bits (the low 21 bits of
// its mantissa field are 0).  Every E2M1 rounding boundary (0.25, 0.75, 1.25,
// 1.75, 2.5, 3.5, 5) is such a number; so are the E2M1 values themselves and
// a few others, which only costs an unneeded exact quotient.  Three
// operations: a test of the boundaries alone measured slower overall.
__device__ __forceinline__ bool near_e2m1_boundary(uint32_t u)
{
    return ((u + 8u) & 0x1FFFFFu) < 16u;
}

// Quotients for round-to-nearest E2M1 encoding: y[i] rounds to the same E2M1
// code (RNE, saturating, sign kept) as RN(x[i] / d).  Worth it only where
// quotients rarely sit on a boundary: on BF16 inputs without the Hadamard
// transform, x / d is exactly 0.75, 1.75 or 3.5 for about 0.1-0.2 % of the
// elements (x with amax's significand, scales 1.5 or 1.75 times a power of
// two: 2688 = 21 * 2^7), which sends a quarter to two thirds of the waves
// through the exact quotient as well, so those paths keep the exact one.  y0 = RN(x r) with
// r = RN(1/d) is within 2.5 ulp of RN(x/d) (two roundings of relative size
// 2^-24 each), so the two encode alike unless an E2M1 rounding boundary lies
// between them or on one of them, i.e. unless y0 is within a few ulps of a
// boundary; those lanes (and blocks whose d is outside Markstein's range)
// take the exact quotient.  Values that underflow in x r are far below 0.25
// and encode as (signed) zero either way.
// The check is wave-wide (any lane near a boundary sends the whole wave
// through the exact quotient), so the common path has no divergent branch.
template <int n>
__device__ __forceinline__ void quotients_rne(const float* x, const BlockDiv& b, float* y)
{
    bool exact = !b.fast;
#pragma unroll
    for (int i = 0; i < n; ++i) {
        y[i] = x[i] * b.r;
        exact |= near_e2m1_boundary(__float_as_uint(y[i]));
    }
    if (__builtin_amdgcn_ballot_w64(exact) != 0) quotients_codes<n>(x, b, y);
}

// Single quotient (block-scale computation).
__device__ __forceinline__ float quotient(float x, const BlockDiv& b)
{
    float y;
    quotients<1>(&x, b, &y);
    return y;
}

// ---------------------------------------------------------------- E2M1

// Two E2M1 codes (RNE, saturating, sign kept) packed into byte `sel` of `old`:
// low nibble = a, high nibble = b.
template <int sel>
__device__ __forceinline__ uint32_t fp4_pack2(uint32_t old, float a, float b)
{
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, sel);
}

// Stochastic rounding of a = |y| (y = RN(x/d)) with the uniform word r.
// Returns the chosen E2M1 magnitude as FP32 (exactly representable, so the
// hardware RNE conversion encodes it unchanged).  With lo <= a < hi the
// neighbouring grid values, the result is hi when r < frac * 2^32,
// frac = (a - lo)/(hi - lo); a >= 6 saturates to 6.  The grid step is 0.5
// below 2, 1 in [2, 4) and 2 in [4, 6]: t = a / step is exact, lo = floor(t)
// * step, frac = t - floor(t) (exact), and frac * 2^32 < 2^32 - 255, so its
// ceiling fits 32 bits and "r < frac * 2^32" is "r < ceil(frac * 2^32)".
__device__ __forceinline__ float e2m1_sr_value(float a, uint32_t r)
{
    a = __builtin_fminf(a, 6.0f);
    // step = 2^(k-2) with k = clamp(exponent of a as m * 2^k, m in [0.5, 1), 1, 3):
    // 0.5 below 2, 1 in [2, 4), 2 in [4, 6]
    const int k = __builtin_amdgcn_frexp_expf(a);
    const int e = 2 - (k < 1 ? 1 : (k > 3 ? 3 : k));
    float t = __builtin_ldexpf(a, e);
    float fl = __builtin_floorf(t);
    float frac = t - fl;
    uint32_t thr = (uint32_t)__builtin_ceilf(frac * 4294967296.0f);
    float up = r < thr ? 1.0f : 0.0f;
    return __builtin_ldexpf(fl + up, -e);
}

// ---------------------------------------------------------------- Philox

// a ^ b ^ c in one gfx950 three-input bitwise op (truth table 0x96).
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c)
{
    return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11): multipliers
// 0xD2511F53 / 0xCD9E8D57, Weyl key increments 0x9E3779B9 / 0xBB67AE85.
// Per round: two 32x32->64 products and two three-way XORs.
__device__ __forceinline__ u32x4 philox4x32_10(u32x4 c, uint32_t k0, uint32_t k1)
{
#pragma unroll
    for (int i = 0; i < 10; ++i) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
        u32x4 n;
        n[0] = xor3((uint32_t)(p1 >> 32), c[1], k0);
        n[1] = (uint32_t)p1;
        n[2] = xor3((uint32_t)(p0 >> 32), c[3], k1);
        n[3] = (uint32_t)p0;
        c = n;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

// The four stochastic-rounding words for flat element indices 4g .. 4g+3.
__device__ __forceinline__ u32x4 sr_words(uint64_t seed, uint32_t stream_id, uint64_t g)
{
    u32x4 c;
    c[0] = (uint32_t)g;
    c[1] = (uint32_t)(g >> 32);
    c[2] = stream_id;
    c[3] = 0u;
    return philox4x32_10(c, (uint32_t)seed, (uint32_t)(seed >> 32));
}

// ---------------------------------------------------------------- RHT16

// y = 1/4 * H16 * D * x on 16 values in registers: sign flips from `mask`
// (bit i set -> element i negated), butterflies at distances 1, 2, 4, 8,
// then the 1/4 scaling.  Same FP32 operation order as the documented
// convention.
// rht16_butterflies is everything but the 1/4: where only max |y| is wanted,
// 0.25 * max |v| over the unscaled v equals the max over the scaled values
// (x -> RN(0.25 x) is monotone), so one multiply per block replaces sixteen.
__device__ __forceinline__ void rht16_butterflies(float v[16], uint32_t mask)
{
#pragma unroll
    for (int i = 0; i < 16; ++i)
        v[i] = __uint_as_float(__float_as_uint(v[i]) ^ (((mask >> i) & 1u) << 31));
#pragma unroll
    for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            if (j & h) continue;
            float a = v[j], b = v[j + h];
            v[j] = a + b;
            v[j + h] = a - b;
        }
    }
}

__device__ __forceinline__ void rht16_inplace(float v[16], uint32_t mask)
{
    rht16_butterflies(v, mask);
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = 0.25f * v[i];
}

// ---------------------------------------------------------------- SwiGLU

// RNE FP32 -> BF16 bits (finite inputs)
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f)
{
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// BF16 bits of two FP32 values rounded to nearest even, a in the low half:
// one v_cvt_pk_bf16_f32, the same bits as f32_to_bf16_bits on each finite
// value (these kernels keep FP32 denormals, so those round like any other).
__device__ __forceinline__ uint32_t bf16_pair(float a, float b)
{
    const float2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// exp(-g) for BF16-valued g: Cody-Waite reduction onto the hardware 2^x
// (v_exp_f32, 1 ulp on [-0.5, 0.5]): with t = -g log2(e) carried as ph + pl
// (log2(e) split into its FP32 rounding and the rest), exp(-g) =
// 2^((ph - e) + pl) * 2^e for e = rint(ph).  g is first clamped to
// [-100, 110], which keeps e and the reduced argument in range (for large |g|
// the rounding error of ph alone would exceed it) and changes nothing that
// matters: from g <= -89 on the BF16 grid 2^e overflows to infinity anyway,
// and from g >= 104 it leaves at most a denormal, where 1 + exp(-g) is 1.
__device__ __forceinline__ float exp_neg(float g)
{
    constexpr float kLog2e = 1.44269502e+00f;     // log2(e) rounded to FP32
    constexpr float kLog2eLo = 1.92596299e-08f;   // log2(e) - kLog2e
    g = __builtin_amdgcn_fmed3f(g, -100.0f, 110.0f);
    const float ph = g * -kLog2e;
    float pl = __builtin_fmaf(g, -kLog2e, -ph);
    pl = __builtin_fmaf(g, -kLog2eLo, pl);
    const float e = __builtin_rintf(ph);
    const float a = (ph - e) + pl;
    return __builtin_ldexpf(__builtin_amdgcn_exp2f(a), (int)e);
}

// silu(g) = g / (1 + exp(-g)) in FP32 for a BF16-valued gate g: silu_den,
// then silu_rcp.  The reciprocal unit (1 ulp) stands in for a correctly
// rounded division, as the result only feeds a BF16 rounding; its output
// flushes below 2^-126, so denominators from 2^126 up (g < -87.3) need the
// IEEE division, which silu_fix applies.  That never happens for g >= -87
// (1 + exp(87) < 2^126), which callers check for a whole wave (swiglu_low,
// or the denominators themselves), so the common path has no division.
__device__ __forceinline__ float silu_den(float g) { return 1.0f + exp_neg(g); }
__device__ __forceinline__ float silu_rcp(float g, float den)
{
    return g * __builtin_amdgcn_rcpf(den);
}
__device__ __forceinline__ bool silu_needs_division(float den) { return den >= 8.5070592e37f; }
__device__ __forceinline__ float silu_fix(float g, float den, float s)
{
    return silu_needs_division(den) ? g / den : s;
}

// act = BF16(BF16(s) * u) for two gate/up pairs, s = silu(g) from the steps
// above, as packed BF16 bits (the first pair in the low half): the rounding
// points of a BF16 framework's silu and multiply.  The standalone SwiGLU pass
// and the GEMM epilogue that fuses it both end here, so their outputs agree
// bit for bit.
__device__ __forceinline__ uint32_t swiglu_pack(float s0, float u0, float s1, float u1)
{
    const uint32_t sb = bf16_pair(s0, s1);
    return bf16_pair(__uint_as_float(sb << 16) * u0, __uint_as_float(sb & 0xFFFF0000u) * u1);
}

// The same from the gate values; kMayDivide = false leaves the division out
// (for waves whose gates are all >= -87).
template <bool kMayDivide>
__device__ __forceinline__ uint32_t swiglu_pair_bits(float g0, float u0, float g1, float u1)
{
    const float d0 = silu_den(g0), d1 = silu_den(g1);
    float s0 = silu_rcp(g0, d0), s1 = silu_rcp(g1, d1);
    if (kMayDivide) {
        s0 = silu_fix(g0, d0, s0);
        s1 = silu_fix(g1, d1, s1);
    }
    return swiglu_pack(s0, u0, s1, u1);
}

// True where silu may need its division (a gate below -87).
__device__ __forceinline__ bool swiglu_low(float g) { return g < -87.0f; }

// ---------------------------------------------------------------- reductions

__device__ __forceinline__ float wave_max(float v)
{
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

}  // namespace nvfp4
