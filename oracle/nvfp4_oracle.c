/*
 * nvfp4_oracle.c -- plain, slow CPU oracle for NVFP4 two-level microscaled
 * quantization, the 16-point random Hadamard transform, dequantization and
 * the NVFP4 GEMM.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, loads or
 * calls this file.  Only the test suite, the package smoke check and the
 * bench's CPU-baseline leg may use it.  It shares no code, header, table or
 * helper with the HIP kernels under nvfp4_bit_microscaled_amd/csrc.
 *
 * Sources (cited by page title and section; the pages carry no formulas):
 *  - "NVFP4: cos'e e come supera FP8 e BF16 nell'intelligenza artificiale"
 *    (guiahardware.es), section "Cos'e NVFP4": E2M1 elements (1 sign, 2
 *    exponent, 1 mantissa bit), an FP8 E4M3 scale per micro-block of 16
 *    values and a global FP32 tensor scale.
 *  - "FP4" (chaitex.ru), section "Matematicheskaya struktura FP4": the same
 *    bit split, 16-element micro-blocks with an E4M3 scale, a 32-bit
 *    tensor-wide multiplier ("two-level metadata").
 *  - readjensen.com news page on the NVFP4 training recipe, recipe
 *    paragraph: 2D block quantization of weights, a random Hadamard
 *    transform on the wgrad inputs, stochastic rounding of gradients; the
 *    three MLP GEMMs take NVFP4 inputs and emit BF16.
 *  - "Mastering Low-Precision AI" (ai-news pages.dev), first and third
 *    paragraphs: per-16 FP8 scales plus a tensor-level scale; stochastic
 *    rounding and Hadamard transforms as stabilisers.
 *
 * The pages fix no arithmetic.  This file implements the convention stated
 * for the build, in FP32 with each operation rounded to nearest-even in the
 * order written:
 *     s_g = amax / (6*448)
 *     e   = E4M3_RNE_sat( a_B / (6*s_g) )            per block
 *     q   = E2M1_RNE_sat( x / (e*s_g) )              per element
 * with zero blocks giving e = 0 and q = 0, and stochastic rounding driven by
 * Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as
 * easy as 1, 2, 3", SC'11) keyed by (seed, element index).
 *
 * The MXFP4 functions near the end follow the open MX standard for the
 * power-of-two format the pages compare NVFP4 with (block size and scale
 * rule are the standard's; the pages give neither).  The KV-cache functions
 * after them store token rows in NVFP4 under a fixed calibration scale, and
 * the SwiGLU function computes the MLP activation between its two GEMMs at
 * BF16 rounding points.
 *
 * Every function is pinned by tests/test_oracle_*.py against something other
 * than itself (torch's float8_e4m3fn and bfloat16 casts, rocRAND's Philox,
 * closed forms, brute force).  No function here is "parity unpinned".
 *
 * Build: gcc -O2 -std=c11 -fopenmp -ffp-contract=off -fPIC -shared
 * (no fast-math: IEEE single-precision rounding and subnormals are relied on).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_DT_BF16 0
#define ORACLE_DT_FP32 1

/* ------------------------------------------------------------------ */
/* Element and scale formats                                           */
/* ------------------------------------------------------------------ */

/* E2M1: bit 3 sign, bits 2..1 exponent (bias 1), bit 0 mantissa.
 * Exponent field 0 is subnormal: 0.m * 2^0.  No infinities, no NaN. */
double oracle_e2m1_value(uint8_t code)
{
    int s = (code >> 3) & 1, E = (code >> 1) & 3, m = code & 1;
    double mag = (E == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, E - 1);
    return s ? -mag : mag;
}

/* E4M3 ("fn" variant): bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0
 * mantissa.  Exponent field 0 is subnormal (m * 2^-9); S.1111.111 is NaN;
 * there is no infinity, so the largest finite magnitude is 448. */
float oracle_e4m3_value(uint8_t code)
{
    int s = (code >> 7) & 1, E = (code >> 3) & 15, m = code & 7;
    double mag;
    if (E == 15 && m == 7) return NAN;
    if (E == 0) mag = ldexp((double)m, -9);
    else mag = ldexp(1.0 + m / 8.0, E - 7);
    return (float)(s ? -mag : mag);
}

/* Round a non-negative FP32 value to the nearest finite E4M3 magnitude,
 * ties to the even code, saturating at 448 (also for +inf).  Written as a
 * search over the 127 non-negative finite codes. */
uint8_t oracle_e4m3_encode(float t)
{
    if (!(t >= 0.0f)) return 0x7F; /* NaN / negative: not produced by the method */
    if (t >= 448.0f) return 0x7E;
    double td = (double)t;
    int best = 0;
    double bestd = td; /* distance to code 0 (value 0) */
    for (int c = 1; c <= 0x7E; ++c) {
        double d = fabs(td - (double)oracle_e4m3_value((uint8_t)c));
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bestd = d;
        }
    }
    return (uint8_t)best;
}

/* Nearest E2M1 magnitude code (0..7) to |y|, ties to the even code,
 * saturating at 6. */
static int e2m1_rne_mag(double a)
{
    if (a >= 6.0) return 7; /* saturation (also for +inf) */
    int best = 0;
    double bestd = a;
    for (int c = 1; c < 8; ++c) {
        double d = fabs(a - oracle_e2m1_value((uint8_t)c));
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bestd = d;
        }
    }
    return best;
}

/* 4-bit code of y under round-to-nearest-even, sign bit kept (so -0 and
 * tiny negatives give 0x8). */
uint8_t oracle_e2m1_encode_rne(float y)
{
    int s = signbit(y) ? 1 : 0;
    return (uint8_t)((s << 3) | e2m1_rne_mag(fabs((double)y)));
}

/* Stochastic rounding of y with a uniform 32-bit word r.  With lo <= |y| < hi
 * the two neighbouring E2M1 magnitudes, the result is hi when
 * r < frac * 2^32 with frac = (|y| - lo)/(hi - lo) (an exact comparison of
 * reals), else lo.  |y| >= 6 saturates to 6. */
uint8_t oracle_e2m1_encode_sr(float y, uint32_t r)
{
    int s = signbit(y) ? 1 : 0;
    double a = fabs((double)y);
    int mag;
    if (a >= 6.0) {
        mag = 7;
    } else {
        int lo = 0;
        for (int c = 1; c < 8; ++c)
            if (oracle_e2m1_value((uint8_t)c) <= a) lo = c;
        double vlo = oracle_e2m1_value((uint8_t)lo);
        double vhi = oracle_e2m1_value((uint8_t)(lo + 1));
        double frac = (a - vlo) / (vhi - vlo);
        mag = ((double)r < frac * 4294967296.0) ? lo + 1 : lo;
    }
    return (uint8_t)((s << 3) | mag);
}

/* ------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon et al., SC'11): 10 rounds of the 4x32 Philox   */
/* S-box with multipliers 0xD2511F53 / 0xCD9E8D57 and Weyl key bumps    */
/* 0x9E3779B9 / 0xBB67AE85, as published with the method.               */
/* ------------------------------------------------------------------ */
void oracle_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int round = 0; round < 10; ++round) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The uniform word that stochastic rounding uses for element idx:
 * key = (seed mod 2^32, seed >> 32), counter = (g mod 2^32, g >> 32,
 * stream_id, 0) with g = idx >> 2, and word (idx & 3) of the output. */
uint32_t oracle_sr_word(uint64_t seed, uint32_t stream_id, uint64_t idx)
{
    uint64_t g = idx >> 2;
    uint32_t ctr[4] = {(uint32_t)g, (uint32_t)(g >> 32), stream_id, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    oracle_philox4x32_10(ctr, key, out);
    return out[idx & 3];
}

/* ------------------------------------------------------------------ */
/* 16-point random Hadamard transform                                  */
/* ------------------------------------------------------------------ */

/* y = 1/4 * H16 * D * x for one group of 16, in FP32: sign flips d_i = -1
 * where bit i of mask is set, then the radix-2 Walsh-Hadamard butterflies
 * at distances 1, 2, 4, 8 (each sum/difference rounded to FP32), then the
 * 1/4 normalisation that makes the transform orthonormal. */
static void rht16_group(const float in[16], uint32_t mask, float out[16])
{
    float v[16];
    for (int i = 0; i < 16; ++i) v[i] = ((mask >> i) & 1u) ? -in[i] : in[i];
    for (int h = 1; h < 16; h <<= 1) {
        for (int j = 0; j < 16; ++j) {
            if (j & h) continue;
            float a = v[j], b = v[j + h];
            v[j] = a + b;
            v[j + h] = a - b;
        }
    }
    for (int i = 0; i < 16; ++i) out[i] = 0.25f * v[i];
}

static float load_elem(const void* x, int dtype, int64_t ld, int64_t r, int64_t c)
{
    if (dtype == ORACLE_DT_BF16) {
        uint16_t b = ((const uint16_t*)x)[r * ld + c];
        uint32_t u = (uint32_t)b << 16;
        float f;
        memcpy(&f, &u, 4);
        return f;
    }
    return ((const float*)x)[r * ld + c];
}

/* Materialise the values that get quantized: the input converted to FP32,
 * optionally passed through RHT16 along `axis` (1: 16 consecutive columns of
 * a row; 0: 16 consecutive rows of a column). Returns a dense rows x cols
 * FP32 buffer the caller frees. */
static float* operand_values(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                             int rht, int axis, uint32_t mask)
{
    float* v = (float*)malloc(sizeof(float) * (size_t)(rows * cols > 0 ? rows * cols : 1));
    if (!v) return NULL;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) v[r * cols + c] = load_elem(x, dtype, ld, r, c);
    if (!rht) return v;
    if (axis == 1) {
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t c0 = 0; c0 < cols; c0 += 16) {
                float in[16], out[16];
                for (int i = 0; i < 16; ++i) in[i] = v[r * cols + c0 + i];
                rht16_group(in, mask, out);
                for (int i = 0; i < 16; ++i) v[r * cols + c0 + i] = out[i];
            }
    } else {
#pragma omp parallel for schedule(static)
        for (int64_t r0 = 0; r0 < rows; r0 += 16)
            for (int64_t c = 0; c < cols; ++c) {
                float in[16], out[16];
                for (int i = 0; i < 16; ++i) in[i] = v[(r0 + i) * cols + c];
                rht16_group(in, mask, out);
                for (int i = 0; i < 16; ++i) v[(r0 + i) * cols + c] = out[i];
            }
    }
    return v;
}

/* Standalone RHT16: FP32 output y[r*ld_y + c]. Returns 0 on success. */
int oracle_rht16(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x, int axis,
                 uint32_t mask, float* y, int64_t ld_y)
{
    if ((axis == 1 && cols % 16) || (axis == 0 && rows % 16)) return -1;
    float* v = operand_values(x, dtype, rows, cols, ld_x, 1, axis, mask);
    if (!v) return -2;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) y[r * ld_y + c] = v[r * cols + c];
    free(v);
    return 0;
}

/* Tensor amax: max |v| over the (optionally transformed) tensor. */
float oracle_amax(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x, int rht,
                  int axis, uint32_t mask)
{
    float* v = operand_values(x, dtype, rows, cols, ld_x, rht, axis, mask);
    if (!v) return NAN;
    float amax = 0.0f;
#pragma omp parallel for reduction(max : amax) schedule(static)
    for (int64_t i = 0; i < rows * cols; ++i) {
        float a = fabsf(v[i]);
        if (a > amax) amax = a;
    }
    free(v);
    return amax;
}

/* ------------------------------------------------------------------ */
/* Quantization                                                         */
/* ------------------------------------------------------------------ */

/* Quantize one block of n values (pointers into the FP32 operand buffer,
 * one per element) and write its scale code and element codes.
 * idx[i] is the element's flat index row*cols+col for the SR stream. */
static void quantize_block(float* const* vals, const int64_t* idx, int n, float s_g, float D6,
                           int sr, uint64_t seed, uint32_t stream_id, uint8_t* e_code,
                           uint8_t* q)
{
    float a_B = 0.0f;
    for (int i = 0; i < n; ++i) {
        float a = fabsf(*vals[i]);
        if (a > a_B) a_B = a;
    }
    uint8_t e = 0;
    float d = 0.0f;
    if (a_B > 0.0f) {
        float t = a_B / D6;               /* FP32 division, RNE */
        e = oracle_e4m3_encode(t);        /* E4M3, RNE, saturating */
        d = oracle_e4m3_value(e) * s_g;   /* FP32 product, RNE */
    }
    if (e == 0 || d == 0.0f) {            /* zero block (or scale underflow) */
        *e_code = 0;
        for (int i = 0; i < n; ++i) q[i] = 0;
        return;
    }
    *e_code = e;
    for (int i = 0; i < n; ++i) {
        float y = *vals[i] / d;           /* FP32 division, RNE */
        q[i] = sr ? oracle_e2m1_encode_sr(y, oracle_sr_word(seed, stream_id, (uint64_t)idx[i]))
                  : oracle_e2m1_encode_rne(y);
    }
}

static void put_code(uint8_t* codes, int64_t cols, int64_t r, int64_t c, uint8_t q)
{
    uint8_t* byte = &codes[r * (cols / 2) + c / 2];
    if (c & 1) *byte = (uint8_t)((*byte & 0x0F) | (q << 4));
    else *byte = (uint8_t)((*byte & 0xF0) | q);
}

/*
 * Quantize a rows x cols tensor (BF16 or FP32, leading dimension ld_x).
 *   block2d = 0: 1x16 blocks; axis 1 = along columns, axis 0 = along rows.
 *   block2d = 1: 16x16 blocks (axis ignored, rht must be 0).
 *   sr = 0: round to nearest even; sr = 1: stochastic rounding.
 *   rht = 1: apply RHT16 with `mask` along the block axis first (1D only).
 *   row0: global row index of row 0 (so a row slice of a larger tensor gets
 *         the same SR words; idx = (row0 + r) * cols + c).
 *   amax_in: if non-NULL, used as the tensor amax instead of computing it.
 * Outputs: codes [rows, cols/2] (byte j = code(2j) | code(2j+1) << 4);
 *   scales: 1D axis 1 [rows, cols/16]; 1D axis 0 [rows/16, cols];
 *           2D [rows/16, cols/16]; tensor_scale[0] = s_g; amax_out[0] = amax.
 * Returns 0, or a negative value on a shape error.
 */
int oracle_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x,
                    int block2d, int axis, int sr, uint64_t seed, uint32_t stream_id, int rht,
                    uint32_t mask, int64_t row0, const float* amax_in, uint8_t* codes,
                    uint8_t* scales, float* tensor_scale, float* amax_out)
{
    if (cols % 2) return -1;
    if (block2d && (rows % 16 || cols % 16 || rht)) return -1;
    if (!block2d && axis == 1 && cols % 16) return -1;
    if (!block2d && axis == 0 && rows % 16) return -1;

    float* v = operand_values(x, dtype, rows, cols, ld_x, rht, axis, mask);
    if (!v) return -2;

    float amax;
    if (amax_in) {
        amax = *amax_in;
    } else {
        amax = 0.0f;
#pragma omp parallel for reduction(max : amax) schedule(static)
        for (int64_t i = 0; i < rows * cols; ++i)
            if (fabsf(v[i]) > amax) amax = fabsf(v[i]);
    }
    float s_g = amax / 2688.0f;   /* 2688 = 6 * 448, FP32 division */
    float D6 = 6.0f * s_g;        /* FP32 product */
    if (tensor_scale) *tensor_scale = s_g;
    if (amax_out) *amax_out = amax;

    if (block2d) {
        int64_t nbr = rows / 16, nbc = cols / 16;
#pragma omp parallel for schedule(dynamic, 16)
        for (int64_t b = 0; b < nbr * nbc; ++b) {
            int64_t br = b / nbc, bc = b % nbc;
            float* vals[256];
            int64_t idx[256];
            uint8_t q[256], e;
            for (int i = 0; i < 16; ++i)
                for (int j = 0; j < 16; ++j) {
                    int64_t r = br * 16 + i, c = bc * 16 + j;
                    vals[i * 16 + j] = &v[r * cols + c];
                    idx[i * 16 + j] = (row0 + r) * cols + c;
                }
            quantize_block(vals, idx, 256, s_g, D6, sr, seed, stream_id, &e, q);
            scales[br * nbc + bc] = e;
            for (int i = 0; i < 16; ++i)
                for (int j = 0; j < 16; ++j)
                    put_code(codes, cols, br * 16 + i, bc * 16 + j, q[i * 16 + j]);
        }
    } else if (axis == 1) {
        int64_t nbc = cols / 16;
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t bc = 0; bc < nbc; ++bc) {
                float* vals[16];
                int64_t idx[16];
                uint8_t q[16], e;
                for (int j = 0; j < 16; ++j) {
                    int64_t c = bc * 16 + j;
                    vals[j] = &v[r * cols + c];
                    idx[j] = (row0 + r) * cols + c;
                }
                quantize_block(vals, idx, 16, s_g, D6, sr, seed, stream_id, &e, q);
                scales[r * nbc + bc] = e;
                for (int j = 0; j < 16; ++j) put_code(codes, cols, r, bc * 16 + j, q[j]);
            }
    } else {
        int64_t nbr = rows / 16;
        /* parallel over block-rows: each thread owns 16 full code rows */
#pragma omp parallel for schedule(static)
        for (int64_t br = 0; br < nbr; ++br)
            for (int64_t c = 0; c < cols; ++c) {
                float* vals[16];
                int64_t idx[16];
                uint8_t q[16], e;
                for (int i = 0; i < 16; ++i) {
                    int64_t r = br * 16 + i;
                    vals[i] = &v[r * cols + c];
                    idx[i] = (row0 + r) * cols + c;
                }
                quantize_block(vals, idx, 16, s_g, D6, sr, seed, stream_id, &e, q);
                scales[br * cols + c] = e;
                for (int i = 0; i < 16; ++i) put_code(codes, cols, br * 16 + i, c, q[i]);
            }
    }
    free(v);
    return 0;
}

/* ------------------------------------------------------------------ */
/* Dequantization                                                       */
/* ------------------------------------------------------------------ */

/* Scale code of element (r, c) of a rows x cols NVFP4 tensor. */
static uint8_t scale_of(const uint8_t* scales, int64_t rows, int64_t cols, int block2d, int axis,
                        int64_t r, int64_t c)
{
    (void)rows;
    if (block2d) return scales[(r / 16) * (cols / 16) + c / 16];
    if (axis == 1) return scales[r * (cols / 16) + c / 16];
    return scales[(r / 16) * cols + c];
}

static uint8_t code_of(const uint8_t* codes, int64_t cols, int64_t r, int64_t c)
{
    uint8_t byte = codes[r * (cols / 2) + c / 2];
    return (c & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0x0F);
}

/* val(code) * e as a double (exact: at most 6 significant bits). */
static double elem_times_scale(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                               int64_t cols, int block2d, int axis, int64_t r, int64_t c)
{
    return oracle_e2m1_value(code_of(codes, cols, r, c)) *
           (double)oracle_e4m3_value(scale_of(scales, rows, cols, block2d, axis, r, c));
}

/* Round an FP32 value to BF16 (nearest, ties to even; NaN kept quiet). */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);
    uint32_t lsb = (u >> 16) & 1u;
    u += 0x7FFFu + lsb;
    return (uint16_t)(u >> 16);
}

/* v = RN32(val * e * s_g) for every element; out_f32 dense rows x cols
 * (ld = cols); out_bf16 (optional) = RNE_bf16(v). */
int oracle_dequantize(const uint8_t* codes, const uint8_t* scales, float s_g, int64_t rows,
                      int64_t cols, int block2d, int axis, float* out_f32, uint16_t* out_bf16)
{
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            double ve = elem_times_scale(codes, scales, rows, cols, block2d, axis, r, c);
            float v = (float)ve * s_g; /* val*e exact in FP32; one FP32 rounding */
            if (out_f32) out_f32[r * cols + c] = v;
            if (out_bf16) out_bf16[r * cols + c] = oracle_f32_to_bf16(v);
        }
    return 0;
}

/*
 * The same NVFP4 tensor stored as its transpose.  Element (r, c) of the
 * rows x cols input is element (c, r) of the cols x rows output, with the
 * same code and the same block scale; the tensor scale is unchanged.  The
 * block of (r, c) becomes the block of (c, r): a 16x16 block stays 16x16,
 * blocks along rows (axis 1) become blocks down the columns (axis 0) and
 * vice versa.  This is what the recipe's 2D weight blocks are for (the
 * readjensen.com recipe paragraph: fprop and dgrad see transpose-consistent
 * values); the function is plain storage work, element by element.
 * Shape rule: rows % 16 == 0 and cols % 16 == 0.  Returns 0, or -1.
 */
int oracle_transpose(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                     int block2d, int axis, uint8_t* codes_t, uint8_t* scales_t)
{
    if (rows % 16 || cols % 16 || (!block2d && axis != 0 && axis != 1)) return -1;
    const int axis_t = block2d ? axis : 1 - axis;
    /* one output row (input column c) per iteration: threads write disjoint rows */
#pragma omp parallel for schedule(static)
    for (int64_t c = 0; c < cols; ++c)
        for (int64_t r = 0; r < rows; ++r) {
            put_code(codes_t, rows, c, r, code_of(codes, cols, r, c));
            const uint8_t e = scale_of(scales, rows, cols, block2d, axis, r, c);
            /* the output tensor is cols x rows; (c, r) is its element */
            if (block2d) scales_t[(c / 16) * (rows / 16) + r / 16] = e;
            else if (axis_t == 1) scales_t[c * (rows / 16) + r / 16] = e;
            else scales_t[(c / 16) * rows + r] = e;
        }
    return 0;
}

/* ------------------------------------------------------------------ */
/* GEMM                                                                 */
/* ------------------------------------------------------------------ */

typedef struct {
    const uint8_t* codes;
    const uint8_t* scales;
    int64_t rows, cols; /* storage shape */
    int block2d, axis;
    int k_is_row;       /* 1 if the contraction index runs along storage rows */
} operand_t;

static double op_value(const operand_t* o, int64_t i, int64_t k)
{
    int64_t r = o->k_is_row ? k : i, c = o->k_is_row ? i : k;
    return elem_times_scale(o->codes, o->scales, o->rows, o->cols, o->block2d, o->axis, r, c);
}

/*
 * NVFP4 GEMM reference on selected outputs, in FP64.
 *   layout 0 (NT): A stored [M, K], B stored [N, K]  (C = A * B^T)
 *   layout 1 (NN): A stored [M, K], B stored [K, N]  (C = A * B)
 *   layout 2 (TN): A stored [K, M], B stored [K, N]  (C = A^T * B)
 * For a 1D operand the block axis is the one along K.
 * ref[p] = s_A * s_B * sum_k (val*e)_A (val*e)_B and
 * absref[p] = s_A * s_B * sum_k |(val*e)_A (val*e)_B| for (ms[p], ns[p]).
 */
int oracle_gemm_pairs(int layout, int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                      const uint8_t* a_scales, float a_ts, int a_block2d, const uint8_t* b_codes,
                      const uint8_t* b_scales, float b_ts, int b_block2d, int64_t npairs,
                      const int64_t* ms, const int64_t* ns, double* ref, double* absref)
{
    operand_t A, B;
    A.codes = a_codes; A.scales = a_scales; A.block2d = a_block2d;
    B.codes = b_codes; B.scales = b_scales; B.block2d = b_block2d;
    if (layout == 0 || layout == 1) { A.rows = M; A.cols = K; A.k_is_row = 0; A.axis = 1; }
    else { A.rows = K; A.cols = M; A.k_is_row = 1; A.axis = 0; }
    if (layout == 0) { B.rows = N; B.cols = K; B.k_is_row = 0; B.axis = 1; }
    else { B.rows = K; B.cols = N; B.k_is_row = 1; B.axis = 0; }
    if (layout < 0 || layout > 2) return -1;
    double sab = (double)a_ts * (double)b_ts;
#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t p = 0; p < npairs; ++p) {
        double s = 0.0, sa = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double t = op_value(&A, ms[p], k) * op_value(&B, ns[p], k);
            s += t;
            sa += fabs(t);
        }
        ref[p] = sab * s;
        absref[p] = sab * sa;
    }
    return 0;
}

/*
 * Weight-only NVFP4 GEMM reference (BF16 activations, NVFP4 weights), NT:
 * A stored [M, K] as BF16 bit patterns with row pitch lda, B an NVFP4 tensor
 * stored [N, K] (1D blocks along K, or 2D).  The juejin.cn page on NVFP4
 * (item 3, ecosystem support) describes models trained at higher precision
 * being quantized to NVFP4 for inference, and "FP4" (chaitex.ru, item 1 of
 * the scaling scheme) quantizes the weight matrix in 16-element blocks; with
 * the activations left in BF16 the product is
 *   ref[p] = s_B * sum_k x[m,k] * (val*e)_B[n,k]
 * in FP64 (each product is exact) and absref[p] = s_B * sum_k |...|.
 */
int oracle_gemm_w4a16_pairs(int64_t M, int64_t N, int64_t K, const uint16_t* a, int64_t lda,
                            const uint8_t* b_codes, const uint8_t* b_scales, float b_ts,
                            int b_block2d, int64_t npairs, const int64_t* ms, const int64_t* ns,
                            double* ref, double* absref)
{
    if (M < 0 || N < 0 || K < 0 || lda < K) return -1;
    operand_t B;
    B.codes = b_codes; B.scales = b_scales; B.block2d = b_block2d;
    B.rows = N; B.cols = K; B.k_is_row = 0; B.axis = 1;
#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t p = 0; p < npairs; ++p) {
        double s = 0.0, sa = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double x = (double)load_elem(a, ORACLE_DT_BF16, lda, ms[p], k);
            double t = x * op_value(&B, ns[p], k);
            s += t;
            sa += fabs(t);
        }
        ref[p] = (double)b_ts * s;
        absref[p] = (double)b_ts * sa;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* MXFP4: the power-of-two-scaled format the pages contrast NVFP4 with */
/* ------------------------------------------------------------------ */
/*
 * "NVFP4: cos'e e come supera FP8 e BF16" (section "Cos'e NVFP4") sets the
 * E4M3-per-16 scheme against simpler power-of-two scaling such as MXFP4, and
 * "FP4" (chaitex.ru, the section comparing NVFP4 with the open standard)
 * says MXFP4 uses larger quantization blocks and coarser scale factors.  The
 * pages give no block size or scale rule; this file takes those of the OCP
 * Microscaling Formats (MX) v1.0 specification, the open standard named:
 *   - 32 consecutive elements share one E8M0 scale X = 2^(u - 127), u the
 *     stored byte (255 is NaN), no tensor-level scale;
 *   - X = 2^(floor(log2(amax)) - 2): 2 is the exponent of E2M1's largest
 *     value 6 = 1.5 * 2^2; the exponent is clamped to the E8M0 range, and a
 *     zero block (or one whose amax is below 2^-125) gets X = 2^-127;
 *   - each element is x / X rounded to E2M1 to nearest-even, saturating at
 *     +-6 (a block whose amax/X lies in (6, 8) clips), sign bit kept.
 */

/* Value of an E8M0 scale byte. */
double oracle_e8m0_value(uint8_t code)
{
    if (code == 255) return NAN;
    return ldexp(1.0, (int)code - 127);
}

/* E8M0 byte of the shared scale of a block with maximum magnitude amax. */
uint8_t oracle_mx_scale_code(float amax)
{
    if (!(amax > 0.0f)) return 0;
    int e;
    (void)frexp((double)amax, &e); /* amax = f * 2^e, 0.5 <= f < 1 */
    int x = (e - 1) - 2;           /* floor(log2(amax)) - 2 */
    if (x < -127) x = -127;
    if (x > 127) x = 127;
    return (uint8_t)(x + 127);
}

/* Quantize rows of x in blocks of 32 consecutive columns (cols % 32 == 0):
 * codes [rows, cols/2] packed as everywhere else (low nibble = even column),
 * scales [rows, cols/32] E8M0.  Returns 0, or -1 on a bad shape. */
int oracle_mx_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x,
                       uint8_t* codes, uint8_t* scales)
{
    if (rows < 0 || cols < 0 || cols % 32 != 0 || ld_x < cols) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b = 0; b < cols / 32; ++b) {
            float v[32], amax = 0.0f;
            for (int i = 0; i < 32; ++i) {
                v[i] = load_elem(x, dtype, ld_x, r, 32 * b + i);
                float a = fabsf(v[i]);
                if (a > amax) amax = a;
            }
            uint8_t u = oracle_mx_scale_code(amax);
            float X = (float)oracle_e8m0_value(u);
            scales[r * (cols / 32) + b] = u;
            for (int i = 0; i < 32; ++i) {
                float y = v[i] / X;
                put_code(codes, cols, r, 32 * b + i, oracle_e2m1_encode_rne(y));
            }
        }
    return 0;
}

/* v = val(code) * X, exact in FP64; FP32 and BF16 (RNE) copies. */
int oracle_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t cols,
                         float* out_f32, uint16_t* out_bf16)
{
    if (rows < 0 || cols < 0 || cols % 32 != 0) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            double v = oracle_e2m1_value(code_of(codes, cols, r, c)) *
                       oracle_e8m0_value(scales[r * (cols / 32) + c / 32]);
            float f = (float)v;
            if (out_f32) out_f32[r * cols + c] = f;
            if (out_bf16) out_bf16[r * cols + c] = oracle_f32_to_bf16(f);
        }
    return 0;
}

/* MXFP4 GEMM reference, NT only: A stored [M, K], B stored [N, K], both in
 * blocks of 32 along K.  ref[p] = sum_k deq(A)[m,k] deq(B)[n,k] in FP64 (each
 * product is exact) and absref[p] = sum_k |...| at (ms[p], ns[p]). */
int oracle_mx_gemm_pairs(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                         const uint8_t* a_scales, const uint8_t* b_codes, const uint8_t* b_scales,
                         int64_t npairs, const int64_t* ms, const int64_t* ns, double* ref,
                         double* absref)
{
    if (K % 32 != 0 || M < 0 || N < 0) return -1;
#pragma omp parallel for schedule(dynamic, 8)
    for (int64_t p = 0; p < npairs; ++p) {
        double s = 0.0, sa = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double a = oracle_e2m1_value(code_of(a_codes, K, ms[p], k)) *
                       oracle_e8m0_value(a_scales[ms[p] * (K / 32) + k / 32]);
            double b = oracle_e2m1_value(code_of(b_codes, K, ns[p], k)) *
                       oracle_e8m0_value(b_scales[ns[p] * (K / 32) + k / 32]);
            s += a * b;
            sa += fabs(a * b);
        }
        ref[p] = s;
        absref[p] = sa;
    }
    return 0;
}

/* ------------------------------------------------------------------ */
/* SwiGLU                                                               */
/* ------------------------------------------------------------------ */
/*
 * The activation between the MLP's two fprop GEMMs (the MLP GEMMs with BF16
 * outputs: readjensen.com recipe paragraph; the Llama 3 models of its
 * benchmark paragraph use SwiGLU), at a BF16 framework's rounding points:
 *   act = BF16( BF16(silu(g)) * u ),  silu(g) = g / (1 + exp(-g)) in FP32
 * for h = [gate | up] in BF16 [rows, 2F] (row pitch ld_h elements); act is
 * written as BF16 bit patterns [rows, F], dense.  exp is the C library's
 * single-precision expf, the division IEEE.
 */
static uint16_t bf16_bits_of(float f)
{
    return oracle_f32_to_bf16(f);
}

static float f32_of_bf16(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* silu(g) in FP32 for one value, and act for one (g, u) pair. */
float oracle_silu_f32(float g)
{
    float den = 1.0f + expf(-g);
    return g / den;
}

uint16_t oracle_swiglu_one(uint16_t g_bf16, uint16_t u_bf16)
{
    float sg = oracle_silu_f32(f32_of_bf16(g_bf16));
    float sb = f32_of_bf16(bf16_bits_of(sg));
    return bf16_bits_of(sb * f32_of_bf16(u_bf16));
}

/* act (and, if sb is not NULL, the BF16 silu values BF16(silu(gate))). */
int oracle_swiglu(const uint16_t* h, int64_t rows, int64_t F, int64_t ld_h, uint16_t* act,
                  uint16_t* sb)
{
    if (rows < 0 || F < 0 || ld_h < 2 * F) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < F; ++c) {
            act[r * F + c] = oracle_swiglu_one(h[r * ld_h + c], h[r * ld_h + F + c]);
            if (sb) sb[r * F + c] = bf16_bits_of(oracle_silu_f32(f32_of_bf16(h[r * ld_h + c])));
        }
    return 0;
}

/* ------------------------------------------------------------------ */
/* NVFP4 KV cache                                                       */
/* ------------------------------------------------------------------ */
/*
 * The NVIDIA-blog translation on juejin.cn (point 3, the ecosystem) names an
 * NVFP4 KV cache among the inference uses of the format; "FP4" (chaitex.ru,
 * mathematical-structure section) gives the inference layout: 16-element
 * micro-blocks with an E4M3 scale and one FP32 tensor scale.  The pages say
 * nothing more, so this file takes the plainest reading:
 *   - a cache holds num_slots rows of `cols` features (heads x head_dim),
 *     1x16 blocks along the features, round to nearest-even;
 *   - the tensor scale is fixed for the cache's lifetime, s_g =
 *     RN(amax / 2688) from a calibration amax the caller supplies (rows
 *     arrive a few at a time, so no amax over the whole cache exists when a
 *     row is written); features beyond the calibration amax saturate;
 *   - writing sends token t to cache row slots[t]; a slot outside
 *     [0, num_slots) skips the token (padding);
 *   - reading gathers cache rows slots[j] and dequantizes them exactly as
 *     the tensor dequantization does; an out-of-range slot gives a zero row.
 * Each written row gets the same codes and scales as quantizing that token
 * alone (rounding to nearest, 1x16 blocks, amax_in = the calibration amax).
 */
int oracle_kv_cache_write(const void* x, int dtype, int64_t tokens, int64_t cols, int64_t ld_x,
                          const int64_t* slots, float amax, int64_t num_slots,
                          uint8_t* cache_codes, uint8_t* cache_scales)
{
    if (tokens < 0 || cols < 0 || cols % 16 != 0 || ld_x < cols || num_slots < 0) return -1;
    float s_g = amax / 2688.0f;   /* FP32 division */
    float D6 = 6.0f * s_g;        /* FP32 product */
    int64_t nbc = cols / 16;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < tokens; ++t) {
        int64_t slot = slots[t];
        if (slot < 0 || slot >= num_slots) continue;
        for (int64_t bc = 0; bc < nbc; ++bc) {
            float buf[16];
            float* vals[16];
            int64_t idx[16];
            uint8_t q[16], e;
            for (int j = 0; j < 16; ++j) {
                buf[j] = load_elem(x, dtype, ld_x, t, bc * 16 + j);
                vals[j] = &buf[j];
                idx[j] = 0; /* no stochastic rounding: the index is unused */
            }
            quantize_block(vals, idx, 16, s_g, D6, 0, 0, 0, &e, q);
            cache_scales[slot * nbc + bc] = e;
            for (int j = 0; j < 16; ++j) put_code(cache_codes, cols, slot, bc * 16 + j, q[j]);
        }
    }
    return 0;
}

/* out row j = dequantized cache row slots[j] (v = RN32(val * e * s_g), and its
 * BF16 rounding), or zeros when slots[j] is outside [0, num_slots). */
int oracle_kv_cache_read(const uint8_t* cache_codes, const uint8_t* cache_scales, float amax,
                         int64_t num_slots, int64_t cols, const int64_t* slots, int64_t n,
                         float* out_f32, uint16_t* out_bf16)
{
    if (n < 0 || cols < 0 || cols % 16 != 0 || num_slots < 0) return -1;
    float s_g = amax / 2688.0f;
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        int64_t slot = slots[j];
        int valid = slot >= 0 && slot < num_slots;
        for (int64_t c = 0; c < cols; ++c) {
            float v = 0.0f;
            if (valid) {
                double ve = elem_times_scale(cache_codes, cache_scales, num_slots, cols, 0, 1,
                                             slot, c);
                v = (float)ve * s_g; /* val*e exact in FP32; one FP32 rounding */
            }
            if (out_f32) out_f32[j * cols + c] = v;
            if (out_bf16) out_bf16[j * cols + c] = oracle_f32_to_bf16(v);
        }
    }
    return 0;
}

/* Number of OpenMP threads a parallel region would use (1 without OpenMP). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
