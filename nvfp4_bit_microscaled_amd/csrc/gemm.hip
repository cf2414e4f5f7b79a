// NVFP4 GEMM for gfx950: C = s_A * s_B * sum_k (q e)_A (q e)_B, FP32 accumulate.
//
// The three MLP GEMMs of the NVFP4 recipe (readjensen.com training-recipe page,
// recipe paragraph): fprop NT, dgrad NN, wgrad TN, NVFP4 in, BF16 out.
//
// Design (CDNA4):
//   global -> LDS   packed E2M1 codes (4 bits/element) and raw E4M3 scale bytes;
//                   operands whose codes run along M/N (the [K, M|N] storage of
//                   NN's B and both TN operands) are nibble-transposed on the way,
//                   so LDS always holds K-contiguous codes and per-row scales.
//   LDS -> VGPR     one 32-bit read gives a lane the 8 K-consecutive codes an
//                   MFMA operand needs; v_cvt_scalef32_pk_f16_fp4 (scale 1.0)
//                   decodes pairs exactly, v_pk_mul_f16 applies the block scale.
//                   E2M1 x E4M3 products need at most 6 significant bits and lie
//                   in [2^-10, 2688], so they are exact FP16 normals.
//   MFMA            v_mfma_f32_32x32x16_f16: K = 16 is exactly one scale block.
//   epilogue        multiply by s_A * s_B, store BF16 (RNE) or FP32.
// FP16 is used rather than BF16 because the VALU has a packed FP16 multiply
// (two scale products per instruction) and the FP16 and BF16 MFMA rates are
// equal; both hold the scaled products exactly.
#include "device_common.h"
#include "launch.h"

namespace nvfp4 {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

struct GemmParams {
    int64_t M, N, K;
    const uint8_t* a_codes;
    const uint8_t* a_scales;
    const uint8_t* b_codes;
    const uint8_t* b_scales;
    const float* a_ts;
    const float* b_ts;
    uint8_t* c;
    int64_t ldc;
};

// 8x8 nibble transpose: in[k] holds element (k, j) in nibble j; out[j] gets
// element (k, j) in nibble k.
__device__ __forceinline__ void transpose8x8_nibbles(const uint32_t in[8], uint32_t out[8])
{
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t o = 0u;
#pragma unroll
        for (int k = 0; k < 8; ++k) o |= ((in[k] >> (4 * j)) & 0xFu) << (4 * k);
        out[j] = o;
    }
}

// Stage one operand's k-tile into LDS as K-contiguous codes [R][BK/2] and
// per-row scale codes [R][BK/16].  rows0: first row (M or N index) of the
// tile; MN: operand extent along rows; k0: first K index.
template <int R, int BK, bool kKMajor, bool k2D>
__device__ __forceinline__ void stage_operand(const uint8_t* __restrict__ codes,
                                              const uint8_t* __restrict__ scales, int64_t MN,
                                              int64_t K, int64_t rows0, int64_t k0,
                                              uint8_t* lds_codes, uint8_t* lds_scales)
{
    constexpr int kCodeRowBytes = BK / 2;
    constexpr int kKB = BK / 16;
    const int tid = threadIdx.x;
    if (kKMajor) {
        // storage [MN, K]: codes row stride K/2 bytes, u32 = 8 K-consecutive codes
        constexpr int kChunks = R * BK / 8;
        for (int c = tid; c < kChunks; c += 256) {
            int r = c / (BK / 8), q = c % (BK / 8);
            int64_t row = rows0 + r, k = k0 + q * 8;
            uint32_t w = 0u;
            if (row < MN && k < K)
                w = *reinterpret_cast<const uint32_t*>(codes + row * (K / 2) + k / 2);
            *reinterpret_cast<uint32_t*>(lds_codes + r * kCodeRowBytes + q * 4) = w;
        }
        for (int c = tid; c < R * kKB; c += 256) {
            int r = c / kKB, j = c % kKB;
            int64_t row = rows0 + r, kb = k0 / 16 + j;
            uint8_t e = 0;
            if (row < MN && kb * 16 < K)
                e = k2D ? scales[(row / 16) * (K / 16) + kb] : scales[row * (K / 16) + kb];
            lds_scales[r * kKB + j] = e;
        }
    } else {
        // storage [K, MN]: codes row stride MN/2 bytes, u32 = 8 MN-consecutive codes
        constexpr int kBlocks = (BK / 8) * (R / 8);
        for (int b = tid; b < kBlocks; b += 256) {
            int kq = b / (R / 8), mq = b % (R / 8);
            int64_t kk = k0 + kq * 8, m = rows0 + mq * 8;
            uint32_t in[8], out[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                in[i] = 0u;
                if (kk + i < K && m < MN)
                    in[i] = *reinterpret_cast<const uint32_t*>(codes + (kk + i) * (MN / 2) + m / 2);
            }
            transpose8x8_nibbles(in, out);
#pragma unroll
            for (int j = 0; j < 8; ++j)
                *reinterpret_cast<uint32_t*>(lds_codes + (mq * 8 + j) * kCodeRowBytes + kq * 4) =
                    out[j];
        }
        for (int c = tid; c < R * kKB; c += 256) {
            int r = c / kKB, j = c % kKB;
            int64_t m = rows0 + r, kb = k0 / 16 + j;
            uint8_t e = 0;
            if (m < MN && kb * 16 < K)
                e = k2D ? scales[kb * (MN / 16) + m / 16] : scales[kb * MN + m];
            lds_scales[r * kKB + j] = e;
        }
    }
}

// Decode the lane's 8 codes (one 32-bit word) times its E4M3 block scale into
// an FP16 MFMA operand.
__device__ __forceinline__ half8_t dequant8(uint32_t w, uint32_t scale_code)
{
    _Float16 e = (_Float16)e4m3_decode(scale_code);
    half2_t s2 = {e, e};
    half2_t p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
    half2_t p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
    half2_t p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
    half2_t p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
    half8_t r;
    r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
    r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
    return r;
}

// Simple tiled kernel: BM x BN tile per workgroup of 256 threads (2 x 2 waves),
// each wave (BM/2) x (BN/2) built from 32x32x16 MFMAs.
template <int BM, int BN, int BK, bool kAK, bool kBK, bool kA2D, bool kB2D, bool kOutBF16>
__global__ __launch_bounds__(256) void k_gemm_simple(GemmParams p)
{
    constexpr int WM = BM / 2, WN = BN / 2;
    constexpr int FM = WM / 32, FN = WN / 32;
    constexpr int kKB = BK / 16;
    __shared__ __attribute__((aligned(16))) uint8_t sa_codes[BM * BK / 2];
    __shared__ __attribute__((aligned(16))) uint8_t sb_codes[BN * BK / 2];
    __shared__ uint8_t sa_scales[BM * kKB];
    __shared__ uint8_t sb_scales[BN * kKB];

    const int64_t m0 = (int64_t)blockIdx.y * BM, n0 = (int64_t)blockIdx.x * BN;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave & 1, wn = wave >> 1;
    const int lr = lane & 31, lk = lane >> 5;

    float16_t acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    for (int64_t k0 = 0; k0 < p.K; k0 += BK) {
        stage_operand<BM, BK, kAK, kA2D>(p.a_codes, p.a_scales, p.M, p.K, m0, k0, sa_codes,
                                         sa_scales);
        stage_operand<BN, BK, kBK, kB2D>(p.b_codes, p.b_scales, p.N, p.K, n0, k0, sb_codes,
                                         sb_scales);
        __syncthreads();
#pragma unroll
        for (int s = 0; s < kKB; ++s) {
            half8_t af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                int row = wm * WM + i * 32 + lr;
                uint32_t w = *reinterpret_cast<const uint32_t*>(sa_codes + row * (BK / 2) +
                                                                 s * 8 + lk * 4);
                af[i] = dequant8(w, sa_scales[row * kKB + s]);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                int row = wn * WN + j * 32 + lr;
                uint32_t w = *reinterpret_cast<const uint32_t*>(sb_codes + row * (BK / 2) +
                                                                 s * 8 + lk * 4);
                bf[j] = dequant8(w, sb_scales[row * kKB + s]);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0,
                                                                        0, 0);
        }
        __syncthreads();
    }

    const float sab = (*p.a_ts) * (*p.b_ts);
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                int64_t row = m0 + wm * WM + i * 32 + 8 * (r / 4) + 4 * lk + (r % 4);
                int64_t col = n0 + wn * WN + j * 32 + lr;
                if (row < p.M && col < p.N) {
                    float v = acc[i][j][r] * sab;
                    if (kOutBF16) {
                        uint32_t u = __float_as_uint(v);
                        u += 0x7FFFu + ((u >> 16) & 1u);
                        reinterpret_cast<uint16_t*>(p.c)[row * p.ldc + col] = (uint16_t)(u >> 16);
                    } else {
                        reinterpret_cast<float*>(p.c)[row * p.ldc + col] = v;
                    }
                }
            }
}

__global__ void k_fill_zero(uint8_t* c, int64_t M, int64_t N, int64_t ldc, int esz)
{
    int64_t total = M * N;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total;
         i += (int64_t)gridDim.x * blockDim.x) {
        int64_t r = i / N, col = i % N;
        uint8_t* dst = c + (r * ldc + col) * esz;
        if (esz == 2) *reinterpret_cast<uint16_t*>(dst) = 0;
        else *reinterpret_cast<float*>(dst) = 0.0f;
    }
}

hipError_t launch_fill_zero(void* c, bool bf16, int64_t M, int64_t N, int64_t ldc, hipStream_t s)
{
    int64_t total = M * N;
    int grid = (int)((total + 255) / 256);
    if (grid > 8192) grid = 8192;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL(k_fill_zero, dim3(grid), dim3(256), 0, s, static_cast<uint8_t*>(c), M, N,
                       ldc, bf16 ? 2 : 4);
    return hipGetLastError();
}

#define NVFP4_BOOL(cond, NAME, ...) \
    do {                            \
        if (cond) {                 \
            constexpr bool NAME = true; \
            __VA_ARGS__;            \
        } else {                    \
            constexpr bool NAME = false; \
            __VA_ARGS__;            \
        }                           \
    } while (0)

hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, const GemmOperand& A,
                       const GemmOperand& B, bool out_bf16, void* c, int64_t ldc, hipStream_t s)
{
    GemmParams p;
    p.M = M; p.N = N; p.K = K;
    p.a_codes = A.codes; p.a_scales = A.scales; p.a_ts = A.ts;
    p.b_codes = B.codes; p.b_scales = B.scales; p.b_ts = B.ts;
    p.c = static_cast<uint8_t*>(c);
    p.ldc = ldc;
    constexpr int BM = 128, BN = 128, BK = 64;
    dim3 grid((unsigned)((N + BN - 1) / BN), (unsigned)((M + BM - 1) / BM));
    NVFP4_BOOL(A.k_major, AK, NVFP4_BOOL(B.k_major, BKM, NVFP4_BOOL(A.block2d != 0, A2,
        NVFP4_BOOL(B.block2d != 0, B2, NVFP4_BOOL(out_bf16, OB,
            hipLaunchKernelGGL((k_gemm_simple<BM, BN, BK, AK, BKM, A2, B2, OB>), grid, dim3(256),
                               0, s, p))))));
    return hipGetLastError();
}

}  // namespace nvfp4
