// Definitions shared by the GEMM kernels (gemm.hip: 256 x 256 tiles and the
// MXFP4 GEMM; gemm_decode.hip: the decode-shape kernels).
#pragma once

#include "device_common.h"

namespace nvfp4 {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

struct GemmParams {
    int64_t M, N, K;
    int64_t kp;   // K-major operands: K extent of a row of the planes (>= K; > K for a K slice)
    const uint8_t* a_codes;
    const uint8_t* a_scales;
    const uint8_t* b_codes;
    const uint8_t* b_scales;
    const float* a_ts;
    const float* b_ts;
    uint8_t* c;
    int64_t ldc;
    bool a2d, b2d, out_bf16;
    bool vec_out;  // C rows allow 8-byte (BF16) / 16-byte (FP32) stores
    const uint16_t* a_bf16;  // weight-only GEMM: BF16 activations [M, K], row pitch lda
    int64_t lda;
    bool vec16;    // C base and row pitch are 16-byte aligned (whole-line epilogue)
    // SwiGLU epilogue (k_gemm_kk<true>): act [M, N/2] BF16, row pitch ld_act;
    // H itself (through c) only when store_h; two amax partials per workgroup
    uint8_t* act;
    int64_t ld_act;
    uint32_t rht_mask;
    float* partials;   // [grid] max|act|, then [grid] max|RHT16 of act down columns|
    bool store_h, act_vec16;
    // K-split of the last round of tiles (k_gemm_kk<.., true>): workgroup b
    // takes K half b % 2 of tile tile_base + b / 2 (K = the half's length,
    // kp the whole K) and writes the FP32 partial to c (half 0) or c2 (half 1)
    uint32_t tile_base;
    uint8_t* c2;
    // k_gemm_kk and k_gemm_mx: when gate is set, the kernel runs only if
    // *gate == gate_want (device-side choice between two launched paths)
    const int32_t* gate;
    int32_t gate_want;
};

// LDS pointer type of the buffer-load-to-LDS builtin
typedef __attribute__((address_space(3))) void lds_void_t;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8)
#define NVFP4_WAIT_VMCNT(n) \
    __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | 0x70 | 0xF00)
// ... and with only the LDS / scalar-memory counter drained (vmcnt left at its
// maximum 63)
#define NVFP4_WAIT_LGKMCNT0() __builtin_amdgcn_s_waitcnt(0xC07F)

// 8 FP16 operand values from 8 codes (one 32-bit word) and the block scale.
__device__ __forceinline__ half8_t dequant_word(uint32_t w, _Float16 e)
{
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

// Eight E2M1 codes times the block scale e as BF16, for the weight-only
// (BF16-activation) GEMM.  val * e needs at most 6 significant bits, so it
// is exact in FP32 and its low 16 bits are zero: the BF16 value is the upper
// half, taken with one v_perm per pair.
__device__ __forceinline__ bf16x8_t dequant_word_bf16(uint32_t w, float e)
{
    u32x4 r;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        float2_t v = q == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0)
                   : q == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1)
                   : q == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2)
                            : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
        r[q] = __builtin_amdgcn_perm(__float_as_uint(v[1] * e), __float_as_uint(v[0] * e),
                                     0x07060302u);
    }
    return __builtin_bit_cast(bf16x8_t, r);
}

// Decode-shape GEMMs (gemm_decode.hip).  gemm_decode_shape: M <= 64, K a
// multiple of 512 and the weight code plane below 2 GiB (32-bit buffer
// offsets); launch_gemm_decode then runs C = s_A s_B A B^T (NT, both K-major,
// kp == K) on the weight-streaming kernels.
bool gemm_decode_shape(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_decode(const GemmParams& p, hipStream_t s);

}  // namespace nvfp4
