// Internal launchers behind the C ABI (include/nvfp4.h).  Arguments have
// already been validated by api.cpp; every launcher enqueues on `stream` and
// returns the hipError_t of the last launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace nvfp4 {

struct QuantArgs {
    const void* x;
    bool bf16;
    int64_t rows, cols, ld;
    int block2d;     // 0: 1x16, 1: 16x16
    int axis;        // 1D only: 1 along columns, 0 along rows
    bool sr;
    uint64_t seed;
    uint32_t stream_id;
    bool rht;
    uint32_t mask;
    uint8_t* codes;
    uint8_t* scales;
    float* tensor_scale;
    float* amax_out;
};

// Number of per-workgroup partial maxima the amax pass writes (<= this).
constexpr int kMaxAmaxPartials = 2048;

// Pass 1: partial maxima of |x| (after the RHT when enabled) into partials[],
// then reduce them into *amax_dst (and *amax_out when non-null).
hipError_t launch_amax(const QuantArgs& a, float* partials, float* amax_dst, hipStream_t s);

// max |x| and max |RHT16 down the columns of x| in one pass (rows % 16 == 0):
// partials[] needs 2 * kMaxAmaxPartials floats.
hipError_t launch_amax_dual(const QuantArgs& a, float* partials, float* amax_dst,
                            float* amax_rht_dst, hipStream_t s);

// act = BF16(BF16(silu(gate)) * up) over h = [gate | up] (BF16 [rows, 2F]),
// plus max |act| and max |RHT16 down the columns of act| (rows % 16 == 0,
// F % 16 == 0); partials[] needs 2 * kMaxAmaxPartials floats.
hipError_t launch_swiglu_amax(const void* h, int64_t rows, int64_t F, int64_t ld_h, void* act,
                              int64_t ld_a, uint32_t mask, float* partials, float* amax,
                              float* amax_rht, hipStream_t s);

// Pass 2: quantize using the amax at *amax_src; writes codes, scales,
// tensor_scale (and amax_out when amax_src is the caller's amax_in).
hipError_t launch_quantize(const QuantArgs& a, const float* amax_src, bool write_amax_out,
                           hipStream_t s);

// Pass 2 for blocks down the columns (1D axis 0 or 2D), written transposed:
// codes [cols, rows/2], scales [cols, rows/16] (1D) / [cols/16, rows/16] (2D).
hipError_t launch_quantize_transposed(const QuantArgs& a, const float* amax_src,
                                      bool write_amax_out, hipStream_t s);

// The NVFP4 tensor [rows, cols] stored as its transpose: codes_t
// [cols, rows/2], scales_t = the input scale plane transposed byte for byte
// (rows % 16 == 0, cols % 16 == 0).
hipError_t launch_transpose(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                            int64_t cols, int block2d, int axis, uint8_t* codes_t,
                            uint8_t* scales_t, hipStream_t s);

// Empty tensor: s_g = 0 and amax = 0.
hipError_t launch_write_zero_scale(float* tensor_scale, float* amax_out, hipStream_t s);

hipError_t launch_rht16(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld_x,
                        int axis, uint32_t mask, float* y, int64_t ld_y, hipStream_t s);

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, const float* ts,
                             int64_t rows, int64_t cols, int block2d, int axis, bool out_bf16,
                             void* out, int64_t ld_out, hipStream_t s);

struct GemmOperand {
    const uint8_t* codes;
    const uint8_t* scales;
    const float* ts;
    int block2d;
    bool k_major;  // true: codes packed along K (storage [MN, K]); false: storage [K, MN]
};

// Longest K one chain of FP32 MFMA accumulations covers.  The matrix unit's
// FP32 accumulation is not round-to-nearest (measured on the MI355X: about a
// quarter of results differ from the correctly rounded sum, with a mean bias
// of -0.02 to -0.2 ulp per instruction), so an all-positive dot product's
// error grows with the chain length: 2e-5 of sum |a*b| at K = 106496, within
// 1e-5 up to 32768.  A longer K is cut into slices of at most this length,
// each accumulated separately and summed in FP32 with IEEE additions.
constexpr int64_t kMaxChainK = 32768;

// Number of K slices of a K-long GEMM and the slice length (a multiple of
// 512; the last slice may be shorter).  1 slice when K <= kMaxChainK.
int gemm_k_slices(int64_t K, int64_t* slice_k);

// Workspace bytes for splitting the last, at most half-full round of output
// tiles along K (both operands K-major); 0 when no split applies on the
// current device.
size_t gemm_split_bytes(bool both_kmajor, int64_t M, int64_t N, int64_t K);

// C = A B^T etc. (layouts by GemmOperand::k_major).  When K > kMaxChainK, ws
// holds gemm_k_slices(K) FP32 planes of M x N (16-byte aligned).  Otherwise
// ws, when not null, holds gemm_split_bytes(...) bytes and the last round's
// tiles are split along K (nullptr: no split).
hipError_t launch_gemm(int64_t M, int64_t N, int64_t K, const GemmOperand& A,
                       const GemmOperand& B, bool out_bf16, void* c, int64_t ldc, float* ws,
                       hipStream_t s);

// NVFP4 GEMM (NT, both K-major, K % 128 == 0, K <= kMaxChainK) on the native
// scaled FP4 MFMA when every 32-K block of both operands maps onto one
// power-of-two scale exactly, else on the FP16 path; *gate (device) ends as 1
// or 0 for the path taken.  ws: gemm_native_bytes(M, N, K) bytes of E8M0
// planes (16-byte aligned).
size_t gemm_native_bytes(int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm_native(int64_t M, int64_t N, int64_t K, const GemmOperand& A,
                              const GemmOperand& B, bool out_bf16, void* c, int64_t ldc,
                              int32_t* gate, uint8_t* ws, hipStream_t s);

// MXFP4 (E2M1 elements, E8M0 scale per 32 along the row): codes
// [rows, cols/2], scales [rows, cols/32]; cols % 32 == 0.
hipError_t launch_mx_quantize(const void* x, bool bf16, int64_t rows, int64_t cols, int64_t ld,
                              uint8_t* codes, uint8_t* scales, hipStream_t s);
hipError_t launch_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                int64_t cols, bool out_bf16, void* out, int64_t ld_out,
                                hipStream_t s);
// MXFP4 GEMM, NT: C[M, N] = A[M, K] B[N, K]^T, both K-major MXFP4, K % 128 == 0.
hipError_t launch_mx_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                          const uint8_t* a_scales, const uint8_t* b_codes, const uint8_t* b_scales,
                          bool out_bf16, void* c, int64_t ldc, hipStream_t s);

// Weight-only GEMM for decode shapes, NT: C[M, N] = A[M, K] B[N, K]^T with
// BF16 activations (row pitch lda) and an NVFP4 weight; M <= 64, K % 512 == 0.
hipError_t launch_gemm_w4a16(int64_t M, int64_t N, int64_t K, const uint16_t* a, int64_t lda,
                             const GemmOperand& B, bool out_bf16, void* c, int64_t ldc,
                             hipStream_t s);

// NVFP4 KV cache: token rows of x [tokens, cols] (cols % 16 == 0) quantized
// (1x16, RNE, s_g = RN(*amax / 2688)) into cache rows slots[t] of codes
// [num_slots, cols/2] and scales [num_slots, cols/16]; the read gathers cache
// rows slots[j] into out [n, cols] (pitch ld_out).  Slots outside
// [0, num_slots) are skipped / read as zeros.
hipError_t launch_kv_cache_write(const void* x, bool bf16, int64_t tokens, int64_t cols,
                                 int64_t ld, const int64_t* slots, int64_t num_slots,
                                 const float* amax, uint8_t* codes, uint8_t* scales,
                                 hipStream_t s);
hipError_t launch_kv_cache_read(const uint8_t* codes, const uint8_t* scales, const float* amax,
                                int64_t num_slots, int64_t cols, const int64_t* slots, int64_t n,
                                bool out_bf16, void* out, int64_t ld_out, hipStream_t s);

// max over partials[0 .. n) into *amax (one workgroup).
hipError_t launch_amax_finalize(const float* partials, int n, float* amax, hipStream_t s);

// GEMM 1 of the MLP with the SwiGLU epilogue (NT, both K-major): B's rows are
// gate/up interleaved in blocks of 64; N % 128 == 0, M % 16 == 0, K % 128 == 0.
// act [M, N/2] BF16 (pitch ld_act), H [M, N] BF16 only when h is non-null;
// partials needs 2 floats per 256 x 256 output tile.
hipError_t launch_gemm_swiglu(int64_t M, int64_t N, int64_t K, const GemmOperand& A,
                              const GemmOperand& B, void* h, int64_t ldh, void* act,
                              int64_t ld_act, uint32_t mask, float* partials, float* amax,
                              float* amax_rht, hipStream_t s);

hipError_t launch_fill_zero(void* c, bool bf16, int64_t M, int64_t N, int64_t ldc, hipStream_t s);

}  // namespace nvfp4
