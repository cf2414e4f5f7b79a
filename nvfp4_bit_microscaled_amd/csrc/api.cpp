// C ABI of the NVFP4 library (declared in include/nvfp4.h): argument
// validation and dispatch to the HIP launchers.  Every check happens before
// anything is enqueued, so a call that returns an error has written nothing.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "launch.h"
#include "nvfp4.h"

using namespace nvfp4;

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool debug_mode()
{
    const char* v = std::getenv("NVFP4_DEBUG");
    return v && v[0] == '1';
}

nvfp4_status from_hip(hipError_t e) { return e == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP; }

constexpr uint64_t kMaxItems = 0xFFFFFFFFull;  // kernels index work items in 32 bits

// Workspace layout: [0, kMaxAmaxPartials) partial maxima, then the amax slot.
constexpr size_t kWorkspaceFloats = kMaxAmaxPartials + 64;

}  // namespace

// Scratch of nvfp4_quantize_noalloc: the amax pass's per-workgroup partial
// maxima and the reduced amax, laid out as nvfp4_quantize's workspace
// (8448 bytes).  Each GPU the library runs on holds its own copy until the
// process ends.  Host code never uses this name as an address: the device
// address comes from hipGetSymbolAddress, once per device.
static __device__ __align__(256) float scratch[kWorkspaceFloats];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call made with that device current, then kept).
nvfp4_status scratch_of_current_device(float** out)
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return NVFP4_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return NVFP4_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return NVFP4_ERR_HIP;
        g_scratch_ptr[dev] = static_cast<float*>(p);
    }
    *out = g_scratch_ptr[dev];
    return NVFP4_OK;
}

}  // namespace

extern "C" {

int nvfp4_version(void) { return 200; }

const char* nvfp4_status_string(nvfp4_status s)
{
    switch (s) {
    case NVFP4_OK: return "NVFP4_OK";
    case NVFP4_ERR_INVALID_ARG: return "NVFP4_ERR_INVALID_ARG";
    case NVFP4_ERR_SHAPE: return "NVFP4_ERR_SHAPE";
    case NVFP4_ERR_ALIGN: return "NVFP4_ERR_ALIGN";
    case NVFP4_ERR_LAYOUT: return "NVFP4_ERR_LAYOUT";
    case NVFP4_ERR_UNSUPPORTED: return "NVFP4_ERR_UNSUPPORTED";
    case NVFP4_ERR_WORKSPACE: return "NVFP4_ERR_WORKSPACE";
    case NVFP4_ERR_HIP: return "NVFP4_ERR_HIP";
    case NVFP4_ERR_NONFINITE: return "NVFP4_ERR_NONFINITE";
    }
    return "NVFP4_ERR_UNKNOWN";
}

size_t nvfp4_quantize_workspace_size(int64_t rows, int64_t cols)
{
    (void)rows;
    (void)cols;
    return kWorkspaceFloats * sizeof(float);
}

nvfp4_status nvfp4_quantize(const void* x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols,
                            int64_t ld_x, nvfp4_block block, int axis, int transpose_out,
                            nvfp4_round rounding,
                            uint64_t seed, uint32_t stream_id, int rht, uint32_t rht_sign_mask,
                            const float* amax_in, float* amax_out, uint8_t* codes,
                            uint8_t* scales, float* tensor_scale, void* workspace,
                            size_t workspace_bytes, void* stream)
{
    if (x_dtype != NVFP4_DTYPE_BF16 && x_dtype != NVFP4_DTYPE_FP32) return NVFP4_ERR_INVALID_ARG;
    if (block != NVFP4_BLOCK_1D && block != NVFP4_BLOCK_2D) return NVFP4_ERR_INVALID_ARG;
    if (rounding != NVFP4_ROUND_RNE && rounding != NVFP4_ROUND_SR) return NVFP4_ERR_INVALID_ARG;
    if (block == NVFP4_BLOCK_1D && axis != 0 && axis != 1) return NVFP4_ERR_INVALID_ARG;
    if (rht != 0 && rht != 1) return NVFP4_ERR_INVALID_ARG;
    if (transpose_out != 0 && transpose_out != 1) return NVFP4_ERR_INVALID_ARG;
    if (rows < 0 || cols < 0) return NVFP4_ERR_INVALID_ARG;
    if (!tensor_scale) return NVFP4_ERR_INVALID_ARG;
    if (rht && block == NVFP4_BLOCK_2D) return NVFP4_ERR_UNSUPPORTED;
    if (transpose_out && block == NVFP4_BLOCK_1D && axis == 1) return NVFP4_ERR_UNSUPPORTED;
    if (cols % 16) return NVFP4_ERR_SHAPE;
    bool along_rows = (block == NVFP4_BLOCK_2D) || axis == 0;
    if (along_rows && rows % 16) return NVFP4_ERR_SHAPE;
    if (ld_x < cols) return NVFP4_ERR_SHAPE;
    if ((uint64_t)rows * (uint64_t)(cols / 8) > kMaxItems) return NVFP4_ERR_UNSUPPORTED;
    size_t esz = x_dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (rows == 0 || cols == 0) return from_hip(launch_write_zero_scale(tensor_scale, amax_out, s));
    if (!x || !codes || !scales) return NVFP4_ERR_INVALID_ARG;
    if (!aligned16(x) || ((size_t)ld_x * esz) % 16) return NVFP4_ERR_ALIGN;
    if (!aligned16(codes) || !aligned16(scales)) return NVFP4_ERR_ALIGN;
    if (!amax_in) {
        if (!workspace || workspace_bytes < nvfp4_quantize_workspace_size(rows, cols))
            return NVFP4_ERR_WORKSPACE;
        if ((reinterpret_cast<uintptr_t>(workspace) & 3u) != 0) return NVFP4_ERR_ALIGN;
    }

    QuantArgs a;
    a.x = x;
    a.bf16 = x_dtype == NVFP4_DTYPE_BF16;
    a.rows = rows;
    a.cols = cols;
    a.ld = ld_x;
    a.block2d = block == NVFP4_BLOCK_2D;
    a.axis = axis;
    a.sr = rounding == NVFP4_ROUND_SR;
    a.seed = seed;
    a.stream_id = stream_id;
    a.rht = rht != 0;
    a.mask = rht_sign_mask & 0xFFFFu;
    a.codes = codes;
    a.scales = scales;
    a.tensor_scale = tensor_scale;
    a.amax_out = amax_out;

    const float* amax_src = amax_in;
    if (!amax_in) {
        float* ws = static_cast<float*>(workspace);
        float* amax_slot = ws + kMaxAmaxPartials;
        hipError_t e = launch_amax(a, ws, amax_slot, s);
        if (e != hipSuccess) return NVFP4_ERR_HIP;
        amax_src = amax_slot;
    }
    if (debug_mode()) {
        float h = 0.0f;
        if (hipMemcpyAsync(&h, amax_src, sizeof(float), hipMemcpyDeviceToHost, s) != hipSuccess)
            return NVFP4_ERR_HIP;
        if (hipStreamSynchronize(s) != hipSuccess) return NVFP4_ERR_HIP;
        if (!std::isfinite(h)) return NVFP4_ERR_NONFINITE;
    }
    if (transpose_out)
        return from_hip(launch_quantize_transposed(a, amax_src, amax_in != nullptr, s));
    return from_hip(launch_quantize(a, amax_src, amax_in != nullptr, s));
}

nvfp4_status nvfp4_quantize_noalloc(const void* x, nvfp4_dtype x_dtype, int64_t rows,
                                    int64_t cols, int64_t ld_x, nvfp4_block block, int axis,
                                    int transpose_out, nvfp4_round rounding, uint64_t seed,
                                    uint32_t stream_id, int rht, uint32_t rht_sign_mask,
                                    const float* amax_in, float* amax_out, uint8_t* codes,
                                    uint8_t* scales, float* tensor_scale, void* stream)
{
    float* ws = nullptr;
    size_t ws_bytes = 0;
    // the scratch is needed only for the amax pass of a non-empty tensor;
    // nvfp4_quantize validates everything else before anything is enqueued
    if (!amax_in && rows > 0 && cols > 0) {
        if (nvfp4_quantize_workspace_size(rows, cols) > sizeof(scratch))
            return NVFP4_ERR_WORKSPACE;
        const nvfp4_status st = scratch_of_current_device(&ws);
        if (st != NVFP4_OK) return st;
        ws_bytes = sizeof(scratch);
    }
    return nvfp4_quantize(x, x_dtype, rows, cols, ld_x, block, axis, transpose_out, rounding,
                          seed, stream_id, rht, rht_sign_mask, amax_in, amax_out, codes, scales,
                          tensor_scale, ws, ws_bytes, stream);
}

nvfp4_status nvfp4_transpose(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                             int64_t cols, nvfp4_block block, int axis, uint8_t* codes_t,
                             uint8_t* scales_t, void* stream)
{
    if (block != NVFP4_BLOCK_1D && block != NVFP4_BLOCK_2D) return NVFP4_ERR_INVALID_ARG;
    if (block == NVFP4_BLOCK_1D && axis != 0 && axis != 1) return NVFP4_ERR_INVALID_ARG;
    if (rows < 0 || cols < 0) return NVFP4_ERR_INVALID_ARG;
    if (rows % 16 || cols % 16) return NVFP4_ERR_SHAPE;
    if ((uint64_t)rows * (uint64_t)(cols / 8) > kMaxItems) return NVFP4_ERR_UNSUPPORTED;
    if (rows == 0 || cols == 0) return NVFP4_OK;
    if (!codes || !scales || !codes_t || !scales_t) return NVFP4_ERR_INVALID_ARG;
    if (!aligned16(codes) || !aligned16(codes_t)) return NVFP4_ERR_ALIGN;
    return from_hip(launch_transpose(codes, scales, rows, cols, block == NVFP4_BLOCK_2D, axis,
                                     codes_t, scales_t, static_cast<hipStream_t>(stream)));
}

size_t nvfp4_amax_workspace_size(int64_t rows, int64_t cols)
{
    (void)rows;
    (void)cols;
    return 2 * kMaxAmaxPartials * sizeof(float);
}

nvfp4_status nvfp4_amax(const void* x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols,
                        int64_t ld_x, uint32_t rht_sign_mask, float* amax, float* amax_rht,
                        void* workspace, size_t workspace_bytes, void* stream)
{
    if (x_dtype != NVFP4_DTYPE_BF16 && x_dtype != NVFP4_DTYPE_FP32) return NVFP4_ERR_INVALID_ARG;
    if (rows < 0 || cols < 0 || !amax) return NVFP4_ERR_INVALID_ARG;
    if (cols % 16) return NVFP4_ERR_SHAPE;
    if (amax_rht && rows % 16) return NVFP4_ERR_SHAPE;
    if (ld_x < cols) return NVFP4_ERR_SHAPE;
    if ((uint64_t)rows * (uint64_t)(cols / 8) > kMaxItems) return NVFP4_ERR_UNSUPPORTED;
    size_t esz = x_dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // an empty tensor: both maxima are 0 (the zero-scale writer stores 0 to
    // its two outputs)
    if (rows == 0 || cols == 0) return from_hip(launch_write_zero_scale(amax, amax_rht, s));
    if (!x) return NVFP4_ERR_INVALID_ARG;
    if (!aligned16(x) || ((size_t)ld_x * esz) % 16) return NVFP4_ERR_ALIGN;
    if (!workspace || workspace_bytes < nvfp4_amax_workspace_size(rows, cols))
        return NVFP4_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 3u) != 0) return NVFP4_ERR_ALIGN;
    QuantArgs a{};
    a.x = x;
    a.bf16 = x_dtype == NVFP4_DTYPE_BF16;
    a.rows = rows;
    a.cols = cols;
    a.ld = ld_x;
    a.axis = 0;
    a.rht = amax_rht != nullptr;
    a.mask = rht_sign_mask & 0xFFFFu;
    float* ws = static_cast<float*>(workspace);
    if (!amax_rht) return from_hip(launch_amax(a, ws, amax, s));
    return from_hip(launch_amax_dual(a, ws, amax, amax_rht, s));
}

nvfp4_status nvfp4_swiglu_amax(const void* h, int64_t rows, int64_t F, int64_t ld_h, void* act,
                               int64_t ld_act, uint32_t rht_sign_mask, float* amax,
                               float* amax_rht, void* workspace, size_t workspace_bytes,
                               void* stream)
{
    if (rows < 0 || F < 0 || !amax || !amax_rht) return NVFP4_ERR_INVALID_ARG;
    if (rows % 16 || F % 16) return NVFP4_ERR_SHAPE;
    if (ld_h < 2 * F || ld_act < F) return NVFP4_ERR_SHAPE;
    if ((uint64_t)rows * (uint64_t)(F / 4) > kMaxItems) return NVFP4_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (rows == 0 || F == 0) return from_hip(launch_write_zero_scale(amax, amax_rht, s));
    if (!h || !act) return NVFP4_ERR_INVALID_ARG;
    if (!aligned16(h) || ((size_t)ld_h * 2) % 16) return NVFP4_ERR_ALIGN;
    if (!aligned16(act) || ((size_t)ld_act * 2) % 16) return NVFP4_ERR_ALIGN;
    if (!workspace || workspace_bytes < nvfp4_amax_workspace_size(rows, F))
        return NVFP4_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 3u) != 0) return NVFP4_ERR_ALIGN;
    return from_hip(launch_swiglu_amax(h, rows, F, ld_h, act, ld_act, rht_sign_mask,
                                       static_cast<float*>(workspace), amax, amax_rht, s));
}

nvfp4_status nvfp4_rht16(const void* x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols,
                         int64_t ld_x, int axis, uint32_t sign_mask, float* y, int64_t ld_y,
                         void* stream)
{
    if (x_dtype != NVFP4_DTYPE_BF16 && x_dtype != NVFP4_DTYPE_FP32) return NVFP4_ERR_INVALID_ARG;
    if (axis != 0 && axis != 1) return NVFP4_ERR_INVALID_ARG;
    if (rows < 0 || cols < 0) return NVFP4_ERR_INVALID_ARG;
    if (axis == 1 && cols % 16) return NVFP4_ERR_SHAPE;
    if (axis == 0 && (rows % 16 || cols % 8)) return NVFP4_ERR_SHAPE;
    if (ld_x < cols || ld_y < cols) return NVFP4_ERR_SHAPE;
    if ((uint64_t)rows * (uint64_t)(cols / 8) > kMaxItems) return NVFP4_ERR_UNSUPPORTED;
    if (rows == 0 || cols == 0) return NVFP4_OK;
    if (!x || !y) return NVFP4_ERR_INVALID_ARG;
    size_t esz = x_dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
    if (!aligned16(x) || ((size_t)ld_x * esz) % 16) return NVFP4_ERR_ALIGN;
    if (!aligned16(y) || ((size_t)ld_y * 4) % 16) return NVFP4_ERR_ALIGN;
    return from_hip(launch_rht16(x, x_dtype == NVFP4_DTYPE_BF16, rows, cols, ld_x, axis,
                                 sign_mask & 0xFFFFu, y, ld_y, static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales,
                              const float* tensor_scale, int64_t rows, int64_t cols,
                              nvfp4_block block, int axis, nvfp4_dtype out_dtype, void* out,
                              int64_t ld_out, void* stream)
{
    if (out_dtype != NVFP4_DTYPE_BF16 && out_dtype != NVFP4_DTYPE_FP32) return NVFP4_ERR_INVALID_ARG;
    if (block != NVFP4_BLOCK_1D && block != NVFP4_BLOCK_2D) return NVFP4_ERR_INVALID_ARG;
    if (block == NVFP4_BLOCK_1D && axis != 0 && axis != 1) return NVFP4_ERR_INVALID_ARG;
    if (rows < 0 || cols < 0) return NVFP4_ERR_INVALID_ARG;
    if (cols % 16) return NVFP4_ERR_SHAPE;
    bool along_rows = (block == NVFP4_BLOCK_2D) || axis == 0;
    if (along_rows && rows % 16) return NVFP4_ERR_SHAPE;
    if (ld_out < cols) return NVFP4_ERR_SHAPE;
    if ((uint64_t)rows * (uint64_t)(cols / 8) > kMaxItems) return NVFP4_ERR_UNSUPPORTED;
    if (rows == 0 || cols == 0) return NVFP4_OK;
    if (!codes || !scales || !tensor_scale || !out) return NVFP4_ERR_INVALID_ARG;
    size_t esz = out_dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
    if (!aligned16(codes) || !aligned16(scales) || !aligned16(out) ||
        ((size_t)ld_out * esz) % 16)
        return NVFP4_ERR_ALIGN;
    return from_hip(launch_dequantize(codes, scales, tensor_scale, rows, cols,
                                      block == NVFP4_BLOCK_2D, axis,
                                      out_dtype == NVFP4_DTYPE_BF16, out, ld_out,
                                      static_cast<hipStream_t>(stream)));
}

size_t nvfp4_gemm_workspace_size(nvfp4_layout layout, int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0 || K <= 0) return 0;
    int64_t ks;
    const int nsl = gemm_k_slices(K, &ks);
    if (nsl > 1) return (size_t)nsl * (size_t)M * (size_t)N * sizeof(float);
    return gemm_split_bytes(layout == NVFP4_LAYOUT_NT, M, N, K);
}

nvfp4_status nvfp4_gemm(nvfp4_layout layout, int64_t M, int64_t N, int64_t K,
                        const uint8_t* a_codes, const uint8_t* a_scales,
                        const float* a_tensor_scale, nvfp4_block a_block,
                        const uint8_t* b_codes, const uint8_t* b_scales,
                        const float* b_tensor_scale, nvfp4_block b_block, nvfp4_dtype out_dtype,
                        void* c, int64_t ldc, void* workspace, size_t workspace_bytes,
                        void* stream)
{
    if (layout != NVFP4_LAYOUT_NT && layout != NVFP4_LAYOUT_NN && layout != NVFP4_LAYOUT_TN)
        return NVFP4_ERR_INVALID_ARG;
    if (a_block != NVFP4_BLOCK_1D && a_block != NVFP4_BLOCK_2D) return NVFP4_ERR_INVALID_ARG;
    if (b_block != NVFP4_BLOCK_1D && b_block != NVFP4_BLOCK_2D) return NVFP4_ERR_INVALID_ARG;
    if (out_dtype != NVFP4_DTYPE_BF16 && out_dtype != NVFP4_DTYPE_FP32) return NVFP4_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K < 0) return NVFP4_ERR_INVALID_ARG;
    if (ldc < N) return NVFP4_ERR_SHAPE;
    if (K % 16) return NVFP4_ERR_SHAPE;
    const bool a_kmajor = layout != NVFP4_LAYOUT_TN;  // A stored [M, K] unless TN
    const bool b_kmajor = layout == NVFP4_LAYOUT_NT;  // B stored [N, K] only for NT
    // dims along which codes are packed but which are not K
    if (!a_kmajor && M % 16) return NVFP4_ERR_SHAPE;
    if (!b_kmajor && N % 16) return NVFP4_ERR_SHAPE;
    // 2D operands need both dims divisible by 16
    if (a_block == NVFP4_BLOCK_2D && M % 16) return NVFP4_ERR_LAYOUT;
    if (b_block == NVFP4_BLOCK_2D && N % 16) return NVFP4_ERR_LAYOUT;
    if (M == 0 || N == 0) return NVFP4_OK;
    if (!c) return NVFP4_ERR_INVALID_ARG;
    size_t esz = out_dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
    if ((reinterpret_cast<uintptr_t>(c) & (esz - 1)) != 0) return NVFP4_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (K == 0) return from_hip(launch_fill_zero(c, out_dtype == NVFP4_DTYPE_BF16, M, N, ldc, s));
    if (!a_codes || !a_scales || !a_tensor_scale || !b_codes || !b_scales || !b_tensor_scale)
        return NVFP4_ERR_INVALID_ARG;
    if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(b_codes) || !aligned16(b_scales))
        return NVFP4_ERR_ALIGN;
    // K slices (K > 32768) need the workspace; the last-round K split only
    // runs when the caller supplied enough of it
    int64_t ks;
    const bool sliced = gemm_k_slices(K, &ks) > 1;
    const size_t need = nvfp4_gemm_workspace_size(layout, M, N, K);
    float* ws = nullptr;
    if (need > 0 && workspace && workspace_bytes >= need) {
        if (!aligned16(workspace)) return NVFP4_ERR_ALIGN;
        ws = static_cast<float*>(workspace);
    } else if (sliced) {
        return NVFP4_ERR_WORKSPACE;
    }
    GemmOperand A{a_codes, a_scales, a_tensor_scale, a_block == NVFP4_BLOCK_2D, a_kmajor};
    GemmOperand B{b_codes, b_scales, b_tensor_scale, b_block == NVFP4_BLOCK_2D, b_kmajor};
    return from_hip(launch_gemm(M, N, K, A, B, out_dtype == NVFP4_DTYPE_BF16, c, ldc, ws, s));
}

nvfp4_status nvfp4_mx_quantize(const void* x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols,
                               int64_t ld_x, uint8_t* codes, uint8_t* scales, void* stream)
{
    if (x_dtype != NVFP4_DTYPE_BF16 && x_dtype != NVFP4_DTYPE_FP32) return NVFP4_ERR_INVALID_ARG;
    if (rows < 0 || cols < 0) return NVFP4_ERR_INVALID_ARG;
    if (cols % 32) return NVFP4_ERR_SHAPE;
    if (ld_x < cols) return NVFP4_ERR_SHAPE;
    if ((uint64_t)rows * (uint64_t)(cols / 32) > kMaxItems) return NVFP4_ERR_UNSUPPORTED;
    if (rows == 0 || cols == 0) return NVFP4_OK;
    if (!x || !codes || !scales) return NVFP4_ERR_INVALID_ARG;
    const size_t esz = x_dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
    if (!aligned16(x) || !aligned16(codes) || ((size_t)ld_x * esz) % 16) return NVFP4_ERR_ALIGN;
    return from_hip(launch_mx_quantize(x, x_dtype == NVFP4_DTYPE_BF16, rows, cols, ld_x, codes,
                                       scales, static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                 int64_t cols, nvfp4_dtype out_dtype, void* out, int64_t ld_out,
                                 void* stream)
{
    if (out_dtype != NVFP4_DTYPE_BF16 && out_dtype != NVFP4_DTYPE_FP32) return NVFP4_ERR_INVALID_ARG;
    if (rows < 0 || cols < 0) return NVFP4_ERR_INVALID_ARG;
    if (cols % 32) return NVFP4_ERR_SHAPE;
    if (ld_out < cols) return NVFP4_ERR_SHAPE;
    if ((uint64_t)rows * (uint64_t)(cols / 8) > kMaxItems) return NVFP4_ERR_UNSUPPORTED;
    if (rows == 0 || cols == 0) return NVFP4_OK;
    if (!codes || !scales || !out) return NVFP4_ERR_INVALID_ARG;
    const size_t esz = out_dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
    if (!aligned16(codes) || !aligned16(out) || ((size_t)ld_out * esz) % 16) return NVFP4_ERR_ALIGN;
    return from_hip(launch_mx_dequantize(codes, scales, rows, cols,
                                         out_dtype == NVFP4_DTYPE_BF16, out, ld_out,
                                         static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_mx_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                           const uint8_t* a_scales, const uint8_t* b_codes,
                           const uint8_t* b_scales, nvfp4_dtype out_dtype, void* c, int64_t ldc,
                           void* stream)
{
    if (out_dtype != NVFP4_DTYPE_BF16 && out_dtype != NVFP4_DTYPE_FP32) return NVFP4_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K < 0) return NVFP4_ERR_INVALID_ARG;
    if (ldc < N) return NVFP4_ERR_SHAPE;
    if (K % 128) return NVFP4_ERR_SHAPE;
    // buffer records of a 256-row tile (and the C offsets) in 32 bits; one
    // FP32 accumulation chain over K
    if ((uint64_t)K / 2 * 256 >= (1ull << 31)) return NVFP4_ERR_UNSUPPORTED;
    if (K > kMaxChainK) return NVFP4_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return NVFP4_OK;
    if (!c) return NVFP4_ERR_INVALID_ARG;
    const size_t esz = out_dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
    if ((reinterpret_cast<uintptr_t>(c) & (esz - 1)) != 0) return NVFP4_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (K == 0) return from_hip(launch_fill_zero(c, out_dtype == NVFP4_DTYPE_BF16, M, N, ldc, s));
    if (!a_codes || !a_scales || !b_codes || !b_scales) return NVFP4_ERR_INVALID_ARG;
    if (!aligned16(a_codes) || !aligned16(b_codes) || !aligned16(a_scales) || !aligned16(b_scales))
        return NVFP4_ERR_ALIGN;
    return from_hip(launch_mx_gemm(M, N, K, a_codes, a_scales, b_codes, b_scales,
                                   out_dtype == NVFP4_DTYPE_BF16, c, ldc, s));
}

size_t nvfp4_gemm_native_workspace_size(int64_t M, int64_t N, int64_t K)
{
    if (M <= 0 || N <= 0 || K <= 0 || K % 128) return 0;
    return gemm_native_bytes(M, N, K);
}

nvfp4_status nvfp4_gemm_native(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                               const uint8_t* a_scales, const float* a_tensor_scale,
                               nvfp4_block a_block, const uint8_t* b_codes,
                               const uint8_t* b_scales, const float* b_tensor_scale,
                               nvfp4_block b_block, nvfp4_dtype out_dtype, void* c, int64_t ldc,
                               int32_t* used_native, void* workspace, size_t workspace_bytes,
                               void* stream)
{
    if (a_block != NVFP4_BLOCK_1D && a_block != NVFP4_BLOCK_2D) return NVFP4_ERR_INVALID_ARG;
    if (b_block != NVFP4_BLOCK_1D && b_block != NVFP4_BLOCK_2D) return NVFP4_ERR_INVALID_ARG;
    if (out_dtype != NVFP4_DTYPE_BF16 && out_dtype != NVFP4_DTYPE_FP32) return NVFP4_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K < 0) return NVFP4_ERR_INVALID_ARG;
    if (ldc < N) return NVFP4_ERR_SHAPE;
    if (K % 128) return NVFP4_ERR_SHAPE;
    if (a_block == NVFP4_BLOCK_2D && M % 16) return NVFP4_ERR_LAYOUT;
    if (b_block == NVFP4_BLOCK_2D && N % 16) return NVFP4_ERR_LAYOUT;
    if ((uint64_t)K / 2 * 256 >= (1ull << 31)) return NVFP4_ERR_UNSUPPORTED;
    if (K > kMaxChainK) return NVFP4_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return NVFP4_OK;
    if (!c) return NVFP4_ERR_INVALID_ARG;
    const size_t esz = out_dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
    if ((reinterpret_cast<uintptr_t>(c) & (esz - 1)) != 0) return NVFP4_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (K == 0) return from_hip(launch_fill_zero(c, out_dtype == NVFP4_DTYPE_BF16, M, N, ldc, s));
    if (!a_codes || !a_scales || !a_tensor_scale || !b_codes || !b_scales || !b_tensor_scale ||
        !used_native)
        return NVFP4_ERR_INVALID_ARG;
    if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(b_codes) || !aligned16(b_scales))
        return NVFP4_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(used_native) & 3u) != 0) return NVFP4_ERR_ALIGN;
    if (!workspace || workspace_bytes < gemm_native_bytes(M, N, K)) return NVFP4_ERR_WORKSPACE;
    if (!aligned16(workspace)) return NVFP4_ERR_ALIGN;
    GemmOperand A{a_codes, a_scales, a_tensor_scale, a_block == NVFP4_BLOCK_2D, true};
    GemmOperand B{b_codes, b_scales, b_tensor_scale, b_block == NVFP4_BLOCK_2D, true};
    return from_hip(launch_gemm_native(M, N, K, A, B, out_dtype == NVFP4_DTYPE_BF16, c, ldc,
                                       used_native, static_cast<uint8_t*>(workspace), s));
}

nvfp4_status nvfp4_gemm_w4a16(int64_t M, int64_t N, int64_t K, const void* a, int64_t lda,
                              const uint8_t* b_codes, const uint8_t* b_scales,
                              const float* b_tensor_scale, nvfp4_block b_block,
                              nvfp4_dtype out_dtype, void* c, int64_t ldc, void* stream)
{
    if (b_block != NVFP4_BLOCK_1D && b_block != NVFP4_BLOCK_2D) return NVFP4_ERR_INVALID_ARG;
    if (out_dtype != NVFP4_DTYPE_BF16 && out_dtype != NVFP4_DTYPE_FP32) return NVFP4_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K < 0) return NVFP4_ERR_INVALID_ARG;
    if (ldc < N || lda < K) return NVFP4_ERR_SHAPE;
    if (K % 512) return NVFP4_ERR_SHAPE;
    if (b_block == NVFP4_BLOCK_2D && N % 16) return NVFP4_ERR_LAYOUT;
    if (M > 64) return NVFP4_ERR_UNSUPPORTED;
    if (K > kMaxChainK) return NVFP4_ERR_UNSUPPORTED;
    if ((uint64_t)N * (uint64_t)K / 2 >= (1ull << 31)) return NVFP4_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return NVFP4_OK;
    if (!c) return NVFP4_ERR_INVALID_ARG;
    const size_t esz = out_dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
    if ((reinterpret_cast<uintptr_t>(c) & (esz - 1)) != 0) return NVFP4_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (K == 0) return from_hip(launch_fill_zero(c, out_dtype == NVFP4_DTYPE_BF16, M, N, ldc, s));
    if (!a || !b_codes || !b_scales || !b_tensor_scale) return NVFP4_ERR_INVALID_ARG;
    if (!aligned16(a) || ((size_t)lda * 2) % 16 || !aligned16(b_codes) || !aligned16(b_scales))
        return NVFP4_ERR_ALIGN;
    GemmOperand B{b_codes, b_scales, b_tensor_scale, b_block == NVFP4_BLOCK_2D, true};
    return from_hip(launch_gemm_w4a16(M, N, K, static_cast<const uint16_t*>(a), lda, B,
                                      out_dtype == NVFP4_DTYPE_BF16, c, ldc, s));
}

nvfp4_status nvfp4_kv_cache_write(const void* x, nvfp4_dtype x_dtype, int64_t tokens,
                                  int64_t cols, int64_t ld_x, const int64_t* slots,
                                  const float* amax, int64_t num_slots, uint8_t* cache_codes,
                                  uint8_t* cache_scales, void* stream)
{
    if (x_dtype != NVFP4_DTYPE_BF16 && x_dtype != NVFP4_DTYPE_FP32) return NVFP4_ERR_INVALID_ARG;
    if (tokens < 0 || cols < 0 || num_slots < 0) return NVFP4_ERR_INVALID_ARG;
    if (cols % 16) return NVFP4_ERR_SHAPE;
    if (ld_x < cols) return NVFP4_ERR_SHAPE;
    if ((uint64_t)tokens * (uint64_t)(cols / 16) > kMaxItems) return NVFP4_ERR_UNSUPPORTED;
    if (tokens == 0 || cols == 0 || num_slots == 0) return NVFP4_OK;
    if (!x || !slots || !amax || !cache_codes || !cache_scales) return NVFP4_ERR_INVALID_ARG;
    const size_t esz = x_dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
    if (!aligned16(x) || !aligned16(cache_codes) || ((size_t)ld_x * esz) % 16 ||
        (reinterpret_cast<uintptr_t>(slots) & 7u))
        return NVFP4_ERR_ALIGN;
    return from_hip(launch_kv_cache_write(x, x_dtype == NVFP4_DTYPE_BF16, tokens, cols, ld_x,
                                          slots, num_slots, amax, cache_codes, cache_scales,
                                          static_cast<hipStream_t>(stream)));
}

nvfp4_status nvfp4_kv_cache_read(const uint8_t* cache_codes, const uint8_t* cache_scales,
                                 const float* amax, int64_t num_slots, int64_t cols,
                                 const int64_t* slots, int64_t n, nvfp4_dtype out_dtype, void* out,
                                 int64_t ld_out, void* stream)
{
    if (out_dtype != NVFP4_DTYPE_BF16 && out_dtype != NVFP4_DTYPE_FP32) return NVFP4_ERR_INVALID_ARG;
    if (n < 0 || cols < 0 || num_slots < 0) return NVFP4_ERR_INVALID_ARG;
    if (cols % 16) return NVFP4_ERR_SHAPE;
    if (ld_out < cols) return NVFP4_ERR_SHAPE;
    if ((uint64_t)n * (uint64_t)(cols / 8) > kMaxItems) return NVFP4_ERR_UNSUPPORTED;
    if (n == 0 || cols == 0) return NVFP4_OK;
    if (!out || !slots || !amax) return NVFP4_ERR_INVALID_ARG;
    if (num_slots > 0 && (!cache_codes || !cache_scales)) return NVFP4_ERR_INVALID_ARG;
    const size_t esz = out_dtype == NVFP4_DTYPE_BF16 ? 2 : 4;
    if (!aligned16(out) || ((size_t)ld_out * esz) % 16 ||
        (reinterpret_cast<uintptr_t>(slots) & 7u))
        return NVFP4_ERR_ALIGN;
    hipStream_t s = static_cast<hipStream_t>(stream);
    // an empty cache has no valid slot: every row reads as zeros, and the
    // gather kernel (which reads slot 0 for out-of-range slots) never runs
    if (num_slots == 0)
        return from_hip(launch_fill_zero(out, out_dtype == NVFP4_DTYPE_BF16, n, cols, ld_out, s));
    if (!aligned16(cache_codes)) return NVFP4_ERR_ALIGN;
    return from_hip(launch_kv_cache_read(cache_codes, cache_scales, amax, num_slots, cols, slots,
                                         n, out_dtype == NVFP4_DTYPE_BF16, out, ld_out, s));
}

size_t nvfp4_gemm_swiglu_workspace_size(int64_t M, int64_t N)
{
    if (M <= 0 || N <= 0) return 2 * sizeof(float);
    const uint64_t t = (uint64_t)((M + 255) / 256) * (uint64_t)((N + 255) / 256);
    return (size_t)(2 * t * sizeof(float));
}

nvfp4_status nvfp4_gemm_swiglu(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                               const uint8_t* a_scales, const float* a_tensor_scale,
                               nvfp4_block a_block, const uint8_t* b_codes,
                               const uint8_t* b_scales, const float* b_tensor_scale,
                               nvfp4_block b_block, void* h, int64_t ldh, void* act,
                               int64_t ld_act, uint32_t rht_sign_mask, float* amax,
                               float* amax_rht, void* workspace, size_t workspace_bytes,
                               void* stream)
{
    if (a_block != NVFP4_BLOCK_1D && a_block != NVFP4_BLOCK_2D) return NVFP4_ERR_INVALID_ARG;
    if (b_block != NVFP4_BLOCK_1D && b_block != NVFP4_BLOCK_2D) return NVFP4_ERR_INVALID_ARG;
    if (M < 0 || N < 0 || K < 0 || !amax || !amax_rht) return NVFP4_ERR_INVALID_ARG;
    if (N % 128 || M % 16) return NVFP4_ERR_SHAPE;
    if (K == 0 || K % 128) return NVFP4_ERR_SHAPE;
    if (ld_act < N / 2 || (h && ldh < N)) return NVFP4_ERR_SHAPE;
    // buffer records of a 256-row tile in 32 bits; tile ids in 31 bits; one
    // FP32 accumulation chain over K
    if ((uint64_t)K / 2 * 256 >= (1ull << 31)) return NVFP4_ERR_UNSUPPORTED;
    if (K > kMaxChainK) return NVFP4_ERR_UNSUPPORTED;
    const uint64_t tiles = (uint64_t)((M + 255) / 256) * (uint64_t)((N + 255) / 256);
    if (tiles >= (1ull << 31)) return NVFP4_ERR_UNSUPPORTED;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (M == 0 || N == 0) return from_hip(launch_write_zero_scale(amax, amax_rht, s));
    if (!act || !a_codes || !a_scales || !a_tensor_scale || !b_codes || !b_scales ||
        !b_tensor_scale)
        return NVFP4_ERR_INVALID_ARG;
    if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(b_codes) || !aligned16(b_scales))
        return NVFP4_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(act) & 7u) != 0 || ld_act % 4) return NVFP4_ERR_ALIGN;
    if (h && (reinterpret_cast<uintptr_t>(h) & 1u) != 0) return NVFP4_ERR_ALIGN;
    if (!workspace || workspace_bytes < nvfp4_gemm_swiglu_workspace_size(M, N))
        return NVFP4_ERR_WORKSPACE;
    if ((reinterpret_cast<uintptr_t>(workspace) & 3u) != 0) return NVFP4_ERR_ALIGN;
    GemmOperand A{a_codes, a_scales, a_tensor_scale, a_block == NVFP4_BLOCK_2D, true};
    GemmOperand B{b_codes, b_scales, b_tensor_scale, b_block == NVFP4_BLOCK_2D, true};
    return from_hip(launch_gemm_swiglu(M, N, K, A, B, h, ldh, act, ld_act, rht_sign_mask,
                                       static_cast<float*>(workspace), amax, amax_rht, s));
}

}  // extern "C"
