/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 library.
 *
 * NVFP4 is a two-level microscaled 4-bit format: E2M1 elements (1 sign,
 * 2 exponent, 1 mantissa bit), one FP8 E4M3 scale per micro-block of 16
 * elements and one FP32 scale per tensor.  Sources: guiahardware.es
 * "NVFP4: cos'e e come supera FP8 e BF16 nell'intelligenza artificiale",
 * section "Cos'e NVFP4"; chaitex.ru "FP4", section on the mathematical
 * structure of FP4 (bullets and numbered items 1-2); "Mastering Low-Precision
 * AI" (ai-news pages.dev), first paragraph.  The training recipe (readjensen.com
 * NVFP4 news page, recipe paragraph) quantizes activations and gradients in
 * 1x16 blocks, weights in 16x16 blocks (so fprop and dgrad see the same
 * values), applies a random Hadamard transform to the wgrad inputs, rounds
 * gradients stochastically, and runs the three MLP GEMMs on NVFP4 inputs
 * with BF16 outputs.
 *
 * Arithmetic convention (the pages give no formulas; every step is one
 * IEEE FP32 operation rounded to nearest-even, in this order):
 *     amax = max |x|  (over the Hadamard-transformed values when rht = 1)
 *     s_g  = amax / 2688                          (2688 = 6 * 448)
 *     per block: a_B = max |x| over the block;  t = a_B / (6 * s_g);
 *                e = E4M3 round-to-nearest-even of t, saturating at 448;
 *                d = e * s_g
 *     per element: y = x / d;  q = E2M1 of y (RNE, or stochastic), saturating at 6
 *     a block with a_B = 0, e = 0 or d = 0 stores e = 0 and q = 0.
 * Stochastic rounding rounds |y| up to the next E2M1 magnitude when
 * r < frac * 2^32 (frac = the position of |y| between its two neighbours),
 * with r the 32-bit word of Philox4x32-10 (Salmon et al., SC'11) at
 * key = (seed mod 2^32, seed >> 32), counter = (g mod 2^32, g >> 32,
 * stream_id, 0), g = idx >> 2, word idx & 3, idx = row * cols + col.
 *
 * Storage (all dense, row-major, caller-owned device memory):
 *   codes   uint8 [rows, cols/2]: byte j of a row holds element 2j in its
 *           low nibble and element 2j+1 in its high nibble.
 *   scales  uint8 E4M3 codes:  1D, axis 1 (blocks along a row):  [rows, cols/16]
 *                              1D, axis 0 (blocks down a column): [rows/16, cols]
 *                              2D (16x16 blocks):                  [rows/16, cols/16]
 *   tensor_scale  one float (s_g) in device memory.
 *
 * Conventions for every entry point:
 *   - All pointers are device pointers unless stated; `stream` is a
 *     hipStream_t (NULL = the default stream).  Work is enqueued on `stream`
 *     and the call returns without synchronizing.  The library allocates no
 *     memory and keeps no state between calls.
 *   - Argument errors are reported before anything is enqueued, so nothing
 *     is written on error.  Launch failures return NVFP4_ERR_HIP.
 *   - Inputs must be finite.  With the environment variable NVFP4_DEBUG=1
 *     nvfp4_quantize synchronizes `stream` and returns NVFP4_ERR_NONFINITE
 *     when the tensor amax is not finite.
 *   - Device pointers must be 16-byte aligned, and leading dimensions must
 *     keep every row 16-byte aligned (NVFP4_ERR_ALIGN otherwise).
 */
#ifndef NVFP4_H_
#define NVFP4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    NVFP4_OK = 0,
    NVFP4_ERR_INVALID_ARG = 1, /* null pointer, bad enum value, negative size */
    NVFP4_ERR_SHAPE = 2,       /* a dimension breaks the block or packing rules */
    NVFP4_ERR_ALIGN = 3,       /* pointer or leading dimension not 16-byte aligned */
    NVFP4_ERR_LAYOUT = 4,      /* a GEMM operand's blocks do not run along K */
    NVFP4_ERR_UNSUPPORTED = 5, /* a valid but unimplemented combination */
    NVFP4_ERR_WORKSPACE = 6,   /* workspace missing or too small */
    NVFP4_ERR_HIP = 7,         /* a HIP runtime call or kernel launch failed */
    NVFP4_ERR_NONFINITE = 8    /* NVFP4_DEBUG=1 only: amax is Inf or NaN */
} nvfp4_status;

typedef enum { NVFP4_DTYPE_BF16 = 0, NVFP4_DTYPE_FP32 = 1 } nvfp4_dtype;
typedef enum { NVFP4_BLOCK_1D = 0, NVFP4_BLOCK_2D = 1 } nvfp4_block;
typedef enum { NVFP4_ROUND_RNE = 0, NVFP4_ROUND_SR = 1 } nvfp4_round;
typedef enum { NVFP4_LAYOUT_NT = 0, NVFP4_LAYOUT_NN = 1, NVFP4_LAYOUT_TN = 2 } nvfp4_layout;

/* Library version as major * 10000 + minor * 100 + patch. */
int nvfp4_version(void);

/* Static, human-readable name of a status code (never NULL). */
const char* nvfp4_status_string(nvfp4_status status);

/*
 * Bytes of device workspace nvfp4_quantize needs for a rows x cols tensor
 * when it computes the tensor amax itself (amax_in == NULL).  The workspace
 * holds per-workgroup partial maxima and the reduced amax; it needs no
 * initialisation and may be reused by later calls on the same stream.
 */
size_t nvfp4_quantize_workspace_size(int64_t rows, int64_t cols);

/*
 * Quantize a rows x cols tensor to NVFP4.
 * Sources: two-level scaling -- guiahardware.es "Cos'e NVFP4"; chaitex.ru
 * "FP4" items 1-2.  2D weight blocks, RHT on wgrad inputs and stochastic
 * rounding of gradients -- readjensen.com recipe paragraph.
 *
 *   x, x_dtype, ld_x   input (BF16 or FP32), row r starts at x + r*ld_x elements
 *   block, axis        NVFP4_BLOCK_1D with axis 1 (16 consecutive columns of a
 *                      row) or axis 0 (16 consecutive rows of a column);
 *                      NVFP4_BLOCK_2D: 16x16 tiles, axis ignored
 *   transpose_out      0: outputs in the storage layout of x (above).
 *                      1 (1D axis 0 or 2D only): the same quantization written
 *                      as that of x^T, blocks along its rows: codes
 *                      [cols, rows/2], scales [cols, rows/16] (1D) or
 *                      [cols/16, rows/16] (2D).  Values, scales, the RHT and
 *                      the stochastic-rounding index (row * cols + col of x)
 *                      are unchanged; only the storage is transposed, so a
 *                      GEMM contracting over the rows of x reads the result
 *                      K-major.  NVFP4_ERR_UNSUPPORTED for 1D axis 1.
 *   rounding, seed, stream_id
 *                      NVFP4_ROUND_RNE, or NVFP4_ROUND_SR with the Philox
 *                      stream keyed by seed and stream_id (see above)
 *   rht, rht_sign_mask rht = 1 applies y = 1/4 * H16 * D * x to each block of
 *                      16 along `axis` before quantizing (1D only), where
 *                      D = diag(d_i), d_i = -1 iff bit i of the mask is set,
 *                      computed in FP32 as four butterfly stages at
 *                      distances 1, 2, 4, 8 followed by the 1/4 scaling
 *   amax_in            NULL: the library computes amax (needs the workspace);
 *                      else a device float used as amax as-is (it must be the
 *                      amax of exactly what is quantized, i.e. after the RHT)
 *   amax_out           NULL, or a device float that receives amax
 *   codes, scales, tensor_scale
 *                      outputs in the storage layout above
 *   workspace, workspace_bytes
 *                      device scratch of nvfp4_quantize_workspace_size bytes
 *                      (may be NULL/0 when amax_in != NULL)
 * Shape rules: rows, cols >= 0; cols % 16 == 0; rows % 16 == 0 for axis 0
 * and for 2D.  ld_x >= cols.  An empty tensor writes s_g = 0 (and amax 0).
 */
nvfp4_status nvfp4_quantize(const void* x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols,
                            int64_t ld_x, nvfp4_block block, int axis, int transpose_out,
                            nvfp4_round rounding,
                            uint64_t seed, uint32_t stream_id, int rht, uint32_t rht_sign_mask,
                            const float* amax_in, float* amax_out, uint8_t* codes,
                            uint8_t* scales, float* tensor_scale, void* workspace,
                            size_t workspace_bytes, void* stream);

/*
 * nvfp4_quantize for callers that cannot allocate device memory or pass a
 * workspace (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  Arguments, outputs and errors are those of
 * nvfp4_quantize without the workspace.  When amax_in is NULL the amax pass
 * uses a scratch array inside the library instead: 8448 bytes per GPU
 * (nvfp4_quantize_workspace_size, which does not depend on the tensor size;
 * a larger need would return NVFP4_ERR_WORKSPACE), held by each GPU the
 * library runs on until the process ends.  The call allocates nothing.  It
 * uses the scratch of the current device, so `stream` must belong to the
 * current device.  All calls on one GPU share that scratch: two calls with
 * amax_in == NULL whose work overlaps on one GPU (different streams, no
 * ordering between them) race and may compute a wrong amax; calls ordered
 * on one stream do not.  Nothing in the scratch needs to start at zero.
 */
nvfp4_status nvfp4_quantize_noalloc(const void* x, nvfp4_dtype x_dtype, int64_t rows,
                                    int64_t cols, int64_t ld_x, nvfp4_block block, int axis,
                                    int transpose_out, nvfp4_round rounding, uint64_t seed,
                                    uint32_t stream_id, int rht, uint32_t rht_sign_mask,
                                    const float* amax_in, float* amax_out, uint8_t* codes,
                                    uint8_t* scales, float* tensor_scale, void* stream);

/*
 * The same NVFP4 tensor stored as its transpose.  The recipe quantizes
 * weights in 16x16 blocks so that fprop (which reads W) and dgrad (which
 * reads W^T) see the same values (readjensen.com NVFP4 training-recipe page,
 * recipe paragraph): a 16x16 block of W is a 16x16 block of W^T with the same
 * scale, and W^T's element (c, r) is W's (r, c) with the same code.  This call
 * writes that W^T from W's codes and scales without reading W again:
 *   codes, scales     the rows x cols input in the storage layout above
 *                     (block, axis)
 *   codes_t           [cols, rows/2] <- codes of the transposed tensor
 *   scales_t          the input's scale plane transposed byte for byte:
 *                     2D [rows/16, cols/16] -> [cols/16, rows/16];
 *                     1D axis 1 [rows, cols/16] -> [cols/16, rows] (the
 *                     output's blocks run down its columns: axis 0);
 *                     1D axis 0 [rows/16, cols] -> [cols, rows/16] (axis 1)
 * The tensor scale is unchanged: the transposed tensor uses the input's
 * tensor_scale.  For 2D blocks, and for 1D round-to-nearest quantizations
 * read with the block axis swapped, the result is bit for bit the
 * quantization of x^T (same amax); stochastically rounded tensors keep the
 * rounding of x's element indices.
 * Shape rules: rows % 16 == 0, cols % 16 == 0.  codes and codes_t 16-byte
 * aligned; the output must not overlap the input.  rows or cols == 0 writes
 * nothing.
 */
nvfp4_status nvfp4_transpose(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                             int64_t cols, nvfp4_block block, int axis, uint8_t* codes_t,
                             uint8_t* scales_t, void* stream);

/*
 * Bytes of device workspace nvfp4_amax needs (per-workgroup partial maxima of
 * both results; no initialisation needed, reusable on the same stream).
 */
size_t nvfp4_amax_workspace_size(int64_t rows, int64_t cols);

/*
 * Tensor amaxes for the first step of the two-level scaling (s_g = amax /
 * 2688; guiahardware.es "Cos'e NVFP4", chaitex.ru "FP4" item 2) of a tensor
 * the recipe quantizes twice (readjensen.com recipe paragraph: row-wise for
 * fprop/dgrad, column-wise with the RHT for wgrad), in one read of x:
 *   amax      device float <- max |x|
 *   amax_rht  NULL, or a device float <- max |y| over y = the 16-point RHT
 *             down the columns of x (16 consecutive rows, sign mask
 *             rht_sign_mask, exactly as nvfp4_quantize with axis 0, rht = 1)
 * Both are exact maxima (order-independent), so passing them as amax_in to
 * nvfp4_quantize gives the same bits as letting it compute its own.
 * Shape rules: rows, cols >= 0; cols % 16 == 0; rows % 16 == 0 when amax_rht
 * is not NULL; ld_x >= cols; x and its rows 16-byte aligned.  An empty
 * tensor writes 0.  Workspace: nvfp4_amax_workspace_size bytes.
 */
nvfp4_status nvfp4_amax(const void* x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols,
                        int64_t ld_x, uint32_t rht_sign_mask, float* amax, float* amax_rht,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * The activation between the two fprop GEMMs of the MLP, fused with both
 * tensor amaxes its quantizations need (the MLP GEMMs on NVFP4 inputs with
 * BF16 outputs: readjensen.com recipe paragraph; the Llama 3 models of its
 * benchmark paragraph use SwiGLU):
 *   h         BF16 [rows, 2F], row r at h + r*ld_h elements: gate = columns
 *             [0, F), up = columns [F, 2F) (the first GEMM's output)
 *   act       BF16 [rows, F] <- BF16(BF16(silu(gate)) * up), silu(g) =
 *             g / (1 + exp(-g)) in FP32 (a BF16 framework's rounding points;
 *             the reciprocal from the hardware unit, within a couple of FP32
 *             ulp, so act may differ from another library's by one BF16 ulp
 *             where silu sits on a BF16 rounding boundary)
 *   amax      device float <- max |act|
 *   amax_rht  device float <- max |RHT16 down the columns of act| (as
 *             nvfp4_amax), the amax of act's wgrad quantization
 * Shape rules: rows % 16 == 0; F % 16 == 0; ld_h >= 2F; ld_act >= F; h, act
 * and their rows 16-byte aligned.  Workspace: nvfp4_amax_workspace_size.
 */
nvfp4_status nvfp4_swiglu_amax(const void* h, int64_t rows, int64_t F, int64_t ld_h, void* act,
                               int64_t ld_act, uint32_t rht_sign_mask, float* amax,
                               float* amax_rht, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Standalone 16-point random Hadamard transform (the wgrad-input transform
 * of the recipe paragraph, readjensen.com; "Hadamard transforms" in
 * "Mastering Low-Precision AI", third paragraph).
 * y[r*ld_y + c] = (1/4 * H16 * D * x) over each group of 16 along `axis`,
 * in FP32 exactly as nvfp4_quantize computes it with rht = 1.
 * Shape rules: cols % 16 == 0 (axis 1) / rows % 16 == 0 (axis 0); cols % 8 == 0.
 */
nvfp4_status nvfp4_rht16(const void* x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols,
                         int64_t ld_x, int axis, uint32_t sign_mask, float* y, int64_t ld_y,
                         void* stream);

/*
 * Dequantize: out[r*ld_out + c] = RN32(val(q) * e * s_g), then (for BF16
 * output) rounded to nearest-even BF16.  The element value times its block
 * scale is exact in FP32; s_g is the product's only rounding.
 * Source: the two-level decode implied by "Cos'e NVFP4" (guiahardware.es)
 * and chaitex.ru "FP4" items 1-2.
 * codes/scales/tensor_scale follow the storage layout above with the given
 * block mode and axis.  Shape rules as for nvfp4_quantize.
 */
nvfp4_status nvfp4_dequantize(const uint8_t* codes, const uint8_t* scales,
                              const float* tensor_scale, int64_t rows, int64_t cols,
                              nvfp4_block block, int axis, nvfp4_dtype out_dtype, void* out,
                              int64_t ld_out, void* stream);

/*
 * NVFP4 GEMM with FP32 accumulation: C = s_A * s_B * sum_k (q*e)_A (q*e)_B.
 * Source: the three MLP GEMMs (fprop, dgrad, wgrad) with NVFP4 inputs and
 * BF16 outputs, readjensen.com recipe paragraph.
 *   NVFP4_LAYOUT_NT (fprop):  A stored [M, K], B stored [N, K];  C = A * B^T
 *   NVFP4_LAYOUT_NN (dgrad):  A stored [M, K], B stored [K, N];  C = A * B
 *   NVFP4_LAYOUT_TN (wgrad):  A stored [K, M], B stored [K, N];  C = A^T * B
 * Each operand is an NVFP4 tensor (codes, scales, device tensor scale) in the
 * storage layout above.  Its scale blocks must run along K: a 1D operand
 * stored with K along its columns uses axis 1, one stored with K along its
 * rows uses axis 0 (the axis is implied by the layout); a 2D operand is
 * accepted in any position (NVFP4_ERR_LAYOUT is returned for 2D operands
 * whose dims are not multiples of 16).
 *   c, ldc, out_dtype  C[m*ldc + n], BF16 (recipe output) or FP32; c needs only
 *                      element alignment and ldc >= N is free
 *   workspace, workspace_bytes
 *                      nvfp4_gemm_workspace_size(layout, M, N, K) bytes of
 *                      device memory, 16-byte aligned, no initialisation
 *                      needed.  Required when K > 32768 (NVFP4_ERR_WORKSPACE
 *                      otherwise).  For K <= 32768 it is optional: with it, a
 *                      last round of 256 x 256 output tiles that would leave
 *                      at least half of the device's compute units idle runs
 *                      as two K halves per tile (two FP32 planes of M x N,
 *                      summed before the output rounding); NULL/0 runs
 *                      every tile whole.  The size depends on the current
 *                      device's compute-unit count.
 * Accumulation: the matrix unit's FP32 accumulation does not round to
 * nearest (a small bias per instruction, measured on the MI355X), so one
 * accumulation chain keeps the error within 1e-5 * sum |a*b| only up to
 * K = 32768 for all-positive products.  Above that, K is cut into slices of
 * at most 32768 (multiples of 512), each slice's s_A s_B * sum goes to its
 * own FP32 plane of the workspace, and the planes are summed in order with
 * IEEE FP32 additions before the BF16 rounding.
 * Shape rules: M, N, K >= 0; K % 16 == 0; a dimension along which codes are
 * packed but which is not K (N for NN, M and N for TN) must be a multiple of
 * 16.  K == 0 writes zeros.
 */
size_t nvfp4_gemm_workspace_size(nvfp4_layout layout, int64_t M, int64_t N, int64_t K);
nvfp4_status nvfp4_gemm(nvfp4_layout layout, int64_t M, int64_t N, int64_t K,
                        const uint8_t* a_codes, const uint8_t* a_scales,
                        const float* a_tensor_scale, nvfp4_block a_block,
                        const uint8_t* b_codes, const uint8_t* b_scales,
                        const float* b_tensor_scale, nvfp4_block b_block, nvfp4_dtype out_dtype,
                        void* c, int64_t ldc, void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Weight-only NVFP4 GEMM for decode shapes (BF16 activations, NVFP4 weights):
 *   C[m, n] = s_B * sum_k a[m, k] (q*e)_B[n, k],  FP32 accumulation.
 * Source: the juejin.cn page on NVFP4 (item 3: models trained at higher
 * precision quantized to NVFP4 and served by inference frameworks) and
 * chaitex.ru "FP4" (item 1 of the scaling scheme: the weight matrix in
 * 16-element blocks with E4M3 scales, a 32-bit tensor scale).  NT only:
 *   a, lda            BF16 activations [M, K], a[m*lda + k]
 *   b_codes/b_scales  NVFP4 weight stored [N, K] (1D blocks along K, or 2D),
 *   /b_tensor_scale   the layout of nvfp4_quantize
 *   c, ldc, out_dtype C[m*ldc + n], BF16 (RNE of the FP32 result) or FP32
 * The weight's block scale times its element is exact in BF16 (at most 6
 * significant bits), so every product is exact and only the accumulation
 * order differs from an FP64 reference.
 * Shape rules: 0 <= M <= 64 (decode; NVFP4_ERR_UNSUPPORTED above), K % 512
 * == 0, K <= 32768 (one FP32 accumulation chain; see nvfp4_gemm), lda >= K
 * with 16-byte aligned rows, N * K / 2 < 2^31, N % 16 == 0 for a 2D weight.
 * K == 0 writes zeros.
 */
nvfp4_status nvfp4_gemm_w4a16(int64_t M, int64_t N, int64_t K, const void* a, int64_t lda,
                              const uint8_t* b_codes, const uint8_t* b_scales,
                              const float* b_tensor_scale, nvfp4_block b_block,
                              nvfp4_dtype out_dtype, void* c, int64_t ldc, void* stream);

/*
 * The first fprop GEMM of the MLP with the activation after it fused into its
 * epilogue (the MLP GEMMs on NVFP4 inputs with BF16 outputs: readjensen.com
 * recipe paragraph; the Llama 3 models of its benchmark paragraph use
 * SwiGLU).  It computes, in one launch (plus two one-workgroup reductions):
 *   H         = s_A s_B A B^T rounded to BF16, exactly as nvfp4_gemm NT with
 *               BF16 output (A [M, K], B [N, K], both blocked along K);
 *               stored to h [M, N] (row pitch ldh) only when h is non-NULL
 *   act       BF16 [M, N/2] (row pitch ld_act) <- the nvfp4_swiglu_amax
 *               arithmetic on H, bit for bit
 *   amax      device float <- max |act|
 *   amax_rht  device float <- max |RHT16 down the columns of act|
 * B's rows are W_gu's gate and up rows interleaved in blocks of 64: rows
 * 128q .. 128q+63 are gate rows 64q .. 64q+63 and rows 128q+64 .. 128q+127
 * the up rows 64q .. 64q+63, so H's column 128q + c (c < 64) is gate column
 * 64q + c and 128q + 64 + c its up column.  act's column 64q + c pairs them.
 * (A weight stored in this row order is an ordinary NVFP4 tensor: quantize,
 * dequantize and the dgrad/wgrad GEMMs treat it like any other.)
 * Shape rules: N % 128 == 0; M % 16 == 0; K % 128 == 0, 0 < K <= 32768 (one
 * FP32 accumulation chain; see nvfp4_gemm); ld_act >= N/2; ldh >= N when h
 * is given.  Code and scale planes
 * 16-byte aligned; act 8-byte aligned with ld_act % 4 == 0.  M == 0 or
 * N == 0 writes only amax = amax_rht = 0.  Workspace:
 * nvfp4_gemm_swiglu_workspace_size(M, N) bytes (two floats per 256 x 256
 * output tile).
 */
size_t nvfp4_gemm_swiglu_workspace_size(int64_t M, int64_t N);
nvfp4_status nvfp4_gemm_swiglu(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                               const uint8_t* a_scales, const float* a_tensor_scale,
                               nvfp4_block a_block, const uint8_t* b_codes,
                               const uint8_t* b_scales, const float* b_tensor_scale,
                               nvfp4_block b_block, void* h, int64_t ldh, void* act,
                               int64_t ld_act, uint32_t rht_sign_mask, float* amax,
                               float* amax_rht, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * NVFP4 GEMM on the native scaled FP4 matrix instruction, where that is
 * exact.  The pages note that CDNA 4's matrix cores support FP4 natively
 * (guiahardware.es, "NVFP4: cos'e e come supera FP8 e BF16", section "Roadmap
 * e disponibilita").  That instruction multiplies each 32 K-consecutive E2M1
 * codes of an operand row by one power of two (E8M0), while NVFP4 scales
 * each 16 with an E4M3 value.  The two agree exactly on a row's 32-K block
 * when each of its two 16-element scales is a power of two or is zero over
 * all-zero codes, and the non-zero ones are equal: then every element's
 * value q * e * s_g is code * 2^k * s_g with one k per 32, and s_A * s_B
 * goes to the epilogue.  Real tensors' E4M3 scales are rarely like that, so
 * this is a path for data that is (for instance quantized with power-of-two
 * block scales), not a replacement for nvfp4_gemm.
 *
 * nvfp4_gemm_native: C[M, N] = s_A s_B sum_k (q e)_A (q e)_B, NT (A [M, K],
 *   B [N, K], both with blocks along K, 1D or 2D), FP32 accumulation, BF16
 *   (RNE) or FP32 out.  The call checks every 32-K block of both operands on
 *   the device, writes the E8M0 planes into the workspace, and runs the
 *   native kernel when every block passes, else the FP16 kernel of
 *   nvfp4_gemm (both are launched; each exits at once unless chosen).  The
 *   result is that of nvfp4_gemm either way, to the same tolerance.
 *   *used_native (device int32, caller-owned) ends as 1 when the native path
 *   ran, 0 otherwise; calls that overlap on one stream must not share it.
 *   Shape rules: K % 128 == 0; K <= 32768 (one FP32 accumulation chain);
 *   2D operands need their rows % 16 == 0; ldc >= N; operand planes and the
 *   workspace 16-byte aligned, used_native 4-byte aligned, c element-aligned.
 *   K == 0 writes zeros and leaves *used_native unchanged.
 * nvfp4_gemm_native_workspace_size: the E8M0 planes, M * K/32 (rounded up to
 *   16) + N * K/32 bytes.
 */
size_t nvfp4_gemm_native_workspace_size(int64_t M, int64_t N, int64_t K);
nvfp4_status nvfp4_gemm_native(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                               const uint8_t* a_scales, const float* a_tensor_scale,
                               nvfp4_block a_block, const uint8_t* b_codes,
                               const uint8_t* b_scales, const float* b_tensor_scale,
                               nvfp4_block b_block, nvfp4_dtype out_dtype, void* c, int64_t ldc,
                               int32_t* used_native, void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * MXFP4, the power-of-two-scaled format the pages compare NVFP4 with
 * ("NVFP4: cos'e e come supera FP8 e BF16", guiahardware.es, section "Cos'e
 * NVFP4": NVFP4's E4M3 scales against power-of-two scaling such as MXFP4;
 * chaitex.ru "FP4", the comparison with the open standard: MXFP4 has larger
 * blocks and coarser scales).  The pages give neither the block size nor the
 * scale rule; these follow the OCP Microscaling Formats (MX) v1.0
 * specification: 32 consecutive elements of a row share one E8M0 scale byte
 * u (X = 2^(u - 127)), X = 2^(floor(log2 amax) - 2) with the exponent clamped
 * to >= -127 (zero blocks get u = 0), and each element is x / X rounded to
 * E2M1 to nearest-even, saturating at +-6, sign kept.  No tensor scale.
 *
 * Storage: codes [rows, cols/2] packed as for NVFP4 (low nibble = even
 * column), scales [rows, cols/32] row-major, one byte each.
 *
 * nvfp4_mx_quantize: x[r*ld_x + c] (BF16 or FP32) -> codes, scales.
 *   Shape rules: cols % 32 == 0; ld_x >= cols; x, codes 16-byte aligned and
 *   x's row pitch a multiple of 16 bytes.  rows or cols == 0 writes nothing.
 * nvfp4_mx_dequantize: out[r*ld_out + c] = val(q) * X (exact in FP32), BF16
 *   output rounded to nearest-even.  cols % 32 == 0; ld_out >= cols.
 * nvfp4_mx_gemm: C[M, N] = A[M, K] * B[N, K]^T (NT: both stored K-major)
 *   with FP32 accumulation on the native scaled FP4 MFMA, BF16 (RNE) or
 *   FP32 out.  K % 128 == 0; K <= 32768 (one FP32 accumulation chain; see
 *   nvfp4_gemm); ldc >= N; c element-aligned, operand planes 16-byte
 *   aligned.  K == 0 writes zeros.
 * All pointers are caller-owned device memory; launches are asynchronous on
 * `stream`; argument errors return before anything is enqueued.
 */
nvfp4_status nvfp4_mx_quantize(const void* x, nvfp4_dtype x_dtype, int64_t rows, int64_t cols,
                               int64_t ld_x, uint8_t* codes, uint8_t* scales, void* stream);
nvfp4_status nvfp4_mx_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                                 int64_t cols, nvfp4_dtype out_dtype, void* out, int64_t ld_out,
                                 void* stream);
nvfp4_status nvfp4_mx_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                           const uint8_t* a_scales, const uint8_t* b_codes,
                           const uint8_t* b_scales, nvfp4_dtype out_dtype, void* c, int64_t ldc,
                           void* stream);

/*
 * NVFP4 KV cache (NVIDIA-blog translation on juejin.cn, point 3: libraries
 * keep the KV cache in NVFP4 for long contexts and large batches; "FP4",
 * chaitex.ru, mathematical-structure section: 16-element micro-blocks with
 * an E4M3 scale and an FP32 tensor scale).  The pages say nothing more; the
 * reading taken:
 *   - a cache holds num_slots rows of `cols` features (e.g. KV heads x head
 *     dim), in 1x16 blocks along the features, rounded to nearest-even;
 *   - its tensor scale is fixed while rows arrive: s_g = RN(*amax / 2688)
 *     from a calibration amax the caller keeps on the device (FP32 scalar);
 *     features beyond it saturate (block scale 448, element +-6);
 *   - every row written equals the 1x16 RNE quantization of that token row
 *     with amax_in = *amax (nvfp4_quantize), and reads equal
 *     nvfp4_dequantize of the rows gathered.
 * Storage: cache_codes [num_slots, cols/2] (low nibble = even column),
 * cache_scales [num_slots, cols/16] row-major E4M3 bytes.
 *
 * nvfp4_kv_cache_write: token t (row t of x, pitch ld_x elements, BF16 or
 *   FP32) goes to cache row slots[t] (int64, device).  A slot outside
 *   [0, num_slots) skips the token (padding); other cache rows are left
 *   untouched.  Two tokens with the same valid slot race (either may win).
 *   cols % 16 == 0; ld_x >= cols; x, cache_codes 16-byte aligned and x's row
 *   pitch a multiple of 16 bytes; slots 8-byte aligned.  tokens == 0 or
 *   cols == 0 writes nothing.
 * nvfp4_kv_cache_read: out row j (pitch ld_out elements, BF16 RNE or FP32)
 *   = v = RN32(val * e * s_g) of cache row slots[j], or zeros when slots[j]
 *   is outside [0, num_slots).  Slots may repeat.  An empty cache
 *   (num_slots == 0; cache_codes and cache_scales may then be NULL) reads
 *   zeros for every row.  cols % 16 == 0; ld_out >= cols; out and
 *   cache_codes 16-byte aligned, out's row pitch a multiple of 16 bytes.
 * All pointers are caller-owned device memory; launches are asynchronous on
 * `stream`; argument errors return before anything is enqueued.
 */
nvfp4_status nvfp4_kv_cache_write(const void* x, nvfp4_dtype x_dtype, int64_t tokens,
                                  int64_t cols, int64_t ld_x, const int64_t* slots,
                                  const float* amax, int64_t num_slots, uint8_t* cache_codes,
                                  uint8_t* cache_scales, void* stream);
nvfp4_status nvfp4_kv_cache_read(const uint8_t* cache_codes, const uint8_t* cache_scales,
                                 const float* amax, int64_t num_slots, int64_t cols,
                                 const int64_t* slots, int64_t n, nvfp4_dtype out_dtype, void* out,
                                 int64_t ld_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H_ */
