// NVFP4 GEMM for decode shapes (M <= 64 activation rows): the packed weights
// dominate the traffic, so these kernels stream them once at full width and
// keep the few activation rows on chip.  Same arithmetic as gemm.hip: E2M1 x
// E4M3 products exact in FP16 (or BF16 for the weight-only GEMM), FP32
// accumulation, s_A s_B applied in the epilogue.
#include "gemm_common.h"
#include "launch.h"

namespace nvfp4 {

// ---------------------------------------------------------------------------
// Weight-only decode GEMM for 17..64 rows (BF16 activations x NVFP4 weights,
// K a multiple of the K chunk KC = 512): C[M, N] = A[M, K] B[N, K]^T.  (Up to
// 16 rows the weight-streaming kernel below takes the weight-only GEMM too.)  The packed
// weights B dominate the traffic (4.5 bits per element) and are streamed
// once: each wave owns 16 rows of B (16 output columns) over all of K.  Inside
// a chunk, lane group g = lane / 16 owns the contiguous K quarter g KC/4 ..
// +KC/4 (one 16-byte code load per 128 K, and its scale bytes for the whole
// chunk in one or two wide loads: the load path is limited by accesses per
// lane, so 2-byte scale loads per step would cost as much as the codes).  The
// few activation rows are copied into LDS as they are (32-element BF16
// pieces, no activation scales), one chunk at a time, in the same
// lane-quarter order (16 bytes of padding per quarter keep the quarters on
// different banks).  Both operands are prefetched into registers one chunk
// ahead, issued after everything the current chunk waits for (vector-memory
// counters drain in order).  Short chunks stream best: with 2048 or 1024 the
// same weights took 15-25% longer (more bytes in flight per wave, in larger
// bursts).  Each weight word is dequantized to BF16 exactly for
// v_mfma_f32_16x16x32_bf16: at step s lane (row l % 16, group g) supplies
// k = kc + g KC/4 + 32 st + 8 s + [0, 8) for both operands.  Rows past M or N
// are clamped to the last valid row (never stored).
// ---------------------------------------------------------------------------
constexpr int kSkN = 64;  // output columns per workgroup

template <int KC, int RMAX>
__global__ __launch_bounds__(256) void k_gemm_w4a16(GemmParams p)
{
    constexpr int kSteps = KC / 128;                 // B steps per chunk
    constexpr int kQ = KC / 4;                       // K of one lane quarter per chunk
    constexpr int kQStride = kQ * 2 + 16;            // LDS bytes per activation row quarter
    constexpr int kRow = 4 * kQStride;               // LDS bytes per activation row
    constexpr int kAPer = RMAX * 16 * KC / 32 / 256; // 32-code activation pieces per thread
    constexpr int kSB = 2 * kSteps;                  // scale bytes per lane and chunk
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int lr = lane & 15, g = lane >> 4;
    const int64_t n = (int64_t)blockIdx.x * kSkN + wave * 16 + lr;  // B row of this lane
    const int64_t nc = n < p.N ? n : p.N - 1;                       // clamped for loads
    const int64_t K = p.K, lds_b = K / 16;
    // B through buffer resources over the whole code / scale planes (below
    // 2 GiB): per-lane offsets in VGPRs, the chunk offset scalar, the step
    // offset an immediate.  Past the last chunk the prefetch goes through
    // resources with no records (out-of-range loads return zeros, touching no
    // memory), so the loop body has no branch around it.
    const __amdgpu_buffer_rsrc_t rc =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.b_codes, (short)0, 0x7FFFFFFF, 0x00020000);
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.b_scales, (short)0, 0x7FFFFFFF, 0x00020000);
    const __amdgpu_buffer_rsrc_t none =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.b_codes, (short)0, 0, 0x00020000);
    // lane group g loads its quarter of the chunk directly, 16 bytes per step
    const int bo = (int)(nc * (K / 2)) + (kQ / 2) * g;
    const int bso = (int)(p.b2d ? (nc / 16) * lds_b : nc * lds_b) + (kQ / 16) * g;
    // Workgroups walk K starting at different chunks: rows are K/2 bytes
    // apart, so if every workgroup read the same chunk at once, all reads
    // would fall in the same few byte ranges of the row pitch (the same
    // memory channels).  The sum over chunks is the same in any order.
    const int nchunks = (int)(K / KC);
    const int rot = (int)(blockIdx.x % (unsigned)nchunks) * KC;
    auto kpos = [&](int kc) { return kc + rot >= (int)K ? kc + rot - (int)K : kc + rot; };
    float4_t acc[RMAX];
#pragma unroll
    for (int r = 0; r < RMAX; ++r) acc[r] = float4_t{0.f, 0.f, 0.f, 0.f};

    // B: lane g owns the contiguous quarter kc + g KC/4 .. +KC/4 of each chunk,
    // 32 codes per step, so its scale bytes for the chunk are one contiguous
    // run of kSB bytes
    u32x4 bc[kSteps], bn[kSteps];
    u32x4 aw[kAPer][4];  // BF16 pieces (64 bytes each)
    uint32_t bs[kSB / 4], bsn[kSB / 4];
    auto load_a = [&](int64_t kc) {
#pragma unroll
        for (int i = 0; i < kAPer; ++i) {
            int idx = threadIdx.x + 256 * i;
            int m = idx / (KC / 32), c = idx % (KC / 32);
            int64_t mc = m < p.M ? m : p.M - 1;
            int64_t k = kc + 32 * c;
            k = k < K ? k : K - 32;  // the prefetch past the last chunk reads a valid piece
            const u32x4* src = reinterpret_cast<const u32x4*>(p.a_bf16 + mc * p.lda + k);
#pragma unroll
            for (int q = 0; q < 4; ++q) aw[i][q] = src[q];
        }
    };
    auto load_b = [&](__amdgpu_buffer_rsrc_t c_rsrc, __amdgpu_buffer_rsrc_t s_rsrc, int kc,
                      u32x4* c, uint32_t* sc) {
#pragma unroll
        for (int st = 0; st < kSteps; ++st)
            c[st] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(c_rsrc, bo + 16 * st, kc / 2, 0));
#pragma unroll
        for (int q = 0; q < kSB / 4; q += (kSB >= 16 ? 4 : 2)) {
            if (kSB >= 16) {
                u32x4 w = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(s_rsrc, bso + 4 * q, kc / 16, 0));
                sc[q] = w[0]; sc[q + 1] = w[1]; sc[q + 2] = w[2]; sc[q + 3] = w[3];
            } else {
                u32x2 w = __builtin_bit_cast(
                    u32x2, __builtin_amdgcn_raw_buffer_load_b64(s_rsrc, bso + 4 * q, kc / 16, 0));
                sc[q] = w[0]; sc[q + 1] = w[1];
            }
        }
    };

    // one chunk: its activations into LDS, the next chunk's operands issued,
    // then the products with the B registers loaded one chunk earlier.  The
    // chunk loop runs in pairs with the two B register sets swapping roles,
    // so no register copy (and no wait for the prefetch) sits in the loop.
    auto chunk = [&](int kc, const u32x4 (&cb)[kSteps], const uint32_t (&cs)[kSB / 4],
                     u32x4 (&nb)[kSteps], uint32_t (&ns)[kSB / 4]) {
        // activations of this chunk -> FP16 in LDS, row-major by lane quarter
        // (the previous chunk's readers are done); rows past M hold the last
        // row again and are never stored.  The barriers only order LDS
        // accesses: a plain s_barrier after draining this wave's LDS counter
        // (a __syncthreads fence would also wait for the prefetch in flight).
        NVFP4_WAIT_LGKMCNT0();
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int i = 0; i < kAPer; ++i) {
            int idx = threadIdx.x + 256 * i;
            int m = idx / (KC / 32), c = idx % (KC / 32);
            const int kl = 32 * c;  // K offset inside the chunk
            uint8_t* dst = lds + m * kRow + (kl / kQ) * kQStride + (kl % kQ) * 2;
#pragma unroll
            for (int q = 0; q < 4; ++q) *reinterpret_cast<u32x4*>(dst + 16 * q) = aw[i][q];
        }
        NVFP4_WAIT_LGKMCNT0();
        __builtin_amdgcn_s_barrier();
        // next chunk's operands, A strictly before B (the next chunk's
        // dequantization then waits for A alone); past the end through the
        // record-less resources
        const bool more = kc + KC < (int)K;
        __builtin_amdgcn_sched_barrier(0);
        load_a(kpos(kc + KC));
        __builtin_amdgcn_sched_barrier(0);
        load_b(more ? rc : none, more ? rs : none, more ? kpos(kc + KC) : 0, nb, ns);
        __builtin_amdgcn_sched_barrier(0);
        u32x4 cq[kSteps];
#pragma unroll
        for (int st = 0; st < kSteps; ++st) cq[st] = cb[st];
#pragma unroll
        for (int st = 0; st < kSteps; ++st) {
            // the step's A fragments first (one LDS latency per step), then
            // its four B dequantizations and MFMAs
            bf16x8_t af[4][RMAX];
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int r = 0; r < RMAX; ++r)
                    af[s][r] = *reinterpret_cast<const bf16x8_t*>(
                        lds + (16 * r + lr) * kRow + g * kQStride + (32 * st + 8 * s) * 2);
            // scale bytes 2 st, 2 st + 1 of the lane's run
            const uint32_t sw = cs[st >> 1] >> (16 * (st & 1));
            const float e0 = __builtin_amdgcn_cvt_f32_fp8((int)sw, 0);
            const float e1 = __builtin_amdgcn_cvt_f32_fp8((int)sw, 1);
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bf16x8_t bf = dequant_word_bf16(cq[st][s], s < 2 ? e0 : e1);
#pragma unroll
                for (int r = 0; r < RMAX; ++r)
                    acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        af[s][r], bf, acc[r], 0, 0, 0);
            }
            __builtin_amdgcn_sched_group_barrier(0x100, 4 * RMAX, 0);   // LDS reads
            __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);         // scale + B dequant
            __builtin_amdgcn_sched_group_barrier(0x008, 4 * RMAX, 0);   // MFMAs
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    __builtin_amdgcn_sched_barrier(0);
    load_a(kpos(0));
    __builtin_amdgcn_sched_barrier(0);
    load_b(rc, rs, kpos(0), bc, bs);
    __builtin_amdgcn_sched_barrier(0);
    // both exits leave the loop, so the loop head is reached only after the
    // second chunk of a pair (its registers are the live ones there)
    for (int kc = 0;; kc += 2 * KC) {
        chunk(kc, bc, bs, bn, bsn);
        if (kc + KC >= (int)K) break;
        chunk(kc + KC, bn, bsn, bc, bs);
        if (kc + 2 * KC >= (int)K) break;
    }
    // lane holds C[16 r + 4 g + j][n] in acc[r][j]
    const float sab = *p.b_ts;
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            int64_t row = 16 * r + 4 * g + j;
            if (row < p.M && n < p.N) {
                float v = acc[r][j] * sab;
                if (p.out_bf16) {
                    uint32_t u = __float_as_uint(v);
                    u += 0x7FFFu + ((u >> 16) & 1u);
                    reinterpret_cast<uint16_t*>(p.c)[row * p.ldc + n] = (uint16_t)(u >> 16);
                } else {
                    reinterpret_cast<float*>(p.c)[row * p.ldc + n] = v;
                }
            }
        }
    }
}

typedef int v8i_t __attribute__((ext_vector_type(8)));

// The E4M3 value of byte e of w, as FP32 (exact).
__device__ __forceinline__ float e4m3_value(uint32_t w, int e)
{
    return e == 0 ? __builtin_amdgcn_cvt_f32_fp8((int)w, 0)
         : e == 1 ? __builtin_amdgcn_cvt_f32_fp8((int)w, 1)
         : e == 2 ? __builtin_amdgcn_cvt_f32_fp8((int)w, 2)
                  : __builtin_amdgcn_cvt_f32_fp8((int)w, 3);
}

// ---------------------------------------------------------------------------
// Weight-streaming decode kernel: C[M, N] = A[M, K] B[N, K]^T for M <= 16 RMAX
// activation rows.  A workgroup owns 64 weight rows (64 output columns) and
// walks K in 512-K chunks.  The weights are read the way HBM streams them
// best: each copy instruction moves four whole 256-byte row pieces (1 KB,
// contiguous per row) straight into LDS (buffer loads with the LDS flag),
// two chunks ahead of use in a three-stage ring (the activations one chunk
// ahead, in registers; a four-stage ring measured slower at every M).  Each
// lane loads the 16-byte
// piece that its LDS slot holds, so the row pieces land XOR-swizzled (piece p
// of row r at position p ^ (r % 16)) and a fragment read's 16 lanes of one
// lane group (16 rows, one piece) hit 16 different bank groups.  Inside a chunk the four waves split
// K: wave w contracts the chunk's K quarter w (128 K) for all 64 columns and
// all activation rows, so every weight byte is read from LDS once and every
// activation element is loaded (from L2: the activations are tiny and shared
// by every workgroup) and dequantized once per workgroup.  Lane (row l % 16,
// group g = l / 16) takes K values 128 w + 32 g + [0, 32) of the chunk: one
// 16-byte fragment read per weight tile and one 16-byte load per activation
// tile, whose four 32-bit words feed four v_mfma_f32_16x16x32_f16 (word s:
// K 8 s + [0, 8) of the lane's 32).  The waves' FP32 partial tiles are summed
// through LDS at the end in a fixed order.  Rows past M or N are clamped to
// the last valid row for loads and never stored.
// ---------------------------------------------------------------------------
constexpr int kDlKC = 512;                   // K per chunk
constexpr int kDlCodes = 64 * 256;           // code bytes per stage (64 rows x 256 B)
constexpr int kDlStage = kDlCodes + 64 * 32; // + 32 scale bytes per row
constexpr int kDlStride = 64 + 4;            // LDS row pitch (floats) of the partial tiles

// LDS of the kernel: the ring of nst stages, reused at the end for the
// partial tiles
__host__ __device__ constexpr int decode_lds_bytes(int rmax, int nst)
{
    return nst * kDlStage > 4 * 16 * rmax * kDlStride * 4 ? nst * kDlStage
                                                          : 4 * 16 * rmax * kDlStride * 4;
}

// NST ring stages: chunk i + NST - 1 is copied while chunk i is computed, and
// the activations of chunk i + NST - 2 are loaded then (NST - 1 register sets).
// kA16: the weight-only GEMM (BF16 activations [M, K], row pitch lda; no
// activation scales): the lane's 32 activation values come as four 16-byte
// loads used as they are, the weight words are dequantized to BF16 exactly
// (dequant_word_bf16) and the products are v_mfma_f32_16x16x32_bf16.
// kRow1: one activation row (M == 1), contracted on the FP4 MFMA with the
// block scales applied to its output: the activation operand's 16 rows are
// the wave's 8 K blocks (row i keeps block i's 16 codes and zeros elsewhere;
// rows 8-15 are zero), so the MFMA (v_mfma_scale_f32_16x16x128_f8f6f4, both
// operands E2M1, unit scales) returns the per-block code dot products
// sum_k a_k w_nk of 16 weight rows exactly (each at most 16 products of
// E2M1 values: multiples of 1/4 below 2^10), and each is then multiplied by
// its block's scale product s_a s_w (exact: two E4M3 values) and summed in
// FP32.  No operand is dequantized.
template <int RMAX, int NST, bool kA16 = false, bool kRow1 = false>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_gemm_decode_lds(GemmParams p)
{
    static_assert(NST == 3 || NST == 4, "three or four ring stages");
    static_assert(!kRow1 || (RMAX == 1 && !kA16), "single activation row, NVFP4");
    constexpr int NA = NST - 1;
    constexpr int AW = kA16 ? 4 : 1;             // 16-byte activation loads per row tile
    constexpr int kAOps = RMAX * (AW + (kA16 ? 0 : 1));  // activation loads per chunk
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lr = lane & 15, g = lane >> 4;
    const int64_t K = p.K, n0 = (int64_t)blockIdx.x * 64;
    const int nch = (int)(K / kDlKC);
    const __amdgpu_buffer_rsrc_t rbc =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.b_codes, (short)0, 0x7FFFFFFF, 0x00020000);
    const __amdgpu_buffer_rsrc_t rbs =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.b_scales, (short)0, 0x7FFFFFFF, 0x00020000);
    const __amdgpu_buffer_rsrc_t rac = __builtin_amdgcn_make_buffer_rsrc(
        kA16 ? (void*)p.a_bf16 : (void*)p.a_codes, (short)0, 0x7FFFFFFF, 0x00020000);
    const __amdgpu_buffer_rsrc_t ras = __builtin_amdgcn_make_buffer_rsrc(
        kA16 ? (void*)p.a_bf16 : (void*)p.a_scales, (short)0, 0x7FFFFFFF, 0x00020000);
    // no records: loads through it return zeros and touch no memory (the
    // copies past the last chunk, which keep the wait counts uniform)
    const __amdgpu_buffer_rsrc_t none =
        __builtin_amdgcn_make_buffer_rsrc((void*)p.b_codes, (short)0, 0, 0x00020000);
    auto clamp_n = [&](int64_t n) { return n < p.N ? n : p.N - 1; };
    // copy offsets: code copy j of this wave moves rows 16 w + 4 j + l / 16,
    // the piece its slot l % 16 holds; scale copy h rows 16 w + 8 h + l / 8,
    // bytes 4 (l % 8) of the row's 32
    int cof[4], sof[2];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 16 * wave + 4 * j + (lane >> 4);
        const int piece = (lane & 15) ^ (r & 15);
        cof[j] = (int)(clamp_n(n0 + r) * (K / 2)) + 16 * piece;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int64_t n = clamp_n(n0 + 16 * wave + 8 * h + (lane >> 3));
        sof[h] = (int)((p.b2d ? n / 16 : n) * (K / 16)) + 4 * (lane & 7);
    }
    int aco[RMAX], aso[RMAX];
#pragma unroll
    for (int r = 0; r < RMAX; ++r) {
        int64_t m = 16 * r + lr;
        m = m < p.M ? m : p.M - 1;
        if constexpr (kA16) {
            aco[r] = (int)(m * p.lda * 2) + 256 * wave + 64 * g;  // bytes of BF16
            aso[r] = 0;
        } else {
            aco[r] = (int)(m * (K / 2)) + 64 * wave + 16 * g;
            aso[r] = (int)((p.a2d ? m / 16 : m) * (K / 16)) + 8 * wave +
                     (kRow1 ? 4 * (g & 1) : 2 * g);
        }
    }
    // chunks start at a per-workgroup offset so the workgroups do not all
    // read the same byte ranges of the row pitch at once
    const int rot = (int)(blockIdx.x % (unsigned)nch);
    auto kpos = [&](int i) {
        const int j = i + rot;
        return (j >= nch ? j - nch : j) * kDlKC;
    };
    // the six copies of chunk i into ring stage st (through `none` past the end)
    auto copy = [&](int i, int st) {
        const bool live = i < nch;
        const __amdgpu_buffer_rsrc_t rc = live ? rbc : none, rs = live ? rbs : none;
        const int kc = live ? kpos(i) : 0;
        uint8_t* base = lds + st * kDlStage;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rc, (lds_void_t*)(base + (16 * wave + 4 * j) * 256), 16, cof[j], kc / 2, 0, 0);
#pragma unroll
        for (int h = 0; h < 2; ++h)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (lds_void_t*)(base + kDlCodes + (16 * wave + 8 * h) * 32), 4, sof[h], kc / 16,
                0, 0);
    };
    u32x4 ac[NA][RMAX][AW];
    uint32_t as[NA][RMAX];
    auto load_a = [&](int i, u32x4 (&c)[RMAX][AW], uint32_t (&sc)[RMAX]) {
        const bool live = i < nch;
        const __amdgpu_buffer_rsrc_t rc = live ? rac : none, rs = live ? ras : none;
        const int kc = live ? kpos(i) : 0;
#pragma unroll
        for (int r = 0; r < RMAX; ++r)
#pragma unroll
            for (int h = 0; h < AW; ++h)
                c[r][h] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(rc, aco[r] + 16 * h,
                                                                 kA16 ? 2 * kc : kc / 2, 0));
        __builtin_amdgcn_sched_barrier(0);  // the same load order in the prologue and the loop
        if constexpr (kRow1) {
            sc[0] = __builtin_amdgcn_raw_buffer_load_b32(rs, aso[0], kc / 16, 0);
        } else if constexpr (!kA16) {
#pragma unroll
            for (int r = 0; r < RMAX; ++r)
                sc[r] = __builtin_amdgcn_raw_buffer_load_b16(rs, aso[r], kc / 16, 0);
        }
    };
    float4_t acc[4][RMAX];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < RMAX; ++r) acc[t][r] = float4_t{0.f, 0.f, 0.f, 0.f};
    // kRow1: the lane's running sum for weight row n0 + 16 t + lr (blocks
    // 4 g .. 4 g + 3 of each wave's 8; lane groups 2 and 3 hold zero rows)
    float ysum[4] = {0.f, 0.f, 0.f, 0.f};
    // kRow1: which half of the lane's 32 activation codes its operand row
    // keeps (row lr is block lr: codes 0-15 of lane group lr / 2)
    const bool keep_lo = lr == 2 * g, keep_hi = lr == 2 * g + 1;
    // fragment address of weight row 16 t + lr in a stage, less 4096 t: piece
    // 4 w + g sits at slot (4 w + g) ^ lr (the row's low four bits are lr)
    const int frag_off = lr * 256 + 16 * ((4 * wave + g) ^ lr);
    // chunk i from ring stage st with the activation registers of chunk i
    auto compute = [&](int st, const u32x4 (&ac)[RMAX][AW], const uint32_t (&as)[RMAX]) {
        const uint8_t* base = lds + st * kDlStage;
        if constexpr (kRow1) {
            u32x4 bc[4];
            uint32_t bs[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                // row 16 t + lr (its piece slot depends on lr only): the
                // lane's address plus a constant per tile
                bc[t] = *reinterpret_cast<const u32x4*>(base + frag_off + 4096 * t);
                // scale bytes of blocks 8 w + 4 (g & 1) .. +3 of the chunk
                bs[t] = *reinterpret_cast<const uint32_t*>(base + kDlCodes + lr * 32 + 512 * t +
                                                           8 * wave + 4 * (g & 1));
            }
            __builtin_amdgcn_sched_barrier(0);
            const u32x4 a = ac[0][0];
            v8i_t af;
            af[0] = keep_lo ? (int)a[0] : 0;
            af[1] = keep_lo ? (int)a[1] : 0;
            af[2] = keep_hi ? (int)a[2] : 0;
            af[3] = keep_hi ? (int)a[3] : 0;
            af[4] = 0; af[5] = 0; af[6] = 0; af[7] = 0;
            float sa[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) sa[e] = e4m3_value(as[0], e);
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                v8i_t bf;
                bf[0] = (int)bc[t][0]; bf[1] = (int)bc[t][1];
                bf[2] = (int)bc[t][2]; bf[3] = (int)bc[t][3];
                bf[4] = 0; bf[5] = 0; bf[6] = 0; bf[7] = 0;
                const float4_t d = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    af, bf, float4_t{0.f, 0.f, 0.f, 0.f}, 4, 4, 0, 127, 0, 127);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    ysum[t] = __builtin_fmaf(d[e], sa[e] * e4m3_value(bs[t], e), ysum[t]);
            }
            return;
        } else {
        u32x4 bc[4];
        uint32_t bs[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            bc[t] = *reinterpret_cast<const u32x4*>(base + frag_off + 4096 * t);
            bs[t] = *reinterpret_cast<const uint16_t*>(base + kDlCodes + lr * 32 + 512 * t +
                                                       8 * wave + 2 * g);
        }
        // all eight LDS reads in flight before the activations' dequantization
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (kA16) {
            // word s of the lane's 32 K: activation load s as it is, weight word
            // s in BF16 with scale byte s / 2 of the pair
            float e[4][2];
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                e[t][0] = __builtin_amdgcn_cvt_f32_fp8((int)bs[t], 0);
                e[t][1] = __builtin_amdgcn_cvt_f32_fp8((int)bs[t], 1);
            }
#pragma unroll
            for (int s = 0; s < 4; ++s) {
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const bf16x8_t bf = dequant_word_bf16(bc[t][s], e[t][s >> 1]);
#pragma unroll
                    for (int r = 0; r < RMAX; ++r)
                        acc[t][r] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                            __builtin_bit_cast(bf16x8_t, ac[r][s]), bf, acc[t][r], 0, 0, 0);
                }
            }
            return;
        } else {
        // Software-pipelined over the four words s: the operands of word
        // s + 1 are dequantized (into the other register set) while the
        // MFMAs of word s run, one MFMA then kV VALU instructions at a time.
        // With one set, each dequantization would overwrite registers that
        // the MFMAs before it still read, and wait for them.
        constexpr int kV = (RMAX + 4) * 8 / (4 * RMAX);  // VALU per MFMA
        half2_t ae[RMAX], be[4];
#pragma unroll
        for (int r = 0; r < RMAX; ++r)
            ae[r] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(as[r], 1.0f, false);
#pragma unroll
        for (int t = 0; t < 4; ++t)
            be[t] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(bs[t], 1.0f, false);
        half8_t af[2][RMAX], bf[2][4];
#pragma unroll
        for (int r = 0; r < RMAX; ++r) af[0][r] = dequant_word(ac[r][0][0], ae[r][0]);
#pragma unroll
        for (int t = 0; t < 4; ++t) bf[0][t] = dequant_word(bc[t][0], be[t][0]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const int c = s & 1, n = c ^ 1;
            if (s < 3) {
#pragma unroll
                for (int r = 0; r < RMAX; ++r)
                    af[n][r] = dequant_word(ac[r][0][s + 1], ae[r][(s + 1) >> 1]);
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    bf[n][t] = dequant_word(bc[t][s + 1], be[t][(s + 1) >> 1]);
            }
#pragma unroll
            for (int t = 0; t < 4; ++t)
#pragma unroll
                for (int r = 0; r < RMAX; ++r)
                    acc[t][r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(af[c][r], bf[c][t], acc[t][r],
                                                                      0, 0, 0);
            if (s < 3) {
#pragma unroll
                for (int q = 0; q < 4 * RMAX; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, kV, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        }
        }
    };
    // Issue order: copy(0), A(0), copy(1), A(1), ... (the activations of chunk
    // j right after the copies of chunk j, before those of chunk j + 1): the
    // prologue issues up to copy(NST - 2), iteration i then A(i + NST - 2) and
    // copy(i + NST - 1).  At the top of iteration i, chunk i's copies and
    // activations have landed once at most the later NST - 2 chunks' copies
    // and NST - 3 chunks' activation loads are in flight.
    // The scheduling barriers keep this order: the compiler would otherwise
    // sink the activation loads below the products and hoist the products'
    // first dequantizations above the wait, leaving the next chunk's copies
    // behind loads an iteration needs at once (in-order counters).
    constexpr int kInFlight = 6 * (NST - 2) + kAOps * (NST - 3);
#pragma unroll
    for (int j = 0; j <= NST - 2; ++j) {
        copy(j, j);
        __builtin_amdgcn_sched_barrier(0);
        if (j <= NST - 3) {
            load_a(j, ac[j], as[j]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    int st = 0;
    // NA iterations per trip, so every activation set index is a constant
    // (chunk i computes with set i % NA and loads chunk i + NA - 1's into set
    // (i + NA - 1) % NA, the one chunk i - 1 used): no register copies
    for (int i0 = 0; i0 < nch; i0 += NA) {
#pragma unroll
        for (int u = 0; u < NA; ++u) {
            const int i = i0 + u;
            if (i >= nch) break;
            // after the barrier every wave's copies of chunk i have landed,
            // and the stage of chunk i - 1 (read in the previous iteration)
            // is free
            __builtin_amdgcn_sched_barrier(0);
            NVFP4_WAIT_VMCNT(kInFlight);
            NVFP4_WAIT_LGKMCNT0();
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            load_a(i + NST - 2, ac[(u + NA - 1) % NA], as[(u + NA - 1) % NA]);
            __builtin_amdgcn_sched_barrier(0);
            copy(i + NST - 1, st == 0 ? NST - 1 : st - 1);
            __builtin_amdgcn_sched_barrier(0);
            compute(st, ac[u], as[u]);
            st = st == NST - 1 ? 0 : st + 1;
        }
    }
    // every wave is done with the ring (and the copies past the end, which
    // write zeros into it, have landed) before it holds the partial tiles:
    // lane's partial C[16 r + 4 g + j][n0 + 16 t + lr] in acc[t][r][j]
    NVFP4_WAIT_VMCNT(0);
    NVFP4_WAIT_LGKMCNT0();
    __builtin_amdgcn_s_barrier();
    if constexpr (kRow1) {
        // lane groups 0 and 1 hold blocks 0-3 and 4-7: their sum is the
        // partial of row 0 (partial tile row 4 g + j = 0: group 0, j = 0)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float o = __shfl_xor(ysum[t], 16);
            acc[t][0] = float4_t{g == 0 ? ysum[t] + o : 0.f, 0.f, 0.f, 0.f};
        }
    }
    float* red = reinterpret_cast<float*>(lds);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int r = 0; r < RMAX; ++r)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                red[(wave * 16 * RMAX + 16 * r + 4 * g + j) * kDlStride + 16 * t + lr] = acc[t][r][j];
    __syncthreads();
    const float sab = kA16 ? *p.b_ts : (*p.a_ts) * (*p.b_ts);
    const int col = threadIdx.x & 63;
    const int64_t n = n0 + col;
    for (int row = threadIdx.x >> 6; row < 16 * RMAX && row < p.M; row += 4) {
        float v = red[row * kDlStride + col] + red[(16 * RMAX + row) * kDlStride + col];
        v += red[(32 * RMAX + row) * kDlStride + col];
        v += red[(48 * RMAX + row) * kDlStride + col];
        v *= sab;
        if (n < p.N) {
            if (p.out_bf16)
                reinterpret_cast<uint16_t*>(p.c)[row * p.ldc + n] = (uint16_t)f32_to_bf16_bits(v);
            else
                reinterpret_cast<float*>(p.c)[row * p.ldc + n] = v;
        }
    }
}

// The dynamic-LDS limit of kernel Kern, raised once per device (not a stream
// operation: repeating it per launch only costs host time, which the short
// decode launches feel, and keeps it out of graph captures after the first
// eager launch).
template <auto Kern>
static void set_lds_limit(int bytes)
{
    static bool done[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = -1;
    if (dev >= 0 && done[dev]) return;
    hipFuncSetAttribute((const void*)Kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (dev >= 0) done[dev] = true;
}

bool gemm_decode_shape(int64_t M, int64_t N, int64_t K)
{
    return M <= 64 && K % 512 == 0 && (uint64_t)N * (uint64_t)K / 2 < (1ull << 31);
}

hipError_t launch_gemm_decode(const GemmParams& p, hipStream_t s)
{
    dim3 g((unsigned)((p.N + kSkN - 1) / kSkN));
#define NVFP4_DECODE_LDS(RMAX, NST, ROW1)                                                      \
    {                                                                                          \
        constexpr auto kern = k_gemm_decode_lds<RMAX, NST, false, ROW1>;                       \
        const int lds = decode_lds_bytes(RMAX, NST);                                           \
        set_lds_limit<kern>(lds);                                                              \
        hipLaunchKernelGGL(kern, g, dim3(256), lds, s, p);                                     \
    }
    if (p.M == 1) NVFP4_DECODE_LDS(1, 3, true)
    else if (p.M <= 16) NVFP4_DECODE_LDS(1, 3, false)
    else if (p.M <= 32) NVFP4_DECODE_LDS(2, 3, false)
    else NVFP4_DECODE_LDS(4, 3, false)
#undef NVFP4_DECODE_LDS
    return hipGetLastError();
}

hipError_t launch_gemm_w4a16(int64_t M, int64_t N, int64_t K, const uint16_t* a, int64_t lda,
                             const GemmOperand& B, bool out_bf16, void* c, int64_t ldc,
                             hipStream_t s)
{
    GemmParams p{};
    p.M = M; p.N = N; p.K = K; p.kp = K;
    p.a_codes = nullptr; p.a_scales = nullptr; p.a_ts = nullptr;
    p.b_codes = B.codes; p.b_scales = B.scales; p.b_ts = B.ts;
    p.c = static_cast<uint8_t*>(c);
    p.ldc = ldc;
    p.a2d = false;
    p.b2d = B.block2d != 0;
    p.out_bf16 = out_bf16;
    p.vec_out = false;
    p.a_bf16 = a;
    p.lda = lda;
    dim3 g((unsigned)((N + 63) / 64));
    // up to 16 rows the weight-streaming kernel (its 16-byte BF16 activation
    // loads are few); with more rows they cost more than the skinny kernel's
    // shared LDS copy of the activations (measured at 32 and 64 rows)
    if (M <= 16) {
        constexpr auto kern = k_gemm_decode_lds<1, 3, true>;
        const int lds = decode_lds_bytes(1, 3);
        set_lds_limit<kern>(lds);
        hipLaunchKernelGGL(kern, g, dim3(256), lds, s, p);
        return hipGetLastError();
    }
#define NVFP4_SKINNY16(RMAX)                                                                   \
    {                                                                                          \
        constexpr auto kern = k_gemm_w4a16<512, RMAX>;                                         \
        const int lds = RMAX * 16 * (512 * 2 + 64);                                            \
        set_lds_limit<kern>(lds);                                                              \
        hipLaunchKernelGGL(kern, g, dim3(256), lds, s, p);                                     \
    }
    if (M <= 32) NVFP4_SKINNY16(2)
    else NVFP4_SKINNY16(4)
#undef NVFP4_SKINNY16
    return hipGetLastError();
}

}  // namespace nvfp4
