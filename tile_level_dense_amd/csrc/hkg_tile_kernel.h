// Large-tile MFMA kernel template for compute-bound shapes: C = A * B^T with
// fp32 accumulation and bf16 out, for bf16 operands and for block-scaled FP8
// (MXFP8: E4M3 operands, one E8M0 scale per 32 k).  hkg_tile.hip instantiates
// the bf16 variants and hkg_tile_mx.hip the MXFP8 ones.
//
// Design (gfx950, MI355X):
//  * One workgroup computes a BM x BN output tile (256 x 256 by default; the
//    HipKittens talk notes, Table 2, show output-tile size dominating BF16
//    GEMM speed on this chip, with all waves doing math and none specialised
//    as producers).
//  * A and B K-slices of 128 bytes per row (64 bf16 or 128 FP8 values) are
//    copied HBM -> LDS by buffer loads that write
//    LDS directly (the "buffer_load ... lds" DMA of the FlyDSL "Prebuilt
//    kernels guide", section 3c), bypassing VGPRs.  Each wave instruction
//    fills 1 KB of LDS contiguously, lane i at byte 16 i, so the bank swizzle
//    is applied on the global address instead (HipKittens talk notes,
//    section 1, asynchronous global loads swizzled on the HBM address).
//  * LDS layout per operand: row r (128 bytes) holds its 16-byte
//    chunk c at position c ^ ((r >> 1) & 7).  A fragment read (ds_read_b128,
//    16 lanes = 16 consecutive rows at one chunk) then touches all 64 banks
//    once per 16-lane phase (64 banks x 4 phases for ds_read_b128: talk
//    notes, section 1, heterogeneous matrix-core shapes).
//  * Two LDS stages; one barrier per K step.  Before the barrier every wave
//    waits for its own DMA (vmcnt) and its LDS reads (lgkmcnt): a direct
//    copy still in flight at a barrier gives wrong results on CDNA4 (hk-dsl
//    page, "The traps it removes").
//  * MFMA v_mfma_f32_16x16x32_bf16 (bf16) or v_mfma_scale_f32_16x16x128_f8f6f4
//    (MXFP8) with the B fragment as the first operand and the A fragment as
//    the second, so each lane ends with four consecutive columns of one row
//    of C (an 8-byte store).
//  * MXFP8 operand layout of the scaled MFMA (measured on gfx950): lane l
//    holds row l % 16 of its 16-row block, k = 16 g .. 16 g + 15 in bytes
//    0-15 and k = 64 + 16 g .. 64 + 16 g + 15 in bytes 16-31 (g = l / 16),
//    i.e. 16-byte chunks g and 4 + g of the row's 128-byte stage: the same
//    two chunks the bf16 path reads for its two 32-k steps.  The scale of
//    row r, 32-k block b is taken from lane 16 b + r (a byte of that lane's
//    scale register chosen by the instruction's op_sel).  Scales come
//    pre-packed so that one dword per lane holds the bytes of four 16-row
//    blocks (byte f = block f of a 64-row group); see mx_pack_kernel.
//  * MXFP4 operand layout of the same instruction with E2M1 operands
//    (measured on gfx950 with one-hot operands and per-lane scales): lane l
//    holds in its first four registers the 32 values of row l % 16, 32-k
//    block g = l / 16 (the last four registers are not read), and that
//    block's scale comes from lane 16 g + r as for MXFP8.  With two E2M1
//    codes per byte, a 128-k step of a row is 64 bytes and the lane's
//    operand is its 16-byte chunk g, so a 256-k stage (128 bytes per row)
//    has exactly the copies, swizzle and fragment reads of a 64-k bf16
//    stage: chunk 4 s + g for step s.  Which code of a chunk pairs with
//    which k inside a block does not matter: A and B are read alike and the
//    block shares one scale.
//  * Workgroup -> tile order: chiplet de-interleave with chunk C and a
//    column-first window of height W (talk notes, section 3, Algorithm 1).
//  * Ragged M, N and K: rows past the matrix and k past K fall outside the
//    buffer resource's range and read as zero; stores are masked.  (MXFP8
//    takes K % 128 == 0; its rows past M or N have zero data and scales.)
#pragma once

#include <type_traits>

#include "hkg_internal.h"
#include "hkg_lds_copy.h"
#include "hkg_store.h"
#include "hkg_tile_order.h"
#include "hkg_tile_kinter.h"
#include "hkg_tile_persistent.h"

namespace hkg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

// gfx9 buffer descriptor word 3 for a raw (unswizzled, stride 0) buffer of
// 32-bit data: out-of-range offsets read as zero.
constexpr int kBufferWord3 = 0x00020000;
// An offset past every range this file creates (ranges are < 2^31 bytes).
constexpr uint32_t kOutOfRange = 0x80000000u;
// Cache-policy operand of buffer loads/stores: sc1, device scope (the
// access is coherent across the XCDs' L2 caches).
constexpr int kDeviceScope = 16;

// Four fp32 values -> four bf16 (nearest-even, v_cvt_pk_bf16_f32) packed in
// two 32-bit words, element r in bits 16 (r % 2) of word r / 2.  Single
// elements are taken out with integer shifts: extracting a lane of a bf16
// vector directly has been seen to store the wrong half.
__device__ __forceinline__ uint2 pack_bf16x4(f32x4 v)
{
    return __builtin_bit_cast(uint2, __builtin_convertvector(v, bf16x4));
}

__device__ __forceinline__ uint16_t bf16_elem(uint2 w, int r)
{
    const uint32_t word = (r >> 1) ? w.y : w.x;
    return (uint16_t)(word >> ((r & 1) * 16));
}

// The 32 bytes of an MXFP8 operand: chunk g (bytes 0-15) and chunk 4 + g.
__device__ __forceinline__ i32x8 mx_operand(bf16x8 lo, bf16x8 hi)
{
    return __builtin_shufflevector(__builtin_bit_cast(i32x4, lo), __builtin_bit_cast(i32x4, hi), 0, 1, 2, 3, 4, 5, 6,
                                   7);
}

// The 16 bytes of an MXFP4 operand (32 E2M1 codes) in the first four
// registers; the instruction does not read the other four.
__device__ __forceinline__ i32x8 fp4_operand(bf16x8 v)
{
    const i32x4 w = __builtin_bit_cast(i32x4, v);
    return i32x8{w[0], w[1], w[2], w[3], 0, 0, 0, 0};
}

// f(integral_constant<int, I>) for I = B .. E - 1: compile-time indices for
// the MFMA's op_sel operands.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

using dma::copy_to_lds;
using dma::rsrc_words;

// Wait until at most N of this wave's buffer->LDS copies are in flight and
// its LDS reads are done, then join the workgroup barrier.
template <int N>
__device__ __forceinline__ void wait_and_barrier()
{
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// `ahead` = stages issued after the one about to be read (0 .. MAXA).
template <int L, int MAXA>
__device__ __forceinline__ void sync_stage(int ahead)
{
    if constexpr (MAXA >= 3) {
        if (ahead >= 3) {
            wait_and_barrier<3 * L>();
            return;
        }
    }
    if constexpr (MAXA >= 2) {
        if (ahead == 2) {
            wait_and_barrier<2 * L>();
            return;
        }
    }
    if constexpr (MAXA >= 1) {
        if (ahead == 1) {
            wait_and_barrier<L>();
            return;
        }
    }
    wait_and_barrier<0>();
}

// MX = false: A, B bf16 (M x K, N x K), BK = 32 or 64.
// MX = true, BK = 128: MXFP8, A, B E4M3 codes, K % 128 == 0; PSA, PSB the
// packed E8M0 scales of A and B (mx_pack_kernel layout).
// MX = true, BK = 256: MXFP4, A, B E2M1 codes two per byte (k even in the
// low nibble; rows of K / 2 bytes), K % 128 == 0, the same packed scales.
// GROUPED = true: the persistent grouped (mixture-of-experts) form, B the
// G x N x K expert weights, offs the G row ends of the experts in A and C.
// Threads of a workgroup: the WM x WN wave grid, twice for schedule 7 (two
// groups, each a WM x WN grid over the whole tile).
template <int WM, int WN, int SCHED>
constexpr int tile_threads() { return WM * WN * 64 * (SCHED == 7 ? 2 : 1); }

template <int BM, int BN, int BK, int STAGES, int WM, int WN, int SCHED, bool EPI, bool MX, bool GROUPED>
__global__ __launch_bounds__(WM * WN * 64 * (SCHED == 7 ? 2 : 1), 2)
void tile_kernel(const void* __restrict__ Av, const void* __restrict__ Bv,
                 uint16_t* __restrict__ C, int M, int N, int K,
                 int tiles_m, int tiles_n, int win_w, int chunk_c,
                 int split_k, float* __restrict__ ws, int* __restrict__ counters,
                 const uint16_t* __restrict__ bias, int epi,
                 const uint32_t* __restrict__ PSA, const uint32_t* __restrict__ PSB,
                 const int* __restrict__ offs, int G, int lda, int ldb, int ldc)
{
    constexpr int NW = WM * WN;
    constexpr bool FP4 = MX && BK == 256;  // MXFP4 (two E2M1 codes per byte)
    constexpr int EB = MX ? 1 : 2;         // bytes per element (MXFP4: per two elements)
    constexpr int KPC = FP4 ? 32 : 16 / EB; // k per 16-byte chunk
    constexpr int RB = FP4 ? BK / 2 : BK * EB; // bytes of one row of a stage
    constexpr int CPR = RB / 16;           // 16-byte chunks per row
    constexpr int RPW = 1024 / RB;         // rows filled by one wave instruction (1 KB)
    constexpr int RPL = 256 / RB;          // rows sharing one 256-byte sweep of the 64 banks
    // 16-byte reads per fragment per stage: bf16 one per 32-k MFMA step,
    // MXFP8 the two halves of one 128-k operand, MXFP4 one per 128-k step.
    constexpr int KS = FP4 ? 2 : MX ? 2 : BK / 32;
    constexpr int SPS = FP4 ? 2 : 1;       // 128-k scale steps per stage (block-scaled)
    constexpr int WTM = BM / WM;           // rows of C per wave
    constexpr int WTN = BN / WN;           // columns of C per wave
    constexpr int FM = WTM / 16;
    constexpr int FN = WTN / 16;
    constexpr int A_BYTES = BM * RB;
    constexpr int B_BYTES = BN * RB;
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int A_LOADS = BM / (RPW * NW);
    constexpr int B_LOADS = BN / (RPW * NW);
    constexpr int L = A_LOADS + B_LOADS;   // copies per wave per stage
    static_assert(MX ? (BK == 128 || BK == 256) : (BK == 32 || BK == 64),
                  "stage k: 32 or 64 (bf16), 128 (MXFP8), 256 (MXFP4)");
    static_assert(!MX || SCHED == 0 || SCHED == 5, "block-scaled: schedules 0 and 5");
    static_assert(SCHED <= 2 || (SCHED >= 5 && SCHED <= 7), "schedules 0, 1, 2, 5, 6 and 7");
    static_assert(SCHED != 7 || (!MX && !GROUPED && BK == 64 && (STAGES == 3 || STAGES == 5)),
                  "schedule 7: bf16 tiles, 3 or 5 stages of 64 k");
    static_assert(!MX || (WTM % 64 == 0 && WTN % 64 == 0), "block-scaled: wave tiles of whole 64-row scale groups");
    static_assert(STAGES >= 2 && STAGES <= 5, "2 to 5 stages");
    static_assert(BM % (RPW * NW) == 0 && BN % (RPW * NW) == 0, "tile rows must split over waves");
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be whole 16x16 blocks");
    // SCHED 5 (and 6, its persistent form) keeps A halves double-buffered and
    // B triple-buffered.
    constexpr bool PINGPONG = SCHED == 5 || SCHED == 6;
    constexpr int SMEM = PINGPONG ? 4 * (BM / 2) * RB + 3 * B_BYTES : STAGES * STAGE;
    static_assert(SMEM <= 160 * 1024, "LDS is 160 KiB per CU");
    static_assert((STAGES - 2) * L <= 63, "vmcnt holds at most 63");

    __shared__ __attribute__((aligned(1024))) char smem[SMEM];

    // SCHED 6: the persistent ping-pong (one workgroup per compute unit
    // walking several tiles or grouped items, hkg_tile_persistent.h); with a
    // fused epilogue, which stages through LDS, the one-tile ping-pong below.
    if constexpr (SCHED == 6 && !EPI && !MX) {
        pingpong_persistent<WM, WN, GROUPED>(Av, Bv, C, M, N, K, tiles_m, tiles_n, win_w, chunk_c, lda, ldb, ldc,
                                             smem, offs, G, split_k, ws, counters);
        return;
    }
    // SCHED 7: the k-interleaved ping-pong (hkg_tile_kinter.h), K not split.
    if constexpr (SCHED == 7) {
        pingpong_kinter<BM, BN, WM, WN, STAGES, EPI>(Av, Bv, C, M, N, K, tiles_m, tiles_n, win_w, chunk_c, lda, ldb,
                                                     ldc, smem, bias, epi);
        return;
    }

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN;
    const int wn = wave - wm * WN;

    // Bytes of k elements of a row.
    auto kbytes = [](int k) { return FP4 ? (uint32_t)k / 2u : (uint32_t)k * (uint32_t)EB; };
    // Row strides in bytes (leading dimensions); block-scaled and grouped
    // launches use dense operands, so there both operands share one stride.
    const uint32_t a_rb = kbytes(lda);
    const uint32_t b_rb = (MX || GROUPED) ? a_rb : kbytes(ldb);
    __shared__ int last_flag;               // split-K: this workgroup arrived last

    // One output tile: C rows [m0, min(m0 + BM, m_lim)) by columns
    // [tn BN, tn BN + BN), from A rows m0.. and rows tn BN.. of b_rows (the
    // tile's N x K operand; an expert's weight in grouped mode), with bias_t
    // the bias row of that operand, over part k_part of k_parts equal parts of
    // K.  tm, tn index split-K's arrival counters (dense mode); in grouped mode
    // a tile split in two (k_parts = 2) is unit `unit` of the last round, whose
    // partial goes to slot `unit` of ws and whose arrivals are counted at
    // counters[unit / 2].
    auto run_tile = [&](int tm, int tn, int m0, int m_lim, const char* b_rows, const uint16_t* bias_t, int k_part,
                        int k_parts, int unit) {
        (void)unit;
        (void)tm;
        // In the persistent loop the lane-derived offsets are recomputed per
        // tile (an opaque copy of the lane id) rather than kept live across
        // tiles beside the accumulators.
        int lane = threadIdx.x & 63;
        if constexpr (GROUPED)
            asm volatile("" : "+v"(lane));
        const int n0 = tn * BN;
        const int rows_a = min(BM, m_lim - m0);
        const int rows_b = min(BN, N - n0);

        const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
            (void*)((const char*)Av + (size_t)m0 * a_rb), 0, (int)(rows_a * a_rb), kBufferWord3);
        const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(b_rows + (size_t)n0 * b_rb), 0, (int)(rows_b * b_rb), kBufferWord3);
        const i32x4 words_a = rsrc_words((const char*)Av + (size_t)m0 * a_rb, (int)(rows_a * a_rb));
        const i32x4 words_b = rsrc_words(b_rows + (size_t)n0 * b_rb, (int)(rows_b * b_rb));

        // LDS layout of a stage: row r holds its logical 16-byte chunk c at
        // position c ^ ((r / RPL) % CPR).  Sixteen consecutive rows read at one
        // logical chunk then hit sixteen distinct 16-byte bank groups.
        //
        // DMA sources of this lane.  Wave instruction i of the A copy fills LDS
        // rows RPW g .. RPW g + RPW - 1 (g = wave + i NW); lane -> row
        // RPW g + lane / CPR, position lane % CPR, which holds logical chunk
        // (lane % CPR) ^ swizzle(row): the swizzle is applied to the source.
        // Consecutive copies of a wave are NW * RPW rows apart, a multiple of
        // RPL * CPR, so the swizzle (and the lane's chunk) is the same for all
        // of them: one base offset per operand, plus a uniform row step.
        static_assert((NW * RPW / RPL) % CPR == 0, "swizzle must repeat across a wave's copies");
        constexpr int COPY_ROWS = NW * RPW;
        const int lrow0 = wave * RPW + lane / CPR;
        const int lchunk = (lane % CPR) ^ ((lrow0 / RPL) % CPR);
        const uint32_t src_off_a = (uint32_t)lrow0 * a_rb + (uint32_t)lchunk * 16u;
        const uint32_t src_off_b = (uint32_t)lrow0 * b_rb + (uint32_t)lchunk * 16u;
        const int src_k = lchunk * KPC;
        const uint32_t copy_step_a = (uint32_t)COPY_ROWS * a_rb;
        const uint32_t copy_step_b = (uint32_t)COPY_ROWS * b_rb;

        // K range of this workgroup: stages [kt0, kt0 + nk) of BK k, part
        // k_part of k_parts (dense split-K: blockIdx.y of split_k).
        const int nk_all = (K + BK - 1) / BK;
        const int per_split = (nk_all + k_parts - 1) / k_parts;
        const int kt0 = min(nk_all, k_part * per_split);
        const int nk = min(nk_all, kt0 + per_split) - kt0;
        const int kbase = kt0 * BK;
        const int k_lim = min(K, (kt0 + nk) * BK);

        auto issue = [&](int stage, int kl) {
            char* base = smem + stage * STAGE;
            const int k0 = kbase + kl;
            const bool k_out = k0 + src_k >= k_lim;  // this lane's chunk past the range
            const uint32_t koff = kbytes(k0);
    #pragma unroll
            for (int i = 0; i < A_LOADS; ++i)
                copy_to_lds(words_a, base + (wave + i * NW) * 1024,
                            k_out ? kOutOfRange : src_off_a + koff + (uint32_t)i * copy_step_a);
    #pragma unroll
            for (int i = 0; i < B_LOADS; ++i)
                copy_to_lds(words_b, base + A_BYTES + (wave + i * NW) * 1024,
                            k_out ? kOutOfRange : src_off_b + koff + (uint32_t)i * copy_step_b);
        };

        // Fragment reads: lane -> row (lane % 16) of a 16-row block, logical
        // chunk 4 s + lane / 16 for read s (bf16: 8 k of the 32-k step s; MXFP8:
        // the two 16-byte halves of the lane's operand).  Every block starts at
        // a multiple of 16 rows, so the swizzle depends on lane only.
        const int lrow = lane & 15;
        const int lgrp = lane >> 4;
        const int swz = (lrow / RPL) % CPR;
        int chunk_off[KS];
    #pragma unroll
        for (int s = 0; s < KS; ++s)
            chunk_off[s] = ((4 * s + lgrp) ^ swz) * 16;
        const int a_frag = (wm * WTM + lrow) * RB;
        const int b_frag = A_BYTES + (wn * WTN + lrow) * RB;

        f32x4 acc[FM][FN];
    #pragma unroll
        for (int i = 0; i < FM; ++i)
    #pragma unroll
            for (int j = 0; j < FN; ++j)
                acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        auto read_frags = [&](const char* base, int s, bf16x8 (&af)[FM], bf16x8 (&bf)[FN]) {
    #pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *(const bf16x8*)(base + a_frag + i * 16 * RB + chunk_off[s]);
    #pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[j] = *(const bf16x8*)(base + b_frag + j * 16 * RB + chunk_off[s]);
        };
        auto mfmas = [&](const bf16x8 (&af)[FM], const bf16x8 (&bf)[FN]) {
    #pragma unroll
            for (int i = 0; i < FM; ++i)
    #pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
        };

        // Block scales.  Packed layout (mx_pack_kernel): for 64-row group R and
        // 128-k step kt, dword R * KT * 64 + kt * 64 + lane holds in byte f the
        // scale of row 64 R + 16 f + lane % 16, block 4 kt + lane / 16: this
        // lane's scale operand for 16-row block f of the group.  A wave's rows
        // are SWA (B: SWB) whole groups; one dword load per group per 128-k
        // step (SPS steps per stage).
        constexpr int SWA = MX ? WTM / 64 : 1;
        constexpr int SWB = MX ? WTN / 64 : 1;
        const int KT = K / 128;
        const __amdgpu_buffer_rsrc_t rsrc_sa = __builtin_amdgcn_make_buffer_rsrc(
            (void*)PSA, 0, MX ? ((M + 63) / 64) * KT * 256 : 0, kBufferWord3);
        const __amdgpu_buffer_rsrc_t rsrc_sb = __builtin_amdgcn_make_buffer_rsrc(
            (void*)PSB, 0, MX ? ((N + 63) / 64) * KT * 256 : 0, kBufferWord3);
        const uint32_t sa_off0 = (uint32_t)(((m0 + wm * WTM) / 64) * KT) * 256u + (uint32_t)lane * 4u;
        const uint32_t sb_off0 = (uint32_t)(((n0 + wn * WTN) / 64) * KT) * 256u + (uint32_t)lane * 4u;
        uint32_t sa_cur[SPS][SWA], sb_cur[SPS][SWB], sa_nxt[SPS][SWA], sb_nxt[SPS][SWB];
        // Scales of local stage t into the *_nxt registers (t past this
        // workgroup's range reads the next split's or out-of-range zeros; such
        // values are never used).  An MXFP4 128-k step past K (the empty half
        // of a last 256-k stage, whose data are zero-filled) reads through an
        // empty descriptor (the choice is uniform across the wave, so it
        // costs no vector register), so it gets code 0 (the finite scale
        // 2^-127) and never the next row group's scales, which may hold NaN
        // codes.
        const __amdgpu_buffer_rsrc_t rsrc_none = __builtin_amdgcn_make_buffer_rsrc((void*)PSA, 0, 0, kBufferWord3);
        auto load_scales = [&](int t) {
            if constexpr (MX) {
    #pragma unroll
                for (int q = 0; q < SPS; ++q) {
                    const int step = (kt0 + t) * SPS + q;
                    const uint32_t st = (uint32_t)step * 256u;
                    const bool past = FP4 && q > 0 && step >= KT;
    #pragma unroll
                    for (int r = 0; r < SWA; ++r)
                        sa_nxt[q][r] = __builtin_amdgcn_raw_buffer_load_b32(
                            past ? rsrc_none : rsrc_sa, sa_off0 + (uint32_t)(r * KT) * 256u + st, 0, 0);
    #pragma unroll
                    for (int r = 0; r < SWB; ++r)
                        sb_nxt[q][r] = __builtin_amdgcn_raw_buffer_load_b32(
                            past ? rsrc_none : rsrc_sb, sb_off0 + (uint32_t)(r * KT) * 256u + st, 0, 0);
                }
            }
        };
        auto take_scales = [&]() {
            if constexpr (MX) {
    #pragma unroll
                for (int q = 0; q < SPS; ++q) {
    #pragma unroll
                    for (int r = 0; r < SWA; ++r)
                        sa_cur[q][r] = sa_nxt[q][r];
    #pragma unroll
                    for (int r = 0; r < SWB; ++r)
                        sb_cur[q][r] = sb_nxt[q][r];
                }
            }
        };
        // One 128-k stage of MXFP8 MFMAs: halves lo (chunk g) and hi (chunk 4 + g).
        auto mfmas_mx = [&](const bf16x8 (&alo)[FM], const bf16x8 (&ahi)[FM], const bf16x8 (&blo)[FN],
                            const bf16x8 (&bhi)[FN]) {
            static_for<0, FM>([&](auto I) {
                constexpr int i = decltype(I)::value;
                const i32x8 av = mx_operand(alo[i], ahi[i]);
                static_for<0, FN>([&](auto J) {
                    constexpr int j = decltype(J)::value;
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        mx_operand(blo[j], bhi[j]), av, acc[i][j], 0, 0, j % 4, (int)sb_cur[0][j / 4], i % 4,
                        (int)sa_cur[0][i / 4]);
                });
            });
        };
        // One 128-k MXFP4 step q (format code 4, E2M1, for both operands).
        auto mfmas_fp4 = [&](auto Q, const bf16x8 (&af)[FM], const bf16x8 (&bf)[FN]) {
            constexpr int q = decltype(Q)::value;
            static_for<0, FM>([&](auto I) {
                constexpr int i = decltype(I)::value;
                const i32x8 av = fp4_operand(af[i]);
                static_for<0, FN>([&](auto J) {
                    constexpr int j = decltype(J)::value;
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        fp4_operand(bf[j]), av, acc[i][j], 4, 4, j % 4, (int)sb_cur[q][j / 4], i % 4,
                        (int)sa_cur[q][i / 4]);
                });
            });
        };

        auto compute = [&](int stage) {
            const char* base = smem + stage * STAGE;
            if constexpr (FP4) {
                bf16x8 af[KS][FM], bf[KS][FN];
    #pragma unroll
                for (int q = 0; q < KS; ++q)
                    read_frags(base, q, af[q], bf[q]);
                static_for<0, KS>([&](auto Q) { mfmas_fp4(Q, af[decltype(Q)::value], bf[decltype(Q)::value]); });
            } else if constexpr (MX) {
                bf16x8 alo[FM], blo[FN], ahi[FM], bhi[FN];
                read_frags(base, 0, alo, blo);
                read_frags(base, 1, ahi, bhi);
                mfmas_mx(alo, ahi, blo, bhi);
            } else if constexpr (SCHED == 0) {
    #pragma unroll
                for (int s = 0; s < KS; ++s) {
                    bf16x8 af[FM], bf[FN];
                    read_frags(base, s, af, bf);
                    mfmas(af, bf);
                }
            } else {
                // Fragments of step s + 1 are read while the MFMAs of step s run:
                // one LDS read between every few MFMAs, so each read has many
                // MFMA cycles to land before its first use.
                bf16x8 af[2][FM], bf[2][FN];
                read_frags(base, 0, af[0], bf[0]);
    #pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const int cur = s & 1;
                    if (s + 1 < KS)
                        read_frags(base, s + 1, af[cur ^ 1], bf[cur ^ 1]);
                    mfmas(af[cur], bf[cur]);
                }
                if constexpr (KS > 1) {
                    constexpr int READS = FM + FN;
                    constexpr int MF = FM * FN;
                    constexpr int PER = MF / READS > 0 ? MF / READS : 1;
                    // first step: its reads were issued above the loop
                    __builtin_amdgcn_sched_group_barrier(0x100, READS, 0);
    #pragma unroll
                    for (int r = 0; r < READS; ++r) {
                        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x008, PER, 0);
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, MF - PER * READS, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, MF, 0);
                }
            }
        };

        if constexpr (SCHED < 2) {
            // K loop over a ring of STAGES buffers, prefetch distance STAGES - 1.
            // At step t: this wave's copy of stage t has landed (vmcnt allows the
            // later stages still in flight), all waves finished reading step t - 1
            // (lgkmcnt + barrier), so buffer (t - 1) % STAGES is refilled with step
            // t + STAGES - 1 while step t is computed.
            // Block-scaled (two stages only): the scales of step t + 1 are loaded
            // just before its copies, so the wait at the top of step t + 1 covers
            // them.
            static_assert(!MX || STAGES == 2, "block-scaled ring: two stages");
            load_scales(0);
    #pragma unroll
            for (int s = 0; s < STAGES - 1; ++s)
                if (s < nk)
                    issue(s, s * BK);
            int read_stage = 0;
            int write_stage = STAGES - 1;
            for (int t = 0; t < nk; ++t) {
                sync_stage<L, STAGES - 2>(min(STAGES - 2, nk - 1 - t));
                take_scales();
                load_scales(t + 1);
                if (t + STAGES - 1 < nk)
                    issue(write_stage, (t + STAGES - 1) * BK);
                compute(read_stage);
                read_stage = read_stage + 1 == STAGES ? 0 : read_stage + 1;
                write_stage = write_stage + 1 == STAGES ? 0 : write_stage + 1;
            }
        } else if constexpr (SCHED == 2 && !MX) {
            // Register-pipelined loop.  Work proceeds in 32-k steps; the
            // fragments of step u + 1 are read from LDS while the MFMAs of step u
            // run.  Before the first read of a new stage every wave waits for its
            // own reads of the previous stage (now in registers) and for its copy
            // of the new stage, then joins the barrier: the previous stage's
            // buffer is then free and is refilled right away with the stage
            // STAGES ahead.  Copies past the end of K are issued with
            // out-of-range offsets (they fill a buffer nobody reads), so the
            // number of copies in flight, and with it every wait count, is the
            // same on every step: the loop body has no branch around LDS reads,
            // copies or waits.
            constexpr int READS = FM + FN;
            constexpr int MF = FM * FN;
            static_assert(MF >= READS, "one MFMA per fragment read at least");
            auto interleave = [&]() {
    #pragma unroll
                for (int r = 0; r < READS; ++r) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                }
                __builtin_amdgcn_sched_group_barrier(0x008, MF - READS, 0);
            };
            auto stage_base = [&](int t) { return smem + (t % STAGES) * STAGE; };
            auto new_stage = [&](int t) {      // about to read stage t + 1
                wait_and_barrier<(STAGES - 2) * L>();
                issue(t % STAGES, (t + STAGES) * BK);
            };
    #pragma unroll
            for (int s = 0; s < STAGES; ++s)
                issue(s, s * BK);
            wait_and_barrier<(STAGES - 1) * L>();
            bf16x8 af0[FM], bf0[FN], af1[FM], bf1[FN];
            read_frags(smem, 0, af0, bf0);
            static_assert(KS == 2, "the register-pipelined loop takes 64-k stages");
            for (int t = 0; t < nk; ++t) {
                mfmas(af0, bf0);
                read_frags(stage_base(t), 1, af1, bf1);
                interleave();
                new_stage(t);
                mfmas(af1, bf1);
                read_frags(stage_base(t + 1), 0, af0, bf0);
                interleave();
            }
            // Leave no copy in flight into LDS that is about to be released.
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        } else if constexpr (PINGPONG) {
            // Ping-pong (HipKittens talk notes, section 2, 8-wave schedule).
            // Waves 0-3 (group 0) and 4-7 (group 1) put one wave on each SIMD
            // and alternate a memory phase (LDS fragment reads of a whole
            // stage, plus copies) with a compute phase (the stage's MFMAs),
            // phases separated by workgroup barriers.  Group 1 joins one extra
            // barrier at the start, so the groups run half a stage apart and
            // each SIMD's matrix unit is fed by one wave while the other reads.
            // Every copy is issued in a memory phase: a copy that the vector
            // memory path cannot take yet stalls its wave, and in a compute
            // phase that would stall the MFMAs too.  That needs these buffer
            // lifetimes: group g alone reads A rows 128 g .. 128 g + 127
            // (double-buffered per group), both groups read B (triple-
            // buffered); 160 KiB of LDS in all.
            // Phase j lies between barriers j and j + 1; group 0 reads stage t
            // in phase 2t and computes it in 2t + 1, group 1 reads it in
            // 2t + 1 and computes it in 2t + 2.  Copies, A first:
            //   group 0, phase 2t:     A rows 0-127 of stage t + 1, B rows
            //                          0-127 of stage t + 2
            //   group 1, phase 2t + 1: A rows 128-255 of stage t + 1, B rows
            //                          128-255 of stage t + 2
            // Each lands in a buffer whose last reader finished before the
            // phase began.  A wave waits for its A copies at the end of its
            // next compute phase and for its B copies one memory phase later
            // (group 1) or one compute phase later (group 0): in every case
            // before the first phase that reads them.
            // Block-scaled: each memory phase starts by taking the scales loaded
            // at the start of the previous one (landed: the waits since then
            // cover them) and loading the next stage's ahead of its copies, so no
            // wait for scales ever holds back a copy issued after them;
            // 2 SPS (SWA + SWB) VGPRs.
            static_assert(BM == 256 && BN == 256 && RB == 128 && NW == 8 && WM <= 4,
                          "split-buffer ping-pong: 256 x 256 tile of 128-byte rows, 8 waves");
            constexpr int HALF = 128 * RB;                  // 128 rows of one stage
            constexpr int CPW = 128 / (RPW * 4);            // copies per half per wave
            char* const a_buf = smem;                       // [group][stage % 2]
            char* const b_buf = smem + 4 * HALF;            // [stage % 3]: rows 0-255
            const int g = wave >> 2;
            const int w4 = wave & 3;
            // DMA source of this lane within a 128-row half (same swizzle rule
            // as the copies above; a group's 4 waves fill 32 rows per round).
            const int prow = w4 * RPW + lane / CPR;
            const int pchunk = (lane % CPR) ^ ((prow / RPL) % CPR);
            const uint32_t p_off_a = (uint32_t)(128 * g + prow) * a_rb + (uint32_t)pchunk * 16u;
            const uint32_t p_off_b = (uint32_t)(128 * g + prow) * b_rb + (uint32_t)pchunk * 16u;
            const int p_k = pchunk * KPC;
            static_assert((4 * RPW / RPL) % CPR == 0, "swizzle must repeat across a group's copies");
            // Grouped mode recomputes the lane-derived offsets at each use from
            // an opaque copy of the lane id, so they are not held in registers
            // through the compute phases (the persistent loop's state needs
            // those registers).
            // (unsigned: the divisions below by powers of two are then plain
            // shifts and masks, with no sign corrections)
            auto fresh_lane = [&]() {
                uint32_t l = threadIdx.x & 63u;
                asm volatile("" : "+v"(l));
                return l;
            };
            auto copy_half = [&](__amdgpu_buffer_rsrc_t rsrc, char* dst, int t, uint32_t p_off, uint32_t rb) {
                int pk = p_k;
                if constexpr (GROUPED) {
                    const uint32_t l = fresh_lane();
                    const uint32_t row = (uint32_t)(w4 * RPW) + l / CPR;
                    const uint32_t ch = (l % CPR) ^ ((row / RPL) % CPR);
                    p_off = ((uint32_t)(128 * g) + row) * rb + ch * 16u;
                    pk = (int)(ch * KPC);
                }
                const int k0 = kbase + t * BK;
                const bool k_out = k0 + pk >= k_lim;
                const uint32_t off0 = k_out ? kOutOfRange : p_off + kbytes(k0);
                const uint32_t p_step = (uint32_t)(4 * RPW) * rb;
    #pragma unroll
                for (int i = 0; i < CPW; ++i)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void*)(dst + (w4 + 4 * i) * 1024), 16,
                                                             k_out ? kOutOfRange : off0 + (uint32_t)i * p_step, 0,
                                                             0, 0);
            };
            auto copy_a = [&](int t) { copy_half(rsrc_a, a_buf + (2 * g + (t & 1)) * HALF, t, p_off_a, a_rb); };
            auto copy_b = [&](int t) { copy_half(rsrc_b, b_buf + (t % 3) * 2 * HALF + g * HALF, t, p_off_b, b_rb); };
            const int a_row = wm * WTM - 128 * g + lrow;    // row within the group's A half
            const int b_row = wn * WTN + lrow;
            bf16x8 af[KS][FM], bf[KS][FN];
            auto read_stage = [&](int t) {
                int ar = a_row, br = b_row;
                int co[KS];
    #pragma unroll
                for (int s = 0; s < KS; ++s)
                    co[s] = chunk_off[s];
                if constexpr (GROUPED) {
                    const uint32_t l = fresh_lane();
                    const uint32_t lr = l & 15u;
                    ar = wm * WTM - 128 * g + (int)lr;
                    br = wn * WTN + (int)lr;
    #pragma unroll
                    for (int s = 0; s < KS; ++s)
                        co[s] = (int)((((uint32_t)(4 * s) + (l >> 4)) ^ ((lr / RPL) % CPR)) * 16u);
                }
                const char* ab = a_buf + (2 * g + (t & 1)) * HALF + ar * RB;
                const char* bb = b_buf + (t % 3) * 2 * HALF + br * RB;
    #pragma unroll
                for (int s = 0; s < KS; ++s) {
    #pragma unroll
                    for (int i = 0; i < FM; ++i)
                        af[s][i] = *(const bf16x8*)(ab + i * 16 * RB + co[s]);
    #pragma unroll
                    for (int j = 0; j < FN; ++j)
                        bf[s][j] = *(const bf16x8*)(bb + j * 16 * RB + co[s]);
                }
            };
            auto mfma_stage = [&]() {
                if constexpr (FP4) {
                    static_for<0, KS>([&](auto Q) { mfmas_fp4(Q, af[decltype(Q)::value], bf[decltype(Q)::value]); });
                } else if constexpr (MX) {
                    mfmas_mx(af[0], af[1], bf[0], bf[1]);
                } else {
    #pragma unroll
                    for (int s = 0; s < KS; ++s)
                        mfmas(af[s], bf[s]);
                }
            };
            auto memory_phase_scales = [&](int t) {
                take_scales();
                load_scales(t + 1);
            };
            auto fence = [&]() { __builtin_amdgcn_sched_barrier(0); };
            auto phase_barrier = [&]() {
                fence();
                asm volatile("s_barrier" ::: "memory");
                fence();
            };
            const bool g1 = g == 1;

            // Prologue: stage 0, and this group's B rows of stage 1.
            load_scales(0);
            copy_a(0);
            copy_b(0);
            copy_b(1);
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CPW) : "memory");
            phase_barrier();
            if (!g1) {
                for (int t = 0; t < nk; ++t) {
                    memory_phase_scales(t);        // phase 2t: memory
                    read_stage(t);
                    fence();
                    copy_a(t + 1);
                    copy_b(t + 2);
                    fence();
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                    phase_barrier();
                    mfma_stage();                  // phase 2t + 1: compute
                    fence();
                    // all but this phase's B copies: A of stage t + 1 and the
                    // B rows of stage t + 1 copied a memory phase earlier
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CPW) : "memory");
                    phase_barrier();
                }
            } else {
                phase_barrier();                   // phase 0: group 0 reads stage 0
                for (int t = 0; t < nk; ++t) {
                    memory_phase_scales(t);        // phase 2t + 1: memory
                    read_stage(t);
                    fence();
                    copy_a(t + 1);
                    copy_b(t + 2);
                    fence();
                    // B rows of stage t + 1 (copied a memory phase earlier)
                    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(2 * CPW) : "memory");
                    phase_barrier();
                    mfma_stage();                  // phase 2t + 2: compute
                    fence();
                    // A of stage t + 1
                    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CPW) : "memory");
                    if (t + 1 < nk)
                        phase_barrier();
                }
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }

        if constexpr (!GROUPED && tile_split_capable(BM, BN, WM, WN, SCHED)) if (split_k > 1) {
            // Split-K: each workgroup writes its fp32 partial tile; the last one
            // of the tile to arrive adds the partials in split order 0, 1, ...
            // (the same order whichever split arrives last, so results are
            // deterministic) and goes on to the rounding store below.  Partials
            // are written and read with device-scope (sc1) accesses, which are
            // coherent across the XCDs' L2 caches without flushing them; every
            // store has completed (vmcnt) before the arrival is counted (the
            // ordering argument is the split-K arrival protocol in
            // hkg_internal.h).
            const int me = k_part;
            const bool vec4 = (N & 3) == 0;
            const int part_bytes = M * N * 4;          // below 2^31: checked by the planner
            auto part = [&](int sp) { return ws + (size_t)sp * (size_t)M * (size_t)N; };
            {
                const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(part(me), 0, part_bytes, kBufferWord3);
    #pragma unroll
                for (int i = 0; i < FM; ++i) {
                    const int m = m0 + wm * WTM + i * 16 + lrow;
                    if (m >= M)
                        continue;
    #pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const int n = n0 + wn * WTN + j * 16 + lgrp * 4;
                        if (vec4 && n + 3 < N) {
                            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), r,
                                                                   (m * N + n) * 4, 0, kDeviceScope);
                        } else {
    #pragma unroll
                            for (int q = 0; q < 4; ++q)
                                if (n + q < N)
                                    __hip_atomic_store(part(me) + (size_t)m * N + n + q, acc[i][j][q], __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
                        }
                    }
                }
            }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            const int tile = tm * tiles_n + tn;
            if (threadIdx.x == 0) {
                const int prev = __hip_atomic_fetch_add(&counters[tile], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                last_flag = (prev == split_k - 1);
            }
            __syncthreads();
            if (!last_flag)
                return;
            // Sums are formed GR block rows at a time (at most 64 registers of
            // running totals beside the accumulators).
            constexpr int GR = FN >= 16 ? 1 : 16 / FN;
    #pragma unroll
            for (int g = 0; g < FM; g += GR) {
                f32x4 tot[GR][FN];
                for (int sp = 0; sp < split_k; ++sp) {
                    const __amdgpu_buffer_rsrc_t r =
                        __builtin_amdgcn_make_buffer_rsrc(part(sp), 0, part_bytes, kBufferWord3);
    #pragma unroll
                    for (int ii = 0; ii < GR; ++ii) {
                        const int i = g + ii;
                        if (i >= FM)
                            break;
                        const int m = m0 + wm * WTM + i * 16 + lrow;
    #pragma unroll
                        for (int j = 0; j < FN; ++j) {
                            const int n = n0 + wn * WTN + j * 16 + lgrp * 4;
                            f32x4 v = acc[i][j];           // this split's own partial
                            if (sp != me && m < M) {
                                if (vec4 && n + 3 < N) {
                                    v = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                                      r, (m * N + n) * 4, 0, kDeviceScope));
                                } else {
    #pragma unroll
                                    for (int q = 0; q < 4; ++q)
                                        v[q] = n + q < N ? __hip_atomic_load(part(sp) + (size_t)m * N + n + q,
                                                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                                         : 0.f;
                                }
                            }
                            tot[ii][j] = sp == 0 ? v : tot[ii][j] + v;
                        }
                    }
                }
    #pragma unroll
                for (int ii = 0; ii < GR; ++ii)
    #pragma unroll
                    for (int j = 0; j < FN; ++j)
                        if (g + ii < FM)
                            acc[g + ii][j] = tot[ii][j];
            }
            if (threadIdx.x == 0)
                __hip_atomic_store(&counters[tile], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }

        if constexpr (GROUPED) if (k_parts == 2) {
            // A tile of the last round split in two halves of K: each half
            // writes its whole fp32 accumulator tile to its own slot (device-
            // scope stores, fragment-major: block (i, j) of wave w fills 1 KiB
            // at ((w FM + i) FN + j) KiB, lane l's four values at 16 l, so each
            // instruction writes 1 KiB contiguously), and the half that
            // arrives second adds the other's partial to its own and goes on
            // to the store.  fp32 addition is commutative, so the sum is the
            // same whichever half arrives second.  The ordering argument is the
            // split-K arrival protocol in hkg_internal.h.
            constexpr int SLOT = BM * BN;
            const __amdgpu_buffer_rsrc_t mine =
                __builtin_amdgcn_make_buffer_rsrc(ws + (size_t)unit * SLOT, 0, SLOT * 4, kBufferWord3);
    #pragma unroll
            for (int i = 0; i < FM; ++i)
    #pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int off = ((wave * FM + i) * FN + j) * 1024 + lane * 16;
                    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), mine, off, 0,
                                                           kDeviceScope);
                }
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            // Every wave is past its last read of the stages: the first word
            // of LDS carries the arrival result (the ping-pong's stages take
            // all 160 KiB, so no separate flag is allocated).
            __syncthreads();
            int* const arrived = (int*)smem;
            if (threadIdx.x == 0)
                *arrived = __hip_atomic_fetch_add(&counters[unit >> 1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __syncthreads();
            if (*arrived != 1)
                return;
            const __amdgpu_buffer_rsrc_t other =
                __builtin_amdgcn_make_buffer_rsrc(ws + (size_t)(unit ^ 1) * SLOT, 0, SLOT * 4, kBufferWord3);
            // RBLK block rows at a time (at most 16 loads, 64 VGPRs, in flight
            // beside the accumulators); each sum is formed here (the empty asm
            // keeps the compiler from sinking the additions into the store
            // branches, which would keep every loaded partial live until then).
            constexpr int RBLK = FN >= 16 ? 1 : (16 / FN < FM ? 16 / FN : FM);
            static_assert(FM % RBLK == 0, "whole groups of block rows");
    #pragma unroll
            for (int i0 = 0; i0 < FM; i0 += RBLK) {
                __builtin_amdgcn_sched_barrier(0);
                f32x4 o[RBLK][FN];
    #pragma unroll
                for (int ii = 0; ii < RBLK; ++ii)
    #pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        const int off = ((wave * FM + i0 + ii) * FN + j) * 1024 + lane * 16;
                        o[ii][j] = __builtin_bit_cast(
                            f32x4, __builtin_amdgcn_raw_buffer_load_b128(other, off, 0, kDeviceScope));
                    }
    #pragma unroll
                for (int ii = 0; ii < RBLK; ++ii)
    #pragma unroll
                    for (int j = 0; j < FN; ++j) {
                        acc[i0 + ii][j] += o[ii][j];
                        asm volatile("" : "+v"(acc[i0 + ii][j]));
                    }
            }
            if (threadIdx.x == 0)
                __hip_atomic_store(&counters[unit >> 1], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }

        const bool vec_ok = ((N | ldc) & 3) == 0;           // 8-byte stores of four columns
        if constexpr (EPI) {
            // Fused epilogue (bias, activation) through LDS: each wave writes
            // its fp32 accumulators, CH block rows at a time, into its own LDS
            // region (rows padded by 16 bytes so the 16 rows of a block land on
            // distinct banks), then walks the region four columns per lane in
            // row order, applying bias and activation once per element (one
            // copy of the activation code instead of one per accumulator
            // register) and storing bf16 rows.
            constexpr int REGION = SMEM / NW;               // bytes per wave
            constexpr int ROWB = WTN * 4 + 16;              // padded fp32 row of a wave tile
            constexpr int CH0 = REGION / (16 * ROWB);       // block rows that fit
            constexpr int CH = CH0 >= FM ? FM : (CH0 >= 8 ? 8 : (CH0 >= 4 ? 4 : (CH0 >= 2 ? 2 : 1)));
            constexpr int QPR = WTN / 4;                    // four-column groups per row
            static_assert(CH0 >= 1 && FM % CH == 0, "epilogue staging needs a block row of LDS per wave");
            // When 64 lanes cover whole rows of the walk (QPR divides 64), a
            // lane's four columns are the same on every row: their bias
            // values are read once, before the barrier; otherwise (48-column
            // wave tiles) per element.
            constexpr bool HOIST = 64 % QPR == 0;
            const int ncol = n0 + wn * WTN + (lane % QPR) * 4;
            float bv[4];
    #pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                bv[rr] = HOIST && ncol + rr < N ? __uint_as_float((uint32_t)bias_t[ncol + rr] << 16) : 0.f;
            __syncthreads();                                // every wave is done with the stages
            char* const wbuf = smem + wave * REGION;
    #pragma unroll
            for (int c = 0; c < FM; c += CH) {
    #pragma unroll
                for (int ii = 0; ii < CH; ++ii)
    #pragma unroll
                    for (int j = 0; j < FN; ++j)
                        *(f32x4*)(wbuf + (ii * 16 + lrow) * ROWB + (j * 16 + lgrp * 4) * 4) = acc[c + ii][j];
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                for (int q = lane; q < CH * 16 * QPR; q += 64) {
                    const int r = q / QPR;
                    const int col = (q - r * QPR) * 4;
                    const int m = m0 + wm * WTM + c * 16 + r;
                    const int n = n0 + wn * WTN + col;
                    if (m >= m_lim)
                        continue;
                    f32x4 v = *(const f32x4*)(wbuf + r * ROWB + col * 4);
    #pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        float bb = bv[rr];
                        if constexpr (!HOIST)
                            bb = n + rr < N ? __uint_as_float((uint32_t)bias_t[n + rr] << 16) : 0.f;
                        v[rr] = epi_activation(v[rr] + bb, epi);
                    }
                    const uint2 h = pack_bf16x4(v);
                    uint16_t* crow = C + (size_t)m * (size_t)ldc;
                    if (vec_ok && n + 3 < N) {
                        *(uint2*)(crow + n) = h;
                    } else {
    #pragma unroll
                        for (int rr = 0; rr < 4; ++rr)
                            if (n + rr < N)
                                crow[n + rr] = bf16_elem(h, rr);
                    }
                }
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // region reads done before the next chunk
            }
            return;
        }

        // Epilogue: one nearest-even rounding per element (v_cvt_pk_bf16_f32);
        // 16-byte stores of 8 rows x 128 bytes (or 16 rows x 64 bytes) when
        // the wave tile has an even number of block columns and C's rows
        // are 16-byte aligned (hkg_store.h), else masked 8-byte stores.
        if constexpr (FN % 2 == 0) {
            if ((ldc & 7) == 0) {
                store_blocks_wide<FM, FN>([&](int i, int j) { return acc[i][j]; }, C, ldc, m0 + wm * WTM, m_lim,
                                          n0 + wn * WTN, N);
                return;
            }
        }
    #pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = m0 + wm * WTM + i * 16 + lrow;
            if (m >= m_lim)
                continue;
            uint16_t* crow = C + (size_t)m * (size_t)ldc;
    #pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = n0 + wn * WTN + j * 16 + lgrp * 4;
                // One block at a time: keeps the compiler from moving every
                // accumulator into VGPRs at once (256 of them in 4-wave tiles).
                __builtin_amdgcn_sched_barrier(0);
                const uint2 h = pack_bf16x4(acc[i][j]);
                if (vec_ok && n + 3 < N) {
                    *(uint2*)(crow + n) = h;
                } else {
    #pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N)
                            crow[n + r] = bf16_elem(h, r);
                }
            }
        }
    };

    if constexpr (!GROUPED) {
        int tm, tn;
        tile_order(blockIdx.x, tiles_m, tiles_n, win_w, chunk_c, tm, tn);
        if (tm >= tiles_m || tn >= tiles_n)    // uniform per workgroup; never taken for a valid order
            return;
        run_tile(tm, tn, tm * BM, M, (const char*)Bv, bias, (int)blockIdx.y, split_k, 0);
    } else {
        // Grouped (mixture-of-experts) mode, a persistent grid (FlyDSL-in-
        // PyTorch blog, grouped GEMM section).  Expert g owns rows
        // [offs[g-1], offs[g]) of A and C and the N x K weight g of B.  The
        // tiles of all experts form one list, expert after expert (empty
        // experts have none), each expert's column-first in windows of 8
        // tile rows: consecutive tiles share a B tile.  Workgroup b visits tiles b, b + P, ... (P = grid size),
        // or, when chunk_c != 0 and the list holds at least P tiles, the
        // list is cut into 8 contiguous parts and workgroups of XCD x
        // (b mod 8 = x under round-robin dispatch) walk part x, so the tiles
        // one XCD holds at a time are neighbours sharing B tiles and A rows
        // in its L2.  Offsets are clamped into [0, M] and made non-
        // decreasing per expert, so any offsets keep every access in bounds.
        static_assert(!MX && SCHED != 1, "grouped mode: bf16 tiles");
        auto expert_rows = [&](int g, int& r0, int& r1) {
            if (offs == nullptr) {          // one expert of M rows (a dense GEMM)
                r0 = 0;
                r1 = M;
                return;
            }
            r0 = g > 0 ? min(max(offs[g - 1], 0), M) : 0;
            r1 = max(r0, min(offs[g], M));
        };
        // Wave-parallel walk over the experts, 64 at a time: lane l holds
        // expert gb + l's tile count and the inclusive prefix over the chunk
        // (64-bit: clamped offsets may overlap, so counts are not bounded by
        // the tiles of C).
        auto chunk = [&](int gb, int64_t& tiles_l, int64_t& incl_l) {
            const int g = gb + lane;
            tiles_l = 0;
            if (g < G) {
                int r0, r1;
                expert_rows(g, r0, r1);
                tiles_l = (int64_t)((r1 - r0 + BM - 1) / BM) * tiles_n;
            }
            incl_l = tiles_l;
#pragma unroll
            for (int d = 1; d < 64; d <<= 1) {
                const int64_t o = __shfl_up(incl_l, d, 64);
                if (lane >= d)
                    incl_l += o;
            }
        };
        auto uniform64 = [](int64_t v) {
            const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
            const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
            return (int64_t)(((uint64_t)hi << 32) | lo);
        };
        int64_t total = 0;
        for (int gb = 0; gb < G; gb += 64) {
            int64_t tl, il;
            chunk(gb, tl, il);
            total += uniform64(__shfl(il, 63, 64));
        }
        const int64_t P = gridDim.x;
        // The last round: when its R tiles (total mod P) fill at most half the
        // grid and split_k is 2, each of them is split into two halves of K
        // (units 2r and 2r + 1 of tile r), so the round takes half a tile's
        // time instead of a whole one.  The tiles before it form whole rounds,
        // walked as above.
        const int nk_all = (K + BK - 1) / BK;
        const int64_t rem = total % P;
        const bool tail_split = split_k == 2 && rem > 0 && 2 * rem <= P && nk_all >= 2;
        const int64_t whole = tail_split ? total - rem : total;
        int64_t first = blockIdx.x, stride = P, limit = whole;
        if (chunk_c != 0 && P % 8 == 0 && whole >= P) {
            const int64_t x = blockIdx.x % 8;
            first = whole * x / 8 + blockIdx.x / 8;
            stride = P / 8;
            limit = whole * (x + 1) / 8;
        }
        int gb = 0;
        int64_t tb = 0;
        // Tile t of the list, over part k_part of k_parts of K (tiles are
        // visited in increasing order, so the walk over experts only moves
        // forward).
        auto visit = [&](int64_t t, int k_part, int k_parts, int unit) {
            int64_t tiles_l, incl_l;
            chunk(gb, tiles_l, incl_l);
            int64_t chunk_total = uniform64(__shfl(incl_l, 63, 64));
            while (t >= tb + chunk_total) {
                tb += chunk_total;
                gb += 64;
                chunk(gb, tiles_l, incl_l);
                chunk_total = uniform64(__shfl(incl_l, 63, 64));
            }
            const uint64_t hit = __ballot(tb + incl_l > t);
            const int l = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
            const int g = gb + l;
            const int64_t t0 = tb + uniform64(__shfl(incl_l - tiles_l, l, 64));
            int r0, r1;
            expert_rows(g, r0, r1);
            r0 = __builtin_amdgcn_readfirstlane(r0);
            r1 = __builtin_amdgcn_readfirstlane(r1);
            const int tiles_mg = (r1 - r0 + BM - 1) / BM;
            const int u = (int)(t - t0);             // below tiles_mg * tiles_n
            // Inside an expert: column-first in windows of 8 tile rows (the
            // dense kernel's window walk), i.e. N-major for experts of at most
            // 8 tile rows, with A's reuse distance bounded for larger ones.
            int tm, tn;
            tile_order(u, tiles_mg, tiles_n, 8, 0, tm, tn);
            __syncthreads();                         // LDS of the previous tile is free
            run_tile(tm, tn, r0 + tm * BM, r1, (const char*)Bv + (size_t)g * (size_t)N * b_rb,
                     EPI ? bias + (size_t)g * (size_t)N : bias, k_part, k_parts, unit);
        };
        // The split round's units u = 2 r + h (half h of its tile r) are cut
        // into 8 contiguous parts and part x goes to workgroups x, x + 8, ...
        // (XCD x under round-robin dispatch), so the units one XCD holds are
        // neighbouring tiles sharing B tiles and A rows in its L2, as in the
        // whole rounds.  Part x has at most ceil(2 rem / 8) <= P / 8 units.
        int unit = -1;
        if (tail_split) {
            const int64_t units = 2 * rem;
            const int64_t x = blockIdx.x % 8, i = blockIdx.x / 8;
            const int64_t u0 = units * x / 8, u1 = units * (x + 1) / 8;
            if (P % 8 == 0) {
                if (u0 + i < u1)
                    unit = (int)(u0 + i);
            } else if ((int64_t)blockIdx.x < units) {
                unit = (int)blockIdx.x;
            }
        }
        // Whole tiles first, then this workgroup's unit of the split round
        // (one loop, so the tile code is instantiated once).
        const int64_t n_whole = first < limit ? (limit - first + stride - 1) / stride : 0;
        const int64_t n_items = n_whole + (unit >= 0 ? 1 : 0);
        for (int64_t j = 0; j < n_items; ++j) {
            const bool half = j == n_whole;
            visit(half ? whole + unit / 2 : first + j * stride, half ? (unit & 1) : 0, half ? 2 : 1,
                  half ? unit : 0);
        }
    }
}

// lda, ldb, ldc: leading dimensions (elements) of A, B, C.
template <int BM, int BN, int BK, int STAGES, int WM, int WN, int SCHED, bool EPI, bool MX>
hipError_t launch_tile_t(const void* A, const void* B, uint16_t* C, int M, int N, int K, int win_w, int chunk_c,
                         int split_k, float* ws, int* counters, const uint16_t* bias, int epi, const uint32_t* psa,
                         const uint32_t* psb, int lda, int ldb, int ldc, hipStream_t stream)
{
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    // the persistent schedule: at most one workgroup per compute unit
    const int grid = (SCHED == 6 && !EPI && !MX) ? min(tiles_m * tiles_n, kPersistentGrid) : tiles_m * tiles_n;
    hipLaunchKernelGGL((tile_kernel<BM, BN, BK, STAGES, WM, WN, SCHED, EPI, MX, false>),
                       dim3(grid, split_k), dim3(tile_threads<WM, WN, SCHED>()), 0, stream, A, B, C, M, N, K, tiles_m,
                       tiles_n, win_w, chunk_c, split_k, ws, counters, bias, epi, psa, psb, nullptr, 0, lda, ldb,
                       ldc);
    return hipGetLastError();
}

// Grouped form on a persistent grid of `grid` workgroups; split_k 2 splits
// the tiles of a last round that fills at most half the grid into two halves
// of K, with ws holding grid partial tiles (BM x BN fp32 each) and counters
// grid / 2 arrival counters, zero on entry and left zero.
template <int BM, int BN, int BK, int STAGES, int WM, int WN, int SCHED, bool EPI>
hipError_t launch_grouped_t(const void* A, const void* B, const int* offs, int G, uint16_t* C, int M, int N, int K,
                            int grid, int xcd_chunks, int split_k, float* ws, int* counters, const uint16_t* bias,
                            int epi, hipStream_t stream)
{
    const int tiles_n = (N + BN - 1) / BN;
    hipLaunchKernelGGL((tile_kernel<BM, BN, BK, STAGES, WM, WN, SCHED, EPI, false, true>), dim3(grid), dim3(WM * WN * 64),
                       0, stream, A, B, C, M, N, K, 0, tiles_n, 0, xcd_chunks, split_k, ws, counters, bias, epi,
                       nullptr, nullptr, offs, G, K, K, N);
    return hipGetLastError();
}

}  // namespace
}  // namespace hkg
