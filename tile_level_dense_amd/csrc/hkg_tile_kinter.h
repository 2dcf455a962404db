// K-interleaved ping-pong (schedule 7): one BM x BN output tile per
// workgroup of 8 waves in two 4-wave groups, where each group covers the
// WHOLE tile (a WM x WN grid of waves, BM / WM x BN / WN of C per wave) and
// the groups take alternate 64-k stages: group 0 stages 0, 2, 4, ..., group
// 1 stages 1, 3, 5, ....  Their two fp32 partial tiles are added through LDS
// at the end.
//
// It is the 256 x 256 ping-pong's phase structure (HipKittens talk notes,
// section 2: the groups alternate a memory phase, the LDS fragment reads of
// a stage plus copies, with a compute phase, the stage's MFMAs from
// registers, phases separated by workgroup barriers) with the same 64 x 128
// tile per wave, for outputs too small to give every compute unit a
// 256 x 256 tile: a 128 x 256 tile has half the area, so M = 2048 at
// N = 4096 (or M = 1024 at N = 8192) makes 256 of them, one per compute
// unit.  Where the 256 x 256 schedule splits its A rows between the groups,
// here the groups share A and B and split K; each phase consumes a whole
// stage, so a stage is copied every phase (the 256 x 256 schedule copies one
// every two).
//
// Phase p lies between barriers p and p + 1.  In phase p, group p % 2 reads
// stage p from LDS into registers and copies stage p + D into buffer
// (p + D) % NB (NB stage buffers, D = NB - 1 = 2 or 4), while the other
// group multiplies stage p - 1.  Buffer lifetimes: stage p + D goes into
// the buffer of stage p - 1, whose reads ended before barrier p (the
// reading group waited for them, lgkmcnt, before it); with D even its only
// reader is the copying group itself, in phase p + D, and each wave of that
// group, at the end of its compute phase p + D - 1, waits for all its
// copies but the D / 2 - 1 batches it issued after them (vmcnt counts its
// copies in order), before barrier p + D.  Stages past K (and a last stage
// that evens out the count) are copied with out-of-range offsets, which
// write zeros, so both groups run the same number of stages and the loop
// has no branch around copies or waits.
//
// Group 0 joins barriers 0 .. nk2 and group 1 barriers 0 .. nk2 - 1 plus
// one extra at the start (phase 0, in which group 1 has nothing to
// multiply): nk2 + 1 each.  After the loop every wave waits for all its
// copies (vmcnt(0)) and no wave reads a stage, so LDS is reused for the
// exchange: each wave writes the half of its accumulator blocks that its
// partner wave (same position in the other group) completes, reads the
// other half from the partner and adds it to its own, and stores its half
// of the tile.  fp32 addition is commutative, so both halves form
// partial(0) + partial(1) identically.
#pragma once

#include <type_traits>

#include "hkg_epilogue.h"
#include "hkg_internal.h"
#include "hkg_store.h"
#include "hkg_tile_order.h"

namespace hkg {
namespace {

template <int BM, int BN, int WM, int WN, int NB, bool EPI>
__device__ __forceinline__ void pingpong_kinter(const void* __restrict__ Av, const void* __restrict__ Bv,
                                                uint16_t* __restrict__ C, int M, int N, int K, int tiles_m,
                                                int tiles_n, int win_w, int chunk_c, int lda, int ldb, int ldc,
                                                char* smem, const uint16_t* __restrict__ bias, int epi)
{
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) void lds_v;
    constexpr int BK = 64, RB = 128;        // k per stage, bytes of a stage row
    constexpr int RPW = 1024 / RB;          // rows per wave copy instruction
    constexpr int RPL = 256 / RB;           // rows per 256-byte sweep of the banks
    constexpr int CPR = RB / 16;            // 16-byte chunks per row
    constexpr int KPC = 8;                  // k per chunk
    constexpr int KS = BK / 32;             // 32-k MFMA steps per stage
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int HN = FN / 2;              // accumulator block columns each wave completes
    constexpr int A_BYTES = BM * RB;
    constexpr int STAGE = (BM + BN) * RB;
    constexpr int A_CP = BM / (4 * RPW);    // copies per wave per stage: A rows, B rows
    constexpr int B_CP = BN / (4 * RPW);
    constexpr int XCH = FM * HN * 1024;     // exchange bytes per wave (one f32x4 per lane per block)
    static_assert(WM * WN == 4, "two groups of four waves");
    static_assert(WTM % 16 == 0 && WTN % 32 == 0, "whole 16 x 16 blocks, an even number of block columns");
    static_assert(BM % (4 * RPW) == 0 && BN % (4 * RPW) == 0, "stage rows split over a group's copies");
    static_assert((4 * RPW / RPL) % CPR == 0, "swizzle must repeat across a wave's copies");
    static_assert(NB == 3 || NB == 5, "stage buffers: copies run NB - 1 (even) stages ahead");
    static_assert(NB * STAGE <= 160 * 1024 && 8 * XCH <= NB * STAGE, "the stages, and the exchange, in LDS");
    constexpr int D = NB - 1;               // copy distance in stages (and phases)
    constexpr int CPS = A_CP + B_CP;        // copies per wave per stage
    constexpr uint32_t kOOR = 0x80000000u;
    constexpr int kW3 = 0x00020000;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int g = wave >> 2, w4 = wave & 3;
    const int wm = w4 / WN, wn = w4 - (w4 / WN) * WN;
    const uint32_t a_rb = (uint32_t)lda * 2u, b_rb = (uint32_t)ldb * 2u;

    int tm, tn;
    tile_order((int)blockIdx.x, tiles_m, tiles_n, win_w, chunk_c, tm, tn);
    if (tm >= tiles_m || tn >= tiles_n)     // uniform per workgroup; never taken for a valid order
        return;
    const int m0 = tm * BM, n0 = tn * BN;
    const int rows_a = min(BM, M - m0), rows_b = min(BN, N - n0);
    const __amdgpu_buffer_rsrc_t ra =
        __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)Av + (size_t)m0 * a_rb), 0, (int)(rows_a * a_rb), kW3);
    const __amdgpu_buffer_rsrc_t rb =
        __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)Bv + (size_t)n0 * b_rb), 0, (int)(rows_b * b_rb), kW3);

    // Copy sources of this lane: copy i of wave w4 fills LDS rows
    // RPW (w4 + 4 i) .. + RPW - 1 of an operand, lane -> row RPW w4 + lane /
    // CPR (plus 4 RPW i), position lane % CPR, which holds logical chunk
    // (lane % CPR) ^ ((row / RPL) % CPR): chunk c of row r is stored at
    // c ^ ((r / RPL) % CPR), as in the other tile schedules.
    const int prow = w4 * RPW + lane / CPR;
    const int pchunk = (lane % CPR) ^ ((prow / RPL) % CPR);
    const uint32_t p_off_a = (uint32_t)prow * a_rb + (uint32_t)pchunk * 16u;
    const uint32_t p_off_b = (uint32_t)prow * b_rb + (uint32_t)pchunk * 16u;
    const int p_k = pchunk * KPC;
    auto copy_stage = [&](int t) {
        char* const base = smem + (t % NB) * STAGE;
        const int k0 = t * BK;
        const bool k_out = k0 + p_k >= K;   // K % 8 == 0: a chunk is wholly inside or outside
        const uint32_t ko = (uint32_t)k0 * 2u;
#pragma unroll
        for (int i = 0; i < A_CP; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_v*)(base + (w4 + 4 * i) * 1024), 16,
                                                     k_out ? kOOR : p_off_a + ko + (uint32_t)(i * 4 * RPW) * a_rb, 0,
                                                     0, 0);
#pragma unroll
        for (int i = 0; i < B_CP; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_v*)(base + A_BYTES + (w4 + 4 * i) * 1024), 16,
                                                     k_out ? kOOR : p_off_b + ko + (uint32_t)(i * 4 * RPW) * b_rb, 0,
                                                     0, 0);
    };

    // Fragment reads: lane -> row lane % 16 of a 16-row block, logical chunk
    // 4 s + lane / 16 for 32-k step s.
    const int lrow = lane & 15, lgrp = lane >> 4;
    const int swz = (lrow / RPL) % CPR;
    int chunk_off[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
        chunk_off[s] = ((4 * s + lgrp) ^ swz) * 16;
    const int a_frag = (wm * WTM + lrow) * RB;
    const int b_frag = A_BYTES + (wn * WTN + lrow) * RB;
    bf16x8 af[KS][FM], bf[KS][FN];
    auto read_stage = [&](int t) {
        const char* const base = smem + (t % NB) * STAGE;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[s][i] = *(const bf16x8*)(base + a_frag + i * 16 * RB + chunk_off[s]);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[s][j] = *(const bf16x8*)(base + b_frag + j * 16 * RB + chunk_off[s]);
        }
    };
    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto mfma_stage = [&]() {
#pragma unroll
        for (int s = 0; s < KS; ++s)
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[s][j], af[s][i], acc[i][j], 0, 0, 0);
    };
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
    auto phase_barrier = [&]() {
        fence();
        asm volatile("s_barrier" ::: "memory");
        fence();
    };

    const int nk = (K + BK - 1) / BK;
    const int pairs = (nk + 1) / 2;         // stages per group

    // Prologue: group g copies its own first stages g, g + 2, ... below D.
    // Each wave then waits for all but its newest D / 2 - 1 batches of
    // copies: the first stage it reads has landed, and the loop's waits (the
    // same count, at the end of every compute phase) cover the rest.
#pragma unroll
    for (int s = 0; s < D; s += 2)
        copy_stage(s + g);
    auto wait_copies = [] {                 // all but the newest D / 2 - 1 batches
        if constexpr (D == 2)
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        else
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CPS * (D / 2 - 1)) : "memory");
    };
    if (g == 0) {
        wait_copies();
        phase_barrier();                    // barrier 0
        for (int q = 0; q < pairs; ++q) {
            const int t = 2 * q;
            read_stage(t);                  // phase t: memory
            fence();
            copy_stage(t + D);
            fence();
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            phase_barrier();
            mfma_stage();                   // phase t + 1: compute
            fence();
            wait_copies();                  // stage t + 2, read in phase t + 2
            phase_barrier();
        }
    } else {
        phase_barrier();                    // barrier 0; phase 0: group 0 reads stage 0
        wait_copies();                      // stage 1
        phase_barrier();
        for (int q = 0; q < pairs; ++q) {
            const int t = 2 * q + 1;
            read_stage(t);                  // phase t: memory
            fence();
            copy_stage(t + D);
            fence();
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            phase_barrier();
            mfma_stage();                   // phase t + 1: compute
            fence();
            wait_copies();
            if (q + 1 < pairs)
                phase_barrier();
        }
    }
    // The last copies (stages past K: zeros nobody reads) land before the
    // exchange reuses LDS.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    // Exchange and store.  Group 0 completes block columns 0 .. HN - 1 of
    // its wave tile, group 1 columns HN .. FN - 1; the exchange slot of
    // block (i, jj) of a wave is 1 KiB, lane l at byte 16 l.
    float bv[HN][4];
    const bool vec_ok = ((N | ldc) & 3) == 0;
    const bool wide_ok = (ldc & 7) == 0;    // 16-byte stores (hkg_store.h)
    auto finish = [&](auto own) {
        constexpr int JO = decltype(own)::value;     // first block column this wave completes
        constexpr int JX = JO == 0 ? HN : 0;         // first block column the partner completes
        if constexpr (EPI) {
#pragma unroll
            for (int jj = 0; jj < HN; ++jj)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int n = n0 + wn * WTN + (JO + jj) * 16 + lgrp * 4 + r;
                    bv[jj][r] = n < N ? __uint_as_float((uint32_t)bias[n] << 16) : 0.f;
                }
        }
        phase_barrier();                    // the last barrier of the stages: LDS is free
        char* const mine = smem + wave * XCH + lane * 16;
        const char* const theirs = smem + (wave ^ 4) * XCH + lane * 16;
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int jj = 0; jj < HN; ++jj)
                *(f32x4*)(mine + (i * HN + jj) * 1024) = acc[i][JX + jj];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        phase_barrier();
        // Block (i, jj) of this wave's half: own partial + the partner's,
        // then the epilogue.
        auto blk = [&](int i, int jj) {
            f32x4 v = acc[i][JO + jj] + *(const f32x4*)(theirs + (i * HN + jj) * 1024);
            if constexpr (EPI) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    v[r] = epi_activation(v[r] + bv[jj][r], epi);
            }
            return v;
        };
        if (wide_ok) {
            store_blocks_wide<FM, HN>(blk, C, ldc, m0 + wm * WTM, M, n0 + wn * WTN + JO * 16, N);
            return;
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = m0 + wm * WTM + i * 16 + lrow;
            uint16_t* const crow = C + (size_t)(m < M ? m : 0) * (size_t)ldc;
#pragma unroll
            for (int jj = 0; jj < HN; ++jj) {
                __builtin_amdgcn_sched_barrier(0);
                const f32x4 v = blk(i, jj);
                const int n = n0 + wn * WTN + (JO + jj) * 16 + lgrp * 4;
                const uint2 h = __builtin_bit_cast(uint2, __builtin_convertvector(v, bf16x4));
                if (m < M) {
                    if (vec_ok && n + 3 < N) {
                        *(uint2*)(crow + n) = h;
                    } else {
#pragma unroll
                        for (int r = 0; r < 4; ++r)
                            if (n + r < N)
                                crow[n + r] = (uint16_t)(((r >> 1) ? h.y : h.x) >> ((r & 1) * 16));
                    }
                }
            }
        }
    };
    if (g == 0)
        finish(std::integral_constant<int, 0>{});
    else
        finish(std::integral_constant<int, HN>{});
}

}  // namespace
}  // namespace hkg
