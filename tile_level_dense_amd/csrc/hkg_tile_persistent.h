// Persistent form of the 256 x 256 ping-pong tile schedule (bf16, no fused
// epilogue, K not split): a grid of at most one workgroup per compute unit,
// each walking its tiles b, b + G, b + 2 G, ... (G = grid size) in the
// chiplet-aware tile order.
//
// Every tile of a workgroup is the same ping-pong as the one-tile kernel
// (hkg_tile_kernel.h, schedule 5: two 4-wave groups alternating memory and
// compute phases, A halves double- and B triple-buffered in LDS, all copies
// issued in memory phases), but the workgroup's tiles form one continuous
// stream of 64-k stages: stage u of the stream is stage u mod nk of tile
// u / nk.  The copies that run ahead of the compute (A one stage, B two
// stages) therefore fetch the next tile's first stages while the current
// tile's last stages are multiplied, where the one-tile kernel issues copies
// past the end of K that read nothing; and each wave stores its part of a
// finished tile right after that tile's last compute phase, while the next
// tile's data is landing, instead of the workgroup ending and a new one
// being dispatched and fetching its first stages from scratch.  LDS
// lifetimes are those of the one-tile schedule, indexed by the stream's
// stage number, so they do not depend on where tiles begin.
//
// Waits: every vmcnt wait counts only the buffer->LDS copies issued after
// the ones it needs (loads complete in order among themselves); the C stores
// of a finished tile can only make such a wait longer, never shorter.
#pragma once

#include <type_traits>

#include "hkg_internal.h"
#include "hkg_tile_order.h"

namespace hkg {
namespace {

template <int WM, int WN>
__device__ __forceinline__ void pingpong_persistent(const void* __restrict__ Av, const void* __restrict__ Bv,
                                                    uint16_t* __restrict__ C, int M, int N, int K, int tiles_m,
                                                    int tiles_n, int win_w, int chunk_c, int lda, int ldb, int ldc,
                                                    char* smem)
{
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    typedef __attribute__((address_space(3))) void lds_v;
    constexpr int BM = 256, BN = 256, BK = 64, RB = 128, NW = WM * WN;
    constexpr int RPW = 1024 / RB;          // rows per wave copy instruction
    constexpr int RPL = 256 / RB;           // rows per 256-byte sweep of the banks
    constexpr int CPR = RB / 16;            // 16-byte chunks per row
    constexpr int KPC = 8;                  // k per chunk
    constexpr int KS = BK / 32;             // 32-k MFMA steps per stage
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 16, FN = WTN / 16;
    constexpr int HALF = 128 * RB;          // 128 rows of one stage
    constexpr int CPW = 128 / (RPW * 4);    // copies per half per wave
    static_assert(NW == 8 && WM <= 4, "two 4-wave groups");
    constexpr uint32_t kOOR = 0x80000000u;
    constexpr int kW3 = 0x00020000;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN, wn = wave - (wave / WN) * WN;
    const int g = wave >> 2, w4 = wave & 3;
    const uint32_t a_rb = (uint32_t)lda * 2u, b_rb = (uint32_t)ldb * 2u;

    // Fragment reads and copy sources of this lane (same swizzle as the
    // one-tile kernel: chunk c of row r stored at c ^ ((r / RPL) % CPR)).
    const int lrow = lane & 15, lgrp = lane >> 4;
    const int swz = (lrow / RPL) % CPR;
    int chunk_off[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s)
        chunk_off[s] = ((4 * s + lgrp) ^ swz) * 16;
    const int prow = w4 * RPW + lane / CPR;
    const int pchunk = (lane % CPR) ^ ((prow / RPL) % CPR);
    const uint32_t p_off_a = (uint32_t)(128 * g + prow) * a_rb + (uint32_t)pchunk * 16u;
    const uint32_t p_off_b = (uint32_t)(128 * g + prow) * b_rb + (uint32_t)pchunk * 16u;
    const int p_k = pchunk * KPC;
    static_assert((4 * RPW / RPL) % CPR == 0, "swizzle must repeat across a group's copies");
    char* const a_buf = smem;
    char* const b_buf = smem + 4 * HALF;
    const int a_row = wm * WTM - 128 * g + lrow;
    const int b_row = wn * WTN + lrow;

    // The workgroup's tiles and its stream of stages.
    const int total = tiles_m * tiles_n;
    const int G = gridDim.x;
    const int ntiles = ((int)blockIdx.x < total) ? (total - (int)blockIdx.x + G - 1) / G : 0;
    const int nk = (K + BK - 1) / BK;
    const int U = ntiles * nk;
    if (U == 0)
        return;

    // A position in the stream: tile j of this workgroup (its m0, n0 and
    // buffer descriptors) and stage s of that tile.
    struct Pos {
        int j, s, m0, n0;
        __amdgpu_buffer_rsrc_t ra, rb;
    };
    auto tile_at = [&](int j, Pos& p) {
        p.j = j;
        p.s = 0;
        int tm = 0, tn = 0;
        if (j < ntiles)
            tile_order((int)blockIdx.x + j * G, tiles_m, tiles_n, win_w, chunk_c, tm, tn);
        p.m0 = tm * BM;
        p.n0 = tn * BN;
        const int rows_a = min(BM, M - p.m0), rows_b = min(BN, N - p.n0);
        p.ra = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)Av + (size_t)p.m0 * a_rb), 0,
                                                 (int)(rows_a * a_rb), kW3);
        p.rb = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)Bv + (size_t)p.n0 * b_rb), 0,
                                                 (int)(rows_b * b_rb), kW3);
    };
    auto advance = [&](Pos& p) {
        if (++p.s == nk)
            tile_at(p.j + 1, p);
    };

    // Copy half g of the stage at `p` (A rows or B rows 128 g ..) into dst;
    // past the workgroup's last tile, or k past K, offsets are out of range
    // and the copy writes zeros nobody reads.
    auto copy_half = [&](const Pos& p, bool is_a, char* dst) {
        const int k0 = p.s * BK;
        const bool k_out = p.j >= ntiles || k0 + p_k >= K;
        const uint32_t rb = is_a ? a_rb : b_rb;
        const uint32_t off0 = k_out ? kOOR : (is_a ? p_off_a : p_off_b) + (uint32_t)k0 * 2u;
        const uint32_t p_step = (uint32_t)(4 * RPW) * rb;
#pragma unroll
        for (int i = 0; i < CPW; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(is_a ? p.ra : p.rb, (lds_v*)(dst + (w4 + 4 * i) * 1024), 16,
                                                     k_out ? kOOR : off0 + (uint32_t)i * p_step, 0, 0, 0);
    };

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    bf16x8 af[KS][FM], bf[KS][FN];
    auto read_stage = [&](int u, int u3) {
        const char* ab = a_buf + (2 * g + (u & 1)) * HALF + a_row * RB;
        const char* bb = b_buf + u3 * 2 * HALF + b_row * RB;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[s][i] = *(const bf16x8*)(ab + i * 16 * RB + chunk_off[s]);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[s][j] = *(const bf16x8*)(bb + j * 16 * RB + chunk_off[s]);
        }
    };
    // A finished tile: one nearest-even rounding per element, masked 8-byte
    // stores, then the accumulators start over for the next tile.
    const bool vec_ok = ((N | ldc) & 3) == 0;
    auto store_tile = [&](const Pos& p) {
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = p.m0 + wm * WTM + i * 16 + lrow;
            uint16_t* crow = C + (size_t)(m < M ? m : 0) * (size_t)ldc;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = p.n0 + wn * WTN + j * 16 + lgrp * 4;
                __builtin_amdgcn_sched_barrier(0);
                const uint2 h = __builtin_bit_cast(uint2, __builtin_convertvector(acc[i][j], bf16x4));
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
                acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
        }
    };
    auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
    auto phase_barrier = [&]() {
        fence();
        asm volatile("s_barrier" ::: "memory");
        fence();
    };

    // Stream positions: the stage being computed, the next A copy (one
    // stage ahead) and the next B copy (two stages ahead).
    Pos pc, pa, pb;
    tile_at(0, pc);
    pa = pc;
    pb = pc;
    // Prologue: stage 0 (A and this group's B rows) and this group's B rows
    // of stage 1.
    copy_half(pa, true, a_buf + (2 * g) * HALF);
    advance(pa);
    copy_half(pb, false, b_buf + g * HALF);
    advance(pb);
    copy_half(pb, false, b_buf + 2 * HALF + g * HALF);
    advance(pb);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CPW) : "memory");
    phase_barrier();

    // The two groups run separate copies of the loop (as the one-tile
    // kernel does), so neither carries the other's waits as branches.
    auto stream = [&](auto group1) {
        constexpr bool G1 = decltype(group1)::value;
        if constexpr (G1)
            phase_barrier();                   // phase 0: group 0 reads stage 0
        int u3 = 0;                            // u % 3
        int pb3 = 2;                           // (u + 2) % 3: B buffer of the next B copy
        for (int u = 0; u < U; ++u) {
            // memory phase: this stage's fragments, the copies running ahead
            read_stage(u, u3);
            fence();
            copy_half(pa, true, a_buf + (2 * g + ((u + 1) & 1)) * HALF);
            copy_half(pb, false, b_buf + pb3 * 2 * HALF + g * HALF);
            fence();
            if constexpr (!G1)
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            else    // B rows of stage u + 1, copied a memory phase earlier
                asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(2 * CPW) : "memory");
            phase_barrier();
            // compute phase
#pragma unroll
            for (int s = 0; s < KS; ++s)
#pragma unroll
                for (int i = 0; i < FM; ++i)
#pragma unroll
                    for (int j = 0; j < FN; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[s][j], af[s][i], acc[i][j], 0, 0, 0);
            fence();
            if (pc.s == nk - 1)
                store_tile(pc);
            fence();
            // all but this phase's B copies
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CPW) : "memory");
            if (!G1 || u + 1 < U)
                phase_barrier();
            advance(pc);
            advance(pa);
            advance(pb);
            u3 = u3 == 2 ? 0 : u3 + 1;
            pb3 = pb3 == 2 ? 0 : pb3 + 1;
        }
    };
    if (g == 1)
        stream(std::integral_constant<bool, true>{});
    else
        stream(std::integral_constant<bool, false>{});
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

}  // namespace
}  // namespace hkg
