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
// of a finished tile, and the loads of expert offsets in grouped mode, can
// only make such a wait longer, never shorter.
//
// GROUPED: the workgroup's items are tiles of the grouped (mixture-of-
// experts) list instead, walked as the one-tile grouped loop walks them (the
// same tiles, order and chiplet parts), the last of them possibly one half
// of K of a tile of a split last round (its partial summed with the other
// half's after the stream ends).  Only the position of the B copies, which
// runs ahead of the others, looks a tile up (a forward scan over the expert
// offsets); the A-copy position is one stage behind it and the compute
// position one stage behind that, so when either crosses into a new item
// the position ahead of it stands on that item's first stage and is copied.
#pragma once

#include <type_traits>

#include "hkg_internal.h"
#include "hkg_store.h"
#include "hkg_tile_order.h"

namespace hkg {
namespace {

template <int WM, int WN, bool GROUPED>
__device__ __forceinline__ void pingpong_persistent(const void* __restrict__ Av, const void* __restrict__ Bv,
                                                    uint16_t* __restrict__ C, int M, int N, int K, int tiles_m,
                                                    int tiles_n, int win_w, int chunk_c, int lda, int ldb, int ldc,
                                                    char* smem, const int* __restrict__ offs, int G, int split_k,
                                                    float* __restrict__ ws, int* __restrict__ counters)
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

    // The workgroup's items and its stream of stages.
    const int nk = (K + BK - 1) / BK;
    int n_items = 0;                        // items of this workgroup
    int n_whole = 0;                        // of which whole tiles (all of K)
    int unit = -1;                          // grouped: unit of the split last round, if any
    int64_t first = blockIdx.x, stride = gridDim.x, whole = 0;
    const int per_split = (nk + 1) / 2;     // stages of a split unit's first half

    // Grouped mode.  Expert g owns rows [offs[g-1], offs[g]) of A and C and
    // the N x K weight g of B; offsets are clamped into [0, M] and made non-
    // decreasing per expert, so any offsets keep every access in bounds.
    auto expert_rows = [&](int e, int& r0, int& r1) {
        if (offs == nullptr) {              // one expert of M rows (a dense GEMM)
            r0 = 0;
            r1 = M;
            return;
        }
        r0 = e > 0 ? min(max(offs[e - 1], 0), M) : 0;
        r1 = max(r0, min(offs[e], M));
    };
    // Lane l: expert gb + l's tile count and the inclusive prefix over the
    // 64 experts from gb (64-bit: clamped offsets may overlap).
    auto chunk = [&](int gb, int64_t& tiles_l, int64_t& incl_l) {
        const int e = gb + lane;
        tiles_l = 0;
        if (e < G) {
            int r0, r1;
            expert_rows(e, r0, r1);
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
    if constexpr (!GROUPED) {
        const int total = tiles_m * tiles_n;
        const int P = gridDim.x;
        n_items = ((int)blockIdx.x < total) ? (total - (int)blockIdx.x + P - 1) / P : 0;
        n_whole = n_items;
    } else {
        // The tiles of all experts form one list, expert after expert, each
        // expert's column-first in windows of 8 tile rows.  Whole rounds of P
        // (grid) tiles: with P a multiple of 8 and chunk_c != 0 the list is
        // cut into 8 contiguous parts and the workgroups of XCD x (b mod 8
        // under round-robin dispatch) walk part x; otherwise b, b + P, ...
        // When the last round's R tiles (total mod P) fill at most half the
        // grid and split_k is 2, each is split into two halves of K (units
        // 2r and 2r + 1 of its tile r), cut into 8 contiguous parts the same
        // way, and a workgroup's unit is its last item.
        int64_t total = 0;
        for (int gb = 0; gb < G; gb += 64) {
            int64_t tl, il;
            chunk(gb, tl, il);
            total += uniform64(__shfl(il, 63, 64));
        }
        const int64_t P = gridDim.x;
        const int64_t rem = total % P;
        const bool tail_split = split_k == 2 && rem > 0 && 2 * rem <= P && nk >= 2;
        whole = tail_split ? total - rem : total;
        int64_t limit = whole;
        if (chunk_c != 0 && P % 8 == 0 && whole >= P) {
            const int64_t x = blockIdx.x % 8;
            first = whole * x / 8 + blockIdx.x / 8;
            stride = P / 8;
            limit = whole * (x + 1) / 8;
        }
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
        n_whole = first < limit ? (int)((limit - first + stride - 1) / stride) : 0;
        n_items = n_whole + (unit >= 0 ? 1 : 0);
    }
    const int unit_k0 = min(nk, (unit & 1) * per_split);
    const int U = n_whole * nk + (unit >= 0 ? min(nk, unit_k0 + per_split) - unit_k0 : 0);
    if (U == 0)
        return;

    // A position in the stream: item j of this workgroup (its C rows m0 ..
    // m_lim - 1, columns n0 .., buffer descriptors, stages s_end - 1 at most)
    // and stage s of it; gb, tb: where the scan over the experts stands.
    struct Pos {
        int j, s, s_end, m0, m_lim, n0;
        __amdgpu_buffer_rsrc_t ra, rb;
        int gb;
        int64_t tb;
    };
    auto tile_at = [&](int j, Pos& p) {
        p.j = j;
        p.s = 0;
        p.s_end = nk;
        if constexpr (!GROUPED) {
            int tm = 0, tn = 0;
            if (j < n_items)
                tile_order((int)blockIdx.x + j * (int)gridDim.x, tiles_m, tiles_n, win_w, chunk_c, tm, tn);
            p.m0 = tm * BM;
            p.n0 = tn * BN;
            p.m_lim = M;
            const int rows_a = min(BM, M - p.m0), rows_b = min(BN, N - p.n0);
            p.ra = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)Av + (size_t)p.m0 * a_rb), 0,
                                                     (int)(rows_a * a_rb), kW3);
            p.rb = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)Bv + (size_t)p.n0 * b_rb), 0,
                                                     (int)(rows_b * b_rb), kW3);
        } else {
            if (j >= n_items)               // past the last item: copies read nothing
                return;
            const bool half = j == n_whole;
            const int64_t t = half ? whole + unit / 2 : first + (int64_t)j * stride;
            if (half) {
                p.s = unit_k0;
                p.s_end = min(nk, unit_k0 + per_split);
            }
            // Expert of list tile t: items come in increasing t, so the scan
            // only moves forward.
            int64_t tiles_l, incl_l;
            chunk(p.gb, tiles_l, incl_l);
            int64_t chunk_total = uniform64(__shfl(incl_l, 63, 64));
            while (t >= p.tb + chunk_total) {
                p.tb += chunk_total;
                p.gb += 64;
                chunk(p.gb, tiles_l, incl_l);
                chunk_total = uniform64(__shfl(incl_l, 63, 64));
            }
            const uint64_t hit = __ballot(p.tb + incl_l > t);
            const int l = __builtin_amdgcn_readfirstlane(__builtin_ctzll(hit));
            const int e = p.gb + l;
            const int64_t t0 = p.tb + uniform64(__shfl(incl_l - tiles_l, l, 64));
            int r0, r1;
            expert_rows(e, r0, r1);
            r0 = __builtin_amdgcn_readfirstlane(r0);
            r1 = __builtin_amdgcn_readfirstlane(r1);
            int tm, tn;
            tile_order((int)(t - t0), (r1 - r0 + BM - 1) / BM, tiles_n, 8, 0, tm, tn);
            p.m0 = r0 + tm * BM;
            p.m_lim = r1;
            p.n0 = tn * BN;
            const char* bg = (const char*)Bv + (size_t)e * (size_t)N * b_rb;
            const int rows_a = min(BM, r1 - p.m0), rows_b = min(BN, N - p.n0);
            p.ra = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)Av + (size_t)p.m0 * a_rb), 0,
                                                     (int)(rows_a * a_rb), kW3);
            p.rb = __builtin_amdgcn_make_buffer_rsrc((void*)(bg + (size_t)p.n0 * b_rb), 0, (int)(rows_b * b_rb),
                                                     kW3);
        }
    };
    auto advance = [&](Pos& p) {
        if (++p.s == p.s_end)
            tile_at(p.j + 1, p);
    };

    // Copy half g of the stage at `p` (A rows or B rows 128 g ..) into dst;
    // past the workgroup's last tile, or k past K, offsets are out of range
    // and the copy writes zeros nobody reads.
    auto copy_half = [&](const Pos& p, bool is_a, char* dst) {
        const int k0 = p.s * BK;
        const bool k_out = p.j >= n_items || k0 + p_k >= K;
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
    // A finished tile: one nearest-even rounding per element, 16-byte stores
    // of 8 rows x 128 bytes (hkg_store.h) when C's rows are 16-byte aligned,
    // else masked 8-byte stores; then the accumulators start over for the
    // next tile.
    const bool vec_ok = ((N | ldc) & 3) == 0;
    const bool wide_ok = (ldc & 7) == 0;
    auto store_tile = [&](const Pos& p) {
        if (wide_ok) {
            store_blocks_wide<FM, FN>([&](int i, int j) { return acc[i][j]; }, C, ldc, p.m0 + wm * WTM, p.m_lim,
                                      p.n0 + wn * WTN, N);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
            return;
        }
#pragma unroll
        for (int i = 0; i < FM; ++i) {
            const int m = p.m0 + wm * WTM + i * 16 + lrow;
            uint16_t* crow = C + (size_t)(m < p.m_lim ? m : 0) * (size_t)ldc;
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int n = p.n0 + wn * WTN + j * 16 + lgrp * 4;
                __builtin_amdgcn_sched_barrier(0);
                const uint2 h = __builtin_bit_cast(uint2, __builtin_convertvector(acc[i][j], bf16x4));
                if (m < p.m_lim) {
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
    pc.gb = 0;
    pc.tb = 0;
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
            if (pc.s == pc.s_end - 1 && (!GROUPED || pc.j < n_whole))
                store_tile(pc);             // (a split unit's partial is summed after the stream)
            fence();
            // all but this phase's B copies
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CPW) : "memory");
            if (!G1 || u + 1 < U)
                phase_barrier();
            if constexpr (GROUPED) {
                // followers take the position ahead of them when they cross
                // into its item (see the head of this file)
                if (++pc.s == pc.s_end)
                    pc = pa;
                if (++pa.s == pa.s_end)
                    pa = pb;
                advance(pb);
            } else {
                advance(pc);
                advance(pa);
                advance(pb);
            }
            u3 = u3 == 2 ? 0 : u3 + 1;
            pb3 = pb3 == 2 ? 0 : pb3 + 1;
        }
    };
    if (g == 1)
        stream(std::integral_constant<bool, true>{});
    else
        stream(std::integral_constant<bool, false>{});
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

    if constexpr (GROUPED) if (unit >= 0) {
        // The last item was half (unit & 1) of K of a tile of the split last
        // round, and acc holds that partial.  Each half writes its fp32 tile
        // to its own slot of ws (device-scope stores), fragment-major: block
        // (i, j) of wave w fills 1 KiB at ((w FM + i) FN + j) KiB, lane l's
        // four values at 16 l, so each store instruction writes 1 KiB
        // contiguously and the other half reads it back with the same
        // geometry; the half that arrives second adds the other's partial to
        // its own and stores the tile.  fp32 addition is commutative, so the
        // sum is the same whichever half arrives second.  The ordering
        // argument is the split-K arrival protocol in hkg_internal.h.
        typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
        constexpr int kDev = 16;            // cache-policy operand: sc1, device scope
        constexpr int SLOT = BM * BN;
        Pos pu;
        pu.gb = 0;
        pu.tb = 0;
        tile_at(n_whole, pu);
        const __amdgpu_buffer_rsrc_t mine =
            __builtin_amdgcn_make_buffer_rsrc(ws + (size_t)unit * SLOT, 0, SLOT * 4, kW3);
#pragma unroll
        for (int i = 0; i < FM; ++i)
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                const int off = ((wave * FM + i) * FN + j) * 1024 + lane * 16;
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, acc[i][j]), mine, off, 0, kDev);
            }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        // Every wave is past its last read of the stages and its copies have
        // landed: the first word of LDS carries the arrival result.
        __syncthreads();
        int* const arrived = (int*)smem;
        if (threadIdx.x == 0)
            *arrived = __hip_atomic_fetch_add(&counters[unit >> 1], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __syncthreads();
        if (*arrived != 1)
            return;
        const __amdgpu_buffer_rsrc_t other =
            __builtin_amdgcn_make_buffer_rsrc(ws + (size_t)(unit ^ 1) * SLOT, 0, SLOT * 4, kW3);
        // RBLK block rows at a time (16 loads in flight beside the
        // accumulators); the empty asm keeps each sum here rather than sunk
        // into the store, which would hold every loaded partial until then.
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
                    o[ii][j] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(other, off, 0, kDev));
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
        store_tile(pu);
    }
}

}  // namespace
}  // namespace hkg
