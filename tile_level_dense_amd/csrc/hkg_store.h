// Wide stores of a wave's bf16 output blocks.
//
// After the MFMAs (B fragment first) lane l of a wave holds, for each 16 x 16
// block of C, row l % 16 and the four consecutive columns 4 (l / 16) .. + 3:
// an 8-byte store per lane writes 16 rows x 32 bytes per instruction, and
// the memory system takes such partial-line writes markedly slower than
// whole-line ones (on MI355X, 256 workgroups writing a 4096 x 4096 bf16 C in
// that pattern took 12.4 us against 8.3 us with 128-byte row pieces and
// 7.0 us with whole rows).  Two in-register exchanges give each lane 16
// contiguous bytes and each store instruction 8 rows x 128 bytes, with the
// values, and so the stored bits, unchanged:
//  * v_permlane16_swap (gfx950) on the packed bf16 words of blocks j and
//    j + 1 swaps the odd 16-lane rows of the first with the even rows of the
//    second.  Lane (r, g) (row r = l % 16, g = l / 16) then holds 8
//    consecutive columns of row r of the block pair: columns
//    16 (g % 2) + 8 (g / 2) .. + 7 of its 32.
//  * For two such pairs (64 columns), a DPP rotation by 8 within each
//    16-lane row hands lane r the values of lane r + 8 (mod 16); selecting
//    own or rotated values by r < 8 gives one instruction that stores rows
//    0-7 of both pairs (lanes r < 8 the first pair, lanes r >= 8 the
//    second) and one that stores rows 8-15.
// Each store is masked by rows (m < m_lim) and by columns: a 16-byte store
// when all eight columns are below N, element stores otherwise.  Callers
// use it when C's leading dimension is a multiple of 8 elements (each
// 16-byte store is then aligned, C itself being 16-byte aligned).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hkg {
namespace {

typedef float store_f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 store_bf16x4 __attribute__((ext_vector_type(4)));

// Nearest-even bf16 of four values, packed two per word (element e in bits
// 16 (e % 2) of word e / 2).
__device__ __forceinline__ uint2 store_pack(store_f32x4 v)
{
    return __builtin_bit_cast(uint2, __builtin_convertvector(v, store_bf16x4));
}

// Blocks j (x) and j + 1 (y) of one block row -> this lane's 8 consecutive
// columns of its row, at column 16 (g % 2) + 8 (g / 2) of the pair.
__device__ __forceinline__ uint4 store_pair(store_f32x4 x, store_f32x4 y)
{
    const uint2 px = store_pack(x), py = store_pack(y);
    const auto lo = __builtin_amdgcn_permlane16_swap(px.x, py.x, false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap(px.y, py.y, false, false);
    return make_uint4(lo[0], hi[0], lo[1], hi[1]);
}

// The value of lane (r + 8) mod 16 of the same 16-lane row (DPP row_ror:8).
__device__ __forceinline__ uint4 store_rot8(uint4 v)
{
    constexpr int kRowRor8 = 0x128;
    return make_uint4((uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.x, kRowRor8, 0xf, 0xf, false),
                      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.y, kRowRor8, 0xf, 0xf, false),
                      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.z, kRowRor8, 0xf, 0xf, false),
                      (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.w, kRowRor8, 0xf, 0xf, false));
}

// Eight bf16 (v) at C[m][n .. n + 7], masked by m < m_lim and n + e < N.
__device__ __forceinline__ void store_put8(uint16_t* __restrict__ C, int64_t ldc, int m, int m_lim, int n, int N,
                                           uint4 v)
{
    if (m >= m_lim)
        return;
    uint16_t* const p = C + (size_t)m * (size_t)ldc + n;
    if (n + 7 < N) {
        *(uint4*)p = v;
    } else {
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (n + e < N)
                p[e] = (uint16_t)(w[e >> 1] >> ((e & 1) * 16));
    }
}

// Store FM x NJ blocks of a wave: block (i, j) covers rows m0 + 16 i .. + 15
// and columns n0 + 16 j .. + 15 of C, and blk(i, j) (compile-time i, j after
// unrolling) returns this lane's four fp32 values of it.  NJ even: pairs of
// blocks (64-byte row pieces) when NJ % 4 != 0, pairs of pairs otherwise.
template <int FM, int NJ, typename F>
__device__ __forceinline__ void store_blocks_wide(F&& blk, uint16_t* __restrict__ C, int64_t ldc, int m0, int m_lim,
                                                  int n0, int N)
{
    static_assert(NJ % 2 == 0, "whole pairs of blocks");
    const int lane = threadIdx.x & 63;
    const int r = lane & 15, g = lane >> 4;
    const int off = (g & 1) * 16 + (g >> 1) * 8;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        if constexpr (NJ % 4 == 0) {
            const bool lo = r < 8;
            const int row = m0 + 16 * i + (r & 7);
#pragma unroll
            for (int q = 0; q < NJ / 4; ++q) {
                __builtin_amdgcn_sched_barrier(0);
                const uint4 u0 = store_pair(blk(i, 4 * q), blk(i, 4 * q + 1));
                const uint4 u1 = store_pair(blk(i, 4 * q + 2), blk(i, 4 * q + 3));
                const uint4 t0 = store_rot8(u0), t1 = store_rot8(u1);
                const int col = n0 + 64 * q + (lo ? 0 : 32) + off;
                store_put8(C, ldc, row, m_lim, col, N, lo ? u0 : t1);
                store_put8(C, ldc, row + 8, m_lim, col, N, lo ? t0 : u1);
            }
        } else {
#pragma unroll
            for (int q = 0; q < NJ / 2; ++q) {
                __builtin_amdgcn_sched_barrier(0);
                const uint4 u = store_pair(blk(i, 2 * q), blk(i, 2 * q + 1));
                store_put8(C, ldc, m0 + 16 * i + r, m_lim, n0 + 32 * q + off, N, u);
            }
        }
    }
}

}  // namespace
}  // namespace hkg
