// Large-tile MFMA kernel for compute-bound shapes: C = A * B^T, bf16 in,
// fp32 accumulation, bf16 out.
//
// Design (gfx950, MI355X):
//  * One workgroup computes a BM x BN output tile (256 x 256 by default; the
//    HipKittens talk notes, Table 2, show output-tile size dominating BF16
//    GEMM speed on this chip, with all waves doing math and none specialised
//    as producers).
//  * A and B K-slices of 64 are copied HBM -> LDS by buffer loads that write
//    LDS directly (the "buffer_load ... lds" DMA of the FlyDSL "Prebuilt
//    kernels guide", section 3c), bypassing VGPRs.  Each wave instruction
//    fills 1 KB of LDS contiguously, lane i at byte 16 i, so the bank swizzle
//    is applied on the global address instead (HipKittens talk notes,
//    section 1, asynchronous global loads swizzled on the HBM address).
//  * LDS layout per operand: row r (128 bytes = 64 k) holds its 16-byte
//    chunk c at position c ^ ((r >> 1) & 7).  A fragment read (ds_read_b128,
//    16 lanes = 16 consecutive rows at one chunk) then touches all 64 banks
//    once per 16-lane phase (64 banks x 4 phases for ds_read_b128: talk
//    notes, section 1, heterogeneous matrix-core shapes).
//  * Two LDS stages; one barrier per K step.  Before the barrier every wave
//    waits for its own DMA (vmcnt) and its LDS reads (lgkmcnt): a direct
//    copy still in flight at a barrier gives wrong results on CDNA4 (hk-dsl
//    page, "The traps it removes").
//  * MFMA v_mfma_f32_16x16x32_bf16 with the B fragment as the first operand
//    and the A fragment as the second, so each lane ends with four
//    consecutive columns of one row of C (an 8-byte store).
//  * Workgroup -> tile order: chiplet de-interleave with chunk C and a
//    column-first window of height W (talk notes, section 3, Algorithm 1).
//  * Ragged M, N and K: rows past the matrix and k past K fall outside the
//    buffer resource's range and read as zero; stores are masked.
#include "hkg_internal.h"
#include "hkg_tile_order.h"

namespace hkg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// gfx9 buffer descriptor word 3 for a raw (unswizzled, stride 0) buffer of
// 32-bit data: out-of-range offsets read as zero.
constexpr int kBufferWord3 = 0x00020000;
// An offset past every range this file creates (ranges are < 2^31 bytes).
constexpr uint32_t kOutOfRange = 0x80000000u;

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

template <int BM, int BN, int WM, int WN>
__global__ __launch_bounds__(WM * WN * 64, 1)
void tile_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                 uint16_t* __restrict__ C, int M, int N, int K,
                 int tiles_m, int tiles_n, int win_w, int chunk_c)
{
    constexpr int BK = 64;                 // k per stage: 128 bytes per row
    constexpr int NW = WM * WN;
    constexpr int WTM = BM / WM;           // rows of C per wave
    constexpr int WTN = BN / WN;           // columns of C per wave
    constexpr int FM = WTM / 16;
    constexpr int FN = WTN / 16;
    constexpr int A_BYTES = BM * BK * 2;
    constexpr int B_BYTES = BN * BK * 2;
    constexpr int STAGE = A_BYTES + B_BYTES;
    constexpr int A_LOADS = BM / (8 * NW);  // 1 KB = 8 rows per wave instruction
    constexpr int B_LOADS = BN / (8 * NW);
    static_assert(BM % (8 * NW) == 0 && BN % (8 * NW) == 0, "tile rows must split over waves");
    static_assert(WTM % 16 == 0 && WTN % 16 == 0, "wave tile must be whole 16x16 blocks");

    __shared__ __attribute__((aligned(1024))) char smem[2 * STAGE];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / WN;
    const int wn = wave - wm * WN;

    int tm, tn;
    tile_order(blockIdx.x, tiles_m, tiles_n, win_w, chunk_c, tm, tn);
    if (tm >= tiles_m || tn >= tiles_n)    // uniform per workgroup; never taken for a valid order
        return;
    const int m0 = tm * BM;
    const int n0 = tn * BN;
    const uint32_t row_bytes = (uint32_t)K * 2u;
    const int rows_a = min(BM, M - m0);
    const int rows_b = min(BN, N - n0);

    const __amdgpu_buffer_rsrc_t rsrc_a = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(A + (size_t)m0 * (size_t)K), 0, (int)(rows_a * row_bytes), kBufferWord3);
    const __amdgpu_buffer_rsrc_t rsrc_b = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(B + (size_t)n0 * (size_t)K), 0, (int)(rows_b * row_bytes), kBufferWord3);

    // DMA sources of this lane.  Wave instruction i of the A copy fills LDS
    // rows 8 g .. 8 g + 7 (g = wave + i NW); lane -> LDS row 8 g + lane / 8,
    // position lane % 8, which holds logical chunk (lane % 8) ^ swizzle(row).
    uint32_t a_off[A_LOADS], b_off[B_LOADS];
    int a_k[A_LOADS], b_k[B_LOADS];
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
        const int row = (wave + i * NW) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ ((row >> 1) & 7);
        a_off[i] = (uint32_t)row * row_bytes + (uint32_t)c * 16u;
        a_k[i] = c * 8;
    }
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
        const int row = (wave + i * NW) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ ((row >> 1) & 7);
        b_off[i] = (uint32_t)row * row_bytes + (uint32_t)c * 16u;
        b_k[i] = c * 8;
    }

    auto issue = [&](int stage, int k0) {
        char* base = smem + stage * STAGE;
        const uint32_t kb = (uint32_t)k0 * 2u;
        const bool tail = k0 + BK > K;
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) {
            uint32_t off = a_off[i] + kb;
            if (tail && k0 + a_k[i] >= K)
                off = kOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_a, (lds_void*)(base + (wave + i * NW) * 1024), 16, off, 0, 0, 0);
        }
#pragma unroll
        for (int i = 0; i < B_LOADS; ++i) {
            uint32_t off = b_off[i] + kb;
            if (tail && k0 + b_k[i] >= K)
                off = kOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc_b, (lds_void*)(base + A_BYTES + (wave + i * NW) * 1024), 16, off, 0, 0, 0);
        }
    };

    // Fragment reads: lane -> row (lane % 16) of a 16-row block, 8 k values
    // at logical chunk 4 s + lane / 16 of the 32-k step s.  The row's swizzle
    // depends only on lane % 16 because every block starts at a multiple of 16.
    const int lrow = lane & 15;
    const int lgrp = lane >> 4;
    const int swz = (lane >> 1) & 7;
    const int chunk0 = ((0 + lgrp) ^ swz) * 16;
    const int chunk1 = ((4 + lgrp) ^ swz) * 16;
    const int a_frag = (wm * WTM + lrow) * 128;
    const int b_frag = A_BYTES + (wn * WTN + lrow) * 128;

    f32x4 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
            acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int stage) {
        const char* base = smem + stage * STAGE;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int ch = s ? chunk1 : chunk0;
            bf16x8 af[FM], bf[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i)
                af[i] = *(const bf16x8*)(base + a_frag + i * 16 * 128 + ch);
#pragma unroll
            for (int j = 0; j < FN; ++j)
                bf[j] = *(const bf16x8*)(base + b_frag + j * 16 * 128 + ch);
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bf[j], af[i], acc[i][j], 0, 0, 0);
        }
    };

    const int nk = (K + BK - 1) / BK;
    issue(0, 0);
    for (int t = 0; t < nk; ++t) {
        // This wave's copy of step t has landed and its reads of step t - 1
        // are done; the barrier extends both to the whole workgroup.
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
        if (t + 1 < nk)
            issue((t + 1) & 1, (t + 1) * BK);
        compute(t & 1);
    }

    // Epilogue: one nearest-even rounding per element (v_cvt_pk_bf16_f32).
    const bool vec_ok = (N & 3) == 0;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
        const int m = m0 + wm * WTM + i * 16 + lrow;
        if (m >= M)
            continue;
        uint16_t* crow = C + (size_t)m * (size_t)N;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
            const int n = n0 + wn * WTN + j * 16 + lgrp * 4;
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
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_tile_t(const uint16_t* A, const uint16_t* B, uint16_t* C, int M, int N, int K,
                         int win_w, int chunk_c, hipStream_t stream)
{
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    hipLaunchKernelGGL((tile_kernel<BM, BN, WM, WN>), dim3(tiles_m * tiles_n), dim3(WM * WN * 64),
                       0, stream, A, B, C, M, N, K, tiles_m, tiles_n, win_w, chunk_c);
    return hipGetLastError();
}

}  // namespace

TileShape tile_shape(int variant)
{
    switch (variant) {
    case TILE_256x256: return {256, 256, 64, 8};
    case TILE_256x128: return {256, 128, 64, 8};
    case TILE_128x128: return {128, 128, 64, 4};
    default: return {0, 0, 0, 0};
    }
}

int tile_lds_bytes(int variant)
{
    const TileShape s = tile_shape(variant);
    return 2 * (s.bm + s.bn) * s.bk * 2;
}

hipError_t launch_tile(int variant, const uint16_t* A, const uint16_t* B, uint16_t* C,
                       int M, int N, int K, int win_w, int chunk_c, hipStream_t stream)
{
    switch (variant) {
    case TILE_256x256: return launch_tile_t<256, 256, 2, 4>(A, B, C, M, N, K, win_w, chunk_c, stream);
    case TILE_256x128: return launch_tile_t<256, 128, 4, 2>(A, B, C, M, N, K, win_w, chunk_c, stream);
    case TILE_128x128: return launch_tile_t<128, 128, 2, 2>(A, B, C, M, N, K, win_w, chunk_c, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace hkg
