// Skinny kernel for decode-shaped GEMMs (M <= 128): C = A * B^T with B
// (the N x K weight) streamed from HBM exactly once.
//
// Design (gfx950, MI355X):
//  * A workgroup owns 16 columns of C (16 rows of B) and a K range; its
//    waves split that range further.  Every lane streams B with 16-byte
//    buffer loads, 8 k values of one B row per lane, 16 rows x 64 bytes per
//    wave instruction, issued U steps ahead of use so many loads are in
//    flight per lane (decode GEMMs that keep too little in flight reach a
//    fraction of HBM bandwidth: hk-dsl page, SGLang decode-GEMM figure).
//  * The 16 x 32 B fragment is the first operand of v_mfma_f32_16x16x32_bf16
//    and is reused for every 16-row block of A (A is small and stays in L2).
//  * Waves reduce through LDS in a fixed order (the wave-level reduction
//    followed by an LDS combine of the FlyDSL "Prebuilt kernels guide",
//    section 1.1); workgroups that share a column block along K (split-K)
//    write fp32 partials and the last one to arrive sums them in split
//    order (split-K on fp32 partials only when the grid underfills the
//    device: same guide, section 3c).  The result is rounded to bf16 once.
#include "hkg_internal.h"

namespace hkg {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));

constexpr int kBufferWord3 = 0x00020000;
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

__device__ __forceinline__ bf16x8 load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// MB: 16-row blocks of A (M <= 16 MB).  WK: waves per workgroup, splitting
// K.  U: 32-k steps loaded ahead per wave.
template <int MB, int WK, int U>
__global__ __launch_bounds__(WK * 64, 1)
void skinny_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                   uint16_t* __restrict__ C, int M, int N, int K, int split_k,
                   float* __restrict__ ws, int* __restrict__ counters)
{
    __shared__ f32x4 red[WK][MB][64];
    __shared__ int last_flag;

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = blockIdx.x * 16;
    const int lrow = lane & 15;
    const int lgrp = lane >> 4;

    // K range, in 32-k steps: workgroup split first, then waves.
    const int steps = (K + 31) >> 5;
    const int per_wg = (steps + split_k - 1) / split_k;
    const int wg_begin = min(steps, (int)blockIdx.y * per_wg);
    const int wg_end = min(steps, wg_begin + per_wg);
    const int per_wave = (wg_end - wg_begin + WK - 1) / WK;
    const int s_begin = min(wg_end, wg_begin + wave * per_wave);
    const int s_end = min(wg_end, s_begin + per_wave);

    const uint32_t row_bytes = (uint32_t)K * 2u;
    const int rows_b = min(16, N - n0);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)(B + (size_t)n0 * (size_t)K), 0, (int)(rows_b * row_bytes), kBufferWord3);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)A, 0, (int)((uint32_t)M * row_bytes), kBufferWord3);

    const uint32_t b_lane = (uint32_t)lrow * row_bytes + (uint32_t)lgrp * 16u;
    const uint32_t a_lane = (uint32_t)lrow * row_bytes + (uint32_t)lgrp * 16u;
    const uint32_t a_block = 16u * row_bytes;    // next 16 rows of A

    f32x4 acc[MB];
#pragma unroll
    for (int i = 0; i < MB; ++i)
        acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int s = s_begin; s < s_end; s += U) {
        bf16x8 bv[U];
        bf16x8 av[U][MB];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int step = s + u;
            const bool ok = step < s_end && step * 32 + lgrp * 8 < K;
            const uint32_t kb = (uint32_t)step * 64u;
            bv[u] = load16(rb, ok ? b_lane + kb : kOutOfRange);
#pragma unroll
            for (int i = 0; i < MB; ++i)
                av[u][i] = load16(ra, ok ? a_lane + (uint32_t)i * a_block + kb : kOutOfRange);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < MB; ++i)
                acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bv[u], av[u][i], acc[i], 0, 0, 0);
    }

    // acc[i] lane: C[16 i + lane % 16][n0 + 4 (lane / 16) + r], r = 0..3.
#pragma unroll
    for (int i = 0; i < MB; ++i)
        red[wave][i][lane] = acc[i];
    __syncthreads();

    const bool vec_ok = (N & 3) == 0;
    const int n = n0 + lgrp * 4;
    for (int i = wave; i < MB; i += WK) {
        f32x4 sum = red[0][i][lane];
#pragma unroll
        for (int w = 1; w < WK; ++w)
            sum += red[w][i][lane];
        const int m = i * 16 + lrow;
        if (split_k == 1) {
            if (m < M) {
                const uint2 h = pack_bf16x4(sum);
                uint16_t* crow = C + (size_t)m * (size_t)N;
                if (vec_ok && n + 3 < N) {
                    *(uint2*)(crow + n) = h;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N)
                            crow[n + r] = bf16_elem(h, r);
                }
            }
        } else if (m < M) {
            float* prow = ws + ((size_t)blockIdx.y * (size_t)M + (size_t)m) * (size_t)N;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (n + r < N)
                    prow[n + r] = sum[r];
        }
    }
    if (split_k == 1)
        return;

    // Split-K: the last workgroup of this column block to finish sums the
    // partials in split order 0, 1, ... (deterministic) and rounds once.
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const int prev = atomicAdd(&counters[blockIdx.x], 1);
        last_flag = (prev == split_k - 1);
    }
    __syncthreads();
    if (!last_flag)
        return;
    __threadfence();
    const int cols = min(16, N - n0);
    for (int e = threadIdx.x; e < M * 16; e += WK * 64) {
        const int m = e >> 4;
        const int c = e & 15;
        if (c >= cols)
            continue;
        float sum = 0.f;
        for (int sp = 0; sp < split_k; ++sp)
            sum += ws[((size_t)sp * (size_t)M + (size_t)m) * (size_t)N + n0 + c];
        C[(size_t)m * (size_t)N + n0 + c] = __builtin_bit_cast(uint16_t, (__bf16)sum);
    }
    if (threadIdx.x == 0)
        counters[blockIdx.x] = 0;
}

template <int MB, int WK, int U>
hipError_t launch_skinny_t(const uint16_t* A, const uint16_t* B, uint16_t* C, int M, int N, int K,
                           int split_k, float* ws, int* counters, hipStream_t stream)
{
    const int col_blocks = (N + 15) / 16;
    hipLaunchKernelGGL((skinny_kernel<MB, WK, U>), dim3(col_blocks, split_k), dim3(WK * 64), 0, stream,
                       A, B, C, M, N, K, split_k, ws, counters);
    return hipGetLastError();
}

}  // namespace

SkinnyShape skinny_shape(int variant)
{
    switch (variant) {
    case SKINNY_M16: return {1, 16, 8};
    case SKINNY_M32: return {2, 16, 8};
    case SKINNY_M64: return {4, 16, 8};
    case SKINNY_M128: return {8, 16, 8};
    default: return {0, 0, 0};
    }
}

int skinny_lds_bytes(int variant)
{
    const SkinnyShape s = skinny_shape(variant);
    return s.waves * s.mblocks * 64 * 16 + 4;
}

hipError_t launch_skinny(int variant, const uint16_t* A, const uint16_t* B, uint16_t* C,
                         int M, int N, int K, int split_k, float* ws, int* counters,
                         hipStream_t stream)
{
    switch (variant) {
    case SKINNY_M16: return launch_skinny_t<1, 8, 8>(A, B, C, M, N, K, split_k, ws, counters, stream);
    case SKINNY_M32: return launch_skinny_t<2, 8, 4>(A, B, C, M, N, K, split_k, ws, counters, stream);
    case SKINNY_M64: return launch_skinny_t<4, 8, 2>(A, B, C, M, N, K, split_k, ws, counters, stream);
    case SKINNY_M128: return launch_skinny_t<8, 8, 2>(A, B, C, M, N, K, split_k, ws, counters, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace hkg
