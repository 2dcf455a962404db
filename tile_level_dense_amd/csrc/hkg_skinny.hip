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
typedef __attribute__((address_space(3))) void lds_void;

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

// Loaded fragments stay int vectors until the MFMA: bf16 vectors carried
// through loop phis get repacked element by element, which forces a wait on
// the load right after it is issued.
template <int CP>
__device__ __forceinline__ i32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off)
{
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CP);
}

__device__ __forceinline__ f32x4 mfma16(i32x4 b, i32x4 a, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, b), __builtin_bit_cast(bf16x8, a),
                                                   c, 0, 0, 0);
}

// MB: 16-row blocks of A (M <= 16 MB).  WK: waves per workgroup, splitting
// K.  U: 32-k steps per chunk of loads; two chunks are in flight per wave
// (the next chunk's loads are issued before the current chunk's MFMAs).
// CP: cache-policy bits of the B loads (B is streamed once).
// AL: 1 = each wave copies its A chunks into its own LDS region with
// contiguous full-line buffer->LDS copies and reads MFMA fragments from
// there; 0 = A fragments are loaded straight from global memory (16 rows x
// 64 bytes per instruction, half cache lines).
template <int MB, int WK, int U, int CP, int AL>
__global__ __launch_bounds__(WK * 64, 1)
void skinny_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                   uint16_t* __restrict__ C, int M, int N, int K, int split_k,
                   float* __restrict__ ws, int* __restrict__ counters)
{
    __shared__ f32x4 red[WK][MB][64];
    __shared__ int last_flag;
    // A staging (AL = 1): per wave two chunk buffers of 16 MB rows x U*64
    // bytes; 16-byte chunk c of row r sits at position c ^ (r % 16), so a
    // fragment read (16 rows, one chunk) hits 16 distinct bank groups.
    constexpr int RS = U * 64;                    // bytes of one row of a chunk
    constexpr int A_CHUNK = 16 * MB * RS;         // bytes of one wave's chunk
    constexpr int RPI = 1024 / RS;                // rows per 1 KB copy
    constexpr int CPRW = RS / 16;                 // 16-byte chunks per row
    constexpr int NCOPY = AL ? 16 * MB / RPI : 0; // copies per chunk
    static_assert(!AL || (RS <= 1024 && 1024 % RS == 0 && CPRW >= 16), "chunk rows must tile 1 KB copies");
    __shared__ __attribute__((aligned(1024))) char a_lds[AL ? WK * 2 * A_CHUNK : 16];

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
    // Wave w takes K slice (w + workgroup) mod WK, so workgroups that run
    // at the same time read different parts of A (which every workgroup
    // reads) instead of all hitting the same L2 channels together.  Partial
    // sums are combined in slice order, so the result does not depend on
    // the rotation.
    const int per_wave = (wg_end - wg_begin + WK - 1) / WK;
    const int slice = (wave + (int)blockIdx.x) % WK;
    const int s_begin = min(wg_end, wg_begin + slice * per_wave);
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

    // Steps past s_end (or k past K) load from an out-of-range offset and
    // read zero, which the MFMA adds exactly; so chunks need no tail code.
    auto load_chunk = [&](int s, i32x4 (&bv)[U], i32x4 (&av)[U][MB]) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int step = s + u;
            const bool ok = step < s_end && step * 32 + lgrp * 8 < K;
            const uint32_t kb = (uint32_t)step * 64u;
            bv[u] = load16<CP>(rb, ok ? b_lane + kb : kOutOfRange);
            if constexpr (!AL) {
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    av[u][i] = load16<0>(ra, ok ? a_lane + (uint32_t)i * a_block + kb : kOutOfRange);
            }
        }
    };
    auto mfma_chunk = [&](const i32x4 (&bv)[U], const i32x4 (&av)[U][MB]) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < MB; ++i)
                acc[i] = mfma16(bv[u], av[u][i], acc[i]);
    };

    i32x4 b0[U], a0[U][MB], b1[U], a1[U][MB];
    // Empty asm statements keep the compiler from sinking the next chunk's
    // loads below the current chunk's MFMAs (which would put one full memory
    // round trip per chunk on the critical path).
    auto fence = [] { asm volatile("" ::: "memory"); };
    if constexpr (!AL) {
        // Chunks c and c + 1 are in flight while chunk c is multiplied.
        const int nch = (s_end - s_begin + U - 1) / U;
        if (nch > 0) {
            load_chunk(s_begin, b0, a0);
            fence();
            load_chunk(s_begin + U, b1, a1);
            fence();
            for (int c = 0; c < nch; c += 2) {
                mfma_chunk(b0, a0);
                fence();
                if (c + 2 < nch)
                    load_chunk(s_begin + (c + 2) * U, b0, a0);
                fence();
                if (c + 1 >= nch)      // odd chunk count: buffer 1 holds an old chunk
                    break;
                mfma_chunk(b1, a1);
                fence();
                if (c + 3 < nch)
                    load_chunk(s_begin + (c + 3) * U, b1, a1);
                fence();
            }
        }
    } else {
        char* my_lds = a_lds + wave * 2 * A_CHUNK;
        const int cr = lane / CPRW;               // row within a copy
        const int cp = lane % CPRW;               // LDS position within the row
        // Copy of A chunk (steps s .. s + U - 1) into buffer `buf`: copy j
        // fills rows j RPI .. j RPI + RPI - 1; lane -> row j RPI + cr,
        // position cp, which holds k-chunk cp ^ (row % 16).
        auto copy_a = [&](int s, int buf) {
            char* dst = my_lds + buf * A_CHUNK;
            const bool live = s < s_end;
#pragma unroll
            for (int j = 0; j < NCOPY; ++j) {
                const int row = j * RPI + cr;
                const int c = cp ^ (row & 15);
                const bool ok = live && s * 32 + c * 8 < K;
                const uint32_t off = (uint32_t)row * row_bytes + (uint32_t)s * 64u + (uint32_t)c * 16u;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(dst + j * 1024), 16,
                                                         ok ? off : kOutOfRange, 0, 0, 0);
            }
        };
        // This wave's copy of `buf` has landed once at most 2 U + NCOPY of
        // its later memory operations are in flight (loads complete in
        // order): the chunk's own B loads and the next chunk's copies and
        // B loads.
        auto read_a = [&](int buf, i32x4 (&av)[U][MB]) {
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * U + NCOPY) : "memory");
            const char* src = my_lds + buf * A_CHUNK;
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int i = 0; i < MB; ++i) {
                    const int row = i * 16 + lrow;
                    const int c = (u * 4 + lgrp) ^ lrow;
                    av[u][i] = *(const i32x4*)(src + row * RS + c * 16);
                }
        };
        // The wait counts in read_a rely on this issue order (copy, then B
        // loads, chunk after chunk); the fences keep it.
        if (s_begin < s_end) {
            copy_a(s_begin, 0);
            fence();
            load_chunk(s_begin, b0, a0);
            fence();
            for (int s = s_begin; s < s_end; s += 2 * U) {
                copy_a(s + U, 1);
                fence();
                load_chunk(s + U, b1, a1);
                fence();
                read_a(0, a0);
                mfma_chunk(b0, a0);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // buffer 0 read before refilled
                copy_a(s + 2 * U, 0);
                fence();
                load_chunk(s + 2 * U, b0, a0);
                fence();
                read_a(1, a1);
                mfma_chunk(b1, a1);
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // buffer 1 read before refilled
            }
            // no copy into LDS may be in flight past this point
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
    }

    // acc[i] lane: C[16 i + lane % 16][n0 + 4 (lane / 16) + r], r = 0..3.
#pragma unroll
    for (int i = 0; i < MB; ++i)
        red[slice][i][lane] = acc[i];
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

template <int MB, int WK, int U, int CP, int AL>
hipError_t launch_skinny_t(const uint16_t* A, const uint16_t* B, uint16_t* C, int M, int N, int K,
                           int split_k, float* ws, int* counters, hipStream_t stream)
{
    const int col_blocks = (N + 15) / 16;
    hipLaunchKernelGGL((skinny_kernel<MB, WK, U, CP, AL>), dim3(col_blocks, split_k), dim3(WK * 64), 0, stream,
                       A, B, C, M, N, K, split_k, ws, counters);
    return hipGetLastError();
}

}  // namespace

SkinnyShape skinny_shape(int variant)
{
    int v = 0;
#define HKG_SHAPE(mb, wk, u, cp, al) \
    if (v++ == variant)          \
        return SkinnyShape{mb, 16, wk, u, cp, al};
    HKG_SKINNY_CONFIGS(HKG_SHAPE)
#undef HKG_SHAPE
    return SkinnyShape{0, 0, 0, 0, 0, 0};
}

int skinny_default_variant(int64_t M)
{
    // smallest MB that covers M; among equal MB the first listed
    int best = -1, best_mb = 1 << 30;
    for (int v = 0; v < SKINNY_NUM_VARIANTS; ++v) {
        const SkinnyShape s = skinny_shape(v);
        if (16 * (int64_t)s.mblocks >= M && s.mblocks < best_mb) {
            best = v;
            best_mb = s.mblocks;
        }
    }
    return best;
}

int skinny_lds_bytes(int variant)
{
    const SkinnyShape s = skinny_shape(variant);
    return s.waves * s.mblocks * 64 * 16 + 4 + (s.a_lds ? s.waves * 2 * 16 * s.mblocks * s.unroll * 64 : 0);
}

hipError_t launch_skinny(int variant, const uint16_t* A, const uint16_t* B, uint16_t* C,
                         int M, int N, int K, int split_k, float* ws, int* counters,
                         hipStream_t stream)
{
    int v = 0;
#define HKG_LAUNCH(mb, wk, u, cp, al) \
    if (v++ == variant)               \
        return launch_skinny_t<mb, wk, u, cp, al>(A, B, C, M, N, K, split_k, ws, counters, stream);
    HKG_SKINNY_CONFIGS(HKG_LAUNCH)
#undef HKG_LAUNCH
    return hipErrorInvalidValue;
}

}  // namespace hkg
