// Skinny kernel for decode-shaped GEMMs (small M): C = A * B^T with B
// (the N x K weight) streamed from HBM exactly once.
//
// Design (gfx950, MI355X):
//  * A workgroup owns NB blocks of 16 columns of C (16 NB rows of B) and a K
//    range; its WK waves split that range further.  Every lane streams B
//    with 16-byte buffer loads, 8 k values of one B row per lane, 16 rows x
//    64 bytes per wave instruction.  All loads of a chunk of U 32-k steps are
//    issued together and two chunks are in flight, so many loads are in
//    flight per lane (decode GEMMs that keep too little in flight reach a
//    fraction of HBM bandwidth: hk-dsl page, SGLang decode-GEMM figure).
//  * The 16 x 32 B fragment is the first operand of v_mfma_f32_16x16x32_bf16;
//    each 16-row block of A (small, read from L2) is the second.  An A
//    fragment feeds NB MFMAs, so covering more B rows per workgroup cuts
//    the A bytes each compute unit must take in per B byte.
//  * With one 16-row block of A (bf16), each wave stages its share of A
//    through LDS: buffer -> LDS copies of 1 KB of consecutive row bytes per
//    instruction, then fragment reads from LDS.  Read straight into
//    registers, a fragment instruction touches 16 rows x 64 bytes, twice the
//    cache lines per byte, and every compute unit reads all of A (as many
//    bytes as its share of B) through its L1.
//  * Waves reduce through LDS in a fixed order (the wave-level reduction
//    followed by an LDS combine of the FlyDSL "Prebuilt kernels guide",
//    section 1.1).  Workgroups that share a column block along K (split-K)
//    write fp32 partials and the last one to arrive sums them in split
//    order (split-K on fp32 partials: same guide, section 3c).  The fused
//    epilogue (bias, activation) acts on the fp32 total, which is then
//    rounded to bf16 once.
//  * MXFP8 mode (E4M3 operands, E8M0 scale per 32 k; FlyDSL-in-PyTorch blog,
//    MXFP section): steps of 128 k, each lane loading the two 16-byte halves
//    of its scaled-MFMA operand (k 16 g .. and 64 + 16 g .., g = lane / 16)
//    from each B row, and its scale dwords from the packed layout of the
//    tile kernel (byte f of dword lane = block f of a 64-row group), or, with
//    NAT, straight from the natural M x K/32 and N x K/32 scale arrays: the
//    dword at row r, byte 4 s of the array holds the row's four blocks of
//    step s, and lane l takes byte l / 16 of it (row l % 16 of the block),
//    which is what the scaled MFMA reads with op_sel 0.
#include <type_traits>

#include "hkg_internal.h"
#include "hkg_lds_copy.h"

namespace hkg {
namespace {

typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

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

template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// MB: 16-row blocks of A (M <= 16 MB).  NB: 16-row blocks of B per
// workgroup.  WK: waves per workgroup, splitting K.  U: steps per chunk of
// loads (32 k, MXFP8 128 k).  CP: cache-policy bits of the B loads (B is
// streamed once).  AL: A staged through LDS (bf16, MB == 1).  MX: E4M3
// operands with packed E8M0 scales PSA / PSB (NAT: natural-layout scales,
// row stride K / 32 bytes).  F4 (with MX): MXFP4, E2M1 codes two per byte
// (rows of K / 2 bytes), steps of 256 k (128 bytes per row, as an MXFP8
// step): the lane's two 16-byte loads of a step are its operands for the
// step's two 128-k halves (format code 4), each with its own packed scales.
template <int MB, int NB, int WK, int U, int CP, bool AL, bool EPI, bool MX, bool NAT, bool F4 = false>
__global__ __launch_bounds__(WK * 64, 1)
void skinny_kernel(const void* __restrict__ Av, const void* __restrict__ Bv,
                   uint16_t* __restrict__ C, int M, int N, int K, int split_k,
                   float* __restrict__ ws, int* __restrict__ counters,
                   const uint16_t* __restrict__ bias, int epi, int lda, int ldb, int ldc,
                   const uint32_t* __restrict__ PSA, const uint32_t* __restrict__ PSB)
{
    constexpr int EB = MX ? 1 : 2;           // bytes per element (MXFP4: per two)
    constexpr int SK = F4 ? 256 : MX ? 128 : 32;   // k per step
    constexpr int SBY = F4 ? 128 : SK * EB;  // bytes of one row per step
    constexpr int KPP = F4 ? 32 : 16 / EB;   // k per 16-byte piece
    typedef std::conditional_t<MX, i32x8, i32x4> frag_t;
    static_assert(!MX || MB <= 4, "block-scaled skinny: one 64-row scale group of A");
    static_assert(MX || !NAT, "natural scales are MXFP8 only");
    static_assert(!F4 || (MX && !NAT), "MXFP4: packed scales");
    constexpr int NBLK = NB * MB;            // 16 x 16 output blocks per wave
    __shared__ f32x4 red[WK][NBLK][64];
    __shared__ int last_flag;
    // A through LDS: per wave two buffers of one chunk of A, 16 MB rows x
    // AROW bytes; row r holds its 16-byte piece c at position c ^ a_swz(r),
    // so 16 lanes reading one piece of 16 consecutive rows cover all 64
    // banks.  NCOPY copies of 1 KB fill a buffer.
    constexpr bool ALDS = AL;
    static_assert(!AL || MB <= 2, "A through LDS: one or two 16-row blocks");
    constexpr int AROW = U * SBY;                     // bytes of a row per chunk
    constexpr int ACH = AROW / 16;                    // 16-byte pieces per row
    constexpr int PPS = SBY / 16;                     // pieces per step
    constexpr int RPI = 1024 / AROW;                  // rows per copy instruction
    constexpr int ABUF = 16 * MB * AROW;
    constexpr int NCOPY = ABUF / 1024;
    static_assert(!ALDS || (AROW <= 1024 && 1024 % AROW == 0), "a chunk row divides a copy instruction");
    static_assert(!ALDS || WK * 2 * ABUF + WK * NBLK * 1024 <= 160 * 1024, "LDS is 160 KiB per CU");
    __shared__ __attribute__((aligned(16))) char a_lds[ALDS ? WK * 2 * ABUF : 16];
    auto a_swz = [](int r) {
        constexpr int RPB = AROW < 256 ? 256 / AROW : 1;  // rows per 64 banks
        constexpr int SW = ACH < 16 ? ACH : 16;
        return (r / RPB) % SW;
    };

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int n0 = blockIdx.x * (16 * NB);
    const int lrow = lane & 15;
    const int lgrp = lane >> 4;

    // K range, in 32-k steps: workgroup split first, then waves.  Wave w
    // takes slice (w + workgroup / 8) mod WK: workgroups are dispatched to
    // the 8 XCDs round-robin, so the ones sharing an XCD (and its L2) read
    // different parts of A at the same time.  Partial sums are combined in
    // slice order, so the result does not depend on the rotation.
    const int steps = (K + SK - 1) / SK;
    const int per_wg = (steps + split_k - 1) / split_k;
    const int wg_begin = min(steps, (int)blockIdx.y * per_wg);
    const int wg_end = min(steps, wg_begin + per_wg);
    const int per_wave = (wg_end - wg_begin + WK - 1) / WK;
    const int slice = (wave + (int)(blockIdx.x >> 3)) % WK;
    const int s_begin = min(wg_end, wg_begin + slice * per_wave);
    const int s_end = min(wg_end, s_begin + per_wave);

    // row strides in bytes (leading dimensions, in elements)
    const uint32_t a_rb = F4 ? (uint32_t)lda / 2u : (uint32_t)lda * (uint32_t)EB;
    const uint32_t b_rb = F4 ? (uint32_t)ldb / 2u : (uint32_t)ldb * (uint32_t)EB;
    const int rows_b = min(16 * NB, N - n0);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const char*)Bv + (size_t)n0 * b_rb), 0, (int)(rows_b * b_rb), kBufferWord3);
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        (void*)Av, 0, (int)((uint32_t)M * a_rb), kBufferWord3);
    const dma::i32x4 words_a = dma::rsrc_words(Av, (int)((uint32_t)M * a_rb));
    // MXFP8 scales: A's 16-row block i is byte i of the lane's dword of
    // group 0; B's block j is byte ((n0 + 16 j) / 16) % 4 of its group's dword.
    // Natural layout: rows past M (N) fall outside the range and read zero.
    const int KT = K / 128;
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
        (void*)PSA, 0, !MX ? 0 : NAT ? M * KT * 4 : ((M + 63) / 64) * KT * 256, kBufferWord3);
    const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
        (void*)PSB, 0, !MX ? 0 : NAT ? N * KT * 4 : ((N + 63) / 64) * KT * 256, kBufferWord3);

    const uint32_t lane_off_a = (uint32_t)lrow * a_rb + (uint32_t)lgrp * 16u;
    const uint32_t lane_off_b = (uint32_t)lrow * b_rb + (uint32_t)lgrp * 16u;
    const uint32_t block16_a = 16u * a_rb;      // next 16 rows
    const uint32_t block16_b = 16u * b_rb;

    // Fused epilogue: the bias of the first block this wave stores is loaded
    // now, so its memory round trip overlaps the K loop instead of following
    // the reduction.
    float bias_pre[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (EPI) {
        if (split_k == 1 && wave < NBLK) {
            const int n = n0 + (wave / MB) * 16 + lgrp * 4;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (n + r < N)
                    bias_pre[r] = __uint_as_float((uint32_t)bias[n + r] << 16);
        }
    }

    f32x4 acc[NB][MB];
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int i = 0; i < MB; ++i)
            acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Steps past s_end (or k past K) load from an out-of-range offset and
    // read zero, which the MFMA adds exactly; so chunks need no tail code.
    // MXFP8 operands are the bytes at k 16 g .. and 64 + 16 g .. of the step;
    // MXFP4 operands of the step's two halves are the bytes at 16 g .. and
    // 64 + 16 g .. (the second half past K when K % 256 == 128: ok_hi).
    auto load_frag = [&](__amdgpu_buffer_rsrc_t r, uint32_t off, bool ok, bool ok_hi, auto cp) -> frag_t {
        constexpr int P = decltype(cp)::value;
        if constexpr (MX) {
            const i32x4 lo = load16<P>(r, ok ? off : kOutOfRange);
            const i32x4 hi = load16<P>(r, ok_hi ? off + 64u : kOutOfRange);
            return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        } else {
            return load16<P>(r, ok ? off : kOutOfRange);
        }
    };
    // A through LDS: the chunk of U steps from step s into buffer abuf of
    // this wave (NCOPY copies; the earlier fragment reads of that buffer
    // have finished first), and its fragments out of the buffer: piece
    // PPS u + g of the row for bf16, pieces PPS u + g and PPS u + 4 + g for
    // the two halves of an MXFP8 operand (g = lane / 16).
    auto copy_a_chunk = [&](int s, int abuf) {
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        const char* dst = a_lds + (wave * 2 + abuf) * ABUF;
#pragma unroll
        for (int q = 0; q < NCOPY; ++q) {
            const int r = q * RPI + lane / ACH;
            const int c = (lane % ACH) ^ a_swz(r);
            const int step = s + c / PPS;
            const bool ok = step < s_end && step * SK + (c % PPS) * KPP < K;
            dma::copy_to_lds(words_a, dst + q * 1024,
                             ok ? (uint32_t)r * a_rb + (uint32_t)step * SBY + (uint32_t)(c % PPS) * 16u
                                : kOutOfRange);
        }
    };
    auto read_a_chunk = [&](int abuf, frag_t (&av)[U][MB]) {
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const char* src = a_lds + (wave * 2 + abuf) * ABUF + (16 * i + lrow) * AROW;
            const int sw = a_swz(16 * i + lrow);
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if constexpr (MX) {
                    const i32x4 lo = *(const i32x4*)(src + ((PPS * u + lgrp) ^ sw) * 16);
                    const i32x4 hi = *(const i32x4*)(src + ((PPS * u + 4 + lgrp) ^ sw) * 16);
                    av[u][i] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                } else {
                    av[u][i] = *(const frag_t*)(src + ((PPS * u + lgrp) ^ sw) * 16);
                }
            }
        }
    };
    // Scale dwords per step: MXFP8 one for A and one per B block (natural
    // layout: one per A row block); MXFP4 the same for each 128-k half.
    constexpr int SWA = F4 ? 2 : MX ? (NAT ? MB : 1) : 0, SWB = F4 ? 2 * NB : MX ? NB : 0;
    constexpr bool NAT_RUN_CHUNK = NAT && AL && (U == 2 || U == 4);
    auto load_chunk = [&](int s, int abuf, frag_t (&bv)[U][NB], frag_t (&av)[U][MB], uint32_t (&sa)[U][SWA + 1],
                          uint32_t (&sb)[U][SWB + 1]) {
        if constexpr (ALDS)
            copy_a_chunk(s, abuf);
        // Natural-layout scales (A through LDS): when the chunk's steps lie
        // inside the row, one 4 U-byte load per row takes them all (steps
        // past the wave's range are zeroed: their data reads zero);
        // otherwise a dword per row and step.
        constexpr bool NAT_RUN = NAT_RUN_CHUNK;
        const bool run = NAT_RUN && s + U <= KT;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int step = s + u;
            const bool ok = step < s_end && step * SK + lgrp * KPP < K;
            const bool ok_hi = F4 ? ok && step * SK + 128 < K : ok;
            const uint32_t kb = (uint32_t)step * (uint32_t)SBY;
#pragma unroll
            for (int j = 0; j < NB; ++j)
                bv[u][j] = load_frag(rb, lane_off_b + kb + (uint32_t)j * block16_b, ok, ok_hi,
                                     std::integral_constant<int, CP>{});
            if constexpr (!ALDS) {
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    av[u][i] = load_frag(ra, lane_off_a + kb + (uint32_t)i * block16_a, ok, ok_hi,
                                         std::integral_constant<int, 0>{});
            }
            if constexpr (NAT) {
                // row r's dword of step s at byte (r KT + s) 4; this lane's
                // scale is byte lgrp (shifted down when it is used)
                if (!run) {
#pragma unroll
                    for (int i = 0; i < MB; ++i)
                        sa[u][i] = __builtin_amdgcn_raw_buffer_load_b32(
                            rsa, ok ? (uint32_t)((16 * i + lrow) * KT + step) * 4u : kOutOfRange, 0, 0);
#pragma unroll
                    for (int j = 0; j < NB; ++j)
                        sb[u][j] = __builtin_amdgcn_raw_buffer_load_b32(
                            rsb, ok ? (uint32_t)((n0 + 16 * j + lrow) * KT + step) * 4u : kOutOfRange, 0, 0);
                }
            } else if constexpr (F4) {
                // 128-k halves 2 step and 2 step + 1 (a half past K reads
                // zero: the finite scale 2^-127 on zero data)
#pragma unroll
                for (int q = 0; q < 2; ++q) {
                    const bool okq = q == 0 ? ok : ok_hi;
                    const uint32_t st = (uint32_t)(2 * step + q) * 256u + (uint32_t)lane * 4u;
                    sa[u][q] = __builtin_amdgcn_raw_buffer_load_b32(rsa, okq ? st : kOutOfRange, 0, 0);
#pragma unroll
                    for (int j = 0; j < NB; ++j) {
                        const int row = n0 + 16 * j;
                        sb[u][2 * j + q] = __builtin_amdgcn_raw_buffer_load_b32(
                            rsb, okq ? (uint32_t)((row / 64) * KT) * 256u + st : kOutOfRange, 0, 0);
                    }
                }
            } else if constexpr (MX) {
                const uint32_t st = (uint32_t)step * 256u + (uint32_t)lane * 4u;
                sa[u][0] = __builtin_amdgcn_raw_buffer_load_b32(rsa, ok ? st : kOutOfRange, 0, 0);
#pragma unroll
                for (int j = 0; j < NB; ++j) {
                    const int row = n0 + 16 * j;
                    sb[u][j] = __builtin_amdgcn_raw_buffer_load_b32(
                        rsb, ok ? (uint32_t)((row / 64) * KT) * 256u + st : kOutOfRange, 0, 0);
                }
            }
        }
        if constexpr (NAT_RUN) {
            if (run) {
                auto take = [&](__amdgpu_buffer_rsrc_t r, int row, auto&& put) {
                    const uint32_t off = (uint32_t)(row * KT + s) * 4u;
                    uint32_t w[U];
                    if constexpr (U == 4) {
                        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
#pragma unroll
                        for (int u = 0; u < 4; ++u)
                            w[u] = v[u];
                    } else {
                        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
                        w[0] = v[0];
                        w[1] = v[1];
                    }
#pragma unroll
                    for (int u = 0; u < U; ++u)
                        put(u, s + u < s_end ? w[u] : 0u);
                };
#pragma unroll
                for (int i = 0; i < MB; ++i)
                    take(rsa, 16 * i + lrow, [&](int u, uint32_t x) { sa[u][i] = x; });
#pragma unroll
                for (int j = 0; j < NB; ++j)
                    take(rsb, n0 + 16 * j + lrow, [&](int u, uint32_t x) { sb[u][j] = x; });
            }
        }
    };
    auto mfma_chunk = [&](const frag_t (&bv)[U][NB], const frag_t (&av)[U][MB], const uint32_t (&sa)[U][SWA + 1],
                          const uint32_t (&sb)[U][SWB + 1]) {
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int j = 0; j < NB; ++j) {
                if constexpr (NAT) {
                    const int bsc = (int)(sb[u][j] >> (8 * lgrp));
                    static_for<0, MB>([&](auto I) {
                        constexpr int i = decltype(I)::value;
                        acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            bv[u][j], av[u][i], acc[j][i], 0, 0, 0, bsc, 0, (int)(sa[u][i] >> (8 * lgrp)));
                    });
                } else if constexpr (F4) {
                    // half q: the first four registers of the operand
                    static_for<0, 2>([&](auto Q) {
                        constexpr int q = decltype(Q)::value;
                        const i32x8 bq = __builtin_shufflevector(bv[u][j], i32x8{}, 4 * q, 4 * q + 1, 4 * q + 2,
                                                                 4 * q + 3, 8, 9, 10, 11);
                        const int bsc = (int)(sb[u][2 * j + q] >> (8 * (((n0 + 16 * j) >> 4) & 3)));
                        static_for<0, MB>([&](auto I) {
                            constexpr int i = decltype(I)::value;
                            const i32x8 aq = __builtin_shufflevector(av[u][i], i32x8{}, 4 * q, 4 * q + 1,
                                                                     4 * q + 2, 4 * q + 3, 8, 9, 10, 11);
                            acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                bq, aq, acc[j][i], 4, 4, 0, bsc, i, (int)sa[u][q]);
                        });
                    });
                } else if constexpr (MX) {
                    const int bsc = (int)(sb[u][j] >> (8 * (((n0 + 16 * j) >> 4) & 3)));
                    static_for<0, MB>([&](auto I) {
                        constexpr int i = decltype(I)::value;
                        acc[j][i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            bv[u][j], av[u][i], acc[j][i], 0, 0, 0, bsc, i, (int)sa[u][0]);
                    });
                } else {
#pragma unroll
                    for (int i = 0; i < MB; ++i)
                        acc[j][i] = mfma16(bv[u][j], av[u][i], acc[j][i]);
                }
            }
    };

    // Chunks c and c + 1 are in flight while chunk c is multiplied.  Empty
    // asm statements keep the compiler from sinking the next chunk's loads
    // below the current chunk's MFMAs (which would put one full memory round
    // trip per chunk on the critical path).  (The compiler's own waits count
    // a conditionally loaded chunk as not issued, so past the first two
    // chunks they also drain the next chunk before the current one's last
    // MFMA; loading past the end unconditionally to keep its counts exact
    // measured slower, 11.8 vs 10.4 us at 16 x 4096 x 4096: out-of-range
    // loads still cost their issue and return.)
    auto fence = [] { asm volatile("" ::: "memory"); };
    // A through LDS: a chunk's A copies are issued before its B loads, and
    // chunk c + 1 (if any) before chunk c is multiplied, so waiting for the
    // copies of chunk c leaves its B loads and chunk c + 1 in flight.
    // Vector-memory instructions a chunk issues after its A copies: B (two
    // per fragment for MXFP8) and the scale loads (the fewest a chunk can
    // issue: natural scales may come as one load per row; a chunk that
    // issues more only makes this wait stricter).
    constexpr int SCL = !MX ? 0 : NAT_RUN_CHUNK ? SWA + SWB : U * (SWA + SWB);
    constexpr int LPC = U * NB * (MX ? 2 : 1) + SCL;
    static_assert(2 * LPC + NCOPY <= 63, "vmcnt holds at most 63");
    auto wait_a = [&](bool next) {
        if constexpr (ALDS) {
            if (next)
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LPC + NCOPY) : "memory");
            else
                asm volatile("s_waitcnt vmcnt(%0)" ::"n"(LPC) : "memory");
        }
    };
    frag_t b0[U][NB], a0[U][MB], b1[U][NB], a1[U][MB];
    uint32_t sa0[U][SWA + 1], sb0[U][SWB + 1], sa1[U][SWA + 1], sb1[U][SWB + 1];
    const int nch = (s_end - s_begin + U - 1) / U;
    if (nch > 0) {
        load_chunk(s_begin, 0, b0, a0, sa0, sb0);
        fence();
        if (nch > 1)
            load_chunk(s_begin + U, 1, b1, a1, sa1, sb1);
        fence();
        for (int c = 0; c < nch; c += 2) {
            if constexpr (ALDS) {
                wait_a(c + 1 < nch);
                read_a_chunk(0, a0);
            }
            mfma_chunk(b0, a0, sa0, sb0);
            fence();
            if (c + 2 < nch)
                load_chunk(s_begin + (c + 2) * U, 0, b0, a0, sa0, sb0);
            fence();
            if (c + 1 >= nch)      // odd chunk count: buffer 1 holds an old chunk
                break;
            if constexpr (ALDS) {
                wait_a(c + 2 < nch);
                read_a_chunk(1, a1);
            }
            mfma_chunk(b1, a1, sa1, sb1);
            fence();
            if (c + 3 < nch)
                load_chunk(s_begin + (c + 3) * U, 1, b1, a1, sa1, sb1);
            fence();
        }
    }

    // acc[j][i] lane: C[16 i + lane % 16][n0 + 16 j + 4 (lane / 16) + r], r = 0..3.
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int i = 0; i < MB; ++i)
            red[slice][j * MB + i][lane] = acc[j][i];
    __syncthreads();

    const bool vec_ok = ((N | ldc) & 3) == 0;
    for (int b = wave; b < NBLK; b += WK) {
        f32x4 sum = red[0][b][lane];
#pragma unroll
        for (int w = 1; w < WK; ++w)
            sum += red[w][b][lane];
        const int m = (b % MB) * 16 + lrow;
        const int n = n0 + (b / MB) * 16 + lgrp * 4;
        if (m >= M)
            continue;
        if (split_k == 1) {
            if (EPI) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < N)
                        sum[r] = b == wave ? epi_activation(sum[r] + bias_pre[r], epi)
                                           : epi_apply(sum[r], bias, n + r, epi);
            }
            const uint2 h = pack_bf16x4(sum);
            uint16_t* crow = C + (size_t)m * (size_t)ldc;
            if (vec_ok && n + 3 < N) {
                *(uint2*)(crow + n) = h;
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < N)
                        crow[n + r] = bf16_elem(h, r);
            }
        } else {
            float* prow = ws + ((size_t)blockIdx.y * (size_t)M + (size_t)m) * (size_t)N;
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (n + r < N)
                    __hip_atomic_store(prow + n + r, sum[r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (split_k == 1)
        return;

    // Split-K: the last workgroup of this column block to finish sums the
    // partials in split order 0, 1, ... (deterministic) and rounds once.
    // Partials are written and read with device-scope accesses (coherent
    // across the XCDs' L2 caches without flushing them); every store has
    // completed (vmcnt) before the workgroup's arrival is counted (the
    // ordering argument is the split-K arrival protocol in hkg_internal.h).
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const int prev = __hip_atomic_fetch_add(&counters[blockIdx.x], 1, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
        last_flag = (prev == split_k - 1);
    }
    __syncthreads();
    if (!last_flag)
        return;
    const int cols = min(16 * NB, N - n0);
    for (int e = threadIdx.x; e < M * 16 * NB; e += WK * 64) {
        const int m = e / (16 * NB);
        const int c = e - m * (16 * NB);
        if (c >= cols)
            continue;
        float sum = 0.f;
        for (int sp = 0; sp < split_k; ++sp)
            sum += __hip_atomic_load(ws + ((size_t)sp * (size_t)M + (size_t)m) * (size_t)N + n0 + c,
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (EPI)
            sum = epi_apply(sum, bias, n0 + c, epi);
        C[(size_t)m * (size_t)ldc + n0 + c] = __builtin_bit_cast(uint16_t, (__bf16)sum);
    }
    if (threadIdx.x == 0)
        __hip_atomic_store(&counters[blockIdx.x], 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int MB, int NB, int WK, int U, int CP, bool AL, bool EPI, bool MX, bool NAT, bool F4 = false>
hipError_t launch_skinny_t(const void* A, const void* B, uint16_t* C, int M, int N, int K, int split_k, float* ws,
                           int* counters, const uint16_t* bias, int epi, int lda, int ldb, int ldc,
                           const uint32_t* psa, const uint32_t* psb, hipStream_t stream)
{
    const int col_blocks = (N + 16 * NB - 1) / (16 * NB);
    hipLaunchKernelGGL((skinny_kernel<MB, NB, WK, U, CP, AL, EPI, MX, NAT, F4>), dim3(col_blocks, split_k), dim3(WK * 64), 0,
                       stream, A, B, C, M, N, K, split_k, ws, counters, bias, epi, lda, ldb, ldc, psa, psb);
    return hipGetLastError();
}

}  // namespace

SkinnyShape skinny_shape(int variant)
{
    int v = 0;
#define HKG_SHAPE(mb, nb, wk, u, cp, al) \
    if (v++ == variant)                  \
        return SkinnyShape{mb, nb, wk, u, cp, al};
    HKG_SKINNY_CONFIGS(HKG_SHAPE)
#undef HKG_SHAPE
    return SkinnyShape{0, 0, 0, 0, 0, 0};
}

int skinny_lds_bytes(int variant)
{
    const SkinnyShape s = skinny_shape(variant);
    const int a_bufs = s.a_lds ? s.waves * 2 * 16 * s.unroll * 64 : 0;   // A through LDS
    return s.waves * s.mblocks * s.nblocks * 64 * 16 + a_bufs + 4;
}

hipError_t launch_skinny(int variant, const uint16_t* A, const uint16_t* B, uint16_t* C,
                         int M, int N, int K, int split_k, float* ws, int* counters,
                         const uint16_t* bias, int epi, int lda, int ldb, int ldc, hipStream_t stream)
{
    int v = 0;
#define HKG_LAUNCH(mb, nb, wk, u, cp, al)                                                                          \
    if (v++ == variant)                                                                                       \
        return epi == EPI_NONE                                                                                \
                   ? launch_skinny_t<mb, nb, wk, u, cp, al, false, false, false>(A, B, C, M, N, K, split_k, ws,  \
                                                                                 counters, bias, epi, lda, ldb,  \
                                                                                 ldc, nullptr, nullptr, stream)  \
                   : launch_skinny_t<mb, nb, wk, u, cp, al, true, false, false>(A, B, C, M, N, K, split_k, ws,   \
                                                                                counters, bias, epi, lda, ldb,   \
                                                                                ldc, nullptr, nullptr, stream);
    HKG_SKINNY_CONFIGS(HKG_LAUNCH)
#undef HKG_LAUNCH
    return hipErrorInvalidValue;
}

SkinnyShape mx_skinny_shape(int variant)
{
    int v = 0;
#define HKG_SHAPE(mb, nb, wk, u, cp, al) \
    if (v++ == variant)                  \
        return SkinnyShape{mb, nb, wk, u, cp, al};
    HKG_MX_SKINNY_CONFIGS(HKG_SHAPE)
#undef HKG_SHAPE
    return SkinnyShape{0, 0, 0, 0, 0, 0};
}

int mx_skinny_lds_bytes(int variant)
{
    const SkinnyShape s = mx_skinny_shape(variant);
    const int a_bufs = s.a_lds ? s.waves * 2 * 16 * s.mblocks * s.unroll * 128 : 0;   // A through LDS
    return s.waves * s.mblocks * s.nblocks * 64 * 16 + a_bufs + 4;
}

hipError_t launch_skinny_mx(int variant, const uint8_t* A, const uint8_t* B, uint16_t* C, int M, int N, int K,
                            int split_k, float* ws, int* counters, const uint16_t* bias, int epi,
                            const uint32_t* psa, const uint32_t* psb, bool natural, hipStream_t stream)
{
    int v = 0;
#define HKG_LAUNCH_NAT(mb, nb, wk, u, cp, al, nat)                                                              \
    return epi == EPI_NONE ? launch_skinny_t<mb, nb, wk, u, cp, al, false, true, nat>(                            \
                                 A, B, C, M, N, K, split_k, ws, counters, bias, epi, K, K, N, psa, psb, stream)   \
                           : launch_skinny_t<mb, nb, wk, u, cp, al, true, true, nat>(                             \
                                 A, B, C, M, N, K, split_k, ws, counters, bias, epi, K, K, N, psa, psb, stream);
#define HKG_LAUNCH(mb, nb, wk, u, cp, al)              \
    if (v++ == variant) {                              \
        if (natural)                                   \
            HKG_LAUNCH_NAT(mb, nb, wk, u, cp, al, true) \
        HKG_LAUNCH_NAT(mb, nb, wk, u, cp, al, false)   \
    }
    HKG_MX_SKINNY_CONFIGS(HKG_LAUNCH)
#undef HKG_LAUNCH
#undef HKG_LAUNCH_NAT
    return hipErrorInvalidValue;
}

SkinnyShape mx4_skinny_shape(int variant)
{
    int v = 0;
#define HKG_SHAPE(mb, nb, wk, u, cp, al) \
    if (v++ == variant)                  \
        return SkinnyShape{mb, nb, wk, u, cp, al};
    HKG_MX4_SKINNY_CONFIGS(HKG_SHAPE)
#undef HKG_SHAPE
    return SkinnyShape{0, 0, 0, 0, 0, 0};
}

int mx4_skinny_lds_bytes(int variant)
{
    const SkinnyShape s = mx4_skinny_shape(variant);
    const int a_bufs = s.a_lds ? s.waves * 2 * 16 * s.mblocks * s.unroll * 128 : 0;   // A through LDS
    return s.waves * s.mblocks * s.nblocks * 64 * 16 + a_bufs + 4;
}

// Packed scales only; leading dimensions in elements (K).
hipError_t launch_skinny_mx4(int variant, const uint8_t* A, const uint8_t* B, uint16_t* C, int M, int N, int K,
                             int split_k, float* ws, int* counters, const uint16_t* bias, int epi,
                             const uint32_t* psa, const uint32_t* psb, hipStream_t stream)
{
    int v = 0;
#define HKG_LAUNCH(mb, nb, wk, u, cp, al)                                                                        \
    if (v++ == variant)                                                                                     \
        return epi == EPI_NONE ? launch_skinny_t<mb, nb, wk, u, cp, al, false, true, false, true>(            \
                                     A, B, C, M, N, K, split_k, ws, counters, bias, epi, K, K, N, psa, psb, stream) \
                               : launch_skinny_t<mb, nb, wk, u, cp, al, true, true, false, true>(             \
                                     A, B, C, M, N, K, split_k, ws, counters, bias, epi, K, K, N, psa, psb, stream);
    HKG_MX4_SKINNY_CONFIGS(HKG_LAUNCH)
#undef HKG_LAUNCH
    return hipErrorInvalidValue;
}

}  // namespace hkg
