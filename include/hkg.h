/*
 * hkg.h -- C ABI of the MI355X (gfx950) dense BF16 GEMM library.
 *
 * Operation (one call computes all of it):
 *
 *     C[i][j] = bf16( sum over k of A[i][k] * B[j][k] ),   0 <= i < M, 0 <= j < N
 *
 *   A is M x K and B is N x K, both row-major with K contiguous (the "NT"
 *   layout of the FlyDSL-in-PyTorch blog post, section "Dense GEMM", and of
 *   the FlyDSL "Prebuilt kernels guide", section 3.1 Preshuffle GEMM:
 *   C[M,N] = A[M,K] @ B[N,K]^T, whose K axis has unit stride in both
 *   operands).  C is M x N row-major.  Products of bf16 values are summed in
 *   fp32 (matrix-core accumulation) and each output is rounded once to bf16,
 *   nearest-even (the gfx950 hardware conversion cvt_pk_bf16_f32, named in
 *   the same guide's section 1.1 "bf16 handling").
 *
 *   The summation order is an implementation detail, fixed for a given plan:
 *   the same plan on the same inputs gives bit-identical results.
 *
 * Memory and ownership
 *   A, B, C are device pointers owned by the caller; the library never
 *   allocates, frees or retains them.  Element type is bf16 (raw 16-bit
 *   patterns).  C must not overlap A or B.  The fast kernels need A, B and C
 *   16-byte aligned and K a multiple of 8; other inputs run a slower,
 *   general kernel (hkg_gemm_bf16) -- nothing is ever rejected for alignment
 *   by hkg_gemm_bf16 itself.
 *   `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *   calls are asynchronous with respect to the host; faults inside a kernel
 *   surface at the caller's next synchronisation, as in HIP.
 *   The library keeps per-device state (device checks) and per-(device,
 *   stream) workspaces: the split-K fp32 partials and arrival counters, the
 *   packed scales of hkg_gemm_mxfp8 and the row-layout copies of
 *   hkg_gemm_bf16_ex.  A workspace is allocated by the first call on that
 *   stream that needs it (outside stream capture: growing one while the
 *   stream is being captured returns HKG_ERR_WORKSPACE, so run a call once
 *   before capturing it) and grows geometrically; an outgrown buffer is kept,
 *   not freed, until the library is unloaded, because a launch in flight or
 *   a captured graph may still use it.
 *
 * Errors
 *   Every argument check happens on the host, before any launch, and is
 *   reported as a status code; nothing is thrown across this ABI.
 *
 * Thread safety
 *   Calls may be made from several host threads and on several streams at
 *   once: each stream has its own workspaces, so calls on different streams
 *   never share scratch, and calls on one stream are ordered by the stream.
 *   (hipStreamPerThread has one workspace per host thread.)  Two cases do
 *   share scratch: a graph captured on stream S uses S's workspace when it
 *   is replayed, so it must not be replayed concurrently with other calls on
 *   S or with another replay of a graph captured on S; and a stream handle
 *   reused after hipStreamDestroy gets the old stream's workspace, so the old
 *   stream's work must have finished first.  Plans are computed per call;
 *   there is no shared plan cache.
 */
#ifndef HKG_H
#define HKG_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define HKG_ABI_VERSION 1

typedef enum {
    HKG_OK = 0,
    HKG_ERR_INVALID_ARG = -1,   /* null pointer with nonzero size, negative dims, a dim >= 2^31,
                                   a matrix of 2^40 or more elements, C overlapping A or B */
    HKG_ERR_MISALIGNED = -2,    /* run_plan with a fast-kernel plan on unaligned pointers or K % 8 != 0 */
    HKG_ERR_UNSUPPORTED = -3,   /* a plan the library cannot run (e.g. edited into an invalid state) */
    HKG_ERR_NO_DEVICE = -4,     /* no HIP device is visible */
    HKG_ERR_ARCH = -5,          /* the current device is not gfx950 */
    HKG_ERR_HIP = -6,           /* a HIP runtime call or launch failed; see hkg_last_hip_error */
    HKG_ERR_WORKSPACE = -7      /* a library workspace (split-K partials, packed MXFP8 scales, layout copies)
                                   could not be allocated, or would have to grow while the stream is captured */
} hkg_status_t;

typedef enum {
    HKG_KERNEL_NONE = 0,        /* M == 0 or N == 0: nothing to do */
    HKG_KERNEL_TILE = 1,        /* large-tile MFMA kernel (compute-bound shapes) */
    HKG_KERNEL_SKINNY = 2,      /* small M: streams B once, split-K over waves / workgroups */
    HKG_KERNEL_GENERIC = 3,     /* any alignment, any K: correctness fallback */
    HKG_KERNEL_ZERO = 4,        /* K == 0: C is the empty sum, +0 (then the epilogue) */
    HKG_KERNEL_MX_TILE = 5,     /* MXFP8 large-tile kernel (scaled MFMA) */
    HKG_KERNEL_GROUPED = 6,     /* grouped (mixture-of-experts) tile kernel, persistent grid */
    HKG_KERNEL_MX_SKINNY = 7,   /* MXFP8 small-M kernel: streams B once, split-K */
    HKG_KERNEL_MX4_TILE = 8,    /* MXFP4 tile kernel (scaled MFMA, E2M1 operands) */
    HKG_KERNEL_MX4_SKINNY = 9   /* MXFP4 small-M kernel: streams B once, split-K */
} hkg_kernel_t;

/*
 * Fused epilogues, applied to the fp32 sum before the one rounding to bf16
 * (the list of the FlyDSL "Prebuilt kernels guide", section 3.1, Preshuffle
 * GEMM, parameter `epilogue`; its bias holds one value per output column in
 * the output dtype):  x = sum + bias[n] and
 *   BIAS       y = x
 *   BIAS_RELU  y = x if x > 0, else +0
 *   BIAS_SILU  y = x / (1 + exp(-x))
 *   BIAS_GELU  y = x * Phi(x), Phi the standard normal CDF (exact GELU,
 *              evaluated as x/2 * erfc(-x / sqrt 2))
 * then C[m][n] = bf16 nearest-even rounding of y.  NONE is the plain GEMM.
 */
typedef enum {
    HKG_EPILOGUE_NONE = 0,
    HKG_EPILOGUE_BIAS = 1,
    HKG_EPILOGUE_BIAS_RELU = 2,
    HKG_EPILOGUE_BIAS_SILU = 3,
    HKG_EPILOGUE_BIAS_GELU = 4
} hkg_epilogue_t;

/*
 * A launch plan.  Plain data owned by the caller.  hkg_gemm_bf16_plan fills
 * it from (M, N, K) alone (no device needed); hkg_gemm_bf16_run_plan runs a
 * plan, possibly edited within the documented ranges for experiments.
 */
typedef struct {
    int32_t abi_version;        /* HKG_ABI_VERSION */
    int32_t kernel_id;          /* hkg_kernel_t */
    int32_t variant;            /* kernel instantiation within kernel_id (tile shape / rows per block) */
    int32_t tile_m, tile_n, tile_k;   /* output tile of one workgroup and the K step of its loop */
    int32_t waves;              /* wavefronts (64 lanes) per workgroup */
    int32_t split_k;            /* workgroups sharing one output tile along K (1 = none) */
    int32_t grid_x, grid_y, grid_z, block_x;
    int32_t xcd_window_w;       /* tile-order window height W (tile rows), 0 = plain row-major order */
    int32_t xcd_chunk_c;        /* consecutive tiles kept on one chiplet (XCD), 0 = no de-interleave */
    int64_t workspace_bytes;    /* library-owned fp32 workspace this plan uses (per stream), 0 if none */
    int32_t lds_bytes;          /* LDS per workgroup */
    int32_t vgprs, agprs, sgprs, scratch_bytes;   /* resource use of the kernel's code object (build-time) */
    int64_t M, N, K;            /* the shape this plan was made for */
    double flops;               /* 2 M N K */
    double algorithmic_bytes;   /* 2 (M K + N K + M N): each operand read once, C written once */
    char kernel_name[64];
    char reason[128];           /* why the selector chose this kernel */
} hkg_plan_t;

/*
 * C = A * B^T as above, on `stream`.  Chooses a plan with
 * hkg_gemm_bf16_plan and runs it; unaligned pointers or K % 8 != 0 run the
 * general kernel instead of failing.  M == 0 or N == 0 launches nothing;
 * K == 0 fills C with +0.  Returns HKG_OK once the work is enqueued.
 */
hkg_status_t hkg_gemm_bf16(const void* A, const void* B, void* C,
                           int64_t M, int64_t N, int64_t K, void* stream);

/*
 * The plan hkg_gemm_bf16 would use for an aligned call of this shape
 * (host only; no device, no allocation).  Shape-based selection after the
 * tile heuristic of the FlyDSL "Prebuilt kernels guide" (section 3c,
 * implicit-GEMM convolution: largest tile that still fills the device,
 * split-K only when the grid underfills it) and the chiplet-aware tile order
 * of the HipKittens talk notes (section 3, Algorithm 1, Table 4).
 */
hkg_status_t hkg_gemm_bf16_plan(int64_t M, int64_t N, int64_t K, hkg_plan_t* out);

/*
 * Runs `plan` on (A, B, C).  M, N, K must equal plan->M, N, K.  A fast-kernel
 * plan on unaligned pointers or K % 8 != 0 returns HKG_ERR_MISALIGNED; an
 * edited plan outside the ranges the library supports returns
 * HKG_ERR_UNSUPPORTED.  Edits that are accepted: xcd_window_w >= 0,
 * xcd_chunk_c >= 0; kernel_id GENERIC for any shape; kernel_id TILE with any
 * tile variant (tile_m/tile_n/tile_k/waves matching it) and split_k in
 * [1, 16] (above 1 only for variants of at most 16 accumulator blocks per
 * wave and M * N < 2^29); kernel_id SKINNY with a variant whose rows cover M
 * and split_k in [1, 64].
 */
hkg_status_t hkg_gemm_bf16_run_plan(const hkg_plan_t* plan, const void* A, const void* B,
                                    void* C, int64_t M, int64_t N, int64_t K, void* stream);

/*
 * C = epilogue(A * B^T + bias) (hkg_epilogue_t above), on `stream`, with the
 * plan and fallbacks of hkg_gemm_bf16; HKG_EPILOGUE_NONE is exactly
 * hkg_gemm_bf16.  bias: device pointer to N bf16 values (one per column of
 * C), caller-owned, 2-byte aligned, not overlapping C; unused (may be NULL)
 * for HKG_EPILOGUE_NONE.  K == 0 gives C = epilogue(bias).
 * Errors, before any device work: an unknown epilogue code, a NULL bias
 * with another code, or bias overlapping C -> HKG_ERR_INVALID_ARG; bias at
 * an odd address -> HKG_ERR_MISALIGNED.
 */
hkg_status_t hkg_gemm_bf16_epilogue(const void* A, const void* B, const void* bias, void* C,
                                    int64_t M, int64_t N, int64_t K, int32_t epilogue, void* stream);

/* hkg_gemm_bf16_run_plan with a fused epilogue (arguments as above). */
hkg_status_t hkg_gemm_bf16_run_plan_epilogue(const hkg_plan_t* plan, const void* A, const void* B,
                                             const void* bias, void* C, int64_t M, int64_t N, int64_t K,
                                             int32_t epilogue, void* stream);

/*
 * Block-scaled FP8 GEMM (MXFP8), the block-scaled format of the
 * FlyDSL-in-PyTorch blog post (MXFP section: E4M3 values with one E8M0
 * scale per 32 values along K, K a multiple of 128 for the scaled MFMA):
 *
 *   C[i][j] = bf16( sum over k of  a(i,k) 2^(SA[i][k/32] - 127) * b(j,k) 2^(SB[j][k/32] - 127) )
 *
 *   A: M x K bytes, OCP FP8 E4M3 codes ("e4m3fn": bias 7, no infinities,
 *      S.1111.111 is NaN, largest finite 448), row-major; B: N x K likewise.
 *   SA: M x K/32 bytes, E8M0 codes (value 2^(e - 127), 0xFF is NaN),
 *      row-major (one code per row per 32 consecutive k); SB: N x K/32.
 *   C: M x N bf16, row-major, nearest-even.  K must be a multiple of 128
 *   (else HKG_ERR_INVALID_ARG); M and N are free.  NaN codes give results
 *   that are not specified here.
 *
 * Accuracy.  Each output is a float sum of scaled products formed by the
 * matrix cores; on gfx950 the scaled FP8 instruction adds the products of
 * each group of 8 consecutive k (one scale block) at a fixed point aligned
 * to the group's largest product, truncating smaller products toward zero
 * to 2^-13 of that product's power of two, and combines groups and the
 * running sum in fp32.  So |C - exact| <= 2^-8 |C| + (truncation of each
 * group: below 7 * 2^-13 of its largest product) + fp32 accumulation.
 *
 * Scale packing.  The tile kernel consumes scales in a packed layout: for
 * each 64-row group of an operand and each 128-k stage, 256 bytes (see
 * hkg_mx_pack_scales).  hkg_gemm_mxfp8 packs SA and SB itself into a
 * library-owned device buffer on every call, except on the small-M kernel
 * (HKG_KERNEL_MX_SKINNY) with 4-byte aligned SA and SB, which reads the
 * natural scales directly; callers with fixed weights pack once with
 * hkg_mx_pack_scales and call hkg_gemm_mxfp8_prepacked.
 *
 * Pointers: A, B, C 16-byte aligned, packed scales 4-byte aligned (else
 * HKG_ERR_MISALIGNED), all device memory owned by the caller; C overlaps
 * no input.  bias / epilogue as in hkg_gemm_bf16_epilogue.  Shapes whose
 * packed scales reach 2^31 bytes, or K above 8388480, give
 * HKG_ERR_UNSUPPORTED.  The packed scales of hkg_gemm_mxfp8 go to the
 * stream's library-owned workspace (see "Thread safety" above).
 */

/* The plan an MXFP8 call of this shape uses (host only, no device). */
hkg_status_t hkg_gemm_mxfp8_plan(int64_t M, int64_t N, int64_t K, hkg_plan_t* out);

/* C = epilogue(MXFP8 A * B^T + bias) with natural-layout scales SA, SB. */
hkg_status_t hkg_gemm_mxfp8(const void* A, const void* SA, const void* B, const void* SB, const void* bias,
                            void* C, int64_t M, int64_t N, int64_t K, int32_t epilogue, void* stream);

/*
 * Bytes of the packed form of `rows` x K/32 scales: ceil(rows / 64) * 64 *
 * K / 32.  -1 for negative sizes or K % 128 != 0.
 */
int64_t hkg_mx_packed_scales_bytes(int64_t rows, int64_t K);

/*
 * Packs S (rows x K/32 E8M0 codes, row-major, device memory) into P
 * (hkg_mx_packed_scales_bytes(rows, K) bytes, 4-byte aligned, device
 * memory, not overlapping S) on `stream`.  Layout: for 64-row group R, stage
 * t (128 k) and lane l in 0..63, the 4 bytes at offset ((R * K/128 + t) * 64
 * + l) * 4 hold, in byte f, the code of row 64 R + 16 f + l % 16, block
 * 4 t + l / 16 (0 past the last row).
 */
hkg_status_t hkg_mx_pack_scales(const void* S, void* P, int64_t rows, int64_t K, void* stream);

/* hkg_gemm_mxfp8 with packed scales PA (of A, M rows) and PB (of B, N rows). */
hkg_status_t hkg_gemm_mxfp8_prepacked(const void* A, const void* PA, const void* B, const void* PB,
                                      const void* bias, void* C, int64_t M, int64_t N, int64_t K,
                                      int32_t epilogue, void* stream);

/*
 * Runs an MXFP8 plan (from hkg_gemm_mxfp8_plan, possibly edited: variant
 * with matching tile fields, split_k in [1, 16] for split-capable variants,
 * xcd fields >= 0) on packed scales; other plans give HKG_ERR_UNSUPPORTED.
 */
hkg_status_t hkg_gemm_mxfp8_run_plan(const hkg_plan_t* plan, const void* A, const void* PA, const void* B,
                                     const void* PB, const void* bias, void* C, int64_t M, int64_t N,
                                     int64_t K, int32_t epilogue, void* stream);

/*
 * Block-scaled FP4 GEMM (MXFP4), the packed-FP4 form of the same MXFP
 * section of the FlyDSL-in-PyTorch blog (E2M1 values stored two per byte,
 * one E8M0 scale per 32 values along K, fp32 accumulation, bf16 output):
 *
 *   C[i][j] = bf16( sum over k of  a(i,k) 2^(SA[i][k/32] - 127) * b(j,k) 2^(SB[j][k/32] - 127) )
 *
 *   A: M x K/2 bytes, row-major; byte c of row i holds a(i, 2c) in its low
 *      nibble and a(i, 2c + 1) in its high nibble, each an E2M1 code (OCP
 *      MX: 1 sign bit, 2 exponent bits with bias 1, 1 fraction bit; values
 *      0, 0.5, 1, 1.5, 2, 3, 4, 6 and their negatives; no infinities or
 *      NaNs).  B: N x K/2 bytes likewise.
 *   SA: M x K/32 bytes, SB: N x K/32 bytes, E8M0 codes as for MXFP8.
 *   C: M x N bf16, row-major, nearest-even.  K must be a multiple of 128
 *   (else HKG_ERR_INVALID_ARG); M and N are free.  NaN scale codes give
 *   unspecified results in the outputs whose sums they enter and leave
 *   every other output as specified.
 *
 * Accuracy.  A product of two E2M1 values is a multiple of 1/4 below 37,
 * and the 32 products of one scale block share one power-of-two scale, so
 * the matrix cores form every block's partial sums exactly; they combine
 * them with the running sum in fp32.  So |C - exact| <= 2^-8 |C| + fp32
 * accumulation (at most 17 roundings of 2^-24 relative per 128 k).
 *
 * Scales are consumed in the packed layout of hkg_mx_pack_scales (the same
 * as MXFP8's); hkg_gemm_mxfp4 packs SA and SB into the stream's
 * library-owned workspace on every call, hkg_gemm_mxfp4_prepacked takes
 * packed scales.  Pointers: A, B, C 16-byte aligned, packed scales 4-byte
 * aligned (else HKG_ERR_MISALIGNED), device memory owned by the caller; C
 * overlaps no input.  bias / epilogue as in hkg_gemm_bf16_epilogue.  Shapes
 * whose packed scales reach 2^31 bytes, or K above 16777088, give
 * HKG_ERR_UNSUPPORTED.
 */

/* The plan an MXFP4 call of this shape uses (host only, no device). */
hkg_status_t hkg_gemm_mxfp4_plan(int64_t M, int64_t N, int64_t K, hkg_plan_t* out);

/* C = epilogue(MXFP4 A * B^T + bias) with natural-layout scales SA, SB. */
hkg_status_t hkg_gemm_mxfp4(const void* A, const void* SA, const void* B, const void* SB, const void* bias,
                            void* C, int64_t M, int64_t N, int64_t K, int32_t epilogue, void* stream);

/* hkg_gemm_mxfp4 with packed scales PA (of A, M rows) and PB (of B, N rows). */
hkg_status_t hkg_gemm_mxfp4_prepacked(const void* A, const void* PA, const void* B, const void* PB,
                                      const void* bias, void* C, int64_t M, int64_t N, int64_t K,
                                      int32_t epilogue, void* stream);

/*
 * Runs an MXFP4 plan (from hkg_gemm_mxfp4_plan, possibly edited: variant
 * with matching tile fields, split_k in [1, 16] for split-capable tile
 * variants and in [1, 64] for the small-M kernel, xcd fields >= 0) on packed
 * scales; other plans give HKG_ERR_UNSUPPORTED.  The planner takes the
 * small-M kernel (HKG_KERNEL_MX4_SKINNY) for M <= 32.
 */
hkg_status_t hkg_gemm_mxfp4_run_plan(const hkg_plan_t* plan, const void* A, const void* PA, const void* B,
                                     const void* PB, const void* bias, void* C, int64_t M, int64_t N,
                                     int64_t K, int32_t epilogue, void* stream);

/*
 * Operand layouts and leading dimensions (the FlyDSL-in-PyTorch blog,
 * section "Dense GEMM", measures all four layouts).  The logical operation is
 * unchanged, C = epilogue(A * B^T + bias) with A M x K and B N x K; only where
 * element (i, k) of A (j, k of B) lives changes:
 *   HKG_LAYOUT_ROW  a(i,k) = A[i * lda + k]   (K contiguous, lda >= K)
 *   HKG_LAYOUT_COL  a(i,k) = A[k * lda + i]   (stored K x M, lda >= M)
 * and likewise b(j,k) = B[j * ldb + k] (ROW, ldb >= K) or B[k * ldb + j]
 * (COL: B stored K x N, ldb >= N); C[i * ldc + j] with ldc >= N (elements in
 * between are not touched).  In the usual names for C = op(A) op(B) with a
 * row-major K x N second operand: NT = (ROW, ROW), NN = (ROW, COL),
 * TN = (COL, COL), TT = (COL, ROW).
 */
typedef enum {
    HKG_LAYOUT_ROW = 0,
    HKG_LAYOUT_COL = 1
} hkg_layout_t;

/*
 * C = epilogue(A * B^T + bias) in any layouts (above), on `stream`.
 * ROW operands with 16-byte aligned pointers and leading dimensions (ld % 8
 * == 0) and K % 8 == 0 run the fast kernels in place; a COL operand is first
 * transposed into a library-owned device buffer (one extra pass over it; to
 * avoid it for a fixed weight, pack it once with hkg_pack_bf16); anything
 * else runs the general kernel, which reads every layout directly.
 * Errors (before any device work): unknown layout, a leading dimension below
 * its minimum (or above 2^31 - 1), null pointers with nonzero extent, C
 * overlapping A or B -> HKG_ERR_INVALID_ARG; epilogue errors as
 * hkg_gemm_bf16_epilogue.  The transposed copies go to the stream's
 * library-owned workspace (see "Thread safety" above).
 */
hkg_status_t hkg_gemm_bf16_ex(const void* A, int64_t lda, int32_t a_layout, const void* B, int64_t ldb,
                              int32_t b_layout, const void* bias, void* C, int64_t ldc, int64_t M, int64_t N,
                              int64_t K, int32_t epilogue, void* stream);

/*
 * Offline pre-pack of an operand into the layout the fast kernels read: Y
 * (rows x K bf16, K contiguous, dense) from X of `rows` logical rows in
 * `layout` with leading dimension ldx (a weight stored K x N for x @ W is
 * layout COL, rows = N).  Y is then passed as a ROW operand with ld = K.
 * Device pointers, Y not overlapping X.  Errors as hkg_gemm_bf16_ex.
 */
hkg_status_t hkg_pack_bf16(const void* X, int64_t ldx, int32_t layout, void* Y, int64_t rows, int64_t K,
                           void* stream);

/*
 * Grouped GEMM for mixture-of-experts layers (FlyDSL-in-PyTorch blog,
 * grouped GEMM section: concatenated activations, one weight per expert,
 * cumulative row offsets, one launch on a persistent grid):
 *
 *   C[i][j] = epilogue( sum over k of A[i][k] * B[g][j][k] + bias[g][j] ),
 *             for offs[g-1] <= i < offs[g]  (offs[-1] = 0)
 *
 *   A: M x K bf16, the rows of all experts concatenated; B: G x N x K bf16,
 *   expert g's weight N x K with K contiguous (the NT layout of
 *   hkg_gemm_bf16; the blog's B[G, K, N] with unit stride along K); offs: G
 *   int32 row ends, device memory, non-decreasing, at most M; C: M x N bf16.
 *   Rows at or past offs[G-1] are not written.  bias: G x N bf16 (one row per
 *   expert) for epilogues other than NONE.  Empty experts (equal offsets)
 *   cost nothing.  Offsets are read on the device: values outside [0, M] are
 *   clamped and a decreasing offset makes its expert empty, so no offsets
 *   can make the kernel access memory outside A, B, C; the result for such
 *   offsets is not specified.
 *   A, B, C 16-byte aligned, offs 4-byte aligned, K % 8 == 0 (else
 *   HKG_ERR_MISALIGNED / HKG_ERR_UNSUPPORTED; there is no general fallback).
 *   M, N or G == 0 launches nothing.  Rounding as hkg_gemm_bf16.
 *   Tiles form one list over the experts, walked in rounds of grid_x
 *   workgroups.  When the last round's tiles fill at most half the grid and
 *   the plan's split_k is 2 (K of at least two stages), each of those tiles
 *   is computed as two halves of K whose fp32 sums are added once (in either
 *   order: the result is the same) before the rounding; the partials use
 *   the stream's workspace (workspace_bytes of the plan, grid_x tiles of
 *   fp32), allocated as for split-K of hkg_gemm_bf16.  While the stream is
 *   being captured and its workspace is smaller than that (it never grows
 *   during capture), the call runs every tile whole: correct, but its
 *   last-round tiles may differ in the last bit from an eager call's.
 *   Otherwise results are deterministic run to run.
 */
hkg_status_t hkg_grouped_gemm_bf16_plan(int64_t G, int64_t M, int64_t N, int64_t K, hkg_plan_t* out);

hkg_status_t hkg_grouped_gemm_bf16(const void* A, const void* B, const void* offs, const void* bias, void* C,
                                   int64_t G, int64_t M, int64_t N, int64_t K, int32_t epilogue, void* stream);

/* Runs a grouped plan (variant, grid_x >= 1, xcd_chunk_c and split_k 1 or 2
 * may be edited). */
hkg_status_t hkg_grouped_gemm_bf16_run_plan(const hkg_plan_t* plan, const void* A, const void* B, const void* offs,
                                            const void* bias, void* C, int64_t G, int64_t M, int64_t N, int64_t K,
                                            int32_t epilogue, void* stream);

/* ------------------------------------------------------ without allocation
 * hkg_gemm_bf16_noalloc: hkg_gemm_bf16 for callers that cannot allocate
 * device memory -- code under stream capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, plan, kernels and results as
 * hkg_gemm_bf16 (bit-identical output), but the split-K partials and arrival
 * counters live in a fixed device array of the library (16 MiB of partials
 * and 16384 counters per device, held until the process ends) instead of a
 * workspace the library allocates; the call itself allocates nothing.
 * Every split-K plan the library chooses fits (at most 256 x 128 x 128 fp32
 * partials); a plan needing more returns HKG_ERR_WORKSPACE.  One exception
 * to bit-identity: where hkg_gemm_bf16's plan splits the last round of
 * 256 x 256 tiles in two halves of K (one 256 KiB partial per workgroup,
 * 64 MiB), this entry point runs those tiles whole, with the same kernel's
 * persistent schedule: the output is then within the library's accuracy
 * bound of the same sum, accumulated in another order.
 * All calls on one device share the array: calls that overlap in time on
 * one device (on different streams, or a captured graph replayed beside
 * another call) race and give wrong results; calls on one stream are
 * ordered.  The first call on a device finds the array's address and, when
 * its stream is not being captured, clears the counters (synchronously).
 */
hkg_status_t hkg_gemm_bf16_noalloc(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K,
                                   void* stream);

/* Static description of a status code. */
const char* hkg_status_string(hkg_status_t status);

/* Text of the last HIP error seen by this thread ("" if none). */
const char* hkg_last_hip_error(void);

/* HKG_ABI_VERSION of the loaded library. */
int32_t hkg_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* HKG_H */
