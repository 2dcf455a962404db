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
 *   The library keeps per-device state (device checks, split-K workspace)
 *   that it allocates on first use on a device and frees at unload.
 *
 * Errors
 *   Every argument check happens on the host, before any launch, and is
 *   reported as a status code; nothing is thrown across this ABI.
 *
 * Thread safety
 *   Calls may be made from several host threads and on several streams.
 *   Calls that use a split-K workspace on one device are serialised by
 *   stream order only if they share a stream; see hkg_plan_t.workspace_bytes.
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
    HKG_ERR_WORKSPACE = -7      /* the split-K workspace could not be allocated */
} hkg_status_t;

typedef enum {
    HKG_KERNEL_NONE = 0,        /* M == 0 or N == 0: nothing to do */
    HKG_KERNEL_TILE = 1,        /* large-tile MFMA kernel (compute-bound shapes) */
    HKG_KERNEL_SKINNY = 2,      /* small M: streams B once, split-K over waves / workgroups */
    HKG_KERNEL_GENERIC = 3,     /* any alignment, any K: correctness fallback */
    HKG_KERNEL_ZERO = 4         /* K == 0: C is the empty sum, +0 (then the epilogue) */
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
    int64_t workspace_bytes;    /* library-owned fp32 workspace this plan uses, 0 if none */
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
