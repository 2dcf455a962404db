// Internal interface between the C ABI (hkg_abi.cpp) and the kernel files.
// Not installed; no HIP types beyond hipStream_t cross it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "hkg.h"
#include "hkg_epilogue.h"
#include "hkg_skinny_configs.h"
#include "hkg_tile_configs.h"

namespace hkg {

// Tile-kernel instantiations (plan.variant for HKG_KERNEL_TILE): the rows
// of HKG_TILE_CONFIGS in hkg_tile_configs.h, in order.
constexpr int TILE_NUM_VARIANTS = 0
#define HKG_COUNT_TILE(bm, bn, bk, st, wm, wn, sc) +1
    HKG_TILE_CONFIGS(HKG_COUNT_TILE)
#undef HKG_COUNT_TILE
    ;

// MXFP8 tile-kernel instantiations (plan.variant for HKG_KERNEL_MX_TILE):
// the rows of HKG_MX_TILE_CONFIGS.
constexpr int MX_TILE_NUM_VARIANTS = 0
#define HKG_COUNT_TILE(bm, bn, bk, st, wm, wn, sc) +1
    HKG_MX_TILE_CONFIGS(HKG_COUNT_TILE)
#undef HKG_COUNT_TILE
    ;

// MXFP4 tile-kernel instantiations (plan.variant for HKG_KERNEL_MX4_TILE):
// the rows of HKG_MX4_TILE_CONFIGS.
constexpr int MX4_TILE_NUM_VARIANTS = 0
#define HKG_COUNT_TILE(bm, bn, bk, st, wm, wn, sc) +1
    HKG_MX4_TILE_CONFIGS(HKG_COUNT_TILE)
#undef HKG_COUNT_TILE
    ;

// Grouped-GEMM instantiations (plan.variant for HKG_KERNEL_GROUPED): the
// rows of HKG_GROUPED_CONFIGS; the planner's two (the 256 x 256 ping-pong
// streaming its tiles' stages, and the 128 x 128 tile).
constexpr int kGroupedPingPong = 3;
constexpr int kGroupedSmall = 1;
constexpr int GROUPED_NUM_VARIANTS = 0
#define HKG_COUNT_TILE(bm, bn, bk, st, wm, wn, sc) +1
    HKG_GROUPED_CONFIGS(HKG_COUNT_TILE)
#undef HKG_COUNT_TILE
    ;

// Planner's tiles (variant indices): the compute-bound ladder (256 x 256
// ping-pong on the persistent grid, two-stage 128 x 128), then the 4-stage
// streaming tiles, largest first (128 x 128, 128 x 96, 128 x 64, 64 x 128,
// 64 x 96, 64 x 64), for shapes that read their operands only a few times.  The persistent
// ping-pong against the one-tile form (variant 0), MI355X, uniform bf16:
// 8192^3 0.717 vs 0.725 ms, 4096 x 4096 x 12288 equal (one tile per
// workgroup), 3072 x 4096 x 4096 0.0838 vs 0.0843 ms.
constexpr int TILE_LADDER[] = {11, 2};
constexpr int STREAM_TILES[] = {8, 13, 10, 9, 12, 7};
// The k-interleaved ping-pong tiles (schedule 7), 128 x 256 and 128 x 128
// (copies 2 and 4 stages ahead), for outputs that fill one round of compute
// units with them.
constexpr int TILE_KINTER[] = {14, 15, 16};

// MXFP8 skinny instantiations (plan.variant for HKG_KERNEL_MX_SKINNY).
constexpr int MX_SKINNY_NUM_VARIANTS = 0
#define HKG_COUNT_SKINNY(mb, nb, wk, u, cp, al) +1
    HKG_MX_SKINNY_CONFIGS(HKG_COUNT_SKINNY)
#undef HKG_COUNT_SKINNY
    ;

// MXFP4 skinny instantiations (plan.variant for HKG_KERNEL_MX4_SKINNY).
constexpr int MX4_SKINNY_NUM_VARIANTS = 0
#define HKG_COUNT_SKINNY(mb, nb, wk, u, cp, al) +1
    HKG_MX4_SKINNY_CONFIGS(HKG_COUNT_SKINNY)
#undef HKG_COUNT_SKINNY
    ;

// Skinny-kernel instantiations (plan.variant for HKG_KERNEL_SKINNY): the
// rows of HKG_SKINNY_CONFIGS in hkg_skinny_configs.h, in order.
constexpr int SKINNY_NUM_VARIANTS = 0
#define HKG_COUNT_SKINNY(mb, nb, wk, u, cp, al) +1
    HKG_SKINNY_CONFIGS(HKG_COUNT_SKINNY)
#undef HKG_COUNT_SKINNY
    ;

struct TileShape { int bm, bn, bk, stages, waves, wm, wn, sched; };
// Grid of the persistent schedule (SCHED 6): one workgroup per compute unit
// of MI355X (256 CUs; its 160 KiB of LDS admit one per CU).  A multiple of
// the 8 XCDs, so workgroup b keeps the XCD of the tiles b + k G it walks.
constexpr int kPersistentGrid = 256;
// Split-K is built into tile variants whose waves hold at most 16 blocks
// of 16 x 16 accumulators (the split sums need as many registers again),
// other than the k-interleaved schedule 7, whose groups already divide K.
constexpr bool tile_split_capable(int bm, int bn, int wm, int wn, int sched)
{
    return sched != 7 && (bm / wm / 16) * (bn / wn / 16) <= 16;
}
TileShape tile_shape(int variant);
int tile_lds_bytes(int variant);

TileShape mx_tile_shape(int variant);
TileShape mx4_tile_shape(int variant);
TileShape grouped_shape(int variant);
int mx_tile_lds_bytes(int variant);
int mx4_tile_lds_bytes(int variant);
// Bytes of the packed scales of `rows` rows (rows rounded up to 64).
int64_t mx_packed_scale_bytes(int64_t rows, int64_t K);

struct SkinnyShape { int mblocks, nblocks, waves, unroll, cache_policy, a_lds; };
SkinnyShape skinny_shape(int variant);
SkinnyShape mx_skinny_shape(int variant);
SkinnyShape mx4_skinny_shape(int variant);
int skinny_lds_bytes(int variant);
int mx_skinny_lds_bytes(int variant);
int mx4_skinny_lds_bytes(int variant);

// Split-K arrival protocol (tile and skinny kernels).  Each workgroup of a
// split writes its fp32 partials with agent-scope relaxed atomic stores or
// buffer stores with the sc1 cache-policy bit (the same encoding the
// compiler emits for agent-scope relaxed atomics on gfx950: written through
// the XCD's L2 to the device coherence point), then every wave executes
// s_waitcnt vmcnt(0), which on gfx9 counts stores too and returns only when
// they are acknowledged at that point, and joins s_barrier.  Only then does
// one lane count the workgroup's arrival with an agent-scope atomic add.  The
// counter's modification order is device-wide, so the workgroup that sees
// split_k - 1 earlier arrivals knows every other split's partials were
// complete at the coherence point before their increments.  It reads them
// with agent-scope (sc1) loads, which are served from that point rather than
// from a possibly stale L1 or L2 line, and it issues them only after its own
// atomic has returned: the returned value reaches every wave through LDS and
// s_barrier before any load.  The argument rests on gfx9's completion
// counters, not on C++ happens-before between relaxed atomics; a release /
// acquire fence pair would give that too but writes back and invalidates
// the whole L2 (measured about 8x slower).  The last arriver resets the
// counter to zero, so counters are zero between calls on one stream.

// Launchers: enqueue one kernel on `stream`; return the launch error.
// Every launcher takes the fused epilogue (`epi`, an EPI_* code, and `bias`,
// N bf16 values; bias is not read when epi == EPI_NONE).
// split_k == 1: plain launch.  split_k > 1: K divided across workgroups,
// fp32 partials in `ws` (split_k * M * N floats) and per-tile arrival
// counters in `counters` (one per output tile, zero on entry and on exit).
// lda, ldb, ldc: leading dimensions (elements) of A (M x K), B (N x K), C.
hipError_t launch_tile(int variant, const uint16_t* A, const uint16_t* B, uint16_t* C,
                       int M, int N, int K, int win_w, int xcd_chunk, int split_k, float* ws,
                       int* counters, const uint16_t* bias, int epi, int lda, int ldb, int ldc, hipStream_t stream);

// MXFP8 tile kernel: A, B E4M3 codes, K % 128 == 0, psa / psb the packed
// scales (launch_mx_pack) of A and B; other arguments as launch_tile.
hipError_t launch_tile_mx(int variant, const uint8_t* A, const uint8_t* B, uint16_t* C, int M, int N, int K,
                          int win_w, int chunk_c, int split_k, float* ws, int* counters, const uint16_t* bias,
                          int epi, const uint32_t* psa, const uint32_t* psb, hipStream_t stream);

// MXFP4 tile kernel: A, B E2M1 codes two per byte (rows of K / 2 bytes),
// K % 128 == 0, packed scales as launch_tile_mx; other arguments likewise.
hipError_t launch_tile_mx4(int variant, const uint8_t* A, const uint8_t* B, uint16_t* C, int M, int N, int K,
                           int win_w, int chunk_c, int split_k, float* ws, int* counters, const uint16_t* bias,
                           int epi, const uint32_t* psa, const uint32_t* psb, hipStream_t stream);

// Grouped GEMM: A (M x K), B (G x N x K), offs (G row ends, device int32),
// C (M x N), bias G x N when epi != EPI_NONE; `grid` persistent workgroups,
// xcd_chunks != 0 for the chiplet-contiguous tile walk.  split_k 2: the tiles
// of a last round that fills at most half the grid are split into two halves
// of K, with grouped_workspace_bytes(variant, grid) of partials in ws and
// grid / 2 zeroed arrival counters (left zero); split_k 1 uses neither.
hipError_t launch_grouped(int variant, const uint16_t* A, const uint16_t* B, const int* offs, int G, uint16_t* C,
                          int M, int N, int K, int grid, int xcd_chunks, int split_k, float* ws, int* counters,
                          const uint16_t* bias, int epi, hipStream_t stream);

// MXFP8 skinny kernel (M <= 16 MB): packed scales as launch_tile_mx, or with
// natural the M x K/32 and N x K/32 scale arrays themselves (4-byte aligned);
// split-K as launch_skinny.
hipError_t launch_skinny_mx(int variant, const uint8_t* A, const uint8_t* B, uint16_t* C, int M, int N, int K,
                            int split_k, float* ws, int* counters, const uint16_t* bias, int epi,
                            const uint32_t* psa, const uint32_t* psb, bool natural, hipStream_t stream);

// MXFP4 skinny kernel (M <= 16 MB): packed scales only; split-K as
// launch_skinny.
hipError_t launch_skinny_mx4(int variant, const uint8_t* A, const uint8_t* B, uint16_t* C, int M, int N, int K,
                             int split_k, float* ws, int* counters, const uint16_t* bias, int epi,
                             const uint32_t* psa, const uint32_t* psb, hipStream_t stream);

// Packs rows x (K / 32) E8M0 codes S into the tile kernel's layout P
// (mx_packed_scale_bytes(rows, K) bytes, 4-byte aligned).
hipError_t launch_mx_pack(const uint8_t* S, uint32_t* P, int64_t rows, int64_t K, hipStream_t stream);

// split_k == 1: plain launch.  split_k > 1: fp32 partials in `ws`
// (split_k * M * N floats) and per-column-block arrival counters in `counters`
// (grid_x ints, zero on entry and left zero on exit).
hipError_t launch_skinny(int variant, const uint16_t* A, const uint16_t* B, uint16_t* C,
                         int M, int N, int K, int split_k, float* ws, int* counters,
                         const uint16_t* bias, int epi, int lda, int ldb, int ldc, hipStream_t stream);

// a_col / b_col: the operand is stored in column layout (a(i,k) = A[k lda + i]).
hipError_t launch_generic(const uint16_t* A, int64_t lda, int a_col, const uint16_t* B, int64_t ldb, int b_col,
                          uint16_t* C, int64_t ldc, int64_t M, int64_t N, int64_t K, const uint16_t* bias, int epi,
                          hipStream_t stream);

// K == 0: C[i][n] = epilogue(+0) (the empty sum).
hipError_t launch_zero(uint16_t* C, int64_t ldc, int64_t M, int64_t N, const uint16_t* bias, int epi,
                       hipStream_t stream);

// Y[r ldy + c] = X[c ldx + r], r < R, c < CC (column layout -> row layout).
hipError_t launch_transpose(const uint16_t* X, int64_t ldx, uint16_t* Y, int64_t ldy, int64_t R, int64_t CC,
                            hipStream_t stream);

// Split-K scratch supplied by the caller instead of the stream's library
// workspace: ws_bytes of fp32 partials at ws, `counters` arrival counters
// at counter_base (zero between calls).
struct FixedScratch {
    float* ws;
    size_t ws_bytes;
    int* counter_base;
    size_t counters;
};

// hkg_gemm_bf16 with split-K scratch from `scratch` (no allocation); a plan
// that needs more returns HKG_ERR_WORKSPACE.  Defined in hkg_abi.cpp.
hkg_status_t gemm_fixed_scratch(const void* A, const void* B, void* C, int64_t M, int64_t N, int64_t K, void* stream,
                                const FixedScratch& scratch);

// Build-time resource figures of each kernel (filled by the generated
// hkg_resources.inc; -1 where unknown).
struct KernelResources { const char* name; int vgprs, agprs, sgprs, scratch, lds; };
const KernelResources* tile_resources(int variant);
const KernelResources* mx_tile_resources(int variant);
const KernelResources* mx4_tile_resources(int variant);
const KernelResources* grouped_resources(int variant);
const KernelResources* skinny_resources(int variant);
const KernelResources* mx_skinny_resources(int variant);
const KernelResources* mx4_skinny_resources(int variant);
const KernelResources* generic_resources();

}  // namespace hkg
