// Internal interface between the C ABI (hkg_abi.cpp) and the kernel files.
// Not installed; no HIP types beyond hipStream_t cross it.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hkg {

// Tile-kernel instantiations (plan.variant for HKG_KERNEL_TILE).
enum TileVariant : int {
    TILE_256x256 = 0,   // 8 waves, 2 x 4 wave grid, 128 x 64 per wave
    TILE_256x128 = 1,   // 8 waves, 4 x 2 wave grid,  64 x 64 per wave
    TILE_128x128 = 2,   // 4 waves, 2 x 2 wave grid,  64 x 64 per wave
    TILE_NUM_VARIANTS = 3
};

// Skinny-kernel instantiations (plan.variant for HKG_KERNEL_SKINNY): the
// number of 16-row blocks of A the kernel covers (M <= 16 * mblocks).
enum SkinnyVariant : int {
    SKINNY_M16 = 0,     // M <= 16
    SKINNY_M32 = 1,     // M <= 32
    SKINNY_M64 = 2,     // M <= 64
    SKINNY_M128 = 3,    // M <= 128
    SKINNY_NUM_VARIANTS = 4
};

struct TileShape { int bm, bn, bk, waves; };
TileShape tile_shape(int variant);
int tile_lds_bytes(int variant);

struct SkinnyShape { int mblocks, rows_n, waves; };
SkinnyShape skinny_shape(int variant);
int skinny_lds_bytes(int variant);

// Launchers: enqueue one kernel on `stream`; return the launch error.
hipError_t launch_tile(int variant, const uint16_t* A, const uint16_t* B, uint16_t* C,
                       int M, int N, int K, int win_w, int xcd_chunk, hipStream_t stream);

// split_k == 1: plain launch.  split_k > 1: fp32 partials in `ws`
// (split_k * M * N floats) and per-column-block arrival counters in `counters`
// (grid_x ints, zero on entry and left zero on exit).
hipError_t launch_skinny(int variant, const uint16_t* A, const uint16_t* B, uint16_t* C,
                         int M, int N, int K, int split_k, float* ws, int* counters,
                         hipStream_t stream);

hipError_t launch_generic(const uint16_t* A, const uint16_t* B, uint16_t* C,
                          int64_t M, int64_t N, int64_t K, hipStream_t stream);

hipError_t launch_zero(uint16_t* C, int64_t count, hipStream_t stream);

// Build-time resource figures of each kernel (filled by the generated
// hkg_resources.inc; -1 where unknown).
struct KernelResources { const char* name; int vgprs, agprs, sgprs, scratch, lds; };
const KernelResources* tile_resources(int variant);
const KernelResources* skinny_resources(int variant);
const KernelResources* generic_resources();

}  // namespace hkg
