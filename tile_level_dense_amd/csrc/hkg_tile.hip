// BF16 instantiations of the large-tile MFMA kernel (hkg_tile_kernel.h):
// the variants of HKG_TILE_CONFIGS, each with and without the fused
// epilogue, and the grouped (mixture-of-experts) variants of
// HKG_GROUPED_CONFIGS.
#include "hkg_tile_kernel.h"

namespace hkg {

TileShape tile_shape(int variant)
{
    int v = 0;
#define HKG_SHAPE(bm, bn, bk, st, wm, wn, sc) \
    if (v++ == variant)                   \
        return TileShape{bm, bn, bk, st, (wm) * (wn) * ((sc) == 7 ? 2 : 1), wm, wn, sc};
    HKG_TILE_CONFIGS(HKG_SHAPE)
#undef HKG_SHAPE
    return TileShape{0, 0, 0, 0, 0, 0, 0, 0};
}

int tile_lds_bytes(int variant)
{
    const TileShape s = tile_shape(variant);
    if (s.sched == 5 || s.sched == 6)   // A halves double-, B triple-buffered
        return (4 * (s.bm / 2) + 3 * s.bn) * s.bk * 2;
    return s.stages * (s.bm + s.bn) * s.bk * 2;
}

hipError_t launch_tile(int variant, const uint16_t* A, const uint16_t* B, uint16_t* C,
                       int M, int N, int K, int win_w, int chunk_c, int split_k, float* ws, int* counters,
                       const uint16_t* bias, int epi, int lda, int ldb, int ldc, hipStream_t stream)
{
    int v = 0;
#define HKG_LAUNCH(bm, bn, bk, st, wm, wn, sc) \
    if (v++ == variant)                        \
        return epi == EPI_NONE                                                                               \
                   ? launch_tile_t<bm, bn, bk, st, wm, wn, sc, false, false>(A, B, C, M, N, K, win_w, chunk_c,     \
                                                                             split_k, ws, counters, bias, epi,   \
                                                                             nullptr, nullptr, lda, ldb, ldc,    \
                                                                             stream)                             \
                   : launch_tile_t<bm, bn, bk, st, wm, wn, sc, true, false>(A, B, C, M, N, K, win_w, chunk_c,      \
                                                                            split_k, ws, counters, bias, epi,    \
                                                                            nullptr, nullptr, lda, ldb, ldc,     \
                                                                            stream);
    HKG_TILE_CONFIGS(HKG_LAUNCH)
#undef HKG_LAUNCH
    return hipErrorInvalidValue;
}

TileShape grouped_shape(int variant)
{
    int v = 0;
#define HKG_SHAPE(bm, bn, bk, st, wm, wn, sc) \
    if (v++ == variant)                   \
        return TileShape{bm, bn, bk, st, (wm) * (wn), wm, wn, sc};
    HKG_GROUPED_CONFIGS(HKG_SHAPE)
#undef HKG_SHAPE
    return TileShape{0, 0, 0, 0, 0, 0, 0, 0};
}

hipError_t launch_grouped(int variant, const uint16_t* A, const uint16_t* B, const int* offs, int G, uint16_t* C,
                          int M, int N, int K, int grid, int xcd_chunks, int split_k, float* ws, int* counters,
                          const uint16_t* bias, int epi, hipStream_t stream)
{
    int v = 0;
#define HKG_LAUNCH(bm, bn, bk, st, wm, wn, sc)                                                                     \
    if (v++ == variant)                                                                                           \
        return epi == EPI_NONE                                                                                    \
                   ? launch_grouped_t<bm, bn, bk, st, wm, wn, sc, false>(A, B, offs, G, C, M, N, K, grid,         \
                                                                         xcd_chunks, split_k, ws, counters, bias, \
                                                                         epi, stream)                             \
                   : launch_grouped_t<bm, bn, bk, st, wm, wn, sc, true>(A, B, offs, G, C, M, N, K, grid,          \
                                                                        xcd_chunks, split_k, ws, counters, bias,  \
                                                                        epi, stream);
    HKG_GROUPED_CONFIGS(HKG_LAUNCH)
#undef HKG_LAUNCH
    return hipErrorInvalidValue;
}

}  // namespace hkg
