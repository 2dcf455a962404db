// MXFP8 and MXFP4 instantiations of the large-tile MFMA kernel
// (hkg_tile_kernel.h) and the scale packer that feeds them.
//
// Block-scaled formats as the FlyDSL-in-PyTorch blog describes them (MXFP
// section): E4M3 elements (MXFP8) or packed E2M1 elements (MXFP4) with one
// E8M0 power-of-two scale per 32 values along K, consumed by gfx950's scaled
// MFMA, K a multiple of 128.
#include "hkg_tile_kernel.h"

namespace hkg {
namespace {

// Scale packing.  S: rows x (K / 32) E8M0 codes, row-major.  P: for every
// 64-row group R and 128-k stage kt, 64 dwords; dword (R * KT + kt) * 64 + l
// holds in byte f the code of row 64 R + 16 f + l % 16, block 4 kt + l / 16
// (0 for rows past `rows`).  That dword is lane l's scale operand of the
// scaled MFMA for the group's 16-row block f (byte chosen by op_sel), so the
// GEMM loads one coalesced dword per lane per group and stage.
__global__ __launch_bounds__(256) void mx_pack_kernel(const uint8_t* __restrict__ S, uint32_t* __restrict__ P,
                                                      int64_t rows, int KB, int KT, int64_t total)
{
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= total)
        return;
    const int lane = (int)(idx & 63);
    const int64_t q = idx >> 6;
    const int kt = (int)(q % KT);
    const int64_t group = q / KT;
    const int col = 4 * kt + lane / 16;
    uint32_t w = 0;
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        const int64_t row = 64 * group + 16 * f + (lane & 15);
        if (row < rows)
            w |= (uint32_t)S[row * KB + col] << (8 * f);
    }
    P[idx] = w;
}

}  // namespace

TileShape mx_tile_shape(int variant)
{
    int v = 0;
#define HKG_SHAPE(bm, bn, bk, st, wm, wn, sc) \
    if (v++ == variant)                   \
        return TileShape{bm, bn, bk, st, (wm) * (wn), wm, wn, sc};
    HKG_MX_TILE_CONFIGS(HKG_SHAPE)
#undef HKG_SHAPE
    return TileShape{0, 0, 0, 0, 0, 0, 0, 0};
}

int mx_tile_lds_bytes(int variant)
{
    const TileShape s = mx_tile_shape(variant);
    if (s.sched == 5)
        return (4 * (s.bm / 2) + 3 * s.bn) * s.bk;
    return s.stages * (s.bm + s.bn) * s.bk;
}

TileShape mx4_tile_shape(int variant)
{
    int v = 0;
#define HKG_SHAPE(bm, bn, bk, st, wm, wn, sc) \
    if (v++ == variant)                   \
        return TileShape{bm, bn, bk, st, (wm) * (wn), wm, wn, sc};
    HKG_MX4_TILE_CONFIGS(HKG_SHAPE)
#undef HKG_SHAPE
    return TileShape{0, 0, 0, 0, 0, 0, 0, 0};
}

int mx4_tile_lds_bytes(int variant)
{
    const TileShape s = mx4_tile_shape(variant);   // rows of bk / 2 bytes
    if (s.sched == 5)
        return (4 * (s.bm / 2) + 3 * s.bn) * (s.bk / 2);
    return s.stages * (s.bm + s.bn) * (s.bk / 2);
}

int64_t mx_packed_scale_bytes(int64_t rows, int64_t K) { return (rows + 63) / 64 * 64 * (K / 32); }

hipError_t launch_mx_pack(const uint8_t* S, uint32_t* P, int64_t rows, int64_t K, hipStream_t stream)
{
    const int64_t total = mx_packed_scale_bytes(rows, K) / 4;
    if (total == 0)
        return hipSuccess;
    const int64_t blocks = (total + 255) / 256;
    hipLaunchKernelGGL(mx_pack_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, S, P, rows, (int)(K / 32),
                       (int)(K / 128), total);
    return hipGetLastError();
}

hipError_t launch_tile_mx(int variant, const uint8_t* A, const uint8_t* B, uint16_t* C, int M, int N, int K,
                          int win_w, int chunk_c, int split_k, float* ws, int* counters, const uint16_t* bias,
                          int epi, const uint32_t* psa, const uint32_t* psb, hipStream_t stream)
{
    int v = 0;
#define HKG_LAUNCH(bm, bn, bk, st, wm, wn, sc)                                                                    \
    if (v++ == variant)                                                                                          \
        return epi == EPI_NONE                                                                                   \
                   ? launch_tile_t<bm, bn, bk, st, wm, wn, sc, false, true>(A, B, C, M, N, K, win_w, chunk_c,    \
                                                                            split_k, ws, counters, bias, epi,  \
                                                                            psa, psb, K, K, N, stream)         \
                   : launch_tile_t<bm, bn, bk, st, wm, wn, sc, true, true>(A, B, C, M, N, K, win_w, chunk_c,     \
                                                                           split_k, ws, counters, bias, epi,   \
                                                                           psa, psb, K, K, N, stream);
    HKG_MX_TILE_CONFIGS(HKG_LAUNCH)
#undef HKG_LAUNCH
    return hipErrorInvalidValue;
}

// Leading dimensions are passed in elements (K), as for MXFP8; the kernel
// takes a row of the MXFP4 operands as K / 2 bytes.
hipError_t launch_tile_mx4(int variant, const uint8_t* A, const uint8_t* B, uint16_t* C, int M, int N, int K,
                           int win_w, int chunk_c, int split_k, float* ws, int* counters, const uint16_t* bias,
                           int epi, const uint32_t* psa, const uint32_t* psb, hipStream_t stream)
{
    int v = 0;
#define HKG_LAUNCH(bm, bn, bk, st, wm, wn, sc)                                                                    \
    if (v++ == variant)                                                                                          \
        return epi == EPI_NONE                                                                                   \
                   ? launch_tile_t<bm, bn, bk, st, wm, wn, sc, false, true>(A, B, C, M, N, K, win_w, chunk_c,    \
                                                                            split_k, ws, counters, bias, epi,  \
                                                                            psa, psb, K, K, N, stream)         \
                   : launch_tile_t<bm, bn, bk, st, wm, wn, sc, true, true>(A, B, C, M, N, K, win_w, chunk_c,     \
                                                                           split_k, ws, counters, bias, epi,   \
                                                                           psa, psb, K, K, N, stream);
    HKG_MX4_TILE_CONFIGS(HKG_LAUNCH)
#undef HKG_LAUNCH
    return hipErrorInvalidValue;
}

}  // namespace hkg
