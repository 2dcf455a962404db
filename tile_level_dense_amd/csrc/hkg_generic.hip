// General fallback for shapes, layouts and pointers the fast kernels do not
// take (K % 8 != 0, pointers or leading dimensions not 16-byte aligned):
// C = A * B^T with one thread per output element, each operand in row layout
// (a(i,k) = A[i lda + k]) or column layout (a(i,k) = A[k lda + i]), bf16
// loads of any alignment, fp32 fused multiply-add over k ascending, the fused
// epilogue, and one nearest-even rounding to bf16.  Also the K == 0 case:
// C = epilogue(+0), the empty sum.  And the transpose that turns a column-
// layout operand into the K-contiguous form the fast kernels read.
#include "hkg_internal.h"

namespace hkg {
namespace {

__device__ __forceinline__ float bf16_to_f32(uint16_t h)
{
    return __uint_as_float((uint32_t)h << 16);
}

__global__ __launch_bounds__(256)
void generic_kernel(const uint16_t* __restrict__ A, int64_t lda, int a_col, const uint16_t* __restrict__ B,
                    int64_t ldb, int b_col, uint16_t* __restrict__ C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                    const uint16_t* __restrict__ bias, int epi)
{
    // 16 x 16 threads per block; blockIdx.x walks N, blockIdx.y strides over M.
    const int64_t j = (int64_t)blockIdx.x * 16 + (threadIdx.x & 15);
    if (j >= N)
        return;
    // element k of the operand's row (i or j) sits at base + k * step
    const uint16_t* b = B + (b_col ? j : j * ldb);
    const int64_t b_step = b_col ? ldb : 1;
    const int64_t a_step = a_col ? lda : 1;
    for (int64_t i = (int64_t)blockIdx.y * 16 + (threadIdx.x >> 4); i < M; i += (int64_t)gridDim.y * 16) {
        const uint16_t* a = A + (a_col ? i : i * lda);
        float acc = 0.f;
        for (int64_t k = 0; k < K; ++k)
            acc = __builtin_fmaf(bf16_to_f32(a[k * a_step]), bf16_to_f32(b[k * b_step]), acc);
        if (epi != EPI_NONE)
            acc = epi_apply(acc, bias, j, epi);
        C[i * ldc + j] = __builtin_bit_cast(uint16_t, (__bf16)acc);
    }
}

__global__ __launch_bounds__(256)
void zero_kernel(uint16_t* __restrict__ C, int64_t ldc, int64_t count, int64_t N, const uint16_t* __restrict__ bias,
                 int epi)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < count; t += stride) {
        const int64_t i = t / N, j = t - i * N;
        C[i * ldc + j] =
            epi == EPI_NONE ? (uint16_t)0 : __builtin_bit_cast(uint16_t, (__bf16)epi_apply(0.f, bias, j, epi));
    }
}

// Y[r * ldy + c] = X[c * ldx + r] for r < R, c < CC: a column-layout operand
// (stored CC x R with leading dimension ldx) into row layout (R x CC).  64 x 64
// tiles through LDS (rows padded by 2 elements so the transposed reads of a
// tile column spread over the banks); reads run along X's rows and writes
// along Y's rows, so both sides are coalesced.  Tile columns beyond grid y
// are walked in a loop.
//
// With VEC (X, Y 16-byte aligned, ldx and ldy multiples of 8) interior tiles
// move 16 bytes per access: each thread reads two 8-element pieces of X rows
// and writes two 8-element pieces of Y rows (the transposed gather happens in
// LDS); edge tiles take the element path.
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

template <bool VEC>
__global__ __launch_bounds__(256)
void transpose_kernel(const uint16_t* __restrict__ X, int64_t ldx, uint16_t* __restrict__ Y, int64_t ldy, int64_t R,
                      int64_t CC)
{
    __shared__ uint16_t tile[64][66];
    const int t = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * 64;
    for (int64_t c0 = (int64_t)blockIdx.y * 64; c0 < CC; c0 += (int64_t)gridDim.y * 64) {
        if (VEC && r0 + 64 <= R && c0 + 64 <= CC) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int q = t + 256 * h;                  // 512 pieces: X row c0 + q / 8, elements 8 (q % 8)
                const int cl = q >> 3, rl = (q & 7) * 8;
                const u16x8 v = *(const u16x8*)(X + (c0 + cl) * ldx + r0 + rl);
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    tile[cl][rl + e] = v[e];
            }
            __syncthreads();
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int q = t + 256 * h;                  // Y row r0 + q / 8, elements 8 (q % 8)
                const int rl = q >> 3, cl = (q & 7) * 8;
                u16x8 v;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    v[e] = tile[cl + e][rl];
                *(u16x8*)(Y + (r0 + rl) * ldy + c0 + cl) = v;
            }
            __syncthreads();
            continue;
        }
        {
            const int cl = t >> 2, rl = (t & 3) * 16;       // X row c0 + cl, 16 elements from r0 + rl
            const int64_t c = c0 + cl;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int64_t r = r0 + rl + e;
                tile[cl][rl + e] = (c < CC && r < R) ? X[c * ldx + r] : (uint16_t)0;
            }
        }
        __syncthreads();
        {
            const int rl = t >> 2, cl = (t & 3) * 16;       // Y row r0 + rl, 16 elements from c0 + cl
            const int64_t r = r0 + rl;
            if (r < R) {
#pragma unroll
                for (int e = 0; e < 16; ++e) {
                    const int64_t c = c0 + cl + e;
                    if (c < CC)
                        Y[r * ldy + c] = tile[cl + e][rl];
                }
            }
        }
        __syncthreads();
    }
}

}  // namespace

hipError_t launch_generic(const uint16_t* A, int64_t lda, int a_col, const uint16_t* B, int64_t ldb, int b_col,
                          uint16_t* C, int64_t ldc, int64_t M, int64_t N, int64_t K, const uint16_t* bias, int epi,
                          hipStream_t stream)
{
    int64_t gy = (M + 15) / 16;
    if (gy > 65535)
        gy = 65535;
    const dim3 grid((unsigned)((N + 15) / 16), (unsigned)gy);
    hipLaunchKernelGGL(generic_kernel, grid, dim3(256), 0, stream, A, lda, a_col, B, ldb, b_col, C, ldc, M, N, K, bias,
                       epi);
    return hipGetLastError();
}

hipError_t launch_zero(uint16_t* C, int64_t ldc, int64_t M, int64_t N, const uint16_t* bias, int epi,
                       hipStream_t stream)
{
    const int64_t count = M * N;
    int64_t blocks = (count + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    if (blocks < 1)
        blocks = 1;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, C, ldc, count, N, bias, epi);
    return hipGetLastError();
}

hipError_t launch_transpose(const uint16_t* X, int64_t ldx, uint16_t* Y, int64_t ldy, int64_t R, int64_t CC,
                            hipStream_t stream)
{
    if (R <= 0 || CC <= 0)
        return hipSuccess;
    const int64_t gx = (R + 63) / 64;
    int64_t gy = (CC + 63) / 64;
    if (gy > 65535)
        gy = 65535;
    if (gx > INT32_MAX)
        return hipErrorInvalidValue;
    const bool vec = ((uintptr_t)X & 15u) == 0 && ((uintptr_t)Y & 15u) == 0 && ldx % 8 == 0 && ldy % 8 == 0;
    if (vec)
        hipLaunchKernelGGL(transpose_kernel<true>, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, stream, X, ldx, Y,
                           ldy, R, CC);
    else
        hipLaunchKernelGGL(transpose_kernel<false>, dim3((unsigned)gx, (unsigned)gy), dim3(256), 0, stream, X, ldx,
                           Y, ldy, R, CC);
    return hipGetLastError();
}

}  // namespace hkg
