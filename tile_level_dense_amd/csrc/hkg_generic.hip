// General fallback for shapes and pointers the fast kernels do not take
// (K % 8 != 0, pointers not 16-byte aligned): C = A * B^T with one thread
// per output element, bf16 loads of any alignment, fp32 fused multiply-add
// over k ascending, the fused epilogue, and one nearest-even rounding to
// bf16.  Also the K == 0 case: C = epilogue(+0), the empty sum.
#include "hkg_internal.h"

namespace hkg {
namespace {

__device__ __forceinline__ float bf16_to_f32(uint16_t h)
{
    return __uint_as_float((uint32_t)h << 16);
}

__global__ __launch_bounds__(256)
void generic_kernel(const uint16_t* __restrict__ A, const uint16_t* __restrict__ B,
                    uint16_t* __restrict__ C, int64_t M, int64_t N, int64_t K,
                    const uint16_t* __restrict__ bias, int epi)
{
    // 16 x 16 threads per block; blockIdx.x walks N, blockIdx.y strides over M.
    const int64_t j = (int64_t)blockIdx.x * 16 + (threadIdx.x & 15);
    if (j >= N)
        return;
    const uint16_t* b = B + j * K;
    for (int64_t i = (int64_t)blockIdx.y * 16 + (threadIdx.x >> 4); i < M; i += (int64_t)gridDim.y * 16) {
        const uint16_t* a = A + i * K;
        float acc = 0.f;
        for (int64_t k = 0; k < K; ++k)
            acc = __builtin_fmaf(bf16_to_f32(a[k]), bf16_to_f32(b[k]), acc);
        if (epi != EPI_NONE)
            acc = epi_apply(acc, bias, j, epi);
        C[i * N + j] = __builtin_bit_cast(uint16_t, (__bf16)acc);
    }
}

__global__ __launch_bounds__(256)
void zero_kernel(uint16_t* __restrict__ C, int64_t count, int64_t N, const uint16_t* __restrict__ bias, int epi)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < count; t += stride)
        C[t] = epi == EPI_NONE ? (uint16_t)0 : __builtin_bit_cast(uint16_t, (__bf16)epi_apply(0.f, bias, t % N, epi));
}

}  // namespace

hipError_t launch_generic(const uint16_t* A, const uint16_t* B, uint16_t* C,
                          int64_t M, int64_t N, int64_t K, const uint16_t* bias, int epi, hipStream_t stream)
{
    int64_t gy = (M + 15) / 16;
    if (gy > 65535)
        gy = 65535;
    const dim3 grid((unsigned)((N + 15) / 16), (unsigned)gy);
    hipLaunchKernelGGL(generic_kernel, grid, dim3(256), 0, stream, A, B, C, M, N, K, bias, epi);
    return hipGetLastError();
}

hipError_t launch_zero(uint16_t* C, int64_t M, int64_t N, const uint16_t* bias, int epi, hipStream_t stream)
{
    const int64_t count = M * N;
    int64_t blocks = (count + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    if (blocks < 1)
        blocks = 1;
    hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, C, count, N, bias, epi);
    return hipGetLastError();
}

}  // namespace hkg
