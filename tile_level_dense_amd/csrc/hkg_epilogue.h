// Fused epilogue of the GEMM kernels: y = act(acc + bias[n]) in fp32, then
// the one nearest-even rounding to bf16 (FlyDSL "Prebuilt kernels guide",
// section 3.1, Preshuffle GEMM: epilogues "bias", "bias_relu", "bias_silu",
// "bias_gelu" with one bias value per output column, in the output dtype).
//   bias_relu  x if x > 0, else +0
//   bias_silu  x / (1 + e^-x)
//   bias_gelu  x * Phi(x), the exact GELU (not the tanh form), Phi the
//              standard normal CDF from Abramowitz & Stegun 7.1.26 (below)
// The exponentials use the hardware exp2 (v_exp_f32) and the divisions the
// hardware reciprocal: each activation is within about 1e-7 |x| of its
// exact value, far inside one bf16 rounding (2^-9 relative).
// The codes are those of hkg_epilogue_t in include/hkg.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hkg {

enum : int { EPI_NONE = 0, EPI_BIAS = 1, EPI_BIAS_RELU = 2, EPI_BIAS_SILU = 3, EPI_BIAS_GELU = 4 };

// Phi(x) for the GELU.  Abramowitz & Stegun, Handbook of Mathematical
// Functions, formula 7.1.26 (Hastings' approximation of erf, absolute error
// below 1.5e-7): with z = |x| / sqrt 2 and t = 1 / (1 + p z),
//   erfc(z) ~ t (a1 + t (a2 + t (a3 + t (a4 + t a5)))) exp(-z^2).
// Phi(x) = erfc(z) / 2 for x < 0 and 1 - erfc(z) / 2 otherwise, so the left
// tail is formed directly rather than as a difference of nearly equal values.
__device__ __forceinline__ float epi_normal_cdf(float x)
{
    const float z = fabsf(x) * 0.70710678118654752f;
    const float t = __builtin_amdgcn_rcpf(__builtin_fmaf(0.3275911f, z, 1.f));
    float poly = __builtin_fmaf(t, 1.061405429f, -1.453152027f);
    poly = __builtin_fmaf(t, poly, 1.421413741f);
    poly = __builtin_fmaf(t, poly, -0.284496736f);
    poly = __builtin_fmaf(t, poly, 0.254829592f);
    const float half_erfc = 0.5f * t * poly * __expf(-z * z);
    return x < 0.f ? half_erfc : 1.f - half_erfc;
}

__device__ __forceinline__ float epi_activation(float x, int epi)
{
    switch (epi) {
    case EPI_BIAS_RELU:
        return x > 0.f ? x : 0.f;
    case EPI_BIAS_SILU:
        // x / (1 + e^-x); 1 + e^-x is +inf below x ~ -88, and x * rcp(inf) = -0
        return x * __builtin_amdgcn_rcpf(1.f + __expf(-x));
    case EPI_BIAS_GELU:
        return x * epi_normal_cdf(x);
    default:
        return x;
    }
}

// Value of output column n after the epilogue (epi != EPI_NONE).
__device__ __forceinline__ float epi_apply(float acc, const uint16_t* __restrict__ bias, int64_t n, int epi)
{
    const float b = __uint_as_float((uint32_t)bias[n] << 16);
    return epi_activation(acc + b, epi);
}

}  // namespace hkg
