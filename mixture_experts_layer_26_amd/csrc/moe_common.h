// moe_common.h -- device helpers shared by the gfx950 kernels of libmoe.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

#define MOE_LDS __attribute__((address_space(3)))

namespace moe {

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, round-robin WG dispatch

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Exact-erf GELU in fp32: u * Phi(u) = 0.5 u (1 + erf(u / sqrt 2)), using the
// device library's erff.
__device__ __forceinline__ float gelu_erf(float u) {
    return 0.5f * u * (1.0f + erff(u * 0.70710678118654752440f));
}

// GELU through the erf approximation of Abramowitz & Stegun, Handbook of
// Mathematical Functions, eq. 7.1.26: for z >= 0,
//   erfc(z) = (a1 t + a2 t^2 + a3 t^3 + a4 t^4 + a5 t^5) exp(-z^2) + eps,
//   t = 1 / (1 + p z),  |eps| <= 1.5e-7.
// With z = |u| / sqrt 2, q = erfc(z) / 2 = Phi(-|u|) and
//   GELU(u) = u (1 - q) for u >= 0,  u q for u < 0,
// which keeps GELU(u) - GELU(-u) = u and a small relative error in the
// negative tail.  Used where h is rounded to bf16 (8 mantissa bits), far
// coarser than this error.
__device__ __forceinline__ float gelu_as(float u) {
    // t = 1 / (1 + p z) with z = |u| / sqrt 2; the polynomial carries the
    // factor 1/2 of q; exp(-z^2) = exp2(-u^2 log2(e) / 2)
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f * 0.70710678118654752440f, fabsf(u), 1.0f));
    float poly = fmaf(t, 0.5f * 1.061405429f, 0.5f * -1.453152027f);
    poly = fmaf(t, poly, 0.5f * 1.421413741f);
    poly = fmaf(t, poly, 0.5f * -0.284496736f);
    poly = fmaf(t, poly, 0.5f * 0.254829592f);
    const float e = __builtin_amdgcn_exp2f(u * (u * (-0.5f * 1.44269504088896340736f)));
    const float q = poly * t * e;
    // u (1 - q) for u >= 0 and u q for u < 0, as max(u, 0) - |u| q; |u| is
    // clamped to the largest float so that u = +-inf gives +inf and 0
    // (q = 0 there) and a NaN stays NaN
    return fmaxf(u, 0.0f) - fminf(fabsf(u), 3.40282347e38f) * q;
}

// GELU and its derivative from one evaluation of the erf approximation of
// gelu_as: with q = Phi(-|u|), Phi(u) = 1 - q for u >= 0 and q for u < 0, and
// GELU'(u) = Phi(u) + u phi(u) with phi(u) = exp(-u^2 / 2) / sqrt(2 pi).
// u must be finite.
__device__ __forceinline__ void gelu_and_grad_as(float u, float& h, float& hg) {
    const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f * 0.70710678118654752440f, fabsf(u), 1.0f));
    float poly = fmaf(t, 0.5f * 1.061405429f, 0.5f * -1.453152027f);
    poly = fmaf(t, poly, 0.5f * 1.421413741f);
    poly = fmaf(t, poly, 0.5f * -0.284496736f);
    poly = fmaf(t, poly, 0.5f * 0.254829592f);
    const float e = __builtin_amdgcn_exp2f(u * (u * (-0.5f * 1.44269504088896340736f)));
    const float q = poly * t * e;
    h = fmaxf(u, 0.0f) - fabsf(u) * q;
    hg = (u >= 0.0f ? 1.0f - q : q) + u * (e * 0.39894228040143267794f);
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

// Inclusive prefix sum over the threads of a block (blockDim.x <= 1024),
// `tmp` is __shared__ scratch of at least 32 ints.  Every thread must call it.
__device__ __forceinline__ int block_inclusive_scan(int v, int* tmp) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const int nw = (blockDim.x + kWave - 1) / kWave;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int o = __shfl_up(v, off, kWave);
        if (lane >= off) v += o;
    }
    if (lane == kWave - 1) tmp[wid] = v;
    __syncthreads();
    if (wid == 0) {
        int s = (lane < nw) ? tmp[lane] : 0;
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            int o = __shfl_up(s, off, kWave);
            if (lane >= off) s += o;
        }
        if (lane < nw) tmp[lane] = s;
    }
    __syncthreads();
    if (wid > 0) v += tmp[wid - 1];
    __syncthreads();
    return v;
}

}  // namespace moe
