// combine.hip -- routing-weighted combine, fills and the balance loss.
//
// [PithTrain] section 4.1: every expert's output row, scaled by the token's
// routing weight for that expert, is accumulated into the token's output.
// Here the separate (unfused) form: y[t] = sum_j w[t,j] * out_perm[slot[t,j]]
// over kept slots, in j order, one workgroup per token, float4 wide.
// [EP] section 2.3: balance loss lambda * sum_e p_e q_e with q_e = 1/E.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

__global__ __launch_bounds__(256) void zero_f32_kernel(float4* p, int64_t n4) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4;
         i += (int64_t)gridDim.x * blockDim.x)
        p[i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

__global__ __launch_bounds__(256) void combine_kernel(int64_t T, int d, int k,
                                                      const float* __restrict__ out_perm,
                                                      const int32_t* __restrict__ slot,
                                                      const float* __restrict__ w,
                                                      float* __restrict__ y) {
    const int64_t t = blockIdx.x;
    const int d4 = d / 4;
    for (int c = threadIdx.x; c < d4; c += blockDim.x) {
        float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int j = 0; j < k; ++j) {
            const int r = slot[t * k + j];
            if (r < 0) continue;
            const float wt = w[t * k + j];
            const float4 o = reinterpret_cast<const float4*>(out_perm + (int64_t)r * d)[c];
            acc.x += wt * o.x;
            acc.y += wt * o.y;
            acc.z += wt * o.z;
            acc.w += wt * o.w;
        }
        reinterpret_cast<float4*>(y + t * d)[c] = acc;
    }
}

__global__ __launch_bounds__(64) void aux_kernel(int E, int64_t T, int k, float lambda,
                                                 const int32_t* __restrict__ counts,
                                                 float* __restrict__ aux) {
    long long s = 0;
    for (int e = threadIdx.x; e < E; e += blockDim.x) s += counts[e];
    s = wave_sum(s);
    if (threadIdx.x == 0)
        aux[0] = (float)((double)lambda * ((double)s / ((double)T * (double)k)) / (double)E);
}

hipError_t launch_zero_f32(float* p, int64_t n, hipStream_t st) {
    const int64_t n4 = n / 4;
    int64_t blocks = (n4 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(zero_f32_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                       reinterpret_cast<float4*>(p), n4);
    return hipGetLastError();
}

hipError_t launch_combine(int64_t T, int d, int k, const float* out_perm, const int32_t* slot,
                          const float* w, float* y, hipStream_t st) {
    hipLaunchKernelGGL(combine_kernel, dim3((unsigned)T), dim3(256), 0, st, T, d, k, out_perm, slot,
                       w, y);
    return hipGetLastError();
}

hipError_t launch_aux(int E, int64_t T, int k, float lambda, const int32_t* counts, float* aux,
                      hipStream_t st) {
    hipLaunchKernelGGL(aux_kernel, dim3(1), dim3(64), 0, st, E, T, k, lambda, counts, aux);
    return hipGetLastError();
}

}  // namespace moe
