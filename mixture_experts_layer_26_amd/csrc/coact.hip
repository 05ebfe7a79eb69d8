// coact.hip -- routing heat map and load telemetry.
//
// [EP] section 3.2 step 1: the co-selection matrix of the experts, collected
// from the routing of each batch, is the input of affinity-aware expert
// placement.  The page calls it non-symmetric, which is read here as ordered
// pairs: H[i][j] counts the tokens whose top-k list holds expert i at an
// earlier position than expert j, so H + H^T counts the tokens that chose
// both.  routed[e] is the per-expert load (every slot, before capacity) and
// its statistics: mean, population variance ([PyTorchMoE] section 3.3 item 1,
// the load-variance balance term) and coefficient of variation ([EP]
// section 2.1).
//
// Integer work on T*k indices: every pair is one atomic increment; a thread
// takes one (token, position) at a time and pairs it with the later positions.
//   * E <= 256: each workgroup keeps a private copy of H in LDS as packed
//     16-bit counters (E*E/2 words, 128 KiB at E = 256) and of routed,
//     counts its tokens with LDS atomics and adds its nonzero counters to
//     the global ones.  Hot pairs (tokens of one cluster all choose the same
//     experts) then serialise on LDS rather than on one L2 line.
//   * E > 256: global atomics straight into H.
// A workgroup takes at most 65535 tokens, so a 16-bit counter of distinct
// experts cannot overflow.  Indices outside [0, E) are skipped.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int kCoactThreads = 512;
constexpr int kCoactLdsMaxE = 256;
constexpr int kCoactLdsWords = kCoactLdsMaxE * kCoactLdsMaxE / 2 + kCoactLdsMaxE;
constexpr int64_t kCoactMaxTokensPerBlock = 65535;

__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t* __restrict__ a, int64_t na, int32_t* __restrict__ b,
                                                       int64_t nb) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < na + nb; i += stride) {
        if (i < na) a[i] = 0;
        else b[i - na] = 0;
    }
}

template <bool kLds>
__global__ __launch_bounds__(kCoactThreads) void coact_kernel(const int32_t* __restrict__ idx, int64_t T, int k,
                                                              int E, int64_t tok_per_blk, int32_t* __restrict__ H,
                                                              int32_t* __restrict__ routed) {
    __shared__ uint32_t lds[kLds ? kCoactLdsWords : kCoactLdsMaxE * 4];
    const int hw = kLds ? (E * E + 1) / 2 : 0;   // packed pair counters
    uint32_t* lr = lds + hw;                      // per-expert load
    for (int i = threadIdx.x; i < hw + E; i += blockDim.x) lds[i] = 0u;
    __syncthreads();

    const int64_t t0 = (int64_t)blockIdx.x * tok_per_blk;
    const int64_t t1 = min(T, t0 + tok_per_blk);
    const unsigned uE = (unsigned)E;
    // one (token, position a) per thread and turn: expert i = idx[t][a]
    // against the experts at the later positions of the same token
    const int64_t nq = t1 > t0 ? (t1 - t0) * k : 0;
    for (int64_t q = threadIdx.x; q < nq; q += blockDim.x) {
        const int64_t tq = q / k;
        const int a = (int)(q - tq * k);
        const int32_t* row = idx + (t0 + tq) * k;
        const int i = row[a];
        if ((unsigned)i >= uE) continue;
        atomicAdd(&lr[i], 1u);
        for (int b = a + 1; b < k; ++b) {
            const int j = row[b];
            if ((unsigned)j >= uE) continue;
            const int p = i * E + j;
            if constexpr (kLds) atomicAdd(&lds[p >> 1], 1u << (16 * (p & 1)));
            else atomicAdd(&H[p], 1);
        }
    }
    __syncthreads();

    if constexpr (kLds) {
        const int n = E * E;
        for (int w = threadIdx.x; w < hw; w += blockDim.x) {
            const uint32_t v = lds[w];
            if (v == 0u) continue;
            const int p = 2 * w;
            if (v & 0xffffu) atomicAdd(&H[p], (int)(v & 0xffffu));
            if ((v >> 16) && p + 1 < n) atomicAdd(&H[p + 1], (int)(v >> 16));
        }
    }
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        if (lr[e]) atomicAdd(&routed[e], (int)lr[e]);
}

// mean and population variance of load[0..E) in fp64 by one workgroup of
// 256 threads (two passes: the mean, then the squared deviations); the
// results are valid in thread 0
__device__ __forceinline__ void block_mean_var(const int32_t* __restrict__ routed, int E, double* mean_out,
                                               double* var_out) {
    __shared__ double part[256 / kWave];
    __shared__ double s_mean;
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    long long s = 0;
    for (int e = threadIdx.x; e < E; e += blockDim.x) s += routed[e];
    s = wave_sum(s);
    if (lane == 0) part[wid] = (double)s;
    __syncthreads();
    if (threadIdx.x == 0) {
        double tot = 0.0;
        for (int w = 0; w < 256 / kWave; ++w) tot += part[w];
        s_mean = tot / (double)E;
    }
    __syncthreads();
    const double m = s_mean;
    double q = 0.0;
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        const double dv = (double)routed[e] - m;
        q += dv * dv;
    }
    q = wave_sum(q);
    __syncthreads();   // part[] is reused
    if (lane == 0) part[wid] = q;
    __syncthreads();
    if (threadIdx.x == 0) {
        double tot = 0.0;
        for (int w = 0; w < 256 / kWave; ++w) tot += part[w];
        *mean_out = m;
        *var_out = tot / (double)E;
    }
}

// mean, population variance and CV of the loads
__global__ __launch_bounds__(256) void load_stats_kernel(const int32_t* __restrict__ routed, int E,
                                                         float* __restrict__ stats) {
    double m = 0.0, var = 0.0;
    block_mean_var(routed, E, &m, &var);
    if (threadIdx.x == 0) {
        stats[0] = (float)m;
        stats[1] = (float)var;
        stats[2] = m > 0.0 ? (float)(sqrt(var) / m) : 0.0f;
    }
}

// load-variance balance loss ([PyTorchMoE] section 3.3 item 1)
__global__ __launch_bounds__(256) void aux_variance_kernel(const int32_t* __restrict__ load, int E, float lambda,
                                                           float* __restrict__ aux) {
    double m = 0.0, var = 0.0;
    block_mean_var(load, E, &m, &var);
    if (threadIdx.x == 0) aux[0] = (float)((double)lambda * var);
}

}  // namespace

hipError_t launch_aux_variance(int E, float lambda, const int32_t* load, float* aux, hipStream_t st) {
    hipLaunchKernelGGL(aux_variance_kernel, dim3(1), dim3(256), 0, st, load, E, lambda, aux);
    return hipGetLastError();
}

hipError_t launch_coactivation(int64_t T, int k, int E, const int32_t* idx, int32_t* H, int32_t* routed,
                               float* stats, int cus, hipStream_t st) {
    const int64_t nH = (int64_t)E * E;
    int64_t zb = (nH + E + 255) / 256;
    if (zb > 4096) zb = 4096;
    hipLaunchKernelGGL(zero_i32_kernel, dim3((unsigned)zb), dim3(256), 0, st, H, nH, routed, (int64_t)E);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;

    // about one token per thread, or about 64 pairs per thread where k is
    // large (each thread takes one (token, position) at a time: with every
    // token's whole list on one thread, 1024 tokens choosing all 128 experts
    // ran 8128 pairs per thread on two CUs, 1.8 ms); at most one workgroup
    // per CU, and few enough tokens per workgroup for the 16-bit counters
    const int64_t pairs = T * (int64_t)k * (k - 1) / 2;
    int64_t blocks = (T + kCoactThreads - 1) / kCoactThreads;
    const int64_t by_pairs = (pairs + 64 * kCoactThreads - 1) / (64 * kCoactThreads);
    if (by_pairs > blocks) blocks = by_pairs;
    if (blocks > cus) blocks = cus;
    int64_t per = (T + blocks - 1) / blocks;
    if (per > kCoactMaxTokensPerBlock) {
        per = kCoactMaxTokensPerBlock;
        blocks = (T + per - 1) / per;
    }
    if (E <= kCoactLdsMaxE)
        hipLaunchKernelGGL((coact_kernel<true>), dim3((unsigned)blocks), dim3(kCoactThreads), 0, st, idx, T, k, E,
                           per, H, routed);
    else
        hipLaunchKernelGGL((coact_kernel<false>), dim3((unsigned)blocks), dim3(kCoactThreads), 0, st, idx, T, k,
                           E, per, H, routed);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    if (stats != nullptr) {
        hipLaunchKernelGGL(load_stats_kernel, dim3(1), dim3(256), 0, st, routed, E, stats);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace moe
