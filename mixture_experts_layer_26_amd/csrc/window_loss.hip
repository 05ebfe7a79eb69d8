// window_loss.hip -- balance loss over a sliding window of batches.
//
// [EP] section 2.3: one mini-batch's expert shares are too noisy for the
// balance loss, so the share p_e of each expert is averaged over the last W
// batches (W = 100 on the page) and the loss lambda * sum_e p_e q_e, q_e =
// 1/E, is taken on those averages.  The window is state across calls; it
// lives in caller-owned device memory:
//   [0, 8)                     int64 n, the calls so far
//   [256, 256 + S)             int64 sums[E], counts summed over the window
//   [256 + S, ... + 4 W E)     int32 ring[W][E], the last W count vectors
// with S = 8E rounded up to 256 bytes.  Each call adds its counts to the sums
// and subtracts the vector that leaves the window (exact integers, so no
// drift over any number of calls), then
//   pbar_e = sums_e / (min(n, W) T k),   aux = lambda * sum_e pbar_e / E.
// One workgroup: E <= 1024 values per call.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int kWinThreads = 256;

__host__ __device__ constexpr size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

__global__ __launch_bounds__(kWinThreads) void window_aux_kernel(const int32_t* __restrict__ counts, int E,
                                                                 int64_t W, int64_t T, int k, float lambda,
                                                                 unsigned char* __restrict__ state,
                                                                 float* __restrict__ aux, float* __restrict__ pbar) {
    __shared__ double part[kWinThreads / kWave];
    int64_t* pn = reinterpret_cast<int64_t*>(state);
    int64_t* sums = reinterpret_cast<int64_t*>(state + 256);
    int32_t* ring = reinterpret_cast<int32_t*>(state + 256 + align256(8 * (size_t)E));
    const int64_t n = *pn;
    const int64_t slot = n % W;
    const int64_t m = n + 1 < W ? n + 1 : W;
    const double denom = (double)m * (double)T * (double)k;
    double acc = 0.0;
    for (int e = threadIdx.x; e < E; e += kWinThreads) {
        const int32_t c = counts[e];
        int32_t* r = ring + slot * E + e;
        const int64_t s = sums[e] + c - (n >= W ? (int64_t)*r : 0);
        sums[e] = s;
        *r = c;
        const double pb = (double)s / denom;
        if (pbar != nullptr) pbar[e] = (float)pb;
        acc += pb;
    }
    acc = wave_sum(acc);
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    if (lane == 0) part[wid] = acc;
    __syncthreads();   // every thread has read n before thread 0 advances it
    if (threadIdx.x == 0) {
        double tot = 0.0;
        for (int w = 0; w < kWinThreads / kWave; ++w) tot += part[w];
        aux[0] = (float)((double)lambda * tot / (double)E);
        *pn = n + 1;
    }
}

}  // namespace

size_t window_state_bytes(int64_t E, int64_t W) {
    return 256 + align256(8 * (size_t)E) + align256(4 * (size_t)W * (size_t)E);
}

hipError_t launch_window_aux(int E, int64_t W, int64_t T, int k, float lambda, const int32_t* counts, void* state,
                             float* aux, float* pbar, hipStream_t st) {
    hipLaunchKernelGGL(window_aux_kernel, dim3(1), dim3(kWinThreads), 0, st, counts, E, W, T, k, lambda,
                       static_cast<unsigned char*>(state), aux, pbar);
    return hipGetLastError();
}

}  // namespace moe
