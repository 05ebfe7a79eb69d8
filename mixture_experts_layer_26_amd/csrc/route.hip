// route.hip -- gate GEMM + top-k + softmax over the selected logits (gfx950).
//
// [PithTrain] section 4.1: a linear gate scores every expert, the k best
// are kept and a softmax over those k scores gives the combine weights.
// [EP] section 2.2: the weights may be sharpened by a temperature; the hybrid
// form keeps a coarse top-8 and soft-weights only those.  [EP] section 5.5:
// the routing decision is taken in fp32.
//
// One workgroup owns TB tokens.  Phase 1 accumulates the [TB x E] logit tile
// in fp32 on the vector ALUs (x and Wg staged through LDS in K-chunks, each
// thread a 4x4 register tile).  Phase 2 hands each token to a group of G
// lanes (G = E rounded up to a power of two, at most 64); each lane keeps
// ceil(E/G) logits in registers and k rounds of butterfly arg-max (shuffle
// xor) pick the winners, ties to the lower expert index.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

template <typename XT>
__device__ __forceinline__ float load_x(const XT* p, int64_t i);
template <>
__device__ __forceinline__ float load_x<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_x<uint16_t>(const uint16_t* p, int64_t i) {
    return bf16_bits_to_f32(p[i]);
}

__device__ __forceinline__ bool beats(float av, int ai, float bv, int bi) {
    return av > bv || (av == bv && ai < bi);
}

// Top-k + softmax of one token's logits row[0..E) by a group of G lanes
// (G a power of two <= 64, groups aligned inside the wave).  NV >= ceil(E/G).
// Every lane of the wave must call this (shuffles); only `active` groups
// write.  Lane gl of the group ends up holding the gl-th winner.
template <int NV>
__device__ __forceinline__ void topk_softmax_group(const float* row, int E, int k, float tau, int G,
                                                   int gl, bool active, int32_t* idx_out,
                                                   float* w_out) {
    float v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = gl + G * i;
        v[i] = (active && e < E) ? row[e] : 0.0f;
    }
    uint32_t taken = 0;
    float my_v = 0.0f;
    int my_i = 0;
    for (int r = 0; r < k; ++r) {
        float bv = -INFINITY;
        int bi = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
            const int e = gl + G * i;
            if (e < E && !((taken >> i) & 1u) && beats(v[i], e, bv, bi)) {
                bv = v[i];
                bi = e;
            }
        }
        for (int off = G >> 1; off > 0; off >>= 1) {
            const float ov = __shfl_xor(bv, off, kWave);
            const int oi = __shfl_xor(bi, off, kWave);
            if (beats(ov, oi, bv, bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if ((bi & (G - 1)) == gl) taken |= 1u << (bi / G);
        if (gl == r) {
            my_v = bv;
            my_i = bi;
        }
    }
    const int lane = threadIdx.x & (kWave - 1);
    const float top = __shfl(my_v, lane & ~(G - 1), kWave);  // round 0 winner = max
    float p = (gl < k) ? expf((my_v - top) / tau) : 0.0f;
    float z = p;
    for (int off = G >> 1; off > 0; off >>= 1) z += __shfl_xor(z, off, kWave);
    if (active && gl < k) {
        idx_out[gl] = my_i;
        w_out[gl] = p / z;
    }
}

template <typename XT, int NV>
__global__ __launch_bounds__(256) void route_gate_topk_kernel(RouteArgs a) {
    extern __shared__ __attribute__((aligned(16))) float smem[];
    const int TB = a.TB, Epad = a.Epad, KC = a.KC, KCP = a.KC + 1, LTP = a.Epad + 1;
    float* xs = smem;              // [TB][KCP]
    float* wsm = xs + TB * KCP;    // [KC][Epad]
    float* lt = wsm + KC * Epad;   // [TB][LTP]
    const XT* __restrict__ x = static_cast<const XT*>(a.x);
    const int64_t T = a.T;
    const int d = a.d, E = a.E;
    const int64_t t0 = (int64_t)blockIdx.x * TB;
    const int tid = threadIdx.x;
    const int n_eq = Epad / 4, n_tq = TB / 4;
    const int tq = tid / n_eq, eq = tid % n_eq;
    const bool comp = tid < n_eq * n_tq;

    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

    for (int k0 = 0; k0 < d; k0 += KC) {
        for (int i = tid; i < TB * KC; i += blockDim.x) {
            const int tt = i / KC, kk = i - tt * KC;
            const int64_t t = t0 + tt;
            const int kg = k0 + kk;
            xs[tt * KCP + kk] = (t < T && kg < d) ? load_x<XT>(x, t * d + kg) : 0.0f;
        }
        for (int i = tid; i < KC * Epad; i += blockDim.x) {
            const int kk = i / Epad, e = i - kk * Epad;
            const int kg = k0 + kk;
            wsm[i] = (kg < d && e < E) ? a.Wg[(int64_t)kg * E + e] : 0.0f;
        }
        __syncthreads();
        if (comp) {
            const int kmax = min(KC, d - k0);
            for (int kk = 0; kk < kmax; ++kk) {
                const float4 wv = *reinterpret_cast<const float4*>(&wsm[kk * Epad + 4 * eq]);
                float xv[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) xv[i] = xs[(4 * tq + i) * KCP + kk];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[i][0] = fmaf(xv[i], wv.x, acc[i][0]);
                    acc[i][1] = fmaf(xv[i], wv.y, acc[i][1]);
                    acc[i][2] = fmaf(xv[i], wv.z, acc[i][2]);
                    acc[i][3] = fmaf(xv[i], wv.w, acc[i][3]);
                }
            }
        }
        __syncthreads();
    }
    if (comp) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 4 * eq + j;
            const float b = (a.bg != nullptr && e < E) ? a.bg[e] : 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) lt[(4 * tq + i) * LTP + e] = acc[i][j] + b;
        }
    }
    __syncthreads();
    if (a.logits != nullptr) {
        for (int i = tid; i < TB * E; i += blockDim.x) {
            const int tt = i / E, e = i - tt * E;
            const int64_t t = t0 + tt;
            if (t < T) a.logits[t * E + e] = lt[tt * LTP + e];
        }
    }
    // top-k: groups of G lanes, one token per group
    const int G = a.G;
    const int lane = tid & (kWave - 1), wid = tid / kWave, nwaves = blockDim.x / kWave;
    const int gpw = kWave / G;
    const int gl = lane & (G - 1), gi = lane / G;
    for (int base = wid * gpw; base < TB; base += nwaves * gpw) {
        const int tt = base + gi;
        const int64_t t = t0 + tt;
        const bool active = tt < TB && t < T;
        const float* row = lt + (active ? tt : 0) * LTP;
        topk_softmax_group<NV>(row, E, a.k, a.tau, G, gl, active, a.idx + (active ? t : 0) * a.k,
                               a.w + (active ? t : 0) * a.k);
    }
    // zero this block's rows of y (the fused combine adds into it later)
    if (a.yzero != nullptr) {
        const int64_t nrow = min((int64_t)TB, T - t0);
        const int64_t n4 = nrow * a.ycols / 4;
        float4* yz = reinterpret_cast<float4*>(a.yzero + t0 * a.ycols);
        for (int64_t i = tid; i < n4; i += blockDim.x) yz[i] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
}

// Top-k + softmax of logits already in global memory.
template <int NV>
__global__ __launch_bounds__(256) void route_logits_topk_kernel(RouteArgs a) {
    const int G = a.G;
    const int lane = threadIdx.x & (kWave - 1);
    const int gpw = kWave / G;
    const int gl = lane & (G - 1), gi = lane / G;
    const int64_t gwave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    const int64_t t = gwave * gpw + gi;
    const bool active = t < a.T;
    const float* row = a.logits + (active ? t : 0) * a.E;
    topk_softmax_group<NV>(row, a.E, a.k, a.tau, G, gl, active, a.idx + (active ? t : 0) * a.k,
                           a.w + (active ? t : 0) * a.k);
}

// ---------------------------------------------------------------- host ----

static int route_nv(int E, int G) {
    const int nv = (E + G - 1) / G;
    return nv <= 1 ? 1 : nv <= 2 ? 2 : nv <= 4 ? 4 : nv <= 8 ? 8 : 16;
}

RouteArgs route_config(int64_t T, int d, int E, int k, float tau) {
    RouteArgs a{};
    a.T = T;
    a.d = d;
    a.E = E;
    a.k = k;
    a.tau = tau;
    a.Epad = (E + 3) & ~3;
    const int n_eq = a.Epad / 4;
    int tb = 4 * (256 / n_eq);
    if (tb > 256) tb = 256;
    a.TB = tb;
    int g = 1;
    while (g < E && g < kWave) g <<= 1;
    a.G = g;
    const int budget = 16384;  // floats of LDS per workgroup (64 KiB)
    int kc = 64;
    while (kc > 4 && a.TB * (kc + 1) + kc * a.Epad + a.TB * (a.Epad + 1) > budget) kc >>= 1;
    a.KC = kc;
    return a;
}

size_t route_smem_bytes(const RouteArgs& a) {
    return sizeof(float) * ((size_t)a.TB * (a.KC + 1) + (size_t)a.KC * a.Epad +
                            (size_t)a.TB * (a.Epad + 1));
}

template <typename XT>
static hipError_t launch_gate_t(const RouteArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)((a.T + a.TB - 1) / a.TB)), block(256);
    const size_t sm = route_smem_bytes(a);
    switch (route_nv(a.E, a.G)) {
        case 1: hipLaunchKernelGGL((route_gate_topk_kernel<XT, 1>), grid, block, sm, st, a); break;
        case 2: hipLaunchKernelGGL((route_gate_topk_kernel<XT, 2>), grid, block, sm, st, a); break;
        case 4: hipLaunchKernelGGL((route_gate_topk_kernel<XT, 4>), grid, block, sm, st, a); break;
        case 8: hipLaunchKernelGGL((route_gate_topk_kernel<XT, 8>), grid, block, sm, st, a); break;
        default: hipLaunchKernelGGL((route_gate_topk_kernel<XT, 16>), grid, block, sm, st, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_route_gate(const RouteArgs& a, int dtype, hipStream_t st) {
    return dtype == MOE_BF16 ? launch_gate_t<uint16_t>(a, st) : launch_gate_t<float>(a, st);
}

hipError_t launch_route_logits(const RouteArgs& a, hipStream_t st) {
    const int gpw = kWave / a.G;
    const int64_t waves = (a.T + gpw - 1) / gpw;
    const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    switch (route_nv(a.E, a.G)) {
        case 1: hipLaunchKernelGGL((route_logits_topk_kernel<1>), grid, block, 0, st, a); break;
        case 2: hipLaunchKernelGGL((route_logits_topk_kernel<2>), grid, block, 0, st, a); break;
        case 4: hipLaunchKernelGGL((route_logits_topk_kernel<4>), grid, block, 0, st, a); break;
        case 8: hipLaunchKernelGGL((route_logits_topk_kernel<8>), grid, block, 0, st, a); break;
        default: hipLaunchKernelGGL((route_logits_topk_kernel<16>), grid, block, 0, st, a); break;
    }
    return hipGetLastError();
}

}  // namespace moe
