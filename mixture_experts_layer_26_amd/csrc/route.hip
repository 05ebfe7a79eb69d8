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
// thread an MR x 4 register tile).  Phase 2 hands each token to a group of G
// lanes (G = E rounded up to a power of two, at most 64); each lane keeps
// ceil(E/G) logits in registers and k rounds of butterfly arg-max (shuffle
// xor) pick the winners, ties to the lower expert index.
#include "moe_common.h"
#include "moe_kernels.h"

#include <algorithm>

namespace moe {

__device__ __forceinline__ bool beats(float av, int ai, float bv, int bi) {
    return av > bv || (av == bv && ai < bi);
}

// Top-k + softmax of one token's logits by a group of G lanes (G a power of
// two <= 64, groups aligned inside the wave); lane gl holds logits
// v[i] = L[gl + G i], NV >= ceil(E/G).  Every lane of the wave must call this
// (shuffles); only `active` groups write.  Lane gl of the group ends up
// holding the gl-th winner.
template <int NV>
__device__ __forceinline__ void topk_softmax_regs(const float (&v)[NV], int E, int k, float tau, int G, int gl,
                                                  bool active, int32_t* idx_out, float* w_out) {
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
    topk_softmax_regs<NV>(v, E, k, tau, G, gl, active, idx_out, w_out);
}

// Top-1 over a softmax of all E logits ([PyTorchMoE] sections 2.3, 4.3): the
// largest logit (ties to the lower index) and, as its weight, its softmax
// probability 1 / sum_e exp((L_e - L_max) / tau).  Same lane layout as above.
template <int NV>
__device__ __forceinline__ void top1_full_softmax_regs(const float (&v)[NV], int E, float tau, int G, int gl,
                                                       bool active, int32_t* idx_out, float* w_out) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = gl + G * i;
        if (e < E && beats(v[i], e, bv, bi)) {
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
    float z = 0.0f;
#pragma unroll
    for (int i = 0; i < NV; ++i)
        if (gl + G * i < E) z += expf((v[i] - bv) / tau);
    for (int off = G >> 1; off > 0; off >>= 1) z += __shfl_xor(z, off, kWave);
    if (active && gl == 0) {
        idx_out[0] = bi;
        w_out[0] = 1.0f / z;
    }
}

// Phase 1 geometry (host: route_config): thread (tq, eq) owns an MR x 4
// block of the [TB x E] logit tile; each K-chunk of x (16-byte vectors) and of
// Wg (scalars, rows padded to EP2 = 2^lep) is loaded into registers one chunk
// ahead of its use, so global latency overlaps the FMAs of the previous chunk.
constexpr int kMaxXV = 4;    // 16-byte x vectors per thread per K-chunk
constexpr int kMaxWS = 32;   // Wg scalars per thread per K-chunk

template <typename XT>
__device__ __forceinline__ void unpack16(const uint4& v, float* o);
template <>
__device__ __forceinline__ void unpack16<float>(const uint4& v, float* o) {
    o[0] = __uint_as_float(v.x);
    o[1] = __uint_as_float(v.y);
    o[2] = __uint_as_float(v.z);
    o[3] = __uint_as_float(v.w);
}
template <>
__device__ __forceinline__ void unpack16<uint16_t>(const uint4& v, float* o) {
    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        o[2 * i] = __uint_as_float(u[i] << 16);
        o[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
}

template <typename XT, int MR, int NV>
__global__ __launch_bounds__(256) void route_gate_topk_kernel(RouteArgs a) {
    extern __shared__ __attribute__((aligned(16))) float smem[];
    constexpr int VEC = 16 / sizeof(XT);
    const int TB = a.TB, Epad = a.Epad, KC = a.KC, KCP = a.KC + 1, LTP = a.Epad + 1;
    const int EP2 = 1 << a.lep;
    float* xs = smem;                          // [TB][KCP]
    float* wsm = xs + ((TB * KCP + 3) & ~3);   // [KC][EP2], 16-byte aligned
    float* lt = wsm + KC * EP2;    // [TB][LTP]
    const XT* __restrict__ x = static_cast<const XT*>(a.x);
    const int64_t T = a.T;
    const int d = a.d, E = a.E;
    const int64_t t0 = (int64_t)blockIdx.x * TB;
    const int tid = threadIdx.x;
    const int n_eq = Epad / 4, n_tq = TB / MR;
    const int tq = tid / n_eq, eq = tid % n_eq;
    const bool comp = tid < n_eq * n_tq;
    const int lkv = a.lkv;                 // log2(KC / VEC)
    const int nxv = TB << lkv;             // x vectors per chunk
    const int nws = KC << a.lep;           // Wg scalars per chunk

    float acc[MR][4];
#pragma unroll
    for (int i = 0; i < MR; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

    uint4 xr[kMaxXV];
    float wr[kMaxWS];
    auto load = [&](int k0) {
#pragma unroll
        for (int i = 0; i < kMaxXV; ++i) {
            const int v = tid + 256 * i;
            if (v < nxv) {
                const int tt = v >> lkv, kv = v & ((1 << lkv) - 1);
                const int64_t t = t0 + tt;
                const int kg = k0 + kv * VEC;
                xr[i] = (t < T && kg < d) ? *reinterpret_cast<const uint4*>(x + t * d + kg)
                                          : make_uint4(0u, 0u, 0u, 0u);
            }
        }
#pragma unroll
        for (int j = 0; j < kMaxWS; ++j) {
            const int i = tid + 256 * j;
            if (i < nws) {
                const int kk = i >> a.lep, e = i & (EP2 - 1);
                const int kg = k0 + kk;
                wr[j] = (kg < d && e < E) ? a.Wg[(int64_t)kg * E + e] : 0.0f;
            }
        }
    };
    auto store = [&]() {
#pragma unroll
        for (int i = 0; i < kMaxXV; ++i) {
            const int v = tid + 256 * i;
            if (v < nxv) {
                const int tt = v >> lkv, kv = v & ((1 << lkv) - 1);
                float f[VEC];
                unpack16<XT>(xr[i], f);
#pragma unroll
                for (int q = 0; q < VEC; ++q) xs[tt * KCP + kv * VEC + q] = f[q];
            }
        }
#pragma unroll
        for (int j = 0; j < kMaxWS; ++j) {
            const int i = tid + 256 * j;
            if (i < nws) wsm[i] = wr[j];
        }
    };

    load(0);
    for (int k0 = 0; k0 < d; k0 += KC) {
        store();
        __syncthreads();
        if (k0 + KC < d) load(k0 + KC);
        if (comp) {
            const int kmax = min(KC, d - k0);
            auto step = [&](int kk) {
                const float4 wv = *reinterpret_cast<const float4*>(&wsm[kk * EP2 + 4 * eq]);
                float xv[MR];
#pragma unroll
                for (int i = 0; i < MR; ++i) xv[i] = xs[(MR * tq + i) * KCP + kk];
#pragma unroll
                for (int i = 0; i < MR; ++i) {
                    acc[i][0] = fmaf(xv[i], wv.x, acc[i][0]);
                    acc[i][1] = fmaf(xv[i], wv.y, acc[i][1]);
                    acc[i][2] = fmaf(xv[i], wv.z, acc[i][2]);
                    acc[i][3] = fmaf(xv[i], wv.w, acc[i][3]);
                }
            };
            int kk = 0;
            for (; kk + 8 <= kmax; kk += 8) {   // batches the LDS reads of 8 steps
#pragma unroll
                for (int u = 0; u < 8; ++u) step(kk + u);
            }
            for (; kk < kmax; ++kk) step(kk);
        }
        __syncthreads();
    }
    if (comp) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = 4 * eq + j;
            const float b = (a.bg != nullptr && e < E) ? a.bg[e] : 0.0f;
#pragma unroll
            for (int i = 0; i < MR; ++i) lt[(MR * tq + i) * LTP + e] = acc[i][j] + b;
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

// Top-k of any k <= E <= 1024 by rank, one wave per token: expert e's rank
// is the number of experts that beat it (a larger logit, or an equal one at a
// lower index), which is its place in the order the k rounds of selection
// take; the experts of rank < k go to idx[t, rank] with weights
// exp((l - l_top) / tau) over their sum (l_top: the largest logit, rank 0).
// O(E^2) comparisons per token, the row read from LDS.  For k above the
// register groups' 32, up to the soft MoE over every expert (k = E).
constexpr int kRankMaxE = 1024;

__global__ __launch_bounds__(64) void route_rank_kernel(RouteArgs a) {
    __shared__ float row[kRankMaxE];
    __shared__ int rank_s[kRankMaxE];
    __shared__ float p_s[kRankMaxE];
    const int64_t t = blockIdx.x;
    const int E = a.E, k = a.k, lane = threadIdx.x;
    const float* L = a.logits + t * E;
    float top = -INFINITY;
    for (int e = lane; e < E; e += kWave) {
        row[e] = L[e];
        top = fmaxf(top, L[e]);
    }
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) top = fmaxf(top, __shfl_xor(top, off, kWave));
    __syncthreads();
    float z = 0.0f;
    for (int e = lane; e < E; e += kWave) {
        const float v = row[e];
        int r = 0;
        for (int e2 = 0; e2 < E; ++e2) {
            const float u = row[e2];
            r += (u > v || (u == v && e2 < e)) ? 1 : 0;
        }
        const float p = r < k ? expf((v - top) / a.tau) : 0.0f;
        rank_s[e] = r;
        p_s[e] = p;
        z += p;
    }
    z = wave_sum(z);
    for (int e = lane; e < E; e += kWave) {
        const int r = rank_s[e];
        if (r < k) {
            a.idx[t * k + r] = e;
            a.w[t * k + r] = p_s[e] / z;
        }
    }
}

hipError_t launch_route_rank(const RouteArgs& a, hipStream_t st) {
    if (a.E > kRankMaxE) return hipErrorInvalidValue;
    hipLaunchKernelGGL(route_rank_kernel, dim3((unsigned)a.T), dim3(kWave), 0, st, a);
    return hipGetLastError();
}

// fp32(l + fp32(scale * n)): two roundings, as two fp32 operations; the
// pragma keeps the compiler from contracting them into one fused
// multiply-add (one rounding), which routes differently at near-ties
__device__ __forceinline__ float noisy_logit(float l, float scale, float n) {
#pragma clang fp contract(off)
    const float p = scale * n;
    return l + p;
}

// Router variants on logits in global memory.  With `noise`, the routed
// values are the stable layer's exploration noise of [PyTorchMoE] section 4.3
// in the page's fp32 arithmetic: fp32(L + fp32(scale * n)), product and sum
// rounded separately (no fused multiply-add); `noisy` (optional) receives
// them.  mode MOE_ROUTER_TOPK: top-k + softmax over the selected values;
// MOE_ROUTER_TOP1_FULL (k = 1): top-1 weighted by the full softmax.
template <int NV>
__global__ __launch_bounds__(256) void route_variant_kernel(RouteArgs a, int mode, const float* __restrict__ noise,
                                                           float scale, float* __restrict__ noisy) {
    const int G = a.G;
    const int lane = threadIdx.x & (kWave - 1);
    const int gpw = kWave / G;
    const int gl = lane & (G - 1), gi = lane / G;
    const int64_t gwave = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    const int64_t t = gwave * gpw + gi;
    const bool active = t < a.T;
    const int64_t base = (active ? t : 0) * a.E;
    float v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = gl + G * i;
        const bool in = active && e < a.E;
        float x = in ? a.logits[base + e] : 0.0f;
        if (noise != nullptr && in) x = noisy_logit(x, scale, noise[base + e]);
        if (noisy != nullptr && in) noisy[base + e] = x;
        v[i] = x;
    }
    int32_t* io = a.idx + (active ? t : 0) * a.k;
    float* wo = a.w + (active ? t : 0) * a.k;
    if (mode == MOE_ROUTER_TOP1_FULL) top1_full_softmax_regs<NV>(v, a.E, a.tau, G, gl, active, io, wo);
    else topk_softmax_regs<NV>(v, a.E, a.k, a.tau, G, gl, active, io, wo);
}

// ---------------------------------------------------------------- host ----

static int route_nv(int E, int G) {
    const int nv = (E + G - 1) / G;
    return nv <= 1 ? 1 : nv <= 2 ? 2 : nv <= 4 ? 4 : nv <= 8 ? 8 : 16;
}

static int ilog2(int v) {
    int l = 0;
    while ((1 << l) < v) ++l;
    return l;
}

RouteArgs route_config(int64_t T, int d, int E, int k, float tau, int dtype, int cus) {
    RouteArgs a{};
    a.T = T;
    a.d = d;
    a.E = E;
    a.k = k;
    a.tau = tau;
    a.Epad = (E + 3) & ~3;
    a.lep = ilog2(a.Epad);
    const int EP2 = 1 << a.lep;
    const int n_eq = a.Epad / 4;
    const int n_tq = 256 / n_eq;
    // largest micro-tile height that still gives every CU a workgroup
    int mr = 4;
    while (mr > 1 && (T + (int64_t)std::min(256, mr * n_tq) - 1) / std::min(256, mr * n_tq) < cus) mr >>= 1;
    a.MR = mr;
    a.TB = std::min(256 / mr, n_tq) * mr;
    int g = 1;
    while (g < E && g < kWave) g <<= 1;
    a.G = g;
    const int vec = dtype == MOE_BF16 ? 8 : 4;
    const int budget = 16384;  // floats of LDS per workgroup (64 KiB)
    int kc = 64;
    while (kc > 8 && (a.TB * kc / vec > 256 * kMaxXV || kc * EP2 > 256 * kMaxWS ||
                      a.TB * (kc + 1) + 3 + kc * EP2 + a.TB * (a.Epad + 1) > budget))
        kc >>= 1;
    a.KC = kc;
    a.lkv = ilog2(kc / vec);
    return a;
}

size_t route_smem_bytes(const RouteArgs& a) {
    return sizeof(float) * ((((size_t)a.TB * (a.KC + 1) + 3) & ~size_t(3)) + ((size_t)a.KC << a.lep) +
                            (size_t)a.TB * (a.Epad + 1));
}

template <typename XT, int MR>
static void launch_gate_mr(const RouteArgs& a, dim3 grid, size_t sm, hipStream_t st) {
    switch (route_nv(a.E, a.G)) {
        case 1: hipLaunchKernelGGL((route_gate_topk_kernel<XT, MR, 1>), grid, dim3(256), sm, st, a); break;
        case 2: hipLaunchKernelGGL((route_gate_topk_kernel<XT, MR, 2>), grid, dim3(256), sm, st, a); break;
        case 4: hipLaunchKernelGGL((route_gate_topk_kernel<XT, MR, 4>), grid, dim3(256), sm, st, a); break;
        case 8: hipLaunchKernelGGL((route_gate_topk_kernel<XT, MR, 8>), grid, dim3(256), sm, st, a); break;
        default: hipLaunchKernelGGL((route_gate_topk_kernel<XT, MR, 16>), grid, dim3(256), sm, st, a); break;
    }
}

template <typename XT>
static hipError_t launch_gate_t(const RouteArgs& a, hipStream_t st) {
    const dim3 grid((unsigned)((a.T + a.TB - 1) / a.TB));
    const size_t sm = route_smem_bytes(a);
    if (a.MR == 4) launch_gate_mr<XT, 4>(a, grid, sm, st);
    else if (a.MR == 2) launch_gate_mr<XT, 2>(a, grid, sm, st);
    else launch_gate_mr<XT, 1>(a, grid, sm, st);
    return hipGetLastError();
}

hipError_t launch_route_gate(const RouteArgs& a, int dtype, hipStream_t st) {
    return dtype == MOE_BF16 ? launch_gate_t<uint16_t>(a, st) : launch_gate_t<float>(a, st);
}

hipError_t launch_route_variant(const RouteArgs& a, int mode, const float* noise, float scale, float* noisy,
                                hipStream_t st) {
    const int gpw = kWave / a.G;
    const int64_t waves = (a.T + gpw - 1) / gpw;
    const dim3 grid((unsigned)((waves + 3) / 4)), block(256);
    switch (route_nv(a.E, a.G)) {
        case 1: hipLaunchKernelGGL((route_variant_kernel<1>), grid, block, 0, st, a, mode, noise, scale, noisy); break;
        case 2: hipLaunchKernelGGL((route_variant_kernel<2>), grid, block, 0, st, a, mode, noise, scale, noisy); break;
        case 4: hipLaunchKernelGGL((route_variant_kernel<4>), grid, block, 0, st, a, mode, noise, scale, noisy); break;
        case 8: hipLaunchKernelGGL((route_variant_kernel<8>), grid, block, 0, st, a, mode, noise, scale, noisy); break;
        default: hipLaunchKernelGGL((route_variant_kernel<16>), grid, block, 0, st, a, mode, noise, scale, noisy); break;
    }
    return hipGetLastError();
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
