// route_mfma.hip -- gate GEMM on matrix cores + top-k + softmax (bf16 x, E <= 256).
//
// [PithTrain] section 4.1: linear gate, k best experts, softmax over their
// scores.  [EP] section 5.5: the routing decision is taken in fp32.
//
// fp32-accurate gate from bf16 products: every fp32 weight is the exact sum
// of three bf16 values, w = hi + mid + lo (8 + 8 + 8 significant bits, each
// the round-to-nearest-even bf16 of the remainder left by the previous ones).
// x is bf16, so x*hi, x*mid and x*lo are exact in fp32 and the three
// v_mfma_f32_16x16x32_bf16 accumulations give sum_i x[t,i] Wg[i,e] with
// fp32 accumulation, like an fp32 FMA chain (the order of the additions
// differs).
//
// split_gate_kernel writes the three parts once per call, [3][d][EP2] with
// the expert dimension zero-padded to a power of two EP2 >= 16.
// route_mfma_kernel<EP2, BM>: one workgroup owns BM tokens and all experts;
// K-steps of 32 staged global -> registers -> LDS (two buffers); the four
// waves split the expert columns (and the token rows when EP2 < 64).  The
// logit tile goes to LDS, then groups of G = EP2/4 lanes select the top k of
// each token with butterfly arg-max reductions of compile-time width.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

namespace {

__device__ __forceinline__ bf16x4_t lds_tr(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MOE_LDS bf16x4_t*)(p));
}

__device__ __forceinline__ bool beats(float av, int ai, float bv, int bi) {
    return av > bv || (av == bv && ai < bi);
}

}  // namespace

__global__ __launch_bounds__(256) void split_gate_kernel(const float* __restrict__ Wg, int d, int E, int EP2,
                                                         uint16_t* __restrict__ W3) {
    const int64_t n = (int64_t)d * EP2;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int64_t kk = i / EP2;
        const int e = (int)(i - kk * EP2);
        const float w = e < E ? Wg[kk * E + e] : 0.0f;
        const uint16_t hi = f32_to_bf16_bits(w);
        const float r1 = w - bf16_bits_to_f32(hi);     // exact
        const uint16_t mid = f32_to_bf16_bits(r1);
        const float r2 = r1 - bf16_bits_to_f32(mid);   // exact, fits 8 bits
        W3[i] = hi;
        W3[n + i] = mid;
        W3[2 * n + i] = f32_to_bf16_bits(r2);
    }
}

// Top-k + softmax of one token's logits row[0..E) by a group of G lanes.
// Lane gl holds row[gl + G*i], i < NV (E <= G*NV).  Every lane of the wave
// calls this; only active groups write.  Ties go to the lower expert index.
template <int G, int NV>
__device__ __forceinline__ void topk_group(const float* row, int E, int k, float tau, int gl, bool active,
                                           int32_t* idx_out, float* w_out) {
    float v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = gl + G * i;
        v[i] = (e < E) ? row[e] : -INFINITY;
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
#pragma unroll
        for (int off = G / 2; off > 0; off >>= 1) {
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
    const float top = __shfl(my_v, lane & ~(G - 1), kWave);
    float p = (gl < k) ? expf((my_v - top) / tau) : 0.0f;
    float z = p;
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) z += __shfl_xor(z, off, kWave);
    if (active && gl < k) {
        idx_out[gl] = my_i;
        w_out[gl] = p / z;
    }
}

template <int EP2, int BM>
__global__ __launch_bounds__(256) void route_mfma_kernel(RouteArgs a, const uint16_t* __restrict__ W3) {
    constexpr int BKG = 32;
    constexpr int WN = EP2 / 16 >= 4 ? 4 : EP2 / 16;  // waves across experts
    constexpr int WM = 4 / WN;                          // waves across tokens
    constexpr int NBW = EP2 / 16 / WN;                  // 16-expert blocks per wave
    constexpr int MBW = BM / 16 / WM;                   // 16-token blocks per wave
    static_assert(MBW >= 1 && NBW >= 1, "tile too small for four waves");
    constexpr int XP = BKG + 8;          // LDS pitch of the token tile (elements)
    constexpr int WP = EP2 + 8;          // LDS pitch of a weight tile
    constexpr int XCH = BM * BKG / 8;    // 16-byte chunks of the token tile
    constexpr int WCH = 3 * BKG * EP2 / 8;
    constexpr int LX = (XCH + 255) / 256, LW = (WCH + 255) / 256;
    constexpr int LTP = EP2 + 1;
    struct Smem {
        uint16_t xs[2][BM * XP];
        uint16_t ws[2][3 * BKG * WP];
    };
    __shared__ __attribute__((aligned(16))) union {
        Smem s;
        float lt[BM * LTP];
    } sm;

    const uint16_t* __restrict__ x = static_cast<const uint16_t*>(a.x);
    const int64_t T = a.T;
    const int d = a.d, E = a.E;
    const int64_t t0 = (int64_t)blockIdx.x * BM;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid / WN, wn = wid % WN;
    const int g16 = lane >> 4, i16 = lane & 15;
    const int64_t nW = (int64_t)d * EP2;
    const int nk = (d + BKG - 1) / BKG;

    uint4 rx[LX], rw[LW];
    auto load = [&](int kt) {
        const int k0 = kt * BKG;
#pragma unroll
        for (int j = 0; j < LX; ++j) {
            const int c = tid + 256 * j;
            if (c < XCH) {
                const int r = c >> 2, kc = (c & 3) * 8;
                const int64_t t = t0 + r;
                rx[j] = (t < T && k0 + kc < d) ? *reinterpret_cast<const uint4*>(x + t * d + k0 + kc)
                                               : make_uint4(0u, 0u, 0u, 0u);
            }
        }
#pragma unroll
        for (int j = 0; j < LW; ++j) {
            const int c = tid + 256 * j;
            if (c < WCH) {
                const int s = c / (BKG * EP2 / 8), rem = c % (BKG * EP2 / 8);
                const int kk = rem / (EP2 / 8), ec = (rem % (EP2 / 8)) * 8;
                rw[j] = (k0 + kk < d) ? *reinterpret_cast<const uint4*>(W3 + s * nW + (int64_t)(k0 + kk) * EP2 + ec)
                                      : make_uint4(0u, 0u, 0u, 0u);
            }
        }
    };
    auto store = [&](int buf) {
#pragma unroll
        for (int j = 0; j < LX; ++j) {
            const int c = tid + 256 * j;
            if (c < XCH) *reinterpret_cast<uint4*>(&sm.s.xs[buf][(c >> 2) * XP + (c & 3) * 8]) = rx[j];
        }
#pragma unroll
        for (int j = 0; j < LW; ++j) {
            const int c = tid + 256 * j;
            if (c < WCH) {
                const int s = c / (BKG * EP2 / 8), rem = c % (BKG * EP2 / 8);
                const int kk = rem / (EP2 / 8), ec = (rem % (EP2 / 8)) * 8;
                *reinterpret_cast<uint4*>(&sm.s.ws[buf][(s * BKG + kk) * WP + ec]) = rw[j];
            }
        }
    };

    f32x4_t acc[MBW][NBW];
#pragma unroll
    for (int i = 0; i < MBW; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    load(0);
    store(0);
    __syncthreads();
    for (int kt = 0; kt < nk; ++kt) {
        const int cur = kt & 1;
        if (kt + 1 < nk) load(kt + 1);
        const uint16_t* xs = sm.s.xs[cur];
        const uint16_t* wsb = sm.s.ws[cur];
        bf16x8_t xf[MBW];
#pragma unroll
        for (int mb = 0; mb < MBW; ++mb)
            xf[mb] = *reinterpret_cast<const bf16x8_t*>(&xs[((wm * MBW + mb) * 16 + i16) * XP + 8 * g16]);
#pragma unroll
        for (int s = 0; s < 3; ++s) {
#pragma unroll
            for (int nb = 0; nb < NBW; ++nb) {
                const int col = (wn * NBW + nb) * 16 + 4 * (i16 & 3);
                const int row = s * BKG + 8 * g16 + (i16 >> 2);
                const bf16x4_t lo = lds_tr(&wsb[row * WP + col]);
                const bf16x4_t hi = lds_tr(&wsb[(row + 4) * WP + col]);
                const bf16x8_t wf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
                for (int mb = 0; mb < MBW; ++mb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf, xf[mb], acc[mb][nb], 0, 0, 0);
            }
        }
        if (kt + 1 < nk) store(cur ^ 1);
        __syncthreads();
    }

    // logits (+ bias) -> LDS tile [BM][EP2]
#pragma unroll
    for (int mb = 0; mb < MBW; ++mb) {
        const int tl = (wm * MBW + mb) * 16 + i16;
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int e = (wn * NBW + nb) * 16 + 4 * g16 + q;
                const float b = (a.bg != nullptr && e < E) ? a.bg[e] : 0.0f;
                sm.lt[tl * LTP + e] = acc[mb][nb][q] + b;
            }
        }
    }
    __syncthreads();
    if (a.logits != nullptr) {
        for (int i = tid; i < BM * E; i += 256) {
            const int tl = i / E, e = i - tl * E;
            if (t0 + tl < T) a.logits[(t0 + tl) * E + e] = sm.lt[tl * LTP + e];
        }
    }
    constexpr int G = EP2 / 4 > 64 ? 64 : EP2 / 4;
    constexpr int NV = EP2 / G;
    constexpr int GPW = 64 / G;   // tokens per wave per pass
    const int gl = lane & (G - 1), gi = lane / G;
    for (int base = wid * GPW; base < BM; base += 4 * GPW) {
        const int tl = base + gi;
        const int64_t t = t0 + tl;
        const bool active = tl < BM && t < T;
        topk_group<G, NV>(sm.lt + (tl < BM ? tl : 0) * LTP, E, a.k, a.tau, gl, active,
                          a.idx + (active ? t : 0) * a.k, a.w + (active ? t : 0) * a.k);
    }
}

// ---------------------------------------------------------------- host ----

int route_mfma_ep2(int E) {
    int e = 16;
    while (e < E) e <<= 1;
    return e;
}

// the top-k groups have EP2/4 lanes (at most 64) and lane j keeps the j-th pick
bool route_mfma_supported(int dtype, int E, int k) {
    const int ep2 = route_mfma_ep2(E);
    const int g = ep2 / 4 > 64 ? 64 : ep2 / 4;
    return dtype == MOE_BF16 && E <= 256 && k <= g;
}

size_t route_mfma_ws_bytes(int d, int E) { return (size_t)3 * d * route_mfma_ep2(E) * sizeof(uint16_t); }

template <int EP2, int BM>
static void launch_bm(const RouteArgs& a, const uint16_t* W3, hipStream_t st) {
    const dim3 grid((unsigned)((a.T + BM - 1) / BM));
    hipLaunchKernelGGL((route_mfma_kernel<EP2, BM>), grid, dim3(256), 0, st, a, W3);
}

template <int EP2>
static void launch_ep2(const RouteArgs& a, const uint16_t* W3, int cus, hipStream_t st) {
    // 64-token tiles halve the weight traffic per token once they still fill the CUs
    constexpr int WM = 4 / (EP2 / 16 >= 4 ? 4 : EP2 / 16);
    if constexpr (16 * WM > 32) {
        launch_bm<EP2, 64>(a, W3, st);
    } else {
        if ((a.T + 63) / 64 >= 2 * cus) launch_bm<EP2, 64>(a, W3, st);
        else launch_bm<EP2, 32>(a, W3, st);
    }
}

hipError_t launch_route_mfma(const RouteArgs& a, uint16_t* W3, int cus, hipStream_t st) {
    const int EP2 = route_mfma_ep2(a.E);
    const int64_t n = (int64_t)a.d * EP2;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(split_gate_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a.Wg, a.d, a.E, EP2, W3);
    switch (EP2) {
        case 16: launch_ep2<16>(a, W3, cus, st); break;
        case 32: launch_ep2<32>(a, W3, cus, st); break;
        case 64: launch_ep2<64>(a, W3, cus, st); break;
        case 128: launch_ep2<128>(a, W3, cus, st); break;
        default: launch_ep2<256>(a, W3, cus, st); break;
    }
    return hipGetLastError();
}

}  // namespace moe
