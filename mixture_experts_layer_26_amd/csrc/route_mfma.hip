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
// split_gate_kernel writes the three parts once per call, expert-major and
// K-contiguous: [3][EP2][d], the expert dimension zero-padded to a power of
// two EP2 >= 16.
// route_mfma_kernel<EP2, BM, NS, KS>: one workgroup owns BM tokens and all
// experts.  Each K-step of 32 puts BM token rows and 3 EP2 weight rows of 64
// bytes global -> LDS (buffer_load ... lds); a stage of KS K-steps goes
// through a ring of NS slots, so NS-1 stages of loads are in flight; both
// operands are read back with ds_read_b128 from the same swizzled layout.  The four waves split the
// expert columns (and the token rows when EP2 < 64).  The logit tile goes to
// LDS, then groups of 16 lanes (one DPP row) select the top k of each
// token with arg-max reductions over DPP lane moves.
#include "lds_dma.h"
#include "moe_kernels.h"

namespace moe {

namespace {

__device__ __forceinline__ bool beats(float av, int ai, float bv, int bi) {
    return av > bv || (av == bv && ai < bi);
}

// 128-byte tile rows (two K-steps): logical 16-byte chunk c of row r sits at
// physical chunk c ^ ((r >> 1) & 7), so the 16 rows one 16-lane group reads
// (one chunk each) cover all 16 chunk positions of a 256-byte bank window
__device__ __forceinline__ int w128_swz(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int w128_at(int r, int c) { return r * 64 + 8 * (c ^ w128_swz(r)); }

}  // namespace

__global__ __launch_bounds__(256) void split_gate_kernel(const float* __restrict__ Wg, int d, int E, int EP2,
                                                         uint16_t* __restrict__ W3) {
    const int64_t n = (int64_t)d * EP2;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
        const int e = (int)(i / d);
        const int64_t kk = i - (int64_t)e * d;
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

// Cross-lane moves inside a row of 16 lanes (DPP: no LDS round trip).
// Step 0 pairs lanes 4q+{0,1},{2,3}; step 1 pairs 4q+{0,2},{1,3}; step 2
// mirrors the two quads of each 8 (i <-> 7-i); step 3 mirrors the two
// halves of each 16 (i <-> 15-i).  Each pairing is symmetric and joins two
// disjoint sets whose union is the next power-of-two group, so steps 0..s
// all-reduce groups of 2^(s+1) lanes.
template <int STEP>
__device__ __forceinline__ int dpp_partner(int v) {
    constexpr int ctrl = STEP == 0 ? 0xB1 : STEP == 1 ? 0x4E : STEP == 2 ? 0x141 : 0x140;
    return __builtin_amdgcn_mov_dpp(v, ctrl, 0xF, 0xF, false);
}
template <int STEP>
__device__ __forceinline__ float dpp_partner(float v) {
    return __int_as_float(dpp_partner<STEP>(__float_as_int(v)));
}

// Top-k + softmax of one token's logits row[0..E) by a group of G lanes
// (G = 4, 8 or 16, aligned inside a row of 16).  Lane gl holds
// row[gl + G*i], i < NV (E <= G*NV); round r takes the best value not yet
// taken (ties to the lower expert index) and lane r keeps it.  Every lane of
// the wave calls this; only active groups write.
template <int G, int NV>
__device__ __forceinline__ void topk_group(const float* row, int E, int k, float tau, int gl, bool active,
                                           int32_t* idx_out, float* w_out) {
    static_assert(G == 4 || G == 8 || G == 16, "group inside a DPP row");
    constexpr int STEPS = G == 4 ? 2 : G == 8 ? 3 : 4;
    float v[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = gl + G * i;
        v[i] = (e < E) ? row[e] : -INFINITY;
    }
    uint32_t taken = 0;
    float my_v = 0.0f, top = 0.0f;
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
        for (int st = 0; st < STEPS; ++st) {
            float ov;
            int oi;
            switch (st) {
                case 0: ov = dpp_partner<0>(bv); oi = dpp_partner<0>(bi); break;
                case 1: ov = dpp_partner<1>(bv); oi = dpp_partner<1>(bi); break;
                case 2: ov = dpp_partner<2>(bv); oi = dpp_partner<2>(bi); break;
                default: ov = dpp_partner<3>(bv); oi = dpp_partner<3>(bi); break;
            }
            if (beats(ov, oi, bv, bi)) {
                bv = ov;
                bi = oi;
            }
        }
        if ((bi & (G - 1)) == gl) taken |= 1u << (bi / G);
        if (r == 0) top = bv;
        if (gl == r) {
            my_v = bv;
            my_i = bi;
        }
    }
    const float p = (gl < k) ? expf((my_v - top) / tau) : 0.0f;
    float z = p;
#pragma unroll
    for (int st = 0; st < STEPS; ++st) {
        switch (st) {
            case 0: z += dpp_partner<0>(z); break;
            case 1: z += dpp_partner<1>(z); break;
            case 2: z += dpp_partner<2>(z); break;
            default: z += dpp_partner<3>(z); break;
        }
    }
    if (active && gl < k) {
        idx_out[gl] = my_i;
        w_out[gl] = p / z;
    }
}

// NW = 4 or 8 waves.  With 8 and SE = false, waves w and w + 4 cover the
// same logits and split every stage's K-steps (group w / 4 takes the
// K-steps q with q % 2 == w / 4); their fp32 partial sums are added once at
// the end, group 0's plus group 1's, in that order.  With 8 and SE = true
// (128 experts or more) the eight waves split the experts instead.  Either
// way two waves per SIMD hide each other's LDS and MFMA latencies.
template <int EP2, int BM, int NS, int KS, int NW = 4, bool SE = false>
__global__ __launch_bounds__(64 * NW) void route_mfma_kernel(RouteArgs a, const uint16_t* __restrict__ W3) {
    static_assert(NW == 4 || (NW == 8 && (SE || KS % 2 == 0)),
                  "four waves, or eight splitting the experts or an even K-step count");
    static_assert(!SE || (NW == 8 && EP2 >= 128), "expert split: eight waves of 16-expert blocks");
    constexpr int BKG = 32;
    constexpr int KQ = SE ? 1 : NW / 4;                 // wave groups splitting K
    constexpr int WN = SE ? 8 : EP2 / 16 >= 4 ? 4 : EP2 / 16;   // waves across experts
    constexpr int WM = (SE ? 8 : 4) / WN;               // waves across tokens
    constexpr int NBW = EP2 / 16 / WN;                  // 16-expert blocks per wave
    constexpr int MBW = BM / 16 / WM;                   // 16-token blocks per wave
    static_assert(MBW >= 1 && NBW >= 1, "tile too small for four waves");
    constexpr int ROWS = BM + 3 * EP2;       // 64-byte rows per K-step: tokens, then weight parts
    constexpr int INSTR1 = ROWS / 16;        // 1 KiB wave loads per K-step
    constexpr int INSTR = KS * INSTR1;       // per stage of KS K-steps
    constexpr int PER = (INSTR + NW - 1) / NW;   // per wave; the ones past INSTR fill unused rows
    constexpr int STAGE = NW * PER * 512;    // bf16 elements per slot
    constexpr int LTP = EP2 + 1;
    static_assert(BM % 16 == 0, "token rows in whole wave loads");
    static_assert((NS - 2) * PER < 64, "vmcnt range");
    static_assert(NS * STAGE * 2 <= 160 * 1024 && BM * LTP * 4 <= 160 * 1024, "LDS of one CU");
    __shared__ __attribute__((aligned(1024))) union {
        uint16_t ring[NS][STAGE];
        float lt[BM * LTP];
    } sm;

    const int64_t T = a.T;
    const int d = a.d, E = a.E;
    const int64_t t0 = (int64_t)blockIdx.x * BM;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wq = SE ? 0 : wid / 4, wl = SE ? wid : wid % 4;   // K group, and the wave's logits block
    const int wm = wl / WN, wn = wl % WN;
    const int g16 = lane >> 4, i16 = lane & 15;
    const int nk = (d + BKG - 1) / BKG;          // K-steps
    const int nst = (nk + KS - 1) / KS;          // stages

    // load geometry of this lane.  KS = 1: wave load j = wid * PER + i
    // covers tile rows 16 j .. +15 of the K-step; lane -> row 16 j + lane / 4,
    // physical slot lane % 4, logical chunk c = slot ^ swz(row), i.e. K
    // offset 8 c.  KS = 2: rows are 128 bytes (both K-steps of the stage, a
    // global -> LDS load of 128-byte pieces moves twice the bytes per cycle of
    // one of 64-byte pieces); load j covers rows 8 j .. +7, lane -> row
    // 8 j + lane / 8, physical chunk lane % 8, logical chunk c = chunk ^
    // w128_swz(row), K offset 8 c of the stage.
    static_assert(KS == 1 || KS == 2, "one or two K-steps per stage");
    constexpr bool W128 = KS == 2;
    const int64_t valid = T - t0 < BM ? T - t0 : BM;
    const i32x4_t rsx = make_rsrc(static_cast<const uint16_t*>(a.x) + t0 * d, (uint32_t)(valid * d * 2));
    const i32x4_t rsw = make_rsrc(W3, (uint32_t)(3u * EP2 * (uint32_t)d * 2u));
    int base[PER], c8[PER];
    bool isx[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int j = wid * PER + i;
        const int r = W128 ? 8 * j + (lane >> 3) : 16 * (j % INSTR1) + (lane >> 2);
        const int c = W128 ? (lane & 7) ^ w128_swz(r) : (lane & 3) ^ k64_swz(r);
        const int src_row = r < BM ? r : r - BM;    // token row of the block, or weight row s * EP2 + e
        const int kofs = W128 ? 8 * c : 8 * c + BKG * (j / INSTR1);
        base[i] = (src_row * d + kofs) * 2;
        c8[i] = kofs;
        isx[i] = r < BM;
    }
    auto issue = [&](int st, int slot) {   // st >= nst: every load out of range
        const int k0 = st * KS * BKG;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int j = wid * PER + i;
            const bool ok = j < INSTR && st < nst && k0 + c8[i] < d;
            const int off = ok ? base[i] + 2 * k0 : kOutOfRange;
            dma16(isx[i] ? rsx : rsw, &sm.ring[slot][j * 512], off);
        }
    };

    f32x4_t acc[MBW][NBW];
#pragma unroll
    for (int i = 0; i < MBW; ++i)
#pragma unroll
        for (int j = 0; j < NBW; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    for (int s = 0; s < NS - 1; ++s) issue(s, s);
    int slot = 0;
    for (int st = 0; st < nst; ++st) {
        // stage st has landed for every wave; slot (st - 1) % NS is free
        dma_barrier<(NS - 2) * PER>();
        issue(st + NS - 1, slot == 0 ? NS - 1 : slot - 1);
        const uint16_t* sp = sm.ring[slot];
        // every fragment of the stage first, then the MFMAs (this wave's
        // K-steps of the stage only)
        bf16x8_t xf[KS][MBW], wf[KS][3][NBW];
#pragma unroll
        for (int q = 0; q < KS; ++q) {
            if (q % KQ != wq) continue;
            const uint16_t* sq = sp + q * INSTR1 * 512;
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb)
                xf[q][mb] = *reinterpret_cast<const bf16x8_t*>(
                    W128 ? &sp[w128_at((wm * MBW + mb) * 16 + i16, 4 * q + g16)]
                         : &sq[k64_slot((wm * MBW + mb) * 16 + i16, g16) * 8]);
#pragma unroll
            for (int s = 0; s < 3; ++s)
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb)
                    wf[q][s][nb] = *reinterpret_cast<const bf16x8_t*>(
                        W128 ? &sp[w128_at(BM + s * EP2 + (wn * NBW + nb) * 16 + i16, 4 * q + g16)]
                             : &sq[k64_slot(BM + s * EP2 + (wn * NBW + nb) * 16 + i16, g16) * 8]);
        }
#pragma unroll
        for (int q = 0; q < KS; ++q) {
            if (q % KQ != wq) continue;
#pragma unroll
            for (int s = 0; s < 3; ++s)
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb)
#pragma unroll
                    for (int mb = 0; mb < MBW; ++mb)
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[q][s][nb], xf[q][mb], acc[mb][nb],
                                                                               0, 0, 0);
        }
        slot = slot + 1 == NS ? 0 : slot + 1;
    }
    // the trailing out-of-range loads still write the ring, which the logit
    // tile overlays
    dma_barrier<0>();

    // logits (+ bias) -> LDS tile [BM][EP2]; with two K groups, group 1 puts
    // its partial sums there first and group 0 adds its own to them
    for (int g = KQ - 1; g >= 0; --g) {
        if (wq == g) {
#pragma unroll
            for (int mb = 0; mb < MBW; ++mb) {
                const int tl = (wm * MBW + mb) * 16 + i16;
#pragma unroll
                for (int nb = 0; nb < NBW; ++nb) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int e = (wn * NBW + nb) * 16 + 4 * g16 + q;
                        if (g > 0) {
                            sm.lt[tl * LTP + e] = acc[mb][nb][q];
                        } else {
                            const float b = (a.bg != nullptr && e < E) ? a.bg[e] : 0.0f;
                            const float v = KQ > 1 ? acc[mb][nb][q] + sm.lt[tl * LTP + e] : acc[mb][nb][q];
                            sm.lt[tl * LTP + e] = v + b;
                        }
                    }
                }
            }
        }
        __syncthreads();
    }
    if (a.logits != nullptr) {
        for (int i = tid; i < BM * E; i += 64 * NW) {
            const int tl = i / E, e = i - tl * E;
            if (t0 + tl < T) a.logits[(t0 + tl) * E + e] = sm.lt[tl * LTP + e];
        }
    }
    // one DPP row of 16 lanes per token, whatever the expert count: k up to
    // 16 winners (k = E for the dense soft layer of 16 experts)
    constexpr int G = 16;
    constexpr int NV = EP2 / G;
    constexpr int GPW = 64 / G;   // tokens per wave per pass
    const int gl = lane & (G - 1), gi = lane / G;
    for (int base = wid * GPW; base < BM; base += NW * GPW) {
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

// the top-k groups have 16 lanes and lane j keeps the j-th pick
bool route_mfma_supported(int dtype, int E, int k) {
    return dtype == MOE_BF16 && E <= 256 && k <= 16;
}

size_t route_mfma_ws_bytes(int d, int E) { return (size_t)3 * d * route_mfma_ep2(E) * sizeof(uint16_t); }

template <int EP2, int BM, int NS, int KS, int NW = 4, bool SE = false>
static void launch_bm(const RouteArgs& a, const uint16_t* W3, hipStream_t st) {
    const dim3 grid((unsigned)((a.T + BM - 1) / BM));
    hipLaunchKernelGGL((route_mfma_kernel<EP2, BM, NS, KS, NW, SE>), grid, dim3(64 * NW), 0, st, a, W3);
}

// Tile choice per expert width.  Up to 64 experts: 32- or 64-token tiles,
// two K-steps per stage (one barrier and one batch of LDS reads per 64 of
// K), ring of 4 slots.  128 experts: 32-token tiles, one K-step per stage,
// 4 slots of 32 KiB, eight waves splitting the experts.  256 experts:
// 128-token tiles halve the re-reads of the 3 MiB weight split per token;
// one K-step per stage, 2 slots, eight waves splitting the experts (with
// four, one wave per SIMD, the workload of 256 experts and 32768 tokens took
// 241 us instead of 161; 128 experts and 8192 tokens 42 instead of 36).
#ifndef MOE_ROUTE_NW
#define MOE_ROUTE_NW 8   // waves per workgroup up to 64 experts
#endif
#ifndef MOE_ROUTE_BM64_MIN
#define MOE_ROUTE_BM64_MIN 256   // 64-token tiles from this many workgroups per 256 CUs
#endif

template <int EP2>
static void launch_ep2(const RouteArgs& a, const uint16_t* W3, int cus, hipStream_t st) {
    constexpr int WM = 4 / (EP2 / 16 >= 4 ? 4 : EP2 / 16);
    if constexpr (EP2 == 256) {
        if ((a.T + 127) / 128 >= cus) launch_bm<256, 128, 2, 1, 8, true>(a, W3, st);
        else launch_bm<256, 64, 3, 1>(a, W3, st);
    } else if constexpr (EP2 == 128) {
        launch_bm<128, 32, 4, 1, 8, true>(a, W3, st);
    } else if constexpr (16 * WM > 32) {
        launch_bm<EP2, 64, 4, 2, MOE_ROUTE_NW>(a, W3, st);
    } else {
        // 64-token tiles halve the weight traffic per token once they still fill the CUs
        if ((a.T + 63) / 64 >= MOE_ROUTE_BM64_MIN * cus / 256) launch_bm<EP2, 64, 4, 2, MOE_ROUTE_NW>(a, W3, st);
        else launch_bm<EP2, 32, 4, 2, MOE_ROUTE_NW>(a, W3, st);
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
