// ffn_bf16.hip -- grouped expert GEMMs in bf16 on CDNA4 matrix cores.
//
// [PithTrain] section 4.1 / [PyTorchMoE] section 3.2: each expert is
// Linear(d, d_ff) -> GELU -> Linear(d_ff, d) with biases.  [EP] section 5.5:
// expert math in bf16 while routing stays fp32.
//
//   GEMM1: h[r]   = GELU(x_perm[r] W1[e] + b1[e])          (EPI_GELU_H)
//   GEMM2: y[t]  += w[r] * (h[r] W2[e] + b2[e]), t = perm[r] (EPI_COMBINE)
//      or  out[r] = h[r] W2[e] + b2[e]                      (EPI_STORE_F32)
//
// Tiling: 128x128 output tile per workgroup, K-step 64, four waves of 64x64.
// Operands are staged global -> registers -> LDS with one K-step of
// register prefetch and two LDS buffers.  The inner product is
// v_mfma_f32_16x16x32_bf16 with the weight as the matrix-core A operand and
// the token rows as the B operand, so each lane's accumulator holds four
// consecutive output columns of one row (a vector store / four adjacent
// atomics in the epilogue).  Activation rows are K-contiguous and feed the
// B operand with 16-byte LDS reads; weights are N-contiguous in memory and
// are transposed on the way out of LDS by ds_read_b64_tr_b16.
//
// Edges: rows past an expert's segment are clamped on load and masked on
// store; columns past N likewise (N % 8 == 0); the K tail is zero-filled
// (K % 8 == 0).
#include "ffn_sched.h"
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int AP = BK + 8;   // LDS row pitch of the activation tile (elements)
constexpr int BP = BN + 8;   // LDS row pitch of the weight tile (elements)
constexpr int NTHREADS = 256;

struct __attribute__((aligned(16))) GemmSmem {
    uint16_t a[2][BM * AP];
    uint16_t b[2][BK * BP];
    int mt_pre[1025];
    int tmp[32];
};

__device__ __forceinline__ bf16x4_t lds_read_tr(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MOE_LDS bf16x4_t*)(p));
}

__device__ __forceinline__ bf16x8_t cat8(bf16x4_t lo, bf16x4_t hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

}  // namespace

template <int EPI>
__global__ __launch_bounds__(NTHREADS, 2) void ffn_gemm_bf16_kernel(GemmArgs g) {
    __shared__ GemmSmem sm;
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid / kWave;
    const int wm = wid >> 1, wn = wid & 1;
    const int g16 = lane >> 4, i16 = lane & 15;
    const int E = g.E, K = g.K, N = g.N;
    const int ntn = (N + BN - 1) / BN;
    const int nk = (K + BK - 1) / BK;

    const int total_mt = build_mtile_prefix(g.offsets, E, BM, sm.mt_pre, sm.tmp);
    const ItemRange range = xcd_item_range((int64_t)total_mt * ntn);

    const uint16_t* __restrict__ A = static_cast<const uint16_t*>(g.A);
    const uint16_t* __restrict__ Bw = static_cast<const uint16_t*>(g.B);

    // global -> register staging assignment (4 x 16 B of A and of B per thread)
    const int a_row0 = tid >> 3, a_kc = (tid & 7) * 8;     // rows a_row0 + 32 i
    const int b_row0 = tid >> 4, b_nc = (tid & 15) * 8;    // k-rows b_row0 + 16 i

    for (int64_t item = range.first; item < range.end; item += range.step) {
        const WorkItem wi = decode_item(sm.mt_pre, E, ntn, item);
        const int seg0 = g.offsets[wi.e];
        const int m0 = seg0 + wi.mt * BM;
        const int mrows = min(BM, g.offsets[wi.e + 1] - m0);
        const int n0 = wi.nt * BN;
        const uint16_t* __restrict__ Be = Bw + (int64_t)wi.e * K * N;

        // per-thread source pointers (rows clamped into the segment, columns into [0, N))
        const uint16_t* a_src[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = min(a_row0 + 32 * i, mrows - 1);
            a_src[i] = A + (int64_t)(m0 + r) * K + a_kc;
        }
        const int bcol = min(n0 + b_nc, N - 8);

        uint4 ra[4], rb[4];
        auto load_regs = [&](int kt) {
            const int k0 = kt * BK;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kg = k0 + a_kc;
                ra[i] = (kg < K) ? *reinterpret_cast<const uint4*>(a_src[i] + k0) : make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kg = k0 + b_row0 + 16 * i;
                rb[i] = (kg < K) ? *reinterpret_cast<const uint4*>(Be + (int64_t)kg * N + bcol)
                                 : make_uint4(0, 0, 0, 0);
            }
        };
        auto store_lds = [&](int buf) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<uint4*>(&sm.a[buf][(a_row0 + 32 * i) * AP + a_kc]) = ra[i];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *reinterpret_cast<uint4*>(&sm.b[buf][(b_row0 + 16 * i) * BP + b_nc]) = rb[i];
        };

        f32x4_t acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        load_regs(0);
        store_lds(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < nk) load_regs(kt + 1);
            const uint16_t* as = sm.a[cur];
            const uint16_t* bs = sm.b[cur];
#pragma unroll
            for (int ks = 0; ks < BK; ks += 32) {
                bf16x8_t tf[4], wf[4];
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
                    tf[mb] = *reinterpret_cast<const bf16x8_t*>(
                        &as[(wm * 64 + mb * 16 + i16) * AP + ks + 8 * g16]);
#pragma unroll
                for (int nb = 0; nb < 4; ++nb) {
                    const int col = wn * 64 + nb * 16 + 4 * (i16 & 3);
                    const int row = ks + 8 * g16 + (i16 >> 2);
                    const bf16x4_t lo = lds_read_tr(&bs[row * BP + col]);
                    const bf16x4_t hi = lds_read_tr(&bs[(row + 4) * BP + col]);
                    wf[nb] = cat8(lo, hi);
                }
#pragma unroll
                for (int mb = 0; mb < 4; ++mb)
#pragma unroll
                    for (int nb = 0; nb < 4; ++nb)
                        acc[mb][nb] =
                            __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[nb], tf[mb], acc[mb][nb], 0, 0, 0);
            }
            if (kt + 1 < nk) store_lds(cur ^ 1);
            __syncthreads();
        }

        // epilogue: lane holds out[m][n..n+3]
        const float* __restrict__ bias = g.bias + (int64_t)wi.e * N;
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) {
            const int ml = wm * 64 + mb * 16 + i16;
            if (ml >= mrows) continue;
            const int64_t row = m0 + ml;
#pragma unroll
            for (int nb = 0; nb < 4; ++nb) {
                const int n = n0 + wn * 64 + nb * 16 + 4 * g16;
                if (n >= N) continue;
                const float4 bv = *reinterpret_cast<const float4*>(bias + n);
                float v0 = acc[mb][nb][0] + bv.x, v1 = acc[mb][nb][1] + bv.y;
                float v2 = acc[mb][nb][2] + bv.z, v3 = acc[mb][nb][3] + bv.w;
                if constexpr (EPI == EPI_GELU_H) {
                    uint2 pk;
                    pk.x = (uint32_t)f32_to_bf16_bits(gelu_erf(v0)) |
                           ((uint32_t)f32_to_bf16_bits(gelu_erf(v1)) << 16);
                    pk.y = (uint32_t)f32_to_bf16_bits(gelu_erf(v2)) |
                           ((uint32_t)f32_to_bf16_bits(gelu_erf(v3)) << 16);
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.out) + row * N + n) = pk;
                } else if constexpr (EPI == EPI_STORE_F32) {
                    *reinterpret_cast<float4*>(static_cast<float*>(g.out) + row * N + n) =
                        make_float4(v0, v1, v2, v3);
                } else {
                    const int64_t t = g.perm[row];
                    const float wt = g.row_w[row];
                    float* yp = static_cast<float*>(g.out) + t * N + n;
                    atomicAdd(yp + 0, wt * v0);
                    atomicAdd(yp + 1, wt * v1);
                    atomicAdd(yp + 2, wt * v2);
                    atomicAdd(yp + 3, wt * v3);
                }
            }
        }
    }
}

template <int EPI>
static int persistent_grid() {
    static int blocks = 0;
    if (blocks == 0) {
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ffn_gemm_bf16_kernel<EPI>, NTHREADS,
                                                         0) != hipSuccess ||
            per_cu < 1)
            per_cu = 1;
        blocks = per_cu * device_cu_count();
        if (blocks < kXcds) blocks = kXcds;
    }
    return blocks;
}

hipError_t launch_ffn_gemm_bf16(const GemmArgs& g, int epi, hipStream_t st) {
    switch (epi) {
        case EPI_GELU_H:
            hipLaunchKernelGGL(ffn_gemm_bf16_kernel<EPI_GELU_H>, dim3(persistent_grid<EPI_GELU_H>()),
                               dim3(NTHREADS), 0, st, g);
            break;
        case EPI_STORE_F32:
            hipLaunchKernelGGL(ffn_gemm_bf16_kernel<EPI_STORE_F32>,
                               dim3(persistent_grid<EPI_STORE_F32>()), dim3(NTHREADS), 0, st, g);
            break;
        default:
            hipLaunchKernelGGL(ffn_gemm_bf16_kernel<EPI_COMBINE>, dim3(persistent_grid<EPI_COMBINE>()),
                               dim3(NTHREADS), 0, st, g);
            break;
    }
    return hipGetLastError();
}

}  // namespace moe
