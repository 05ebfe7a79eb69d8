// ffn_fp32.hip -- grouped expert GEMMs for fp32 layers on the vector ALUs.
//
// Same work list, epilogues and edge handling as the bf16 path (see
// ffn_bf16.hip and ffn_sched.h); used when x, W1, W2 and h are fp32.
// 64x64 output tile per workgroup, K-step 16, each of the 256 threads a
// 4x4 register tile; the activation tile is stored K-major in LDS so both
// operands are read as float4.
#include "ffn_sched.h"
#include "moe_kernels.h"

namespace moe {

namespace {
constexpr int FBM = 64, FBN = 64, FBK = 16;
constexpr int FAP = FBM + 4, FBP = FBN + 4;
}  // namespace

template <int EPI>
__global__ __launch_bounds__(256) void ffn_gemm_f32_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(16))) float as[FBK * FAP];
    __shared__ __attribute__((aligned(16))) float bs[FBK * FBP];
    __shared__ int mt_pre[1025];
    __shared__ int tmp[32];
    const int tid = threadIdx.x;
    const int ty = tid >> 4, tx = tid & 15;
    const int E = g.E, K = g.K, N = g.N;
    const int ntn = (N + FBN - 1) / FBN;
    const int total_mt = build_mtile_prefix(g.offsets, E, FBM, mt_pre, tmp);
    const ItemRange range = xcd_item_range((int64_t)total_mt * ntn);
    const float* __restrict__ A = static_cast<const float*>(g.A);
    const float* __restrict__ Bw = static_cast<const float*>(g.B);
    const int a_row = tid >> 2, a_kc = (tid & 3) * 4;
    const int b_row = tid >> 4, b_nc = (tid & 15) * 4;

    for (int64_t item = range.first; item < range.end; item += range.step) {
        const WorkItem wi = decode_item(mt_pre, E, ntn, item);
        const int m0 = g.offsets[wi.e] + wi.mt * FBM;
        const int mrows = min(FBM, g.offsets[wi.e + 1] - m0);
        const int n0 = wi.nt * FBN;
        const float* __restrict__ Be = Bw + (int64_t)wi.e * K * N;
        const float* a_src = A + (int64_t)(m0 + min(a_row, mrows - 1)) * K;
        const int bcol = min(n0 + b_nc, N - 4);
        float acc[4][4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;
        for (int k0 = 0; k0 < K; k0 += FBK) {
            const int ka = k0 + a_kc;
            const float4 av = (ka < K) ? *reinterpret_cast<const float4*>(a_src + ka)
                                       : make_float4(0.f, 0.f, 0.f, 0.f);
            as[(a_kc + 0) * FAP + a_row] = av.x;
            as[(a_kc + 1) * FAP + a_row] = av.y;
            as[(a_kc + 2) * FAP + a_row] = av.z;
            as[(a_kc + 3) * FAP + a_row] = av.w;
            const int kb = k0 + b_row;
            *reinterpret_cast<float4*>(&bs[b_row * FBP + b_nc]) =
                (kb < K) ? *reinterpret_cast<const float4*>(Be + (int64_t)kb * N + bcol)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
            __syncthreads();
#pragma unroll
            for (int kk = 0; kk < FBK; ++kk) {
                const float4 a4 = *reinterpret_cast<const float4*>(&as[kk * FAP + ty * 4]);
                const float4 b4 = *reinterpret_cast<const float4*>(&bs[kk * FBP + tx * 4]);
                const float ar[4] = {a4.x, a4.y, a4.z, a4.w};
                const float br[4] = {b4.x, b4.y, b4.z, b4.w};
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(ar[i], br[j], acc[i][j]);
            }
            __syncthreads();
        }
        const float* __restrict__ bias = g.bias + (int64_t)wi.e * N;
        const int n = n0 + tx * 4;
        if (n >= N) continue;
        const float4 bv = *reinterpret_cast<const float4*>(bias + n);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ml = ty * 4 + i;
            if (ml >= mrows) continue;
            const int64_t row = m0 + ml;
            float v0 = acc[i][0] + bv.x, v1 = acc[i][1] + bv.y;
            float v2 = acc[i][2] + bv.z, v3 = acc[i][3] + bv.w;
            if constexpr (EPI == EPI_GELU_H) {
                *reinterpret_cast<float4*>(static_cast<float*>(g.out) + row * N + n) =
                    make_float4(gelu_erf(v0), gelu_erf(v1), gelu_erf(v2), gelu_erf(v3));
            } else {
                *reinterpret_cast<float4*>(static_cast<float*>(g.out) + row * N + n) =
                    make_float4(v0, v1, v2, v3);
            }
        }
    }
}

template <int EPI>
static int persistent_grid_f32() {
    static int blocks = 0;
    if (blocks == 0) {
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ffn_gemm_f32_kernel<EPI>, 256, 0) !=
                hipSuccess ||
            per_cu < 1)
            per_cu = 1;
        blocks = per_cu * device_cu_count();
        if (blocks < kXcds) blocks = kXcds;
    }
    return blocks;
}

hipError_t launch_ffn_gemm_f32(const GemmArgs& g, int epi, hipStream_t st) {
    if (epi == EPI_GELU_H)
        hipLaunchKernelGGL(ffn_gemm_f32_kernel<EPI_GELU_H>, dim3(persistent_grid_f32<EPI_GELU_H>()), dim3(256), 0,
                           st, g);
    else
        hipLaunchKernelGGL(ffn_gemm_f32_kernel<EPI_STORE_F32>, dim3(persistent_grid_f32<EPI_STORE_F32>()),
                           dim3(256), 0, st, g);
    return hipGetLastError();
}

}  // namespace moe
