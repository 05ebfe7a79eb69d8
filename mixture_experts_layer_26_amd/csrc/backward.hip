// backward.hip -- backward of the MoE layer forward (gfx950).
//
// Gradients of sum(dy * y) with the forward's routing decisions (selection,
// capacity, drops) fixed; they are piecewise constant.  [PithTrain] section
// 4.1's layer is differentiated as autograd would: the combine y[t] +=
// w[t,j] o[r], the expert FFN o = GELU(x W1 + b1) W2 + b2 and the gate
// w = softmax(l_sel / tau), l = x Wg (+ bg).  Only experts that received rows
// get weight gradients; the others are zero ([EP] section 4.3, expert-grained
// gradients).
//
// Launch sequence (moe_layer_backward):
//   1. combine_backward: per kept slot, dw[t,j] = dy[t] . o[r] and the
//      expert-output gradient g[r] = w[t,j] dy[t] (packed rows);
//   2. recompute per row a = x_perm W1 + b1 -> h = GELU(a), h' = GELU'(a);
//   3. dh = g W2^T, da = dh * h'           (rows of each expert);
//   4. dx_perm = da W1^T                   (rows of each expert);
//   5. dW2[e] = h^T g, dW1[e] = x_perm^T da (sums over each expert's rows);
//   6. db2[e], db1[e]: column sums of g and da over each expert's rows;
//   7. gate: dl[t, idx_j] = w_j (dw_j - sum_i w_i dw_i) / tau (zero at the
//      other E - k logits), dWg = x^T dl and dbg = column sums of dl, each a
//      sum over the tokens that selected the expert (grouped by expert);
//   8. dx[t] = sum_j dx_perm[slot[t,j]] + sum_j dl[t, idx_j] Wg[:, idx_j].
// Arithmetic.  fp32 layers: every GEMM in fp32 on the vector ALUs (one
// tiled kernel, 64 x 64 outputs per workgroup, 4 x 4 per thread, K in steps
// of 16 through LDS), GELU and GELU' from the device library's erff.  bf16
// layers: the expert GEMMs run on bf16 matrix cores with fp32 accumulation
// (the forward's pipelined 256 x 256 kernel for large problems,
// bw_mfma_kernel otherwise); their operands g = w dy and da = dh GELU'(a)
// are rounded to bf16 (a 2^-9 relative rounding each, like h; GELU'(a) is
// kept in bf16 between the recompute and the dh GEMM), h is recomputed in
// bf16 and GELU / GELU' use the forward's erf approximation
// (Abramowitz & Stegun 7.1.26); bias gradients are column sums of the bf16 g
// and da in fp32.  The gate's gradients (both layer types) are fp32 sums of
// the k nonzero terms per token (bf16 x widened exactly).  Three operand
// patterns:
//   NN: A rows of a segment, K-contiguous; B = W[e] [K][N]
//   NT: A rows of a segment, K-contiguous; B = W[e] stored [N][K]
//   TN: A and B both rows of a segment; K runs over the segment's rows
#include "ffn_sched.h"
#include "moe_kernels.h"

#include <type_traits>

namespace moe {

namespace {

constexpr int BW_BM = 64, BW_BN = 64, BW_BK = 16, BW_THREADS = 256;
constexpr int BW_PAD = 4;   // LDS row padding (floats)

enum { BW_NN = 0, BW_NT = 1, BW_TN = 2 };
enum { BWE_HGRAD = 0, BWE_DA = 1, BWE_STORE = 2, BWE_WGRAD = 3 };

template <typename T>
__device__ __forceinline__ float ld_elem(const T* p, int64_t i);
template <>
__device__ __forceinline__ float ld_elem<float>(const float* p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float ld_elem<uint16_t>(const uint16_t* p, int64_t i) { return bf16_bits_to_f32(p[i]); }

template <typename T>
__device__ __forceinline__ void st_elem(T* p, int64_t i, float v);
template <>
__device__ __forceinline__ void st_elem<float>(float* p, int64_t i, float v) { p[i] = v; }
template <>
__device__ __forceinline__ void st_elem<uint16_t>(uint16_t* p, int64_t i, float v) { p[i] = f32_to_bf16_bits(v); }

// d/du [u Phi(u)] = Phi(u) + u phi(u), fp32 with the device library's erff
__device__ __forceinline__ float gelu_grad(float u) {
    return 0.5f * (1.0f + erff(u * 0.70710678118654752440f)) +
           u * expf(-0.5f * u * u) * 0.39894228040143267794f;
}

}  // namespace

// C[m][n] = sum_k A(m,k) B(k,n) for every item; see the header comment for
// the operand patterns.  Row segments come from offsets[E+1].
template <int MODE, int EPI, typename TA, typename TB, typename TH>
__global__ __launch_bounds__(BW_THREADS) void bw_gemm_kernel(BwGemmArgs g) {
    __shared__ __attribute__((aligned(16))) float As[BW_BK][BW_BM + BW_PAD];
    __shared__ __attribute__((aligned(16))) float Bs[BW_BK][BW_BN + BW_PAD];
    __shared__ int mt_pre[1025];
    __shared__ int scan_tmp[32];
    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;   // 4 x 4 outputs: rows 4 ty.., cols 4 tx..
    const int ntn = (g.N + BW_BN - 1) / BW_BN;
    const TA* A = static_cast<const TA*>(g.A);
    const TB* B = static_cast<const TB*>(g.B);

    // ---- the item: expert e, rows [m0, m0 + mrows) or K range [k0, k1) ----
    int e, m0, mrows, n0, kb, kend;
    if constexpr (MODE == BW_TN) {
        const int mtn = (g.M + BW_BM - 1) / BW_BM;
        const int64_t item = blockIdx.x;
        e = (int)(item / ((int64_t)mtn * ntn));
        const int rest = (int)(item - (int64_t)e * mtn * ntn);
        m0 = (rest / ntn) * BW_BM;
        n0 = (rest % ntn) * BW_BN;
        mrows = min(BW_BM, g.M - m0);
        kb = g.offsets[e];
        kend = g.offsets[e + 1];
    } else {
        const int total_mt = build_mtile_prefix(g.offsets, g.E, BW_BM, mt_pre, scan_tmp);
        if ((int64_t)blockIdx.x >= (int64_t)total_mt * ntn) return;
        const WorkItem wi = decode_item(mt_pre, g.E, ntn, blockIdx.x);
        e = wi.e;
        m0 = g.offsets[e] + wi.mt * BW_BM;
        mrows = min(BW_BM, g.offsets[e + 1] - m0);
        n0 = wi.nt * BW_BN;
        kb = 0;
        kend = g.K;
    }
    const int64_t bbase = (MODE == BW_TN) ? 0 : (int64_t)e * g.b_estride;

    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

    // staging: each thread moves 4 elements of each 16 x 64 tile
    for (int k0 = kb; k0 < kend; k0 += BW_BK) {
        // A tile, As[k][m]
        if constexpr (MODE == BW_TN) {
            // A(m, k) = A[k lda + m]: 4 consecutive m at one k
            const int kk = tid >> 4, mm = (tid & 15) * 4;
            const int k = k0 + kk;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int m = m0 + mm + q;
                As[kk][mm + q] = (k < kend && mm + q < mrows) ? ld_elem<TA>(A, (int64_t)k * g.lda + m) : 0.0f;
            }
        } else {
            // A(m, k) = A[(m0 + m) lda + k]: 4 consecutive k of one row
            const int mm = tid >> 2, kk = (tid & 3) * 4;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int k = k0 + kk + q;
                As[kk + q][mm] = (mm < mrows && k < kend) ? ld_elem<TA>(A, (int64_t)(m0 + mm) * g.lda + k) : 0.0f;
            }
        }
        // B tile, Bs[k][n]
        if constexpr (MODE == BW_NT) {
            // B(k, n) = B[e: n ldb + k]: 4 consecutive k of one column
            const int nn = tid >> 2, kk = (tid & 3) * 4;
            const int n = n0 + nn;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int k = k0 + kk + q;
                Bs[kk + q][nn] = (n < g.N && k < kend) ? ld_elem<TB>(B, bbase + (int64_t)n * g.ldb + k) : 0.0f;
            }
        } else {
            // NN: B(k, n) = B[e: k ldb + n]; TN: B[k ldb + n] (rows of the segment)
            const int kk = tid >> 4, nn = (tid & 15) * 4;
            const int k = k0 + kk;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int n = n0 + nn + q;
                Bs[kk][nn + q] = (k < kend && n < g.N) ? ld_elem<TB>(B, bbase + (int64_t)k * g.ldb + n) : 0.0f;
            }
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BW_BK; ++kk) {
            const float4 a = *reinterpret_cast<const float4*>(&As[kk][ty * 4]);
            const float4 b = *reinterpret_cast<const float4*>(&Bs[kk][tx * 4]);
            const float av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
        }
        __syncthreads();
    }

    // ---- epilogue ----
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = ty * 4 + i;
        if (m >= mrows) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n >= g.N) continue;
            float v = acc[i][j];
            if constexpr (EPI == BWE_WGRAD) {
                // dW[e][m0 + m][n]
                static_cast<float*>(g.C)[(int64_t)e * g.M * g.N + (int64_t)(m0 + m) * g.N + n] = v;
            } else {
                const int64_t ci = (int64_t)(m0 + m) * g.N + n;
                if constexpr (EPI == BWE_HGRAD) {
                    v += g.bias[(int64_t)e * g.N + n];
                    st_elem<TH>(static_cast<TH*>(g.C), ci, gelu_erf(v));
                    static_cast<float*>(g.C2)[ci] = gelu_grad(v);
                } else if constexpr (EPI == BWE_DA) {
                    static_cast<float*>(g.C)[ci] = v * static_cast<const float*>(g.C2)[ci];
                } else {
                    static_cast<float*>(g.C)[ci] = v;
                }
            }
        }
    }
}

// bf16 layers: the same three patterns on v_mfma_f32_16x16x32_bf16, 128 x
// 128 outputs per workgroup (four waves of 64 x 64), K in steps of 32.  An
// operand keeps its global layout in LDS, staged with 16-byte loads and
// stores: K-contiguous ones as [row][k] (rows padded to 40 elements so the
// 16 rows of a fragment read fall on disjoint banks), read with
// ds_read_b128; M/N-contiguous ones (W1 in the recompute, both operands of
// the weight gradients) as [k][row] (padded to 136), read with
// ds_read_b64_tr_b16, which hands each lane the K-run of its own row.  Two
// LDS buffers: a step multiplies one while the next tile goes into the
// other and the one after is loaded into registers.
constexpr int BWM_BM = 128, BWM_BN = 128, BWM_BK = 32, BWM_LDK = BWM_BK + 8, BWM_LDM = BWM_BM + 8;
constexpr int BWM_TILE = BWM_BM * BWM_LDK > BWM_BK * BWM_LDM ? BWM_BM * BWM_LDK : BWM_BK * BWM_LDM;

template <bool KC>   // KC: the operand is K-contiguous in global memory
__device__ __forceinline__ void bwm_load(const uint16_t* p, int64_t ld, int r0, int rlim, int k0, int kend, int tid,
                                         uint4 (&reg)[2]) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int c = tid + 256 * q;
        if constexpr (KC) {
            const int r = c >> 2, kc = (c & 3) * 8;
            reg[q] = (r < rlim && k0 + kc < kend)
                         ? *reinterpret_cast<const uint4*>(p + (int64_t)(r0 + r) * ld + k0 + kc)
                         : make_uint4(0u, 0u, 0u, 0u);
        } else {
            const int k = c >> 4, rc = (c & 15) * 8;
            reg[q] = (k0 + k < kend && rc < rlim) ? *reinterpret_cast<const uint4*>(p + (int64_t)(k0 + k) * ld + r0 + rc)
                                                  : make_uint4(0u, 0u, 0u, 0u);
        }
    }
}

template <bool KC>
__device__ __forceinline__ void bwm_store(uint16_t* s, int tid, const uint4 (&reg)[2]) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
        const int c = tid + 256 * q;
        if constexpr (KC) {
            const int r = c >> 2, kc = (c & 3) * 8;
            *reinterpret_cast<uint4*>(s + r * BWM_LDK + kc) = reg[q];
        } else {
            const int k = c >> 4, rc = (c & 15) * 8;
            *reinterpret_cast<uint4*>(s + k * BWM_LDM + rc) = reg[q];
        }
    }
}

// fragment of rows base..base+15 (lane l: row base + l % 16, K 8 (l / 16)..+7)
template <bool KC>
__device__ __forceinline__ bf16x8_t bwm_frag(const uint16_t* s, int base, int lane) {
    const int g16 = lane >> 4, i16 = lane & 15;
    if constexpr (KC) {
        return *reinterpret_cast<const bf16x8_t*>(&s[(base + i16) * BWM_LDK + 8 * g16]);
    } else {
        // each 16-lane group reads K rows 8 g16 + (i16 >> 2) (+4) at columns
        // base + 4 (i16 & 3)..+3; the transposing read returns row base + i16
        const int k = 8 * g16 + (i16 >> 2), col = base + 4 * (i16 & 3);
        const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MOE_LDS bf16x4_t*)(&s[k * BWM_LDM + col]));
        const bf16x4_t hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MOE_LDS bf16x4_t*)(&s[(k + 4) * BWM_LDM + col]));
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    }
}

template <int MODE, int EPI>
__global__ __launch_bounds__(256, MODE == BW_TN ? 4 : 1) void bw_mfma_kernel(BwGemmArgs g) {
    // TN: both operands [k][row] (smaller tiles), no item list in LDS, and
    // four workgroups per CU (at most 128 registers a lane): its few K-steps
    // per tile wait on global loads, which more resident workgroups cover
    constexpr int TILE = MODE == BW_TN ? BWM_BK * BWM_LDM : BWM_TILE;
    __shared__ __attribute__((aligned(16))) uint16_t As[2][TILE];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[2][TILE];
    __shared__ int mt_pre[1025];
    __shared__ int scan_tmp[32];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wid = tid / kWave;
    const int wm = wid >> 1, wn = wid & 1;
    const int ntn = (g.N + BWM_BN - 1) / BWM_BN;
    const uint16_t* A = static_cast<const uint16_t*>(g.A);
    const uint16_t* B = static_cast<const uint16_t*>(g.B);

    int e, m0, mrows, n0, kb, kend;
    if constexpr (MODE == BW_TN) {
        // the dispatcher deals workgroups to the XCDs in turn (block b runs on
        // XCD b % 8).  The longer output dimension is cut into 8 ranges and
        // XCD x runs range x of every expert, expert by expert: its L2 holds
        // 1/8 of the larger operand's rows and all of the smaller one's, and
        // every XCD gets the same share of every expert.
        const int mtn = (g.M + BWM_BM - 1) / BWM_BM;
        const int xcd = blockIdx.x % kXcds;
        const int64_t i = blockIdx.x / kXcds;
        const bool split_m = mtn >= ntn;
        const int cut = split_m ? mtn : ntn, other = split_m ? ntn : mtn;
        const int lo = xcd * cut / kXcds, span = (xcd + 1) * cut / kXcds - lo;
        const int64_t per_e = (int64_t)span * other;
        if (i >= (int64_t)g.E * per_e) return;
        e = (int)(i / per_e);
        const int rest = (int)(i - (int64_t)e * per_e);
        const int mt = split_m ? lo + rest / ntn : rest / span;
        const int nt = split_m ? rest % ntn : lo + rest % span;
        m0 = mt * BWM_BM;
        n0 = nt * BWM_BN;
        mrows = min(BWM_BM, g.M - m0);
        kb = g.offsets[e];
        kend = g.offsets[e + 1];
    } else {
        const int total_mt = build_mtile_prefix(g.offsets, g.E, BWM_BM, mt_pre, scan_tmp);
        if ((int64_t)blockIdx.x >= (int64_t)total_mt * ntn) return;
        const WorkItem wi = decode_item(mt_pre, g.E, ntn, blockIdx.x);
        e = wi.e;
        m0 = g.offsets[e] + wi.mt * BWM_BM;
        mrows = min(BWM_BM, g.offsets[e + 1] - m0);
        n0 = wi.nt * BWM_BN;
        kb = 0;
        kend = g.K;
    }
    const int nrows = min(BWM_BN, g.N - n0);
    const uint16_t* Bb = B + ((MODE == BW_TN) ? 0 : (int64_t)e * g.b_estride);

    f32x4_t acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    // A: rows of the segment (K-contiguous) or, for TN, rows k of the segment
    // holding M-contiguous values; B likewise
    constexpr bool AKC = MODE != BW_TN, BKC = MODE == BW_NT;
    uint4 ra[2], rb[2];
    auto load = [&](int k0) {
        if constexpr (AKC) bwm_load<true>(A, g.lda, m0, mrows, k0, kend, tid, ra);
        else bwm_load<false>(A, g.lda, m0, mrows, k0, kend, tid, ra);
        if constexpr (BKC) bwm_load<true>(Bb, g.ldb, n0, nrows, k0, kend, tid, rb);
        else bwm_load<false>(Bb, g.ldb, n0, nrows, k0, kend, tid, rb);
    };
    // two LDS buffers: step s multiplies buffer s & 1 while the tile of step
    // s + 1 (loaded into registers during step s - 1) is stored into the
    // other one and the tile of step s + 2 is loaded; one barrier per step
    if (kb < kend) {
        load(kb);
        bwm_store<AKC>(As[0], tid, ra);
        bwm_store<BKC>(Bs[0], tid, rb);
        if (kb + BWM_BK < kend) load(kb + BWM_BK);
        __syncthreads();
    }
    int buf = 0;
    for (int k0 = kb; k0 < kend; k0 += BWM_BK) {
        bf16x8_t af[4], bfr[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            af[i] = bwm_frag<AKC>(As[buf], wm * 64 + i * 16, lane);
            bfr[i] = bwm_frag<BKC>(Bs[buf], wn * 64 + i * 16, lane);
        }
        if (k0 + BWM_BK < kend) {
            // the other buffer was last read in step s - 1, before the barrier
            bwm_store<AKC>(As[buf ^ 1], tid, ra);
            bwm_store<BKC>(Bs[buf ^ 1], tid, rb);
            if (k0 + 2 * BWM_BK < kend) load(k0 + 2 * BWM_BK);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af[i], acc[i][j], 0, 0, 0);
        __syncthreads();
        buf ^= 1;
    }

    // lane l of block [i][j]: row 16 i + l % 16, columns 16 j + 4 (l / 16)..+3
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = wm * 64 + i * 16 + (lane & 15);
        if (m >= mrows) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + wn * 64 + j * 16 + 4 * (lane >> 4);
            if (n >= g.N) continue;
            f32x4_t v = acc[i][j];
            if constexpr (EPI == BWE_WGRAD) {
                *reinterpret_cast<f32x4_t*>(static_cast<float*>(g.C) + (int64_t)e * g.M * g.N +
                                            (int64_t)(m0 + m) * g.N + n) = v;
            } else {
                const int64_t ci = (int64_t)(m0 + m) * g.N + n;
                if constexpr (EPI == BWE_HGRAD) {
                    const f32x4_t bb = *reinterpret_cast<const f32x4_t*>(g.bias + (int64_t)e * g.N + n);
                    v += bb;
                    // the erf of the forward's GELU (Abramowitz & Stegun 7.1.26),
                    // so h is rounded from the same function the forward stores
                    uint16_t hb[4], gb[4];
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float hv, ga;
                        gelu_and_grad_as(v[q], hv, ga);
                        hb[q] = f32_to_bf16_bits(hv);
                        gb[q] = f32_to_bf16_bits(ga);
                    }
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.C) + ci) =
                        make_uint2(hb[0] | ((uint32_t)hb[1] << 16), hb[2] | ((uint32_t)hb[3] << 16));
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.C2) + ci) =
                        make_uint2(gb[0] | ((uint32_t)gb[1] << 16), gb[2] | ((uint32_t)gb[3] << 16));
                } else if constexpr (EPI == BWE_DA) {
                    // GELU'(a) in bf16, as the recompute stored it
                    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(g.C2) + ci);
                    const f32x4_t gr = {__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                                        __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
                    v *= gr;
                    const uint16_t d0 = f32_to_bf16_bits(v[0]), d1 = f32_to_bf16_bits(v[1]);
                    const uint16_t d2 = f32_to_bf16_bits(v[2]), d3 = f32_to_bf16_bits(v[3]);
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.C) + ci) =
                        make_uint2(d0 | ((uint32_t)d1 << 16), d2 | ((uint32_t)d3 << 16));
                } else {
                    *reinterpret_cast<f32x4_t*>(static_cast<float*>(g.C) + ci) = v;
                }
            }
        }
    }
}

// combine backward: per token, for each kept slot, dw = dy[t] . out[r] and
// g[r] = w dy[t]; dropped slots get dw = 0.  A workgroup takes one token;
// its four waves take the slots (G = 4 / min(k, 4) waves per slot for k < 4,
// their partial dot products added in wave order), each lane four columns
// at a time.
template <typename TG>
__device__ __forceinline__ void st4(TG* p, int64_t i, float4 v);
template <>
__device__ __forceinline__ void st4<float>(float* p, int64_t i, float4 v) {
    *reinterpret_cast<float4*>(p + i) = v;
}
template <>
__device__ __forceinline__ void st4<uint16_t>(uint16_t* p, int64_t i, float4 v) {
    *reinterpret_cast<uint2*>(p + i) = make_uint2(f32_to_bf16_bits(v.x) | ((uint32_t)f32_to_bf16_bits(v.y) << 16),
                                                  f32_to_bf16_bits(v.z) | ((uint32_t)f32_to_bf16_bits(v.w) << 16));
}

template <typename TG>
__global__ __launch_bounds__(256) void combine_backward_kernel(int64_t T, int d, int k, const float* __restrict__ dy,
                                                               const float* __restrict__ out,
                                                               const int32_t* __restrict__ slot,
                                                               const float* __restrict__ w, TG* __restrict__ g,
                                                               float* __restrict__ dw) {
    __shared__ float part[256 / kWave];
    const int64_t t = blockIdx.x;
    const int lane = threadIdx.x & (kWave - 1), wid = threadIdx.x / kWave;
    const int G = k == 1 ? 4 : k == 2 ? 2 : 1;   // waves per slot
    const int NG = 4 / G;                         // slots in flight
    const int sg = wid / G, sub = wid % G;
    for (int j0 = 0; j0 < k; j0 += NG) {          // the same trip count in every wave
        const int j = j0 + sg;
        const int r = j < k ? slot[t * k + j] : -1;
        float s = 0.0f;
        if (r >= 0) {
            const float wt = w[t * k + j];
            for (int c = 4 * (sub * kWave + lane); c < d; c += 4 * kWave * G) {
                const float4 v = *reinterpret_cast<const float4*>(dy + t * d + c);
                const float4 o = *reinterpret_cast<const float4*>(out + (int64_t)r * d + c);
                s = fmaf(v.x, o.x, s);
                s = fmaf(v.y, o.y, s);
                s = fmaf(v.z, o.z, s);
                s = fmaf(v.w, o.w, s);
                st4<TG>(g, (int64_t)r * d + c, make_float4(wt * v.x, wt * v.y, wt * v.z, wt * v.w));
            }
        }
        s = wave_sum(s);
        if (G > 1) {
            if (lane == 0) part[wid] = s;
            __syncthreads();
            if (sub == 0 && lane == 0 && j < k) {
                float tot = part[sg * G];
                for (int q = 1; q < G; ++q) tot += part[sg * G + q];
                dw[t * k + j] = r >= 0 ? tot : 0.0f;
            }
            __syncthreads();
        } else if (lane == 0 && j < k) {
            dw[t * k + j] = r >= 0 ? s : 0.0f;
        }
    }
}

// column sums over row segments: out[e][c] = sum_{r in segment e} src[r][c]
// (fp32, rows in order); one thread per (expert, column) -- fp32 layers
template <typename TS>
__global__ __launch_bounds__(256) void segment_colsum_kernel(const TS* __restrict__ src, const int32_t* offsets,
                                                             int E, int64_t rows, int N, float* __restrict__ out) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)E * N) return;
    const int e = (int)(i / N), c = (int)(i - (int64_t)e * N);
    const int r0 = offsets ? offsets[e] : 0, r1 = offsets ? offsets[e + 1] : (int)rows;
    float s = 0.0f;
    for (int r = r0; r < r1; ++r) s += ld_elem<TS>(src, (int64_t)r * N + c);
    out[i] = s;
}

// column sums over the row segments of a bf16 [rows][N] matrix (N a
// multiple of 8): a workgroup takes one expert and 512 columns; its 256
// threads are 4 row groups x 64 column lanes of 8 columns (16-byte loads),
// the row groups walk rows g, g+4, ... and are added in a fixed order
// (bitwise repeatable)
__global__ __launch_bounds__(256) void segment_colsum_bf16_kernel(const uint16_t* __restrict__ src,
                                                                  const int32_t* __restrict__ offsets, int N,
                                                                  float* __restrict__ out) {
    __shared__ float part[4][512];
    const int e = blockIdx.y;
    const int grp = threadIdx.x >> 6, cl = threadIdx.x & 63;
    const int c0 = blockIdx.x * 512 + cl * 8;
    const int r0 = offsets[e], r1 = offsets[e + 1];
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (c0 < N) {
        // eight of the group's rows in flight, then added in row order (one
        // load at a time waited on each: 94 us for the 64-expert layer's db1)
        constexpr int U = 8;
        for (int rb = r0 + grp; rb < r1; rb += 4 * U) {
            uint4 v[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int r = rb + 4 * u;
                v[u] = r < r1 ? *reinterpret_cast<const uint4*>(src + (int64_t)r * N + c0) : make_uint4(0u, 0u, 0u, 0u);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (rb + 4 * u >= r1) break;
                const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    s[2 * i] += __uint_as_float(w[i] << 16);
                    s[2 * i + 1] += __uint_as_float(w[i] & 0xffff0000u);
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) part[grp][cl * 8 + i] = s[i];
    __syncthreads();
    for (int c = threadIdx.x; c < 512; c += 256) {
        const int col = blockIdx.x * 512 + c;
        if (col < N) out[(int64_t)e * N + col] = ((part[0][c] + part[1][c]) + part[2][c]) + part[3][c];
    }
}

// ---- gate backward ----------------------------------------------------------
// dl[t, e] is nonzero only at the k selected experts of token t, so both gate
// GEMMs are sparse: dWg[:, e] = sum over the tokens that selected e of
// dl[t, e] x[t], and dxg[t] = sum_j dl[t, j] Wg[:, idx_j].  The routed
// (token, expert) pairs are grouped by expert with the dispatch's histogram and
// scatter at unlimited capacity (every pair kept, token order within an
// expert); dWg is then a gather-and-sum over each expert's rows and dxg is
// folded into the assembly of dx.  Work and traffic scale with T k instead of
// T E.

// gate softmax backward over the selected logits, one wave per token (lane
// j takes slots j, j + 64, ...):
// dl_j = w_j (dw_j - sum_i w_i dw_i) / tau (no other logit has a gradient);
// dlsel[t, j] = dl_j and dlr[gslot[t, j]] = dl_j, beside the token's row in the
// expert-grouped order
__global__ __launch_bounds__(256) void gate_backward_kernel(int64_t T, int E, int k, float tau,
                                                            const int32_t* __restrict__ idx,
                                                            const float* __restrict__ w,
                                                            const float* __restrict__ dw,
                                                            const int32_t* __restrict__ gslot,
                                                            float* __restrict__ dlsel, float* __restrict__ dlr) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t t = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave;
    if (t >= T) return;   // wave-uniform
    float s = 0.0f;
    for (int j = lane; j < k; j += kWave) s = fmaf(w[t * k + j], dw[t * k + j], s);
    s = wave_sum(s);
    for (int j = lane; j < k; j += kWave) {
        const int64_t q = t * k + j;
        const int e = idx[q];
        const float v = (unsigned)e < (unsigned)E ? w[q] * (dw[q] - s) / tau : 0.0f;
        dlsel[q] = v;
        const int r = gslot[q];
        if (r >= 0) dlr[r] = v;
    }
}

// wgt[e][c] = Wg[c][e], 64 x 64 tiles through LDS
__global__ __launch_bounds__(256) void transpose_gate_kernel(const float* __restrict__ Wg, int d, int E,
                                                             float* __restrict__ wgt) {
    __shared__ float tile[64][65];
    const int c0 = blockIdx.x * 64, e0 = blockIdx.y * 64;
    const int lo = threadIdx.x & 63, hi = threadIdx.x >> 6;
    for (int cl = hi; cl < 64; cl += 4) {
        const int c = c0 + cl, e = e0 + lo;
        tile[cl][lo] = (c < d && e < E) ? Wg[(int64_t)c * E + e] : 0.0f;
    }
    __syncthreads();
    for (int el = hi; el < 64; el += 4) {
        const int e = e0 + el, c = c0 + lo;
        if (c < d && e < E) wgt[(int64_t)e * d + c] = tile[lo][el];
    }
}

template <typename TX>
__device__ __forceinline__ void load8(const TX* p, float (&v)[8]);
template <>
__device__ __forceinline__ void load8<uint16_t>(const uint16_t* p, float (&v)[8]) {
    const uint4 q = *reinterpret_cast<const uint4*>(p);
    const uint32_t u[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(u[i] << 16);
        v[2 * i + 1] = __uint_as_float(u[i] & 0xffff0000u);
    }
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float (&v)[8]) {
    const float4 a = *reinterpret_cast<const float4*>(p), b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

constexpr int GW_COLS = 512;   // columns of dWg per workgroup: 64 lanes x 8

// partial sums of dWg over row chunks: item i (the mt-th chunk of
// GATE_WGRAD_ROWS rows of expert e) writes part[i][c] = sum over its rows r of
// dlr[r] x[gperm[r]][c], and its first column block also partb[i] = sum of
// dlr[r].  Four row groups (rows r0 + g, r0 + g + 4, ...) are added in a fixed
// order: bitwise repeatable.
template <typename TX>
__global__ __launch_bounds__(256) void gate_wgrad_kernel(const TX* __restrict__ x, const int32_t* __restrict__ gperm,
                                                         const float* __restrict__ dlr,
                                                         const int32_t* __restrict__ goff, int64_t T, int E,
                                                         int d, float* __restrict__ part,
                                                         float* __restrict__ partb) {
    __shared__ int mt_pre[1025];
    __shared__ int scan_tmp[32];
    __shared__ float red[4][GW_COLS];
    const int total = build_mtile_prefix(goff, E, GATE_WGRAD_ROWS, mt_pre, scan_tmp);
    const int item = blockIdx.x;
    if (item >= total) return;
    const WorkItem wi = decode_item(mt_pre, E, 1, item);
    const int r0 = goff[wi.e] + wi.mt * GATE_WGRAD_ROWS;
    const int r1 = min(r0 + GATE_WGRAD_ROWS, goff[wi.e + 1]);
    const int grp = threadIdx.x >> 6, cl = threadIdx.x & 63;
    const int c0 = blockIdx.y * GW_COLS + cl * 8;
    float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    if (c0 < d) {
        // four rows in flight per lane: their token indices, then their x rows
        for (int rb = r0 + grp; rb < r1; rb += 16) {
            int64_t t[4];
            float v[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int r = rb + 4 * u;
                t[u] = r < r1 ? gperm[r] : 0;
                v[u] = r < r1 ? dlr[r] : 0.0f;
            }
            float xv[4][8];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                // (a token index out of range only follows repeated experts in topk_idx)
                if (rb + 4 * u < r1 && (uint64_t)t[u] < (uint64_t)T) load8<TX>(x + t[u] * d + c0, xv[u]);
                else {
#pragma unroll
                    for (int i = 0; i < 8; ++i) xv[u][i] = 0.0f;
                }
            }
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
                for (int i = 0; i < 8; ++i) s[i] = fmaf(v[u], xv[u][i], s[i]);
        }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) red[grp][cl * 8 + i] = s[i];
    __syncthreads();
    for (int c = threadIdx.x; c < GW_COLS; c += 256) {
        const int col = blockIdx.y * GW_COLS + c;
        if (col < d) part[(int64_t)item * d + col] = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
    }
    if (blockIdx.y == 0 && grp == 0) {
        float b = 0.0f;
        for (int r = r0 + cl; r < r1; r += 64) b += dlr[r];
        b = wave_sum(b);
        if (cl == 0) partb[item] = b;
    }
}

// dWg[c][e] = sum of expert e's partial sums in chunk order, dbg[e] likewise.
// A workgroup takes 64 columns x 16 experts and transposes through LDS, so
// that the partial reads (along c) and the dWg writes (along e) are both
// contiguous.  Experts without rows get zeros.
constexpr int GR_E = 16;
__global__ __launch_bounds__(256) void gate_wgrad_reduce_kernel(const float* __restrict__ part,
                                                                const float* __restrict__ partb,
                                                                const int32_t* __restrict__ goff, int E, int d,
                                                                float* __restrict__ dWg, float* __restrict__ dbg) {
    __shared__ int mt_pre[1025];
    __shared__ int scan_tmp[32];
    __shared__ float tile[64][GR_E + 1];
    build_mtile_prefix(goff, E, GATE_WGRAD_ROWS, mt_pre, scan_tmp);
    const int c0 = blockIdx.x * 64, e0 = blockIdx.y * GR_E;
    {
        const int lo = threadIdx.x & 63, hi = threadIdx.x >> 6;
        for (int el = hi; el < GR_E; el += 4) {
            const int e = e0 + el;
            float s = 0.0f;
            if (e < E && c0 + lo < d)
                for (int it = mt_pre[e]; it < mt_pre[e + 1]; ++it) s += part[(int64_t)it * d + c0 + lo];
            tile[lo][el] = s;
        }
    }
    __syncthreads();
    {
        const int lo = threadIdx.x % GR_E, hi = threadIdx.x / GR_E;
        for (int cl = hi; cl < 64; cl += 256 / GR_E) {
            const int c = c0 + cl, e = e0 + lo;
            if (c < d && e < E) dWg[(int64_t)c * E + e] = tile[cl][lo];
        }
    }
    if (blockIdx.x == 0 && threadIdx.x < GR_E) {
        const int e = e0 + threadIdx.x;
        if (e < E) {
            float s = 0.0f;
            for (int it = mt_pre[e]; it < mt_pre[e + 1]; ++it) s += partb[it];
            dbg[e] = s;
        }
    }
}

// dx[t] = sum_j dx_perm[slot[t,j]] over the kept slots, plus the gate's part
// sum_j dl[t,j] Wg[:, idx_j] over the selected experts (both in j order);
// one workgroup per token, 4 columns per thread
__global__ __launch_bounds__(256) void dispatch_backward_kernel(int64_t T, int d, int k, int E,
                                                                const float* __restrict__ dxp,
                                                                const int32_t* __restrict__ slot,
                                                                const int32_t* __restrict__ idx,
                                                                const float* __restrict__ dlsel,
                                                                const float* __restrict__ wgt,
                                                                float* __restrict__ dx) {
    const int64_t t = blockIdx.x;
    for (int c = threadIdx.x * 4; c < d; c += blockDim.x * 4) {
        float4 s = make_float4(0.f, 0.f, 0.f, 0.f), gs = make_float4(0.f, 0.f, 0.f, 0.f);
        for (int j = 0; j < k; ++j) {
            const int r = slot[t * k + j];
            if (r >= 0) {
                const float4 v = *reinterpret_cast<const float4*>(dxp + (int64_t)r * d + c);
                s.x += v.x; s.y += v.y; s.z += v.z; s.w += v.w;
            }
        }
        for (int j = 0; j < k; ++j) {
            const int e = idx[t * k + j];
            if ((unsigned)e < (unsigned)E) {
                const float l = dlsel[t * k + j];
                const float4 wv = *reinterpret_cast<const float4*>(wgt + (int64_t)e * d + c);
                gs.x = fmaf(l, wv.x, gs.x); gs.y = fmaf(l, wv.y, gs.y);
                gs.z = fmaf(l, wv.z, gs.z); gs.w = fmaf(l, wv.w, gs.w);
            }
        }
        *reinterpret_cast<float4*>(dx + t * d + c) = make_float4(s.x + gs.x, s.y + gs.y, s.z + gs.z, s.w + gs.w);
    }
}

int64_t gate_wgrad_items(int64_t T, int k, int E) {
    // each expert's last chunk may be partial: at most one extra item per expert
    return (T * k + GATE_WGRAD_ROWS - 1) / GATE_WGRAD_ROWS + E;
}

// ---- host ------------------------------------------------------------------

template <int MODE, int EPI, typename TA, typename TB, typename TH>
static hipError_t bw_launch(const BwGemmArgs& g, int64_t max_rows, hipStream_t st) {
    const int ntn = (g.N + BW_BN - 1) / BW_BN;
    int64_t blocks;
    if (MODE == BW_TN) blocks = (int64_t)g.E * ((g.M + BW_BM - 1) / BW_BM) * ntn;
    else blocks = ((max_rows + BW_BM - 1) / BW_BM + g.E) * ntn;   // bound; extra blocks exit
    if (blocks < 1) return hipSuccess;
    hipLaunchKernelGGL((bw_gemm_kernel<MODE, EPI, TA, TB, TH>), dim3((unsigned)blocks), dim3(BW_THREADS), 0, st, g);
    return hipGetLastError();
}

#define BW_CHECK(x)                                  \
    do {                                             \
        hipError_t e_ = (x);                         \
        if (e_ != hipSuccess) return e_;             \
    } while (0)

template <int MODE, int EPI>
static hipError_t bwm_launch(const BwGemmArgs& g, int64_t max_rows, hipStream_t st) {
    const int ntn = (g.N + BWM_BN - 1) / BWM_BN, mtn = (g.M + BWM_BM - 1) / BWM_BM;
    // TN: 8 XCD slots of the largest per-XCD share (see bw_mfma_kernel); extra blocks exit
    const int cut = mtn >= ntn ? mtn : ntn, other = mtn >= ntn ? ntn : mtn;
    const int64_t blocks = (MODE == BW_TN) ? (int64_t)kXcds * g.E * ((cut + kXcds - 1) / kXcds) * other
                                           : ((max_rows + BWM_BM - 1) / BWM_BM + g.E) * ntn;   // bound
    if (blocks < 1) return hipSuccess;
    hipLaunchKernelGGL((bw_mfma_kernel<MODE, EPI>), dim3((unsigned)blocks), dim3(256), 0, st, g);
    return hipGetLastError();
}

// steps 2-5: the expert FFN backward.  bf16 layers: matrix cores, with the
// expert-output gradient g and da held in bf16 as GEMM operands; fp32
// layers: vector ALUs in fp32 throughout.
template <typename ET>
static hipError_t ffn_backward_t(const BackwardArgs& b, hipStream_t st) {
    const int d = b.d, E = b.E, F = b.dff;
    constexpr bool kMfma = sizeof(ET) == 2;
    BwGemmArgs g{};
    // 2. recompute h and GELU'(a): x_perm W1[e] + b1[e]
    g.A = b.x_perm; g.lda = d;
    g.B = b.W1; g.ldb = F; g.b_estride = (int64_t)d * F;
    g.offsets = b.offsets; g.E = E; g.K = d; g.N = F;
    g.bias = b.b1; g.C = b.h; g.C2 = b.hgrad;
    if constexpr (kMfma) {
        // large problems: the forward's pipelined GEMM with a GELU + GELU' epilogue
        GemmArgs p{};
        p.A = b.x_perm; p.B = b.W1; p.bias = b.b1; p.offsets = b.offsets;
        p.E = E; p.K = d; p.N = F; p.out = b.h; p.out2 = static_cast<uint16_t*>(b.hgrad);
        hipError_t err = hipSuccess;
        if (launch_ffn_gemm_bf16_pipe(p, EPI_HGRAD, false, b.max_rows, st, &err)) BW_CHECK(err);
        else BW_CHECK((bwm_launch<BW_NN, BWE_HGRAD>(g, b.max_rows, st)));
    } else {
        BW_CHECK((bw_launch<BW_NN, BWE_HGRAD, ET, ET, ET>(g, b.max_rows, st)));
    }
    // 3. dh = g W2[e]^T (W2[e] stored [F][d] = [N][K]), da = dh * GELU'(a)
    g = BwGemmArgs{};
    g.A = b.g; g.lda = d;
    g.B = b.W2; g.ldb = d; g.b_estride = (int64_t)F * d;
    g.offsets = b.offsets; g.E = E; g.K = d; g.N = F;
    g.C = b.da; g.C2 = b.hgrad;
    if constexpr (kMfma) {
        // large problems: the pipelined GEMM, W2[e] read K-contiguous, GELU' product epilogue
        GemmArgs p{};
        p.A = b.g; p.B = b.W2; p.bias = nullptr; p.offsets = b.offsets;
        p.E = E; p.K = d; p.N = F; p.out = b.da; p.out2 = static_cast<uint16_t*>(b.hgrad);
        hipError_t err = hipSuccess;
        if (launch_ffn_gemm_bf16_pipe(p, EPI_DA, true, b.max_rows, st, &err)) BW_CHECK(err);
        else BW_CHECK((bwm_launch<BW_NT, BWE_DA>(g, b.max_rows, st)));
    } else {
        BW_CHECK((bw_launch<BW_NT, BWE_DA, float, ET, float>(g, b.max_rows, st)));
    }
    // 4. dx_perm = da W1[e]^T (W1[e] stored [d][F] = [N][K])
    g = BwGemmArgs{};
    g.A = b.da; g.lda = F;
    g.B = b.W1; g.ldb = F; g.b_estride = (int64_t)d * F;
    g.offsets = b.offsets; g.E = E; g.K = F; g.N = d;
    g.C = b.dx_perm;
    if constexpr (kMfma) {
        // large problems: the pipelined GEMM with W1[e] read K-contiguous
        GemmArgs p{};
        p.A = b.da; p.B = b.W1; p.bias = nullptr; p.offsets = b.offsets;
        p.E = E; p.K = F; p.N = d; p.out = b.dx_perm;
        hipError_t err = hipSuccess;
        if (launch_ffn_gemm_bf16_pipe(p, EPI_STORE_F32, true, b.max_rows, st, &err)) BW_CHECK(err);
        else BW_CHECK((bwm_launch<BW_NT, BWE_STORE>(g, b.max_rows, st)));
    } else {
        BW_CHECK((bw_launch<BW_NT, BWE_STORE, float, ET, float>(g, b.max_rows, st)));
    }
    // 5. dW2[e] = h^T g  ([F][d]), dW1[e] = x_perm^T da  ([d][F])
    g = BwGemmArgs{};
    g.A = b.h; g.lda = F;
    g.B = b.g; g.ldb = d;
    g.offsets = b.offsets; g.E = E; g.M = F; g.N = d;
    g.C = b.dW2;
    // long row segments (>= 1024 rows per expert on average, bounded by
    // max_rows): the pipelined GEMM in its weight-gradient form.  Short ones
    // keep the 128 x 128 kernel: there every 256 x 256 item is a few K-steps
    // followed by 256 KiB of fp32 stores, and the next item's waits (vmcnt
    // counts stores and loads in one order) hold its loads behind them.
    auto wgrad = [&](const BwGemmArgs& w) -> hipError_t {
        if (b.max_rows >= 1024LL * E) {
            GemmArgs p{};
            p.A = w.A; p.B = w.B; p.bias = nullptr; p.offsets = w.offsets;
            p.E = w.E; p.M = w.M; p.N = w.N; p.out = w.C;
            hipError_t err = hipSuccess;
            // a segment holds each token at most once: at most min(T, max_rows) rows
            const int64_t seg_rows = b.T < b.max_rows ? b.T : b.max_rows;
            if (launch_ffn_gemm_bf16_pipe(p, EPI_WGRAD, false, seg_rows, st, &err)) return err;
        }
        return bwm_launch<BW_TN, BWE_WGRAD>(w, b.max_rows, st);
    };
    if constexpr (kMfma) BW_CHECK(wgrad(g));
    else BW_CHECK((bw_launch<BW_TN, BWE_WGRAD, ET, float, float>(g, b.max_rows, st)));
    g = BwGemmArgs{};
    g.A = b.x_perm; g.lda = d;
    g.B = b.da; g.ldb = F;
    g.offsets = b.offsets; g.E = E; g.M = d; g.N = F;
    g.C = b.dW1;
    if constexpr (kMfma) BW_CHECK(wgrad(g));
    else BW_CHECK((bw_launch<BW_TN, BWE_WGRAD, ET, float, float>(g, b.max_rows, st)));
    return hipSuccess;
}

template <typename ET>
static hipError_t layer_backward_t(const BackwardArgs& b, hipStream_t st) {
    const int64_t T = b.T;
    const int d = b.d, E = b.E, k = b.k, F = b.dff;
    // g and da: bf16 operands of the matrix cores in bf16 layers, fp32 otherwise
    using TG = typename std::conditional<sizeof(ET) == 2, uint16_t, float>::type;
    // 1. combine backward
    hipLaunchKernelGGL(combine_backward_kernel<TG>, dim3((unsigned)T), dim3(256), 0, st, T, d, k, b.dy, b.out_perm,
                       b.slot, b.topk_w, reinterpret_cast<TG*>(b.g), b.dw);
    BW_CHECK(hipGetLastError());
    // 2-5. expert FFN
    BW_CHECK(ffn_backward_t<ET>(b, st));
    // 6. bias gradients
    if constexpr (sizeof(ET) == 2) {
        hipLaunchKernelGGL(segment_colsum_bf16_kernel, dim3((unsigned)((d + 511) / 512), (unsigned)E), dim3(256), 0,
                           st, reinterpret_cast<const uint16_t*>(b.g), b.offsets, d, b.db2);
        BW_CHECK(hipGetLastError());
        hipLaunchKernelGGL(segment_colsum_bf16_kernel, dim3((unsigned)((F + 511) / 512), (unsigned)E), dim3(256), 0,
                           st, reinterpret_cast<const uint16_t*>(b.da), b.offsets, F, b.db1);
        BW_CHECK(hipGetLastError());
    } else {
        const int64_t n2 = (int64_t)E * d, n1 = (int64_t)E * F;
        hipLaunchKernelGGL(segment_colsum_kernel<TG>, dim3((unsigned)((n2 + 255) / 256)), dim3(256), 0, st,
                           reinterpret_cast<const TG*>(b.g), b.offsets, E, (int64_t)0, d, b.db2);
        BW_CHECK(hipGetLastError());
        hipLaunchKernelGGL(segment_colsum_kernel<TG>, dim3((unsigned)((n1 + 255) / 256)), dim3(256), 0, st,
                           reinterpret_cast<const TG*>(b.da), b.offsets, E, (int64_t)0, F, b.db1);
        BW_CHECK(hipGetLastError());
    }
    // 7. gate: group the routed (token, expert) pairs by expert, then
    // dl, dWg and dbg over each expert's rows
    DispatchArgs ga{};
    ga.T = T; ga.E = E; ga.k = k;
    ga.cap = T;   // a token holds an expert at most once: nothing is dropped
    ga.max_rows = T * k;
    ga.BT = b.BT; ga.nblk = b.nblk;
    ga.idx = b.topk_idx; ga.blkhist = b.ghist; ga.offsets = b.goff; ga.perm = b.gperm; ga.slot = b.gslot;
    BW_CHECK(launch_hist(ga, st));
    BW_CHECK(launch_scatter(ga, st));
    hipLaunchKernelGGL(gate_backward_kernel, dim3((unsigned)((T + 3) / 4)), dim3(256), 0, st, T, E, k, b.tau,
                       b.topk_idx, b.topk_w, b.dw, b.gslot, b.dlsel, b.dlr);
    BW_CHECK(hipGetLastError());
    hipLaunchKernelGGL(transpose_gate_kernel, dim3((unsigned)((d + 63) / 64), (unsigned)((E + 63) / 64)), dim3(256), 0,
                       st, b.Wg, d, E, b.wgt);
    BW_CHECK(hipGetLastError());
    const dim3 wgrid((unsigned)gate_wgrad_items(T, k, E), (unsigned)((d + GW_COLS - 1) / GW_COLS));
    hipLaunchKernelGGL(gate_wgrad_kernel<ET>, wgrid, dim3(256), 0, st, static_cast<const ET*>(b.x), b.gperm, b.dlr,
                       b.goff, T, E, d, b.gpart, b.gpartb);
    BW_CHECK(hipGetLastError());
    const dim3 rgrid((unsigned)((d + 63) / 64), (unsigned)((E + GR_E - 1) / GR_E));
    hipLaunchKernelGGL(gate_wgrad_reduce_kernel, rgrid, dim3(256), 0, st, b.gpart, b.gpartb, b.goff, E, d, b.dWg,
                       b.dbg);
    BW_CHECK(hipGetLastError());
    // 8. dx, with the gate's part dl Wg^T
    hipLaunchKernelGGL(dispatch_backward_kernel, dim3((unsigned)T), dim3(256), 0, st, T, d, k, E, b.dx_perm, b.slot,
                       b.topk_idx, b.dlsel, b.wgt, b.dx);
    return hipGetLastError();
}

hipError_t launch_layer_backward(const BackwardArgs& b, int dtype, hipStream_t st) {
    return dtype == MOE_BF16 ? layer_backward_t<uint16_t>(b, st) : layer_backward_t<float>(b, st);
}

}  // namespace moe
