// ffn_bf16.hip -- grouped expert GEMMs in bf16 on CDNA4 matrix cores.
//
// [PithTrain] section 4.1 / [PyTorchMoE] section 3.2: each expert is
// Linear(d, d_ff) -> GELU -> Linear(d_ff, d) with biases.  [EP] section 5.5:
// expert math in bf16 while routing stays fp32.
//
//   GEMM1: h[r]   = GELU(x_perm[r] W1[e] + b1[e])   (EPI_GELU_H)
//   GEMM2: out[r] = h[r] W2[e] + b2[e]               (EPI_STORE_F32)
// (the weighted sum back to token order is a separate pass, combine.hip:
// fp32 atomics into y cost more than twice the whole GEMM2 on MI355X.)
//
// Work list: persistent workgroups walk (expert, n-tile, m-tile) items, see
// ffn_sched.h.  Per item a BM x BN output tile accumulates over K in steps
// of 32 through an NSTAGE-deep ring of LDS buffers:
//   * operands go global -> LDS with buffer_load_dwordx4 ... lds (no VGPR
//     staging); each wave instruction fills 1 KiB of LDS, lane L the L-th
//     16 bytes.  The buffer descriptor's range ends at the expert's last row
//     (activations) or matrix end (weights), so rows past the segment and
//     the K tail read as zeros; the column tail is steered out of range.
//   * loads run NSTAGE-1 steps ahead; one s_waitcnt vmcnt + s_barrier per
//     step publishes the oldest stage and frees the one consumed before it;
//     the next item's first stages are issued before the current item's
//     epilogue, so its arithmetic and stores overlap those loads.
//   * GEMM1's epilogue is bias + GELU (Abramowitz & Stegun 7.1.26 erf, error
//     below 1.5e-7, well under the bf16 rounding of h) + bf16 rounding.
//   * v_mfma_f32_16x16x32_bf16 with the weight as the A operand and the
//     token rows as the B operand, so each lane's accumulator holds four
//     consecutive output columns of one row.  Activation rows are
//     K-contiguous (16-byte ds_read_b128); weights are N-contiguous and are
//     transposed on the way out of LDS by ds_read_b64_tr_b16.
//   * both LDS tiles are XOR-swizzled at 16-byte granularity so the reads of
//     a 16-lane group fall on distinct banks.
#include "ffn_sched.h"
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int BK = 32;      // K per pipeline stage
constexpr int NSTAGE = 4;   // LDS ring depth

template <int BM_, int BN_, int WM_, int WN_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
    static constexpr int NT = 64 * WM * WN;          // threads
    static constexpr int NW = WM * WN;               // waves
    static constexpr int TM = BM / WM, TN = BN / WN; // wave tile
    static constexpr int MB = TM / 16, NB = TN / 16; // 16x16 blocks per wave
    static constexpr int A_BYTES = BM * BK * 2;      // one stage of activations
    static constexpr int B_BYTES = BK * BN * 2;      // one stage of weights
    static constexpr int A_DMA = A_BYTES / 1024 / NW;  // 1 KiB wave loads per wave per stage
    static constexpr int B_DMA = B_BYTES / 1024 / NW;
    static constexpr int B_ROW_CHUNKS = BN / 8;      // 16-byte chunks per weight row
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be a multiple of 16");
    static_assert(A_DMA * 1024 * NW == A_BYTES && B_DMA * 1024 * NW == B_BYTES, "stage must split into wave loads");
    static_assert(B_ROW_CHUNKS >= 16 && 64 % B_ROW_CHUNKS == 0, "weight row layout (BN 128 or 256)");
};

// Two tile shapes: the large one when the work list still gives every CU a
// few items, the small one otherwise (launch_ffn_gemm_bf16).
#ifndef MOE_TILE_LARGE
#define MOE_TILE_LARGE 256, 256, 2, 4
#endif
#ifndef MOE_TILE_SMALL
#define MOE_TILE_SMALL 128, 128, 2, 2
#endif
using TileLarge = TileCfg<MOE_TILE_LARGE>;
using TileSmall = TileCfg<MOE_TILE_SMALL>;

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// 16 bytes per lane, global -> LDS at (lds + 16 * lane).  Issued as inline asm
// so that the compiler's wait insertion neither tracks it nor adds vmcnt
// waits for it: every wait on these loads is explicit (wait_vm_barrier).
__device__ __forceinline__ void dma16(const i32x4_t& rsrc, const void* lds, int voffset) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds));
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(m0), "v"(voffset), "s"(rsrc) : "memory");
}

// Buffer descriptor: 48-bit base, stride 0, range in bytes, gfx9 data format.
__device__ __forceinline__ i32x4_t make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    i32x4_t r;
    r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)a);
    r[1] = __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xffff);
    r[2] = __builtin_amdgcn_readfirstlane((int)bytes);
    r[3] = 0x00020000;
    return r;
}

constexpr int kOutOfRange = 0x7ff00000;   // byte offset past any range: reads zeros

__device__ __forceinline__ bf16x4_t lds_read_tr(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MOE_LDS bf16x4_t*)(p));
}

__device__ __forceinline__ bf16x8_t cat8(bf16x4_t lo, bf16x4_t hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Activation tile, one stage: row r (BM rows) holds K 0..31 as four 16-byte
// chunks; logical chunk c sits at physical slot c ^ ((r >> 1) & 3), which
// spreads the 16 rows read by one 16-lane group over all banks.
__device__ __forceinline__ int a_swz(int r) { return (r >> 1) & 3; }
__device__ __forceinline__ int a_slot(int r, int c) { return r * 4 + (c ^ a_swz(r)); }
// Weight tile, one stage: row k (32 rows) holds BN columns as BN/8 chunks;
// logical chunk c sits at physical chunk c ^ (2 (k & 3)) ^ (8 ((k >> 3) & 1)):
// a 16-lane transposed read covers rows k..k+3 and two adjacent chunks, and
// the two 16-lane groups served together read rows 8 apart.
__device__ __forceinline__ int b_swz(int k) { return (2 * (k & 3)) ^ (8 * ((k >> 3) & 1)); }
__device__ __forceinline__ int b_chunk(int k, int c) { return c ^ b_swz(k); }

// wait until at most n vector-memory operations of this wave are in flight,
// then meet the other waves of the workgroup
// (one asm statement with a memory clobber, so no LDS access moves across it)
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

}  // namespace

template <class C, int EPI>
__global__ __launch_bounds__(C::NT) void ffn_gemm_bf16_kernel(GemmArgs g) {
    __shared__ __attribute__((aligned(1024))) uint16_t sa[NSTAGE][C::BM * BK];
    __shared__ __attribute__((aligned(1024))) uint16_t sb[NSTAGE][BK * C::BN];
    __shared__ int mt_pre[1025];
    __shared__ int scan_tmp[32];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid / kWave;
    const int wm = wid / C::WN, wn = wid % C::WN;
    const int g16 = lane >> 4, i16 = lane & 15;
    const int E = g.E, K = g.K, N = g.N;
    const int ntn = (N + C::BN - 1) / C::BN;
    const int nk = (K + BK - 1) / BK;

    const int total_mt = build_mtile_prefix(g.offsets, E, C::BM, mt_pre, scan_tmp);
    const ItemRange range = xcd_item_range((int64_t)total_mt * ntn);
    if (range.first >= range.end) return;

    const uint16_t* __restrict__ A = static_cast<const uint16_t*>(g.A);
    const uint16_t* __restrict__ Bw = static_cast<const uint16_t*>(g.B);

    // DMA geometry of this lane (independent of the item):
    //   A: wave instruction covers 16 rows; lane -> (row, physical slot)
    const int a_rl = lane >> 2, a_ps = lane & 3;
    //   B: wave instruction covers 512 / BN rows; lane -> (row, physical chunk)
    constexpr int B_ROWS_PER_DMA = 512 / C::BN;
    const int b_rl = lane / C::B_ROW_CHUNKS, b_pc = lane % C::B_ROW_CHUNKS;

    struct Item {
        int e, m0, mrows, n0;
        i32x4_t rsA, rsB;
        int a_off[C::A_DMA], b_off[C::B_DMA];
    };
    auto setup = [&](int64_t item, Item& it) {
        const WorkItem wi = decode_item(mt_pre, E, ntn, item);
        it.e = wi.e;
        it.m0 = g.offsets[wi.e] + wi.mt * C::BM;
        it.mrows = min(C::BM, g.offsets[wi.e + 1] - it.m0);
        it.n0 = wi.nt * C::BN;
        // activations: the range ends at the expert's last row, so rows past the
        // segment read zeros; a K tail reads the next row's head, which meets the
        // zero weight rows past K (finite inputs)
        it.rsA = make_rsrc(A + (int64_t)it.m0 * K, (uint32_t)it.mrows * (uint32_t)K * 2u);
        it.rsB = make_rsrc(Bw + (int64_t)wi.e * K * N, (uint32_t)K * (uint32_t)N * 2u);
#pragma unroll
        for (int j = 0; j < C::A_DMA; ++j) {
            const int r = (wid * C::A_DMA + j) * 16 + a_rl;   // tile row
            const int c = a_ps ^ a_swz(r);                      // logical chunk
            it.a_off[j] = (r * K + c * 8) * 2;
        }
#pragma unroll
        for (int j = 0; j < C::B_DMA; ++j) {
            const int k = (wid * C::B_DMA + j) * B_ROWS_PER_DMA + b_rl;   // tile k-row
            const int c = b_pc ^ b_swz(k);                                  // logical chunk
            const int col = it.n0 + c * 8;
            it.b_off[j] = (col < N) ? (k * N + col) * 2 : kOutOfRange;
        }
    };
    auto issue = [&](const Item& it, int kt) {
        const int buf = kt % NSTAGE;
        const int k0 = kt * BK;
#pragma unroll
        for (int j = 0; j < C::A_DMA; ++j)
            dma16(it.rsA, &sa[buf][(wid * C::A_DMA + j) * 512], it.a_off[j] + k0 * 2);
#pragma unroll
        for (int j = 0; j < C::B_DMA; ++j) {
            const int off = (it.b_off[j] == kOutOfRange) ? kOutOfRange : it.b_off[j] + k0 * N * 2;
            dma16(it.rsB, &sb[buf][(wid * C::B_DMA + j) * 512], off);
        }
    };
    auto prologue = [&](const Item& it) {
        for (int s = 0; s < NSTAGE - 1 && s < nk; ++s) issue(it, s);
    };

    constexpr int PER = C::A_DMA + C::B_DMA;   // vector-memory ops per stage per lane
    int64_t item = range.first;
    Item cur;
    setup(item, cur);
    prologue(cur);
    while (true) {
        f32x4_t acc[C::MB][C::NB];
#pragma unroll
        for (int i = 0; i < C::MB; ++i)
#pragma unroll
            for (int j = 0; j < C::NB; ++j) acc[i][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

        for (int kt = 0; kt < nk; ++kt) {
            const int ahead = min(NSTAGE - 2, nk - 1 - kt);   // stages issued after kt
            if (kt == 0 || ahead == 0) wait_vm_barrier<0>();   // first step: epilogue stores may be in flight
            else if (ahead >= 2) wait_vm_barrier<2 * PER>();
            else wait_vm_barrier<PER>();
            if (kt + NSTAGE - 1 < nk) issue(cur, kt + NSTAGE - 1);
            const uint16_t* as = sa[kt % NSTAGE];
            const uint16_t* bs = sb[kt % NSTAGE];
            bf16x8_t wf[C::NB];
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) {
                // rows 8 g16 + (i16 >> 2) (+4), columns 4 (i16 & 3) of the 16-column block
                const int col = wn * C::TN + nb * 16 + 4 * (i16 & 3);
                const int k = 8 * g16 + (i16 >> 2);
                const int c = col >> 3, half = (col & 7);
                const bf16x4_t lo = lds_read_tr(&bs[k * C::BN + b_chunk(k, c) * 8 + half]);
                const bf16x4_t hi = lds_read_tr(&bs[(k + 4) * C::BN + b_chunk(k + 4, c) * 8 + half]);
                wf[nb] = cat8(lo, hi);
            }
#pragma unroll
            for (int mb = 0; mb < C::MB; ++mb) {
                const int r = wm * C::TM + mb * 16 + i16;
                const bf16x8_t tf = *reinterpret_cast<const bf16x8_t*>(&as[a_slot(r, g16) * 8]);
#pragma unroll
                for (int nb = 0; nb < C::NB; ++nb)
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(wf[nb], tf, acc[mb][nb], 0, 0, 0);
            }
        }
        // every wave is done reading the ring and every load has landed
        wait_vm_barrier<0>();

        // epilogue inputs first (global loads), then the next item's first
        // stages, then the epilogue arithmetic and stores overlap those loads
        float4 bias4[C::NB];
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
            const int n = min(cur.n0 + wn * C::TN + nb * 16 + 4 * g16, N - 4);
            bias4[nb] = *reinterpret_cast<const float4*>(g.bias + (int64_t)cur.e * N + n);
        }
        const Item done = cur;
        const int64_t next = item + range.step;
        const bool more = next < range.end;
        if (more) {
            // keep the epilogue's loads out of the DMA's vmcnt window
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            setup(next, cur);
            prologue(cur);
        }

#pragma unroll
        for (int mb = 0; mb < C::MB; ++mb) {
            const int ml = wm * C::TM + mb * 16 + i16;
            if (ml >= done.mrows) continue;
            const int64_t row = done.m0 + ml;
#pragma unroll
            for (int nb = 0; nb < C::NB; ++nb) {
                const int n = done.n0 + wn * C::TN + nb * 16 + 4 * g16;
                if (n >= N) continue;
                const float4 bv = bias4[nb];
                const float v0 = acc[mb][nb][0] + bv.x, v1 = acc[mb][nb][1] + bv.y;
                const float v2 = acc[mb][nb][2] + bv.z, v3 = acc[mb][nb][3] + bv.w;
                if constexpr (EPI == EPI_GELU_H) {
                    uint2 pk;
                    pk.x = (uint32_t)f32_to_bf16_bits(gelu_as(v0)) |
                           ((uint32_t)f32_to_bf16_bits(gelu_as(v1)) << 16);
                    pk.y = (uint32_t)f32_to_bf16_bits(gelu_as(v2)) |
                           ((uint32_t)f32_to_bf16_bits(gelu_as(v3)) << 16);
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.out) + row * N + n) = pk;
                } else {
                    *reinterpret_cast<float4*>(static_cast<float*>(g.out) + row * N + n) =
                        make_float4(v0, v1, v2, v3);
                }
            }
        }
        if (!more) break;
        item = next;
    }
}

template <class C, int EPI>
static int persistent_blocks() {
    static int blocks = 0;
    if (blocks == 0) {
        int per_cu = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, ffn_gemm_bf16_kernel<C, EPI>, C::NT, 0) !=
                hipSuccess ||
            per_cu < 1)
            per_cu = 1;
        blocks = per_cu * device_cu_count();
        if (blocks < kXcds) blocks = kXcds;
    }
    return blocks;
}

template <class C, int EPI>
static hipError_t launch_cfg(const GemmArgs& g, hipStream_t st) {
    hipLaunchKernelGGL((ffn_gemm_bf16_kernel<C, EPI>), dim3(persistent_blocks<C, EPI>()), dim3(C::NT), 0, st, g);
    return hipGetLastError();
}

// Upper bound of the work items for tile C: every expert may add one
// partial m-tile on top of max_rows / BM full ones.
template <class C>
static int64_t item_bound(const GemmArgs& g, int64_t max_rows) {
    return ((max_rows + C::BM - 1) / C::BM + g.E) * ((g.N + C::BN - 1) / C::BN);
}

template <int EPI>
static hipError_t launch_epi(const GemmArgs& g, int64_t max_rows, hipStream_t st) {
    // large tiles need about 3 items per CU to keep the tail short
    const int64_t large = item_bound<TileLarge>(g, max_rows);
    if (large >= 3 * (int64_t)persistent_blocks<TileLarge, EPI>()) return launch_cfg<TileLarge, EPI>(g, st);
    return launch_cfg<TileSmall, EPI>(g, st);
}

hipError_t launch_ffn_gemm_bf16(const GemmArgs& g, int epi, int64_t max_rows, hipStream_t st) {
    return epi == EPI_GELU_H ? launch_epi<EPI_GELU_H>(g, max_rows, st) : launch_epi<EPI_STORE_F32>(g, max_rows, st);
}

}  // namespace moe
