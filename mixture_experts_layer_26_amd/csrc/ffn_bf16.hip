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
// of 32 through a ring of NSTAGE LDS slots:
//   * operands go global -> LDS with buffer_load_dwordx4 ... lds (no VGPR
//     staging); each wave instruction fills 1 KiB of LDS, lane L the L-th
//     16 bytes.  The buffer descriptor's range ends at the expert's last row
//     (activations) or matrix end (weights), so rows past the segment and
//     the K tail read as zeros; the column tail is steered out of range.
//   * the weight is the MFMA A operand and the token rows the B operand, so
//     each lane's accumulator holds runs of four consecutive output columns
//     of one row.  Activation rows are K-contiguous (16-byte ds_read_b128);
//     weights are N-contiguous and are transposed on the way out of LDS by
//     ds_read_b64_tr_b16.  Both LDS tiles are XOR-swizzled at 16-byte
//     granularity so the lanes served together fall on distinct banks.
//   * GEMM1's epilogue is bias + GELU (Abramowitz & Stegun 7.1.26 erf, error
//     below 1.5e-7, well under the bf16 rounding of h) + bf16 rounding.
//   * h, which only GEMM1 writes and GEMM2 reads, is stored in 16-row x
//     32-column tiles (1 KiB each) over expert segments padded to 16 rows:
//     one K-step of 16 rows is then one contiguous 1 KiB global -> LDS load
//     instead of sixteen 64-byte row pieces (GEMM2 ~7% faster).  Padded row
//     p, column c sits at element ((p / 16) KT + c / 32) 512 + (p % 16) 32 +
//     c % 32 with KT = ceil(d_ff / 32); GEMM1 writes zeros into columns
//     [d_ff, 32 KT), so GEMM2's K tail multiplies zeros.  Padding rows are
//     never written; each feeds only its own output row, which is not stored.
//   * in the fused forward GEMM1's activations come in the same tile layout
//     (x_perm over ceil(d / 32) column tiles, written by the dispatch's tiled
//     copy): a global -> LDS load of 64-byte row pieces moves half the bytes
//     per cycle of one of contiguous KiBs.  moe_grouped_ffn's GEMM1 reads the
//     caller's row-major x_perm.
//
// Two schedules:
//   * large problems: 256 x 256 tiles on eight waves (two per SIMD), each a
//     128 x 64 quarter-column of the tile on v_mfma_f32_32x32x16_bf16 (one
//     wave issues these back to back; the 16x16x32 form with accumulators in
//     VGPRs cannot).  Every wave reads the next step's fragments into a second
//     register set while its MFMAs run, and the ring continues across items.
//   * small problems: 128 x 128 tiles, four waves on v_mfma_f32_16x16x32_bf16,
//     one barrier per step (read, then multiply).
// Expert tails (an expert's last 1..128 rows) run on 128 x 256 tiles of the
// same eight waves in ffn_gemm_bf16_split_kernel: on workgroups of their own
// beside the full items, or after each workgroup's full items where a die has
// few of them (see there).
#include "ffn_sched.h"
#include "lds_dma.h"
#include "moe_kernels.h"

namespace moe {

namespace {

constexpr int BK = 32;      // K per pipeline stage
constexpr int NSTAGE = 4;   // LDS ring depth

// MF: 16 (v_mfma_f32_16x16x32_bf16) or 32 (v_mfma_f32_32x32x16_bf16)
template <int BM_, int BN_, int WM_, int WN_, int MF_>
struct TileCfg {
    static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, MF = MF_;
    static constexpr int NT = 64 * WM * WN;          // threads
    static constexpr int NW = WM * WN;               // waves
    static constexpr int TM = BM / WM, TN = BN / WN; // wave tile
    static constexpr int MB = TM / MF, NB = TN / MF; // MFMA blocks per wave
    static constexpr int A_BYTES = BM * BK * 2;      // one stage of activations
    static constexpr int B_BYTES = BK * BN * 2;      // one stage of weights
    static constexpr int A_DMA = A_BYTES / 1024 / NW;  // 1 KiB wave loads per wave per stage
    static constexpr int B_DMA = B_BYTES / 1024 / NW;
    static constexpr int B_ROW_CHUNKS = BN / 8;      // 16-byte chunks per weight row
    static_assert(MF == 16 || MF == 32, "MFMA shape");
    static_assert(TM % MF == 0 && TN % MF == 0, "wave tile must be a multiple of the MFMA block");
    static_assert(A_DMA * 1024 * NW == A_BYTES && B_DMA * 1024 * NW == B_BYTES, "stage must split into wave loads");
    static_assert(B_ROW_CHUNKS >= 16 && 64 % B_ROW_CHUNKS == 0, "weight row layout (BN 128 or 256)");
};

#ifndef MOE_TILE_SMALL
#define MOE_TILE_SMALL 128, 128, 2, 2, 16
#endif
#ifndef MOE_TILE_PIPE
#define MOE_TILE_PIPE 256, 256, 2, 4, 32
#endif
using TileSmall = TileCfg<MOE_TILE_SMALL>;
using TilePipe = TileCfg<MOE_TILE_PIPE>;
#ifndef MOE_PIPE_NS
#define MOE_PIPE_NS 4   // LDS ring slots of the pipelined kernel
#endif

typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ bf16x4_t lds_read_tr(const uint16_t* p) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((MOE_LDS bf16x4_t*)(p));
}

__device__ __forceinline__ bf16x8_t cat8(bf16x4_t lo, bf16x4_t hi) {
    return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Activation tile, one stage: row r (BM rows) holds K 0..31 as four 16-byte
// chunks; logical chunk c sits at physical slot c ^ a_swz<MF>(r), which puts
// the rows read together by one fragment read on distinct banks (both
// choices measured conflict-free with SQ_LDS_BANK_CONFLICT on MI355X).
template <int MF>
__device__ __forceinline__ int a_swz(int r) { return MF == 16 ? (r >> 1) & 3 : (r >> 2) & 3; }
template <int MF>
__device__ __forceinline__ int a_slot(int r, int c) { return r * 4 + (c ^ a_swz<MF>(r)); }

// Weight tile, one stage: row k (32 rows) holds BN columns as BN/8 chunks;
// logical chunk c sits at physical chunk c ^ b_swz<MF>(k).  A 16-lane
// transposed read covers rows k..k+3 and two adjacent chunks.
//   MF 16: the two 16-lane groups served together read rows 8 apart:
//          c ^ (2 (k & 3)) ^ (8 ((k >> 3) & 1)).
//   MF 32: they read the same rows and the next two chunks: c ^ (4 (k & 3)),
//          so the four rows of a 4-chunk window land on distinct banks.
// (both measured conflict-free with SQ_LDS_BANK_CONFLICT on MI355X)
template <int MF>
__device__ __forceinline__ int b_swz(int k) {
    return MF == 16 ? (2 * (k & 3)) ^ (8 * ((k >> 3) & 1)) : 4 * (k & 3);
}
template <int MF>
__device__ __forceinline__ int b_chunk(int k, int c) { return c ^ b_swz<MF>(k); }

// wait until at most n vector-memory operations of this wave are in flight,
// then meet the other waves of the workgroup
// (one asm statement with a memory clobber, so no LDS access moves across it)
template <int N>
__device__ __forceinline__ void wait_vm_barrier() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(N) : "memory");
}

template <int VM>
__device__ __forceinline__ void pipe_barrier() { dma_barrier<VM>(); }

// fp32 pair -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    typedef __bf16 b2 __attribute__((ext_vector_type(2)));
    const f2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, b2));
}

// element index of padded row p, column c in the h tile layout
__device__ __forceinline__ int64_t h_tile_index(int64_t p, int c, int KT) {
    return ((p >> 4) * KT + (c >> 5)) * 512 + (p & 15) * 32 + (c & 31);
}

// GEMM1 (GELU epilogue) writes h in the tile layout; GEMM2 reads it as A
template <int EPI>
constexpr bool kOutTiled = EPI == EPI_GELU_H;
template <int EPI>
constexpr bool kATiled = EPI == EPI_STORE_F32;

// element index of output row `row` (padded row `prow` in the tile layout)
template <int EPI>
__device__ __forceinline__ int64_t out_index(const GemmArgs& g, int64_t row, int64_t prow, int n) {
    if constexpr (kOutTiled<EPI>) return h_tile_index(prow, n, (g.N + 31) >> 5);
    else return row * g.N + n;
}

// bias + activation + store of four consecutive columns of one row
template <int EPI>
__device__ __forceinline__ void store4(const GemmArgs& g, int64_t row, int64_t prow, int n, f32x4_t v) {
    if constexpr (EPI == EPI_GELU_H) {
        uint2 pk;
        pk.x = pack_bf16x2(gelu_as(v[0]), gelu_as(v[1]));
        pk.y = pack_bf16x2(gelu_as(v[2]), gelu_as(v[3]));
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.out) + out_index<EPI>(g, row, prow, n)) = pk;
    } else {
        *reinterpret_cast<f32x4_t*>(static_cast<float*>(g.out) + out_index<EPI>(g, row, prow, n)) = v;
    }
}

// Per-lane global -> LDS load geometry and the work item it streams from.
template <class C>
struct Item {
    int e, m0, mrows, n0;
    int pm0;         // first padded row (h tile layout)
    int nk, nks;     // K-steps of the item, and rounded up to even
    int mc0, k0;     // transposed form: first column of A, first segment row
    i32x4_t rsA, rsB;
    int a_off[C::A_DMA], b_off[C::B_DMA];
};

// AT: A in the h tile layout; BKC: B stored [E, N, K] (K-contiguous rows of
// N, staged like the activations) instead of [E, K, N].
// TN (weight gradients): out[e] [M, N] = A[seg(e)]^T B[seg(e)], both operands
// [rows, M] / [rows, N] row-major over the expert's segment of rows, so K is
// the segment and varies per item; A is staged like the weights ([k][m]
// rows) and read with transposing reads.  Items are (expert, m-tile,
// n-tile) over every expert; an expert without rows has no K-steps and gets
// zeros.
template <class C, bool AT, bool BKC = false, bool TN = false>
struct Loader {
    const uint16_t* A;
    const uint16_t* Bw;
    const int* s_off;    // expert row offsets, copied to LDS
    const int* mt_pre;   // m-tile prefix, LDS
    const int* s_poff;   // padded expert row offsets (h tile layout), LDS
    int E, K, N, M, ntn, mtn, wid;
    int a_rl, a_ps, b_rl, b_pc;   // BKC: b_rl, b_pc as a_rl, a_ps
    int a_kt;            // A in the tile layout: 32-column tiles per 16-row block
    bool tail = false;   // items are the experts' tails (mt_pre counts them; see the split kernel)
    static constexpr int B_ROWS_PER_DMA = 512 / C::BN;

    __device__ __forceinline__ Loader(const GemmArgs& g, const int* off, const int* pre, const int* poff, int ntn_,
                                      int wid_, int lane)
        : A(static_cast<const uint16_t*>(g.A)), Bw(static_cast<const uint16_t*>(g.B)), s_off(off),
          mt_pre(pre), s_poff(poff), E(g.E), K(g.K), N(g.N), M(g.M), ntn(ntn_), wid(wid_) {
        a_kt = (g.K + 31) >> 5;
        mtn = (g.M + C::BM - 1) / C::BM;
        // A: a wave instruction covers 16 rows; lane -> (row, physical slot)
        // (TN: 512 / BM k-rows; lane -> (k-row, physical chunk))
        a_rl = TN ? lane / (C::BM / 8) : lane >> 2;
        a_ps = TN ? lane % (C::BM / 8) : lane & 3;
        // B: a wave instruction covers 512 / BN k-rows; lane -> (k-row, physical chunk)
        // (BKC: 16 rows of N, as A)
        b_rl = BKC ? lane >> 2 : lane / C::B_ROW_CHUNKS;
        b_pc = BKC ? lane & 3 : lane % C::B_ROW_CHUNKS;
    }

    // expert, first row, row count and first column of an item (LDS reads only)
    __device__ __forceinline__ void decode(int64_t item, Item<C>& it) const {
        if constexpr (TN) {
            const int per_e = mtn * ntn;
            const int e = __builtin_amdgcn_readfirstlane((int)(item / per_e));
            const int rest = __builtin_amdgcn_readfirstlane((int)(item - (int64_t)e * per_e));
            const int mt = rest / ntn;
            it.e = e;
            it.mc0 = mt * C::BM;
            it.m0 = __builtin_amdgcn_readfirstlane(e * M + it.mc0);   // output row of out [E M, N]
            it.mrows = __builtin_amdgcn_readfirstlane(min(C::BM, M - it.mc0));
            it.n0 = __builtin_amdgcn_readfirstlane((rest - mt * ntn) * C::BN);
            it.pm0 = 0;
            it.k0 = __builtin_amdgcn_readfirstlane(s_off[e]);
            it.nk = __builtin_amdgcn_readfirstlane((s_off[e + 1] - it.k0 + BK - 1) / BK);
            it.nks = it.nk + (it.nk & 1);
            return;
        }
        const WorkItem wi = decode_item(mt_pre, E, ntn, item);
        const int e = __builtin_amdgcn_readfirstlane(wi.e);
        // a tail item starts after the expert's whole 256-row blocks
        const int r0 = tail ? (s_off[e + 1] - s_off[e]) & ~255 : wi.mt * C::BM;
        const int m0 = __builtin_amdgcn_readfirstlane(s_off[e] + r0);
        it.e = e;
        it.m0 = m0;
        it.mrows = __builtin_amdgcn_readfirstlane(min(C::BM, s_off[e + 1] - m0));
        it.n0 = __builtin_amdgcn_readfirstlane(wi.nt * C::BN);
        it.pm0 = __builtin_amdgcn_readfirstlane(s_poff[e] + r0);
        it.nk = (K + BK - 1) / BK;
        it.nks = it.nk + (it.nk & 1);
    }

    __device__ __forceinline__ void setup(int64_t item, Item<C>& it) const {
        decode(item, it);
        // activations: the range ends at the expert's last row, so rows past the
        // segment read zeros; a K tail reads the next row's head, which meets the
        // zero weight rows past K (finite inputs)
        if constexpr (TN) {
            // both operands: the expert's rows; rows past the segment read zeros
            const uint32_t rows = (uint32_t)(s_off[it.e + 1] - it.k0);
            it.rsA = make_rsrc(A + (int64_t)it.k0 * M, rows * (uint32_t)M * 2u);
            it.rsB = make_rsrc(Bw + (int64_t)it.k0 * N, rows * (uint32_t)N * 2u);
#pragma unroll
            for (int j = 0; j < C::A_DMA; ++j) {
                const int k = (wid * C::A_DMA + j) * (512 / C::BM) + a_rl;   // tile k-row
                const int c = a_ps ^ b_swz<C::MF>(k);                          // logical chunk
                const int col = it.mc0 + c * 8;
                it.a_off[j] = (col < M) ? (k * M + col) * 2 : kOutOfRange;
            }
        } else if constexpr (AT) {
            // the item's 16-row blocks; rows past the segment inside its last
            // block are padding, later blocks read zeros
            it.rsA = make_rsrc(A + (int64_t)(it.pm0 >> 4) * a_kt * 512,
                               (uint32_t)((it.mrows + 15) >> 4) * (uint32_t)a_kt * 1024u);
        } else {
            it.rsA = make_rsrc(A + (int64_t)it.m0 * K, (uint32_t)it.mrows * (uint32_t)K * 2u);
        }
        if constexpr (!TN) it.rsB = make_rsrc(Bw + (int64_t)it.e * K * N, (uint32_t)K * (uint32_t)N * 2u);
#pragma unroll
        for (int j = 0; j < C::A_DMA; ++j) {
            if constexpr (TN) break;
            const int r = (wid * C::A_DMA + j) * 16 + a_rl;   // tile row
            const int c = a_ps ^ a_swz<C::MF>(r);               // logical chunk
            it.a_off[j] = AT ? ((r >> 4) * a_kt * 512 + (r & 15) * 32 + c * 8) * 2 : (r * K + c * 8) * 2;
        }
#pragma unroll
        for (int j = 0; j < C::B_DMA; ++j) {
            if constexpr (BKC) {
                const int r = (wid * C::B_DMA + j) * 16 + b_rl;   // tile row (column n0 + r of the output)
                const int c = b_pc ^ a_swz<C::MF>(r);              // logical chunk
                it.b_off[j] = (it.n0 + r < N) ? ((it.n0 + r) * K + c * 8) * 2 : kOutOfRange;
            } else {
                const int k = (wid * C::B_DMA + j) * B_ROWS_PER_DMA + b_rl;   // tile k-row
                const int c = b_pc ^ b_swz<C::MF>(k);                           // logical chunk
                const int col = it.n0 + c * 8;
                it.b_off[j] = (col < N) ? (k * N + col) * 2 : kOutOfRange;
            }
        }
    }

    // PER = A_DMA + B_DMA loads of K-step kt of `it` into one ring slot
    __device__ __forceinline__ void issue(const Item<C>& it, int kt, uint16_t* sa_buf, uint16_t* sb_buf) const {
        const int k0 = kt * BK;
        const int a_step = TN ? k0 * M * 2 : AT ? kt * 1024 : k0 * 2;   // bytes to K-step kt
#pragma unroll
        for (int j = 0; j < C::A_DMA; ++j) {
            const int off = (TN && it.a_off[j] == kOutOfRange) ? kOutOfRange : it.a_off[j] + a_step;
            dma16(it.rsA, sa_buf + (wid * C::A_DMA + j) * 512, off);
        }
#pragma unroll
        for (int j = 0; j < C::B_DMA; ++j) {
            const int step = BKC ? k0 * 2 : k0 * N * 2;
            const int off = (it.b_off[j] == kOutOfRange) ? kOutOfRange : it.b_off[j] + step;
            dma16(it.rsB, sb_buf + (wid * C::B_DMA + j) * 512, off);
        }
    }

    // the item's BN bias values (fp32, 1 KiB) into LDS: one wave instruction,
    // columns past N (and every column without a bias) read zeros
    __device__ __forceinline__ void issue_bias(const Item<C>& it, const float* bias, int lane, float* dst) const {
        static_assert(C::BN == 256, "one wave instruction per bias slice");
        const i32x4_t rs = bias ? make_rsrc(bias + (int64_t)it.e * N, (uint32_t)N * 4u) : make_rsrc(bias, 0u);
        dma16(rs, dst, (it.n0 + 4 * lane) * 4);
    }

    // the same number of loads, all out of range: they fill the slot with
    // zeros and touch no memory (keeps every wave's load count per step fixed)
    __device__ __forceinline__ void issue_zero(const Item<C>& it, uint16_t* sa_buf, uint16_t* sb_buf) const {
#pragma unroll
        for (int j = 0; j < C::A_DMA; ++j) dma16(it.rsA, sa_buf + (wid * C::A_DMA + j) * 512, kOutOfRange);
#pragma unroll
        for (int j = 0; j < C::B_DMA; ++j) dma16(it.rsB, sb_buf + (wid * C::B_DMA + j) * 512, kOutOfRange);
    }
};

// ---- 16x16x32 fragments (small tiles) ------------------------------------
// One K-step of a wave tile: NB weight fragments (transposed out of LDS) and
// MB activation fragments; lane l holds row / column l % 16, K 8 (l / 16)..+7.
template <class C>
struct Frags16 {
    bf16x8_t w[C::NB];
    bf16x8_t t[C::MB];
};

template <class C>
__device__ __forceinline__ void read_frags16(Frags16<C>& f, const uint16_t* as, const uint16_t* bs, int wm, int wn,
                                             int lane) {
    const int g16 = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb) {
        // rows 8 g16 + (i16 >> 2) (+4), columns 4 (i16 & 3) of the 16-column block
        const int col = wn * C::TN + nb * 16 + 4 * (i16 & 3);
        const int k = 8 * g16 + (i16 >> 2);
        const int c = col >> 3, half = (col & 7);
        const bf16x4_t lo = lds_read_tr(&bs[k * C::BN + b_chunk<16>(k, c) * 8 + half]);
        const bf16x4_t hi = lds_read_tr(&bs[(k + 4) * C::BN + b_chunk<16>(k + 4, c) * 8 + half]);
        f.w[nb] = cat8(lo, hi);
    }
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
        const int r = wm * C::TM + mb * 16 + i16;
        f.t[mb] = *reinterpret_cast<const bf16x8_t*>(&as[a_slot<16>(r, g16) * 8]);
    }
}

template <class C>
__device__ __forceinline__ void mfma_step16(f32x4_t (&acc)[C::MB][C::NB], const Frags16<C>& f) {
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.w[nb], f.t[mb], acc[mb][nb], 0, 0, 0);
}

// accumulator [mb][nb] of lane l: row 16 mb + l % 16, columns 16 nb + 4 (l / 16)..+3
template <class C, int EPI>
__device__ __forceinline__ void epilogue16(const GemmArgs& g, const Item<C>& it, const f32x4_t (&acc)[C::MB][C::NB],
                                           const f32x4_t (&bias4)[C::NB], int wm, int wn, int lane) {
    const int g16 = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
        const int ml = wm * C::TM + mb * 16 + i16;
        if (ml >= it.mrows) continue;
        const int64_t row = it.m0 + ml, prow = it.pm0 + ml;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
            const int n = it.n0 + wn * C::TN + nb * 16 + 4 * g16;
            if (n >= g.N) {
                // tile layout: zeros up to the 32-column boundary for the next GEMM's K tail
                if (kOutTiled<EPI> && n < ((g.N + 31) & ~31))
                    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(g.out) + out_index<EPI>(g, row, prow, n)) =
                        make_uint2(0u, 0u);
                continue;
            }
            store4<EPI>(g, row, prow, n, acc[mb][nb] + bias4[nb]);
        }
    }
}

// ---- 32x32x16 fragments (large tiles) ------------------------------------
// One K-step = two K-halves of 16.  Weight fragment [nb][h]: lane l holds
// column 32 nb + l % 32, K 16 h + 8 (l / 32)..+7; activation fragment
// [mb][h]: row 32 mb + l % 32, the same K.
template <class C>
struct Frags32 {
    bf16x8_t w[C::NB][2];
    bf16x8_t t[C::MB][2];
};

template <class C, bool BKC = false, bool TN = false>
__device__ __forceinline__ void read_frags32(Frags32<C>& f, const uint16_t* as, const uint16_t* bs, int wm, int wn,
                                             int lane) {
    const int g16 = lane >> 4, i16 = lane & 15;
#pragma unroll
    for (int nb = 0; nb < C::NB; ++nb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if constexpr (BKC) {
                // K-contiguous weight rows, laid out like the activations
                const int col = wn * C::TN + nb * 32 + (lane & 31);
                f.w[nb][h] = *reinterpret_cast<const bf16x8_t*>(&bs[a_slot<32>(col, 2 * h + (lane >> 5)) * 8]);
                continue;
            }
            // the 16-lane group g16 covers columns 16 (g16 & 1)..+15 of the block and
            // K rows 16 h + 8 (g16 >> 1)..+7: lane i16 points at row (i16 >> 2) (+4),
            // columns 4 (i16 & 3)..+3 of that 4 x 16 window
            const int col = wn * C::TN + nb * 32 + 16 * (g16 & 1) + 4 * (i16 & 3);
            const int k = 16 * h + 8 * (g16 >> 1) + (i16 >> 2);
            const int c = col >> 3, half = (col & 7);
            const bf16x4_t lo = lds_read_tr(&bs[k * C::BN + b_chunk<32>(k, c) * 8 + half]);
            const bf16x4_t hi = lds_read_tr(&bs[(k + 4) * C::BN + b_chunk<32>(k + 4, c) * 8 + half]);
            f.w[nb][h] = cat8(lo, hi);
        }
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if constexpr (TN) {
                // [k][m] rows, read like the weights
                const int col = wm * C::TM + mb * 32 + 16 * (g16 & 1) + 4 * (i16 & 3);
                const int k = 16 * h + 8 * (g16 >> 1) + (i16 >> 2);
                const int c = col >> 3, half = (col & 7);
                const bf16x4_t lo = lds_read_tr(&as[k * C::BM + b_chunk<32>(k, c) * 8 + half]);
                const bf16x4_t hi = lds_read_tr(&as[(k + 4) * C::BM + b_chunk<32>(k + 4, c) * 8 + half]);
                f.t[mb][h] = cat8(lo, hi);
                continue;
            }
            const int r = wm * C::TM + mb * 32 + (lane & 31);
            f.t[mb][h] = *reinterpret_cast<const bf16x8_t*>(&as[a_slot<32>(r, 2 * h + (lane >> 5)) * 8]);
        }
}

// scheduling groups: M MFMAs, each followed by its share of R LDS reads
// (spread evenly: MFMA i takes reads floor(i R / M) .. floor((i+1) R / M))
template <int M, int R, int I = 0>
__device__ __forceinline__ void interleave_mfma_reads() {
    if constexpr (I < M) {
        constexpr int n = (I + 1) * R / M - I * R / M;
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if constexpr (n > 0) __builtin_amdgcn_sched_group_barrier(0x100, n, 0);
        interleave_mfma_reads<M, R, I + 1>();
    }
}

// Accumulators in AGPRs: an empty asm statement with an AGPR operand marks
// the kernel as using AGPRs, so the compiler picks the MFMA forms that keep
// C/D there and leaves the VGPRs to fragments and addresses (measured ~4%
// faster than C/D in VGPRs on GEMM2's 256 x 256 tiles).
__device__ __forceinline__ void request_agpr_accumulators() { asm volatile("" ::"a"(0.f)); }

// the MFMAs of K-half h of one step
template <class C>
__device__ __forceinline__ void mfma_half32(f32x16_t (&acc)[C::MB][C::NB], const Frags32<C>& f, int h) {
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb)
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.w[nb][h], f.t[mb][h], acc[mb][nb], 0, 0, 0);
}

// accumulator [mb][nb] of lane l, elements 4q..4q+3: row 32 mb + l % 32,
// columns 32 nb + 8 q + 4 (l / 32)..+3; bias quads re-read from the item's
// LDS slice.  Rows outermost: the stores that fill one row's 128-byte lines
// issue back to back (row pieces spread over the epilogue measured up to
// twice the HBM write bytes).
// bf16 h: the two lanes of a row each hold 8-byte pieces; the upper half of
// the wave trades its quad q for the lower half's quad q + 1 (q even), so each
// lane stores 8 consecutive columns and a store covers 32 contiguous bytes
// of a row.
template <class C, int EPI>
__device__ __forceinline__ void epilogue32(const GemmArgs& g, const Item<C>& it, const f32x16_t (&acc)[C::MB][C::NB],
                                           const float* sbias, int wm, int wn, int lane) {
    const int h = lane >> 5;
#pragma unroll
    for (int mb = 0; mb < C::MB; ++mb) {
        // a block of 32 rows wholly past the item (padding of a short expert)
        // stores nothing: the fp32 store epilogue skips it (wave-uniform;
        // 2-3.5% off GEMM2; the same skip made GEMM1 ~1.5% slower)
        if (EPI == EPI_STORE_F32 && wm * C::TM + mb * 32 >= it.mrows) continue;
        const int ml = wm * C::TM + mb * 32 + (lane & 31);
        const bool row_ok = ml < it.mrows;
        const int64_t row = it.m0 + ml, prow = it.pm0 + ml;
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
            if constexpr (EPI == EPI_GELU_H || EPI == EPI_HGRAD || EPI == EPI_DA) {
#pragma unroll
                for (int q = 0; q < 4; q += 2) {
                    const int nl = wn * C::TN + nb * 32 + 8 * q + 4 * h;
                    const int n = it.n0 + wn * C::TN + nb * 32 + 8 * q + 8 * h;
                    uint32_t p[2][2];
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const f32x4_t b = *reinterpret_cast<const f32x4_t*>(&sbias[nl + 8 * j]);
                        const int e = 4 * (q + j);
                        if constexpr (EPI == EPI_DA) {
                            // dh * GELU'(a): the bf16 factor read from out2 (a global
                            // load here waits for the loads issued before it, in order)
                            const int ng = it.n0 + nl + 8 * j;
                            f32x4_t gv = {0.f, 0.f, 0.f, 0.f};
                            if (row_ok && ng < g.N) {
                                const uint2 u = *reinterpret_cast<const uint2*>(g.out2 + row * g.N + ng);
                                gv = f32x4_t{__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                                             __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u)};
                            }
                            p[j][0] = pack_bf16x2(acc[mb][nb][e] * gv[0], acc[mb][nb][e + 1] * gv[1]);
                            p[j][1] = pack_bf16x2(acc[mb][nb][e + 2] * gv[2], acc[mb][nb][e + 3] * gv[3]);
                        } else if constexpr (EPI == EPI_HGRAD) {
                            // GELU'(a) of this lane's quad straight to out2 in bf16; h as below
                            float hv[4], ga[4];
#pragma unroll
                            for (int i = 0; i < 4; ++i) gelu_and_grad_as(acc[mb][nb][e + i] + b[i], hv[i], ga[i]);
                            const int ng = it.n0 + nl + 8 * j;
                            if (row_ok && ng < g.N)
                                *reinterpret_cast<uint2*>(g.out2 + row * g.N + ng) =
                                    make_uint2(pack_bf16x2(ga[0], ga[1]), pack_bf16x2(ga[2], ga[3]));
                            p[j][0] = pack_bf16x2(hv[0], hv[1]);
                            p[j][1] = pack_bf16x2(hv[2], hv[3]);
                        } else {
                            p[j][0] = pack_bf16x2(gelu_as(acc[mb][nb][e] + b[0]), gelu_as(acc[mb][nb][e + 1] + b[1]));
                            p[j][1] =
                                pack_bf16x2(gelu_as(acc[mb][nb][e + 2] + b[2]), gelu_as(acc[mb][nb][e + 3] + b[3]));
                        }
                    }
                    const auto x = __builtin_amdgcn_permlane32_swap(p[0][0], p[1][0], false, false);
                    const auto y = __builtin_amdgcn_permlane32_swap(p[0][1], p[1][1], false, false);
                    if (!row_ok) continue;
                    uint4 o = {x[0], y[0], x[1], y[1]};
                    if (n >= g.N) {
                        // tile layout: zeros up to the 32-column boundary for the next GEMM's K tail
                        if (!kOutTiled<EPI> || n >= ((g.N + 31) & ~31)) continue;
                        o = make_uint4(0u, 0u, 0u, 0u);
                    }
                    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(g.out) + out_index<EPI>(g, row, prow, n)) = o;
                }
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int nl = wn * C::TN + nb * 32 + 8 * q + 4 * h;
                    const int n = it.n0 + nl;
                    if (!row_ok || n >= g.N) continue;
                    const f32x4_t b = EPI == EPI_WGRAD ? f32x4_t{0.f, 0.f, 0.f, 0.f}
                                                       : *reinterpret_cast<const f32x4_t*>(&sbias[nl]);
                    const f32x4_t v = {acc[mb][nb][4 * q], acc[mb][nb][4 * q + 1], acc[mb][nb][4 * q + 2],
                                       acc[mb][nb][4 * q + 3]};
                    store4<EPI>(g, row, prow, n, v + b);
                }
            }
        }
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// Small tiles: every wave reads and multiplies each step; one s_waitcnt
// vmcnt + s_barrier per step publishes the oldest stage and frees the one
// consumed before it.
template <class C, int EPI, bool AT = kATiled<EPI>>
__global__ __launch_bounds__(C::NT) void ffn_gemm_bf16_kernel(GemmArgs g) {
    static_assert(C::MF == 16, "small tiles use the 16x16x32 form");
    __shared__ __attribute__((aligned(1024))) uint16_t sa[NSTAGE][C::BM * BK];
    __shared__ __attribute__((aligned(1024))) uint16_t sb[NSTAGE][BK * C::BN];
    __shared__ int mt_pre[1025];
    __shared__ int s_off[1025];
    __shared__ int s_poff[1025];
    __shared__ int scan_tmp[32];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = tid / kWave;
    const int wm = wid / C::WN, wn = wid % C::WN;
    const int g16 = lane >> 4;
    const int E = g.E, K = g.K, N = g.N;
    const int ntn = (N + C::BN - 1) / C::BN;
    const int nk = (K + BK - 1) / BK;

    for (int i = tid; i <= E; i += C::NT) s_off[i] = g.offsets[i];
    const int total_mt = build_mtile_prefix(g.offsets, E, C::BM, mt_pre, scan_tmp);   // ends with a barrier
    build_padded_offsets(s_off, E, s_poff, scan_tmp);
    const ItemRange range = xcd_item_range((int64_t)total_mt * ntn);
    if (range.first >= range.end) return;
    const Loader<C, AT> ld(g, s_off, mt_pre, s_poff, ntn, wid, lane);

    constexpr int PER = C::A_DMA + C::B_DMA;   // vector-memory ops per stage per lane
    int64_t item = range.first;
    Item<C> cur;
    ld.setup(item, cur);
    for (int s = 0; s < NSTAGE - 1 && s < nk; ++s) ld.issue(cur, s, sa[s], sb[s]);
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
            if (kt + NSTAGE - 1 < nk) {
                const int b = (kt + NSTAGE - 1) % NSTAGE;
                ld.issue(cur, kt + NSTAGE - 1, sa[b], sb[b]);
            }
            Frags16<C> f;
            read_frags16<C>(f, sa[kt % NSTAGE], sb[kt % NSTAGE], wm, wn, lane);
            mfma_step16<C>(acc, f);
        }
        // every wave is done reading the ring and every load has landed
        wait_vm_barrier<0>();

        // epilogue inputs first (global loads), then the next item's first
        // stages, then the epilogue arithmetic and stores overlap those loads
        f32x4_t bias4[C::NB];
#pragma unroll
        for (int nb = 0; nb < C::NB; ++nb) {
            // clamped into the row for a column tail; those columns are never stored
            const int n = min(cur.n0 + wn * C::TN + nb * 16 + 4 * g16, N - 4);
            bias4[nb] = *reinterpret_cast<const f32x4_t*>(g.bias + (int64_t)cur.e * N + n);
        }
        const Item<C> done = cur;
        const int64_t next = item + range.step;
        const bool more = next < range.end;
        if (more) {
            // keep the epilogue's loads out of the DMA's vmcnt window
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            ld.setup(next, cur);
            for (int s = 0; s < NSTAGE - 1 && s < nk; ++s) ld.issue(cur, s, sa[s], sb[s]);
        }
        epilogue16<C, EPI>(g, done, acc, bias4, wm, wn, lane);
        if (!more) break;
        item = next;
    }
}

// ---------------------------------------------------------------------------
// Large tiles, pipelined: each wave reads the next step's fragments from LDS
// into a second register set while its MFMAs run on the current set.
//
// The ring of NS slots runs on across items (the next item's loads start
// while the current one finishes; past the last item out-of-range loads keep
// every wave's count per step at PER).  Items take an even number of steps
// (an odd K-step count gets one all-zero step), so the two fragment sets
// swap roles in a loop unrolled by two.  Global step j:
//   * opens with vmcnt((NS-2) PER) lgkmcnt(0) and the barrier: stage j+1
//     (read during step j) has landed for every wave; the fragments of step
//     j are in registers, so slot j % NS is free for every wave;
//   * issues stage j+NS into that slot, reads stage j+1 into the other set,
//     multiplies the current set.
// Wave 0 loads each item's bias slice into LDS with the item's first stage
// (one extra load only makes that wave's later vmcnt waits stricter), so no
// global load in the loop leaves the compiler to insert a wait for every
// load in flight.  The load cursor runs NS steps ahead; an item has two
// steps or more, so it is at most ceil(NS / 2) items ahead and NS bias slots
// (NS >= 3) never overwrite one still in use.

// The pipelined K-loop over one workgroup's items `range`; the ring, the
// bias slots and the loader's LDS tables come from the caller.
template <class C, int NS, int EPI, bool AT, bool BKC, bool TN>
__device__ __forceinline__ void pipe_run(const GemmArgs& g, const Loader<C, AT, BKC, TN>& ld, const ItemRange range,
                                         uint16_t (*sa)[C::BM * BK], uint16_t (*sb)[BK * C::BN],
                                         float (*s_bias)[C::BN], int wid, int lane) {
    const int wm = wid / C::WN, wn = wid % C::WN;
    constexpr int PER = C::A_DMA + C::B_DMA;
    constexpr bool kBias = EPI != EPI_WGRAD;

    // load cursor: item, K-step, ring slot and bias slot of the next stage;
    // it passes over items without K-steps (TN)
    Item<C> lit;
    int64_t l_item = range.first;
    int l_kt = 0, l_slot = 0, l_bslot = 0;
    ld.setup(l_item, lit);
    if constexpr (TN) {
        while (lit.nks == 0) {
            l_item += range.step;
            if (l_item >= range.end) break;
            ld.setup(l_item, lit);
        }
    }
    auto issue_next = [&]() {
        if (l_item < range.end) {
            if (kBias && l_kt == 0 && wid == 0) ld.issue_bias(lit, g.bias, lane, s_bias[l_bslot]);
            if (l_kt < lit.nk) ld.issue(lit, l_kt, sa[l_slot], sb[l_slot]);
            else ld.issue_zero(lit, sa[l_slot], sb[l_slot]);
        } else {
            ld.issue_zero(lit, sa[l_slot], sb[l_slot]);
        }
        if (++l_slot == NS) l_slot = 0;
        if (++l_kt == lit.nks) {
            l_kt = 0;
            if (++l_bslot == NS) l_bslot = 0;
            while (true) {
                l_item += range.step;
                if (l_item >= range.end) break;
                ld.setup(l_item, lit);
                if (!TN || lit.nks > 0) break;
            }
        }
    };
    for (int s = 0; s < NS; ++s) issue_next();
    pipe_barrier<(NS - 1) * PER>();   // stage 0 landed everywhere

    // GEMM2 keeps C/D in AGPRs (about 4% faster); GEMM1's GELU epilogue does
    // not fit the remaining 128 VGPRs and stays on the VGPR forms
    if constexpr (EPI == EPI_STORE_F32 || EPI == EPI_WGRAD) request_agpr_accumulators();
    Frags32<C> fa, fb;
    read_frags32<C, BKC, TN>(fa, sa[0], sb[0], wm, wn, lane);
    int c_slot = 0, c_bslot = 0;
    int64_t item = range.first;
    f32x16_t acc[C::MB][C::NB];
    auto step = [&](Frags32<C>& cur, Frags32<C>& nxt) {
        pipe_barrier<(NS - 2) * PER>();
        const int ns = c_slot + 1 == NS ? 0 : c_slot + 1;
        // the next step's fragment reads interleaved with the first K-half of
        // MFMAs (one MFMA, then two reads: a wave whose reads all came first
        // waited on the LDS queue before its first MFMA), then this step's
        // global -> LDS loads, then the second K-half: the loads of eight waves
        // take the TA ~500 cycles per step, and issued right after the barrier
        // they held back the MFMAs
        read_frags32<C, BKC, TN>(nxt, sa[ns], sb[ns], wm, wn, lane);
        mfma_half32<C>(acc, cur, 0);
        interleave_mfma_reads<C::MB * C::NB, (BKC ? 2 : 4) * C::NB + (TN ? 4 : 2) * C::MB>();
        __builtin_amdgcn_sched_barrier(0);
        issue_next();
        __builtin_amdgcn_sched_barrier(0);
        mfma_half32<C>(acc, cur, 1);
        c_slot = ns;
    };
    while (true) {
        Item<C> cur;
        ld.decode(item, cur);
#pragma unroll
        for (int i = 0; i < C::MB; ++i)
#pragma unroll
            for (int j = 0; j < C::NB; ++j)
#pragma unroll
                for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
        for (int kt = 0; kt < cur.nks; kt += 2) {
            step(fa, fb);
            step(fb, fa);
        }
        // the bias slice landed with the item's first stage, several barriers ago
        epilogue32<C, EPI>(g, cur, acc, s_bias[c_bslot], wm, wn, lane);
        if (!TN || cur.nks > 0)
            if (++c_bslot == NS) c_bslot = 0;
        item += range.step;
        if (item >= range.end) break;
    }
    // the trailing out-of-range loads still write the ring
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// WPE: waves per SIMD the kernel is built for (register budget 512 / WPE).
// AT: A in the h tile layout; BKC: B stored K-contiguous ([E, N, K]); TN:
// the weight-gradient form of Loader (K-steps per item vary; items without
// any K-step skip the ring and store zeros).
template <class C, int NS, int EMAX, int WPE, int EPI, bool AT, bool BKC, bool TN>
__global__ __launch_bounds__(C::NT, WPE) void ffn_gemm_bf16_pipe_kernel(GemmArgs g) {
    static_assert(C::MF == 32 && C::BN == 256, "256-column tiles on 32x32x16 MFMAs");
    static_assert(NS >= 3 && NS <= 4, "ring depth");
    __shared__ __attribute__((aligned(1024))) uint16_t sa[NS][C::BM * BK];
    __shared__ __attribute__((aligned(1024))) uint16_t sb[NS][BK * C::BN];
    __shared__ int mt_pre[EMAX + 1];
    __shared__ int s_off[EMAX + 1];
    __shared__ int s_poff[EMAX + 1];
    __shared__ int scan_tmp[32];
    __shared__ __attribute__((aligned(16))) float s_bias[NS][C::BN];   // by item number mod NS
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);   // wave-uniform: scalar branches
    const int E = g.E, N = g.N;
    const int ntn = (N + C::BN - 1) / C::BN;

    for (int i = tid; i <= E; i += C::NT) s_off[i] = g.offsets[i];
    int64_t total;
    if constexpr (TN) {
        __syncthreads();
        total = (int64_t)E * ((g.M + C::BM - 1) / C::BM) * ntn;
    } else {
        total = (int64_t)build_mtile_prefix(g.offsets, E, C::BM, mt_pre, scan_tmp) * ntn;   // ends with a barrier
        build_padded_offsets(s_off, E, s_poff, scan_tmp);
    }
    const ItemRange range = xcd_item_range(total);
    if (range.first >= range.end) return;
    const Loader<C, AT, BKC, TN> ld(g, s_off, mt_pre, s_poff, ntn, wid, lane);
    pipe_run<C, NS, EPI, AT, BKC, TN>(g, ld, range, sa, sb, s_bias, wid, lane);
}

#ifndef MOE_TAIL_WEIGHT
#define MOE_TAIL_WEIGHT 75   // a tail item's work in hundredths of a full item's
#endif
#ifndef MOE_TILE_TAIL
#define MOE_TILE_TAIL 128, 256, 2, 4, 32
#endif
using TileTail = TileCfg<MOE_TILE_TAIL>;

// The first grouped GEMM (and the backward's recompute and dh GEMMs of the
// same shape) with the experts' short tails on 128-row tiles.  An expert
// of r rows has floor(r / 256) whole 256-row blocks; a remainder above 128
// rows is one more 256-row item, one of 1..128 rows a tail item on a
// 128 x 256 tile (a 128-row tile costs about two thirds of a 256-row one on
// whole launches).  Tails and full items run at the same time in one
// launch, on workgroups of two roles: the last nB of each die's workgroups
// take the tail items, the others the full ones, nB in proportion to each
// role's work (tail items weighted 0.75: the best of 0.65, 0.75 and 0.9 on
// the 64-expert workloads).  Both lists run expert by expert, so an
// expert's tail and full items share its weight tiles in the die's L2, and
// no workgroup mixes stage sizes.  Every workgroup derives nB from the same
// offsets.  Each role runs the pipeline of ffn_gemm_bf16_pipe_kernel with
// its own tile shape over one LDS ring.
//
// Where a die has at most MOE_SEQ_MAX_FULL full items per workgroup (the
// second GEMM at the 64-expert workload: 2, at 128 experts: 4; the first at
// 16 experts: 2), one more full item for some workgroups decides the launch
// time and the roles cannot help (measured: sequenced wins up to 4, roles at
// 8).  Such a die runs sequenced instead: every workgroup takes both
// kinds, its full items first and its tails after them.  The die's full items
// go round robin over all its workgroups, exactly as in
// ffn_gemm_bf16_pipe_kernel, and its tails round robin from the first
// workgroup left with one full item fewer: the busiest workgroups then run
// e.g. two full items and one tail instead of three full items.  The tails run
// as a last round and re-read their weight tiles (their experts' full items
// ran earlier).  Every workgroup of a die takes the same decision; dies
// decide apart (their full-item counts may differ by one), and either way a
// die covers exactly its own share of both lists.
#ifndef MOE_SEQ_MAX_FULL
#define MOE_SEQ_MAX_FULL 4
#endif
template <int NS, int EPI, bool AT, bool BKC = false>
__global__ __launch_bounds__(TilePipe::NT, 2) void ffn_gemm_bf16_split_kernel(GemmArgs g) {
    using CA = TilePipe;
    using CB = TileTail;
    static_assert(CA::NT == CB::NT && CA::BN == 256 && CB::BN == 256 && CA::BM == 256 && CB::BM == 128,
                  "256- and 128-row tiles of 256 columns on the same waves");
    static_assert(NS >= 3 && NS <= 4, "ring depth");
    constexpr int RING_A = NS * (CA::BM * BK + BK * CA::BN), RING_B = NS * (CB::BM * BK + BK * CB::BN);
    __shared__ __attribute__((aligned(1024))) uint16_t ring[RING_A > RING_B ? RING_A : RING_B];
    __shared__ int mt_full[1025], mt_tail[1025], s_off[1025], s_poff[1025], scan_tmp[32];
    __shared__ __attribute__((aligned(16))) float s_bias[NS][CA::BN];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int E = g.E;
    const int ntn = (g.N + CA::BN - 1) / CA::BN;
    for (int i = tid; i <= E; i += CA::NT) s_off[i] = g.offsets[i];
    const int64_t full = (int64_t)build_mtile_prefix(g.offsets, E, 256, mt_full, scan_tmp, kTilesFull) * ntn;
    const int64_t tails = (int64_t)build_mtile_prefix(g.offsets, E, 256, mt_tail, scan_tmp, kTilesTail) * ntn;
    build_padded_offsets(s_off, E, s_poff, scan_tmp);

    const int P8 = gridDim.x / kXcds, xcd = blockIdx.x % kXcds, slot = blockIdx.x / kXcds;
    const int64_t f0 = full * xcd / kXcds, f1 = full * (xcd + 1) / kXcds;
    if (tails > 0 && f1 - f0 <= (int64_t)MOE_SEQ_MAX_FULL * P8) {
        const int64_t t0 = tails * xcd / kXcds, t1 = tails * (xcd + 1) / kXcds;
        const int remF = (int)((f1 - f0) % P8);
        const ItemRange rf{f0 + slot, f1, P8};
        const ItemRange rt{t0 + (slot - remF + P8) % P8, t1, P8};
        if (rf.first < rf.end) {
            const Loader<CA, AT, BKC, false> ld(g, s_off, mt_full, s_poff, ntn, wid, lane);
            pipe_run<CA, NS, EPI, AT, BKC, false>(g, ld, rf, reinterpret_cast<uint16_t(*)[CA::BM * BK]>(ring),
                                                    reinterpret_cast<uint16_t(*)[BK * CA::BN]>(ring + NS * CA::BM * BK),
                                                    s_bias, wid, lane);
        }
        if (rt.first < rt.end) {
            // every wave is done with the ring and the bias slots of the full items
            __syncthreads();
            Loader<CB, AT, BKC, false> ld(g, s_off, mt_tail, s_poff, ntn, wid, lane);
            ld.tail = true;
            pipe_run<CB, NS, EPI, AT, BKC, false>(g, ld, rt, reinterpret_cast<uint16_t(*)[CB::BM * BK]>(ring),
                                                    reinterpret_cast<uint16_t(*)[BK * CB::BN]>(ring + NS * CB::BM * BK),
                                                    s_bias, wid, lane);
        }
        return;
    }
    // roles: per die, P8 workgroups (the launch is a multiple of 8 of them)
    int nB = 0;
    if (tails > 0) {
        if (full == 0) {
            nB = P8;
        } else {
            const int64_t wa = 100 * full, wb = MOE_TAIL_WEIGHT * tails;
            nB = (int)(((int64_t)P8 * wb + (wa + wb) / 2) / (wa + wb));
            nB = nB < 1 ? 1 : nB > P8 - 1 ? P8 - 1 : nB;
        }
    }
    const bool is_tail = slot >= P8 - nB;
    const int64_t total = is_tail ? tails : full;
    ItemRange range;
    range.first = total * xcd / kXcds + (is_tail ? slot - (P8 - nB) : slot);
    range.end = total * (xcd + 1) / kXcds;
    range.step = is_tail ? nB : P8 - nB;
    if (range.first >= range.end) return;
    if (is_tail) {
        Loader<CB, AT, BKC, false> ld(g, s_off, mt_tail, s_poff, ntn, wid, lane);
        ld.tail = true;
        pipe_run<CB, NS, EPI, AT, BKC, false>(g, ld, range, reinterpret_cast<uint16_t(*)[CB::BM * BK]>(ring),
                                                reinterpret_cast<uint16_t(*)[BK * CB::BN]>(ring + NS * CB::BM * BK),
                                                s_bias, wid, lane);
    } else {
        const Loader<CA, AT, BKC, false> ld(g, s_off, mt_full, s_poff, ntn, wid, lane);
        pipe_run<CA, NS, EPI, AT, BKC, false>(g, ld, range, reinterpret_cast<uint16_t(*)[CA::BM * BK]>(ring),
                                                reinterpret_cast<uint16_t(*)[BK * CA::BN]>(ring + NS * CA::BM * BK),
                                                s_bias, wid, lane);
    }
}

template <class KernelFn>
static int persistent_blocks(KernelFn kernel, int threads) {
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess || per_cu < 1)
        per_cu = 1;
    const int blocks = per_cu * device_cu_count();
    return blocks < kXcds ? kXcds : blocks;
}

template <class C, int EPI, bool AT>
static int small_blocks() {
    static const int blocks = persistent_blocks(ffn_gemm_bf16_kernel<C, EPI, AT>, C::NT);
    return blocks;
}

// Large tiles: 256 x 256 on eight waves (two per SIMD), four 32 KiB stages.
// (Two workgroups per CU on 128 x 256 tiles measured slower where weight
// tiles are shared by several m-tiles: each re-reads them from HBM.)
template <class C, int NS, int EMAX, int WPE, int EPI, bool AT, bool BKC, bool TN>
static int pipe_blocks() {
    static const int blocks =
        persistent_blocks(ffn_gemm_bf16_pipe_kernel<C, NS, EMAX, WPE, EPI, AT, BKC, TN>, C::NT);
    return blocks;
}

// Upper bound of the work items for tile C: every expert may add one
// partial m-tile on top of max_rows / BM full ones.
template <class C>
static int64_t item_bound(const GemmArgs& g, int64_t max_rows) {
    return ((max_rows + C::BM - 1) / C::BM + g.E) * ((g.N + C::BN - 1) / C::BN);
}

template <class C, int NS, int EMAX, int WPE, int EPI, bool AT = kATiled<EPI>, bool BKC = false, bool TN = false>
static bool try_pipe(const GemmArgs& g, int64_t max_rows, hipStream_t st, hipError_t* err) {
    const int blocks = pipe_blocks<C, NS, EMAX, WPE, EPI, AT, BKC, TN>();
    // large tiles from half an item per workgroup: on the 16-expert layer's
    // GEMM2 (192 items bound, 156 used, on 256 workgroups) they take 102 us
    // against 143 us for 128 x 128 tiles; below that the small tiles spread
    // the work over more CUs
    const int64_t items = TN ? (int64_t)g.E * ((g.M + C::BM - 1) / C::BM) * ((g.N + C::BN - 1) / C::BN)
                             : item_bound<C>(g, max_rows);
    if (g.E > EMAX || 2 * items < (int64_t)blocks) return false;
    // TN: buffer ranges and byte offsets over a whole segment are 32-bit
    // (max_rows bounds a segment's rows here)
    if (TN && max_rows * (int64_t)(g.M > g.N ? g.M : g.N) * 2 >= (int64_t(1) << 31)) return false;
    hipLaunchKernelGGL((ffn_gemm_bf16_pipe_kernel<C, NS, EMAX, WPE, EPI, AT, BKC, TN>), dim3(blocks), dim3(C::NT), 0,
                       st, g);
    *err = hipGetLastError();
    return true;
}

#ifndef MOE_TAIL_SPLIT
#define MOE_TAIL_SPLIT 1   // the first GEMM's short expert tails on 128-row tiles (ffn_gemm_bf16_split_kernel)
#endif
#ifndef MOE_TAIL_SPLIT2
#define MOE_TAIL_SPLIT2 1   // the second GEMM's and dx_perm's too (roles or sequenced, per die)
#endif

// the split kernel in place of the pipelined one, under the same conditions
template <int EPI, bool AT, bool BKC = false>
static bool try_split(const GemmArgs& g, int64_t max_rows, hipStream_t st, hipError_t* err) {
    static const int blocks = [] {
        const int b = persistent_blocks(ffn_gemm_bf16_split_kernel<MOE_PIPE_NS, EPI, AT, BKC>, TilePipe::NT);
        return b / kXcds * kXcds;   // whole dies: each die splits its workgroups into the two roles
    }();
    if (g.E > 1024 || blocks < 2 * kXcds || 2 * item_bound<TilePipe>(g, max_rows) < (int64_t)blocks) return false;
    hipLaunchKernelGGL((ffn_gemm_bf16_split_kernel<MOE_PIPE_NS, EPI, AT, BKC>), dim3(blocks), dim3(TilePipe::NT),
                       0, st, g);
    *err = hipGetLastError();
    return true;
}

template <int EPI, bool AT = kATiled<EPI>>
static hipError_t launch_epi(const GemmArgs& g, int64_t max_rows, hipStream_t st) {
    hipError_t err = hipSuccess;
    if constexpr (MOE_TAIL_SPLIT && EPI == EPI_GELU_H)
        if (try_split<EPI, AT>(g, max_rows, st, &err)) return err;
    if constexpr (MOE_TAIL_SPLIT2 && EPI == EPI_STORE_F32)
        if (try_split<EPI, AT>(g, max_rows, st, &err)) return err;
    if (try_pipe<TilePipe, MOE_PIPE_NS, 1024, TilePipe::NW >= 8 ? 2 : 1, EPI, AT>(g, max_rows, st, &err)) return err;
    hipLaunchKernelGGL((ffn_gemm_bf16_kernel<TileSmall, EPI, AT>), dim3(small_blocks<TileSmall, EPI, AT>()),
                       dim3(TileSmall::NT), 0, st, g);
    return hipGetLastError();
}

hipError_t launch_ffn_gemm_bf16(const GemmArgs& g, int epi, int64_t max_rows, hipStream_t st, bool a_tiled) {
    if (epi == EPI_GELU_H)
        return a_tiled ? launch_epi<EPI_GELU_H, true>(g, max_rows, st) : launch_epi<EPI_GELU_H>(g, max_rows, st);
    return launch_epi<EPI_STORE_F32>(g, max_rows, st);
}

bool launch_ffn_gemm_bf16_pipe(const GemmArgs& g, int epi, bool b_kc, int64_t max_rows, hipStream_t st,
                               hipError_t* err) {
    constexpr int WPE = TilePipe::NW >= 8 ? 2 : 1;
    if (b_kc && g.K % BK != 0) return false;   // both operands K-contiguous: no zero rows under a K tail
    // the recompute and dh have GEMM1's shape: expert tails on 128-row tiles too
    if constexpr (MOE_TAIL_SPLIT) {
        if (epi == EPI_HGRAD && !b_kc && try_split<EPI_HGRAD, false>(g, max_rows, st, err)) return true;
        if (epi == EPI_DA && b_kc && try_split<EPI_DA, false, true>(g, max_rows, st, err)) return true;
    }
    if (epi == EPI_HGRAD && !b_kc) return try_pipe<TilePipe, MOE_PIPE_NS, 1024, WPE, EPI_HGRAD, false, false>(g, max_rows, st, err);
    // dx_perm has the second GEMM's shape
    if constexpr (MOE_TAIL_SPLIT2)
        if (epi == EPI_STORE_F32 && b_kc && try_split<EPI_STORE_F32, false, true>(g, max_rows, st, err)) return true;
    if (epi == EPI_STORE_F32 && b_kc)
        return try_pipe<TilePipe, MOE_PIPE_NS, 1024, WPE, EPI_STORE_F32, false, true>(g, max_rows, st, err);
    if (epi == EPI_DA && b_kc) return try_pipe<TilePipe, MOE_PIPE_NS, 1024, WPE, EPI_DA, false, true>(g, max_rows, st, err);
    if (epi == EPI_WGRAD && !b_kc)
        return try_pipe<TilePipe, MOE_PIPE_NS, 1024, WPE, EPI_WGRAD, false, false, true>(g, max_rows, st, err);
    return false;
}

}  // namespace moe
