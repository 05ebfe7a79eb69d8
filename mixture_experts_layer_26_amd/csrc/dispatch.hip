// dispatch.hip -- capacity-limited, stable dispatch into expert-contiguous rows.
//
// [PithTrain] section 4.3 item 1: an expert takes at most `cap` tokens, the
// rest are dropped.  [EP] sections 4.1-4.2: gathering each expert's tokens
// with a separate concatenation step is costly; rows are instead written
// straight into a per-expert bucket.  Here the buckets are packed: expert e
// owns rows [offsets[e], offsets[e+1]) and keeps its slots in token order.
//
// Three launches, none of which relies on the order of atomics:
//   hist    : per token block (BT tokens) an LDS histogram of the k*BT slots;
//   scatter : every block re-derives, from the [nblk x E] histogram matrix,
//             its per-expert base (slots of earlier blocks), the routed and
//             kept totals and the offsets; the in-block rank of a slot is a
//             popcount over a per-expert bitmask of the block's tokens (a
//             token holds each expert at most once), so ranks follow token
//             order exactly;  kept slots write perm and slot;
//             block 0 also writes routed, counts, offsets and the balance
//             loss ([EP] section 2.3);
//   gather  : x_perm[row] = x[perm[row]] with 16-byte vector copies, one
//             wave per row; pads perm with -1 past the used rows (the fused
//             bf16 forward uses gather_tiled_kernel instead: the same rows
//             in the grouped GEMM's tile layout, copied token by token).
// gather_slots_kernel is the backward's copy of the rows, by slot.
#include "ffn_sched.h"
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

int dispatch_block_tokens(int64_t T, int E, int k) {
    // bitmask bytes E * BT / 8 kept <= 32 KiB
    int bt = E <= 256 ? 1024 : E <= 512 ? 512 : 256;
    // aim at <= 2048 slots per block and at least 16 blocks: with k = 8 or 16
    // choices per token a 1024-token block leaves most CUs idle (8 blocks for
    // 8192 tokens) while each thread walks 8-16 slots, and 4 or 8 blocks of
    // two choices per token left the scatter 2 us slower (4096 and 8192
    // tokens).  Every scatter block reads the whole [nblk x E] histogram, so
    // blocks are not split past 256 of them.
    while (bt > 64 && (bt * k > 2048 || (T + bt - 1) / bt < 16) && (T + bt / 2 - 1) / (bt / 2) <= 256) bt >>= 1;
    return bt;
}

int dispatch_threads(int BT, int k) {
    // J = blockDim / BT threads per token, each taking every J-th of its
    // slots: with many choices per token one thread walking all k of them
    // in turn waits on each load (k = 128: 77 us for the scatter of 1024
    // tokens on 16 blocks of 64 threads)
    int j = 1;
    while (2 * j <= k && 2 * j * BT <= 1024) j *= 2;
    return j * BT;
}

__global__ __launch_bounds__(1024) void hist_kernel(DispatchArgs a) {
    extern __shared__ int h[];  // [E]
    const int E = a.E;
    for (int e = threadIdx.x; e < E; e += blockDim.x) h[e] = 0;
    __syncthreads();
    const int J = blockDim.x / a.BT;
    const int64_t t = (int64_t)blockIdx.x * a.BT + threadIdx.x % a.BT;
    if (t < a.T) {
        for (int j = threadIdx.x / a.BT; j < a.k; j += J) {
            const int e = a.idx[t * a.k + j];
            if ((unsigned)e < (unsigned)E) atomicAdd(&h[e], 1);
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) a.blkhist[(int64_t)blockIdx.x * E + e] = h[e];
}

__global__ __launch_bounds__(1024) void scatter_kernel(DispatchArgs a) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    const int E = a.E, BT = a.BT, MW = BT / 64;
    unsigned long long* mask = reinterpret_cast<unsigned long long*>(smem_raw);  // [E][MW]
    int* base_s = reinterpret_cast<int*>(mask + (size_t)E * MW);                // [E]
    int* cnt_s = base_s + E;                                                      // [E]
    int* off_s = cnt_s + E;                                                       // [E+1]
    __shared__ int scan_tmp[32];
    const int tid = threadIdx.x;
    const int blk = blockIdx.x;

    // 1. per-expert base of this block, routed and kept totals
    for (int e = tid; e < E; e += blockDim.x) {
        int before = 0, total = 0;
        for (int b = 0; b < a.nblk; ++b) {
            const int hv = a.blkhist[(int64_t)b * E + e];
            before += (b < blk) ? hv : 0;
            total += hv;
        }
        base_s[e] = before;
        const int kept = (int64_t)total < a.cap ? total : (int)a.cap;
        cnt_s[e] = kept;
        if (blk == 0) {
            if (a.routed) a.routed[e] = total;
            if (a.counts) a.counts[e] = kept;
        }
    }
    for (int i = tid; i < E * MW; i += blockDim.x) mask[i] = 0ull;
    __syncthreads();

    // 2. offsets = exclusive scan of kept counts (each thread a contiguous chunk)
    const int per = (E + blockDim.x - 1) / blockDim.x;
    const int lo = tid * per;
    int local = 0;
    for (int e = lo; e < lo + per && e < E; ++e) local += cnt_s[e];
    const int incl = block_inclusive_scan(local, scan_tmp);
    int run = incl - local;
    for (int e = lo; e < lo + per && e < E; ++e) {
        off_s[e] = run;
        run += cnt_s[e];
    }
    if (tid == blockDim.x - 1) off_s[E] = incl;
    __syncthreads();
    if (blk == 0) {
        for (int e = tid; e <= E; e += blockDim.x) a.offsets[e] = off_s[e];
        if (tid == 0 && a.aux != nullptr) {
            // lambda * sum_e (kept_e / (T k)) * (1/E), evaluated in double
            const double S = (double)off_s[E];
            a.aux[0] = (float)((double)a.lambda * (S / ((double)a.T * (double)a.k)) / (double)E);
        }
    }

    // 3. per-expert token bitmask of this block (J threads per token, each
    // taking every J-th slot)
    const int tl = tid % BT, J = blockDim.x / BT, j0 = tid / BT;
    const int64_t t = (int64_t)blk * BT + tl;
    const bool live = t < a.T;
    const int word = tl >> 6;
    const unsigned long long bit = 1ull << (tl & 63);
    if (live) {
        for (int j = j0; j < a.k; j += J) {
            const int e = a.idx[t * a.k + j];
            if ((unsigned)e < (unsigned)E) atomicOr(&mask[(size_t)e * MW + word], bit);
        }
    }
    __syncthreads();

    // 4. rank in token order -> row, or drop
    if (live) {
        for (int j = j0; j < a.k; j += J) {
            const int64_t s = t * a.k + j;
            const int e = a.idx[s];
            int row = -1;
            if ((unsigned)e < (unsigned)E) {
                const unsigned long long* m = mask + (size_t)e * MW;
                int rank = __popcll(m[word] & (bit - 1ull));
                for (int wv = 0; wv < word; ++wv) rank += __popcll(m[wv]);
                const int64_t p = (int64_t)base_s[e] + rank;
                if (p < a.cap) {
                    row = off_s[e] + (int)p;
                    a.perm[row] = (int32_t)t;
                }
            }
            a.slot[s] = row;
        }
    }
}

// one wave per row of the expert-contiguous buffer
__global__ __launch_bounds__(256) void gather_kernel(DispatchArgs a) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t S = a.offsets[a.E];
    const int64_t n16 = a.row_bytes / 16;
    const int64_t wstride = (int64_t)gridDim.x * (blockDim.x / kWave);
    for (int64_t r = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave; r < a.max_rows;
         r += wstride) {
        if (r < S) {
            const int64_t src = a.perm[r];
            if ((uint64_t)src >= (uint64_t)a.T) continue;  // only with invalid topk_idx
            const uint4* s4 = reinterpret_cast<const uint4*>(static_cast<const char*>(a.x) +
                                                             src * a.row_bytes);
            uint4* d4 = reinterpret_cast<uint4*>(static_cast<char*>(a.x_perm) + r * a.row_bytes);
            for (int64_t c = lane; c < n16; c += kWave) d4[c] = s4[c];
        } else if (lane == 0) {
            a.perm[r] = -1;
        }
    }
}

// The fused bf16 forward's copy of the kept rows into the grouped GEMM's
// 16-row x 32-column tile layout over expert segments padded to 16 rows:
// padded row p, column c at ((p / 16) KT + c / 32) 512 + (p % 16) 32 + c % 32,
// KT = ceil(d / 32).  In that layout one K-step of 16 rows of GEMM1's
// activation operand is one contiguous KiB: a global -> LDS load of 64-byte
// row pieces moves half as many bytes per cycle as one of contiguous KiBs.
// Columns d .. 32 KT - 1 are zeros (the weight rows past d read as zeros, so
// the K tail must be finite).  Two ways, chosen in the kernel from the kept
// row count S (offsets[E]):
//   by token: a wave copies two tokens at a time, each row of x read once
//     (1 KiB per load) and written to its k kept slots in 64-byte tile row
//     pieces (4 lanes each), the slots' destinations found by k lanes at
//     once; padding rows are not written (the grouped GEMM computes them but
//     never stores their outputs);
//   by block: a workgroup takes 16-row blocks, each wave a quarter of the
//     block's tiles, each lane one 16-byte piece of row 16 pb + lane / 4 -- the gathered
//     rows are read in 64-byte pieces and every tile is one contiguous KiB
//     store; padding rows are written as zeros.
// The token way reads T rows instead of the block way's S (with its
// re-reads of a row's other copies, from cache) but scatters 64-byte writes,
// which merge into whole lines while the written rows and x fit in the
// last-level cache (256 MB).  It is taken when S >= 1.5 T, x is at least 12
// MiB (below that the re-reads stay in cache) and (T + S) d 2 bytes <= 192
// MiB, with k <= 32.  Measured on MI355X (us, token / block way): 64 experts top-2 18.7 /
// 21.8, 128 experts top-8 27.1 / 41.6, the 16-expert soft layer (k = 16,
// x 8 MiB) 29.6 / 25.8, 16 experts top-2 8.4 / 9.0, 256 experts at T = 32768
// 80.3 / 74.7, the literal Zipf bias (most slots dropped) 13.0 / 10.7.
// Both pad perm with -1 past the used rows; the row-major x_perm is not
// written.
constexpr int GT_TOKENS = 16;   // tokens per workgroup pass (4 per wave)
constexpr int GT_CPL = 8;       // 16-byte chunks per lane and token in one pass (d <= 4096)
constexpr int GB_TILES = 8;     // tiles per wave in flight (block way)

#ifndef MOE_GATHER_FORCE
#define MOE_GATHER_FORCE 0   // 1: token way, 2: block way (timing builds only)
#endif

__global__ __launch_bounds__(256) void gather_tiled_kernel(DispatchArgs a, uint16_t* __restrict__ x_pt, int d) {
    __shared__ int s_off[1025];
    __shared__ int s_poff[1025];
    __shared__ int scan_tmp[32];
    const int E = a.E, k = a.k;
    for (int i = threadIdx.x; i <= E; i += blockDim.x) s_off[i] = a.offsets[i];
    __syncthreads();
    build_padded_offsets(s_off, E, s_poff, scan_tmp);   // ends with a barrier
    const int lane = threadIdx.x & (kWave - 1);
    const int wid = threadIdx.x / kWave;
    const int KT = (d + 31) >> 5;
    const int nch = KT * 4;   // 16-byte chunks of a tiled row
    const int d16 = d / 8;    // of them, the ones holding x (d is a multiple of 8)
    const uint4* __restrict__ x4 = static_cast<const uint4*>(a.x);
    uint4* __restrict__ t4 = reinterpret_cast<uint4*>(x_pt);
    const int64_t S = s_off[E];
    // (the token way holds a token's slots in 32 lanes: k <= 32)
    bool by_token = k <= 32 && 2 * S >= 3 * a.T && a.T * (int64_t)d * 2 >= (int64_t(12) << 20) &&
                    (a.T + S) * (int64_t)d * 2 <= (int64_t(192) << 20);
    if (MOE_GATHER_FORCE) by_token = MOE_GATHER_FORCE == 1;
    if (by_token) {
        const int64_t step = (int64_t)gridDim.x * GT_TOKENS;
        for (int64_t t0 = (int64_t)blockIdx.x * GT_TOKENS; t0 < a.T; t0 += step) {
            // wave w copies tokens t0 + w + 4 u, two at a time
            for (int u = 0; u < GT_TOKENS / 4; u += 2) {
                const int64_t ta = t0 + wid + 4 * u, tb = ta + 4;
                // lane j (< k) finds the tile row start of copy j of token a,
                // lane 32 + j that of token b (k <= 32); -1: dropped
                int64_t dst = -1;
                {
                    const int j = lane & 31;
                    const int64_t t = lane < 32 ? ta : tb;
                    if (j < k && t < a.T) {
                        const int r = a.slot[t * k + j];
                        const int e = a.idx[t * k + j];
                        if (r >= 0 && (unsigned)e < (unsigned)E) {
                            const int64_t p = (int64_t)r - s_off[e] + s_poff[e];
                            dst = (p >> 4) * KT * 64 + (p & 15) * 4;
                        }
                    }
                }
                const int dlo = (int)(uint32_t)(uint64_t)dst, dhi = (int)(uint32_t)((uint64_t)dst >> 32);
                for (int cb = 0; cb < nch; cb += kWave * GT_CPL) {
                    uint4 va[GT_CPL], vb[GT_CPL];
#pragma unroll
                    for (int i = 0; i < GT_CPL; ++i) {
                        const int c = cb + lane + kWave * i;
                        va[i] = make_uint4(0u, 0u, 0u, 0u);
                        vb[i] = make_uint4(0u, 0u, 0u, 0u);
                        if (c < d16) {
                            if (ta < a.T) va[i] = x4[ta * d16 + c];
                            if (tb < a.T) vb[i] = x4[tb * d16 + c];
                        }
                    }
                    for (int h = 0; h < 2; ++h) {
                        for (int j = 0; j < k; ++j) {
                            const int src = 32 * h + j;
                            const int64_t base = (int64_t)(((uint64_t)(uint32_t)__shfl(dhi, src) << 32) |
                                                           (uint32_t)__shfl(dlo, src));
                            if (base < 0) continue;
#pragma unroll
                            for (int i = 0; i < GT_CPL; ++i) {
                                const int c = cb + lane + kWave * i;
                                if (c < nch) t4[base + (c >> 2) * 64 + (c & 3)] = h ? vb[i] : va[i];
                            }
                        }
                    }
                }
            }
        }
    } else {
        const int nblk16 = s_poff[E] >> 4;
        for (int pb = blockIdx.x; pb < nblk16; pb += gridDim.x) {
            // lane l: row p = 16 pb + l / 4 (its source token, or -1 for padding), piece l % 4
            const int p = (pb << 4) + (lane >> 2);
            int lo = 0, hi = E;   // largest e with s_poff[e] <= p: the expert holding the block
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (s_poff[mid] <= p) lo = mid;
                else hi = mid;
            }
            const int local = p - s_poff[lo];
            const int src0 = local < s_off[lo + 1] - s_off[lo] ? a.perm[s_off[lo] + local] : -1;
            const int64_t src = (uint64_t)(int64_t)src0 < (uint64_t)a.T ? src0 : -1;
            const int piece = lane & 3;
            // wave w: a contiguous quarter of the block's tiles, GB_TILES in flight
            const int ct_end = (wid + 1) * KT / 4;
            for (int ct0 = wid * KT / 4; ct0 < ct_end; ct0 += GB_TILES) {
                uint4 v[GB_TILES];
#pragma unroll
                for (int i = 0; i < GB_TILES; ++i) {
                    const int c = (ct0 + i) * 4 + piece;   // 16-byte chunk of the row
                    v[i] = make_uint4(0u, 0u, 0u, 0u);
                    if (ct0 + i < ct_end && src >= 0 && c < d16) v[i] = x4[src * d16 + c];
                }
#pragma unroll
                for (int i = 0; i < GB_TILES; ++i)
                    if (ct0 + i < ct_end) t4[((int64_t)pb * KT + ct0 + i) * 64 + lane] = v[i];
            }
        }
    }
    const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
    for (int64_t r = S + (int64_t)blockIdx.x * blockDim.x + threadIdx.x; r < a.max_rows; r += nthreads)
        a.perm[r] = -1;
}

hipError_t launch_gather_tiled(const DispatchArgs& a, uint16_t* x_pt, int d, hipStream_t st) {
    if (a.E > 1024) return hipErrorInvalidValue;
    // enough workgroups for either way: T / GT_TOKENS token groups or one per 16-row block
    const int64_t by_block = h_tiled_rows(a.max_rows, a.E) / 16;
    const int64_t by_token = (a.T + GT_TOKENS - 1) / GT_TOKENS;
    int64_t blocks = by_block > by_token ? by_block : by_token;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(gather_tiled_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a, x_pt, d);
    return hipGetLastError();
}

// x_perm[slot[t, j]] = x[t] for every kept slot, one wave per token (the
// backward's own copy of the rows when the caller passes no x_perm).
__global__ __launch_bounds__(256) void gather_slots_kernel(int64_t T, int k, int64_t max_rows, int64_t row_bytes,
                                                           const void* __restrict__ x,
                                                           const int32_t* __restrict__ slot,
                                                           void* __restrict__ x_perm) {
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t n16 = row_bytes / 16;
    const int64_t nwaves = (int64_t)gridDim.x * (blockDim.x / kWave);
    for (int64_t t = ((int64_t)blockIdx.x * blockDim.x + threadIdx.x) / kWave; t < T; t += nwaves) {
        const uint4* s4 = reinterpret_cast<const uint4*>(static_cast<const char*>(x) + t * row_bytes);
        // the token's slots 64 at a time, one per lane
        for (int j0 = 0; j0 < k; j0 += kWave) {
            const int my = j0 + lane < k ? slot[t * k + j0 + lane] : -1;
            const uint64_t keep = __ballot((uint64_t)(int64_t)my < (uint64_t)max_rows);
            for (uint64_t m = keep; m != 0; m &= m - 1) {
                const int j = __ffsll((unsigned long long)m) - 1;
                const int64_t row = __shfl(my, j, kWave);
                uint4* d4 = reinterpret_cast<uint4*>(static_cast<char*>(x_perm) + row * row_bytes);
                for (int64_t c = lane; c < n16; c += kWave) d4[c] = s4[c];
            }
        }
    }
}

hipError_t launch_gather_slots(int64_t T, int k, int64_t max_rows, int64_t row_bytes, const void* x,
                               const int32_t* slot, void* x_perm, hipStream_t st) {
    int64_t blocks = (T + 3) / 4;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(gather_slots_kernel, dim3((unsigned)blocks), dim3(256), 0, st, T, k, max_rows, row_bytes, x,
                       slot, x_perm);
    return hipGetLastError();
}

hipError_t launch_hist(const DispatchArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(hist_kernel, dim3(a.nblk), dim3(dispatch_threads(a.BT, a.k)), sizeof(int) * a.E, st, a);
    return hipGetLastError();
}

hipError_t launch_scatter(const DispatchArgs& a, hipStream_t st) {
    const size_t sm = sizeof(unsigned long long) * (size_t)a.E * (a.BT / 64) +
                      sizeof(int) * (3 * (size_t)a.E + 1);
    hipLaunchKernelGGL(scatter_kernel, dim3(a.nblk), dim3(dispatch_threads(a.BT, a.k)), sm, st, a);
    return hipGetLastError();
}

hipError_t launch_gather(const DispatchArgs& a, hipStream_t st) {
    int64_t blocks = (a.max_rows + 3) / 4;
    if (blocks > 65536) blocks = 65536;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(gather_kernel, dim3((unsigned)blocks), dim3(256), 0, st, a);
    return hipGetLastError();
}

}  // namespace moe
