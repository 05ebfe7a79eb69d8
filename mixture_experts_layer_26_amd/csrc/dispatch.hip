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
//             wave per row; pads perm with -1 past the used rows.
#include "moe_common.h"
#include "moe_kernels.h"

namespace moe {

int dispatch_block_tokens(int64_t T, int E, int k) {
    // bitmask bytes E * BT / 8 kept <= 32 KiB
    int bt = E <= 256 ? 1024 : E <= 512 ? 512 : 256;
    // aim at <= 2048 slots per block: with k = 8 or 16 choices per token a
    // 1024-token block leaves most CUs idle (8 blocks for 8192 tokens) while
    // each thread walks 8-16 slots.  Every scatter block reads the whole
    // [nblk x E] histogram, so blocks are not split past 256 of them.
    while (bt > 64 && bt * k > 2048 && (T + bt / 2 - 1) / (bt / 2) <= 256) bt >>= 1;
    return bt;
}

__global__ __launch_bounds__(1024) void hist_kernel(DispatchArgs a) {
    extern __shared__ int h[];  // [E]
    const int E = a.E;
    for (int e = threadIdx.x; e < E; e += blockDim.x) h[e] = 0;
    __syncthreads();
    const int64_t t = (int64_t)blockIdx.x * a.BT + threadIdx.x;
    if (t < a.T) {
        for (int j = 0; j < a.k; ++j) {
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

    // 3. per-expert token bitmask of this block
    const int64_t t = (int64_t)blk * BT + tid;
    const bool live = t < a.T;
    const int word = tid >> 6;
    const unsigned long long bit = 1ull << (tid & 63);
    if (live) {
        for (int j = 0; j < a.k; ++j) {
            const int e = a.idx[t * a.k + j];
            if ((unsigned)e < (unsigned)E) atomicOr(&mask[(size_t)e * MW + word], bit);
        }
    }
    __syncthreads();

    // 4. rank in token order -> row, or drop
    if (live) {
        for (int j = 0; j < a.k; ++j) {
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

hipError_t launch_hist(const DispatchArgs& a, hipStream_t st) {
    hipLaunchKernelGGL(hist_kernel, dim3(a.nblk), dim3(a.BT), sizeof(int) * a.E, st, a);
    return hipGetLastError();
}

hipError_t launch_scatter(const DispatchArgs& a, hipStream_t st) {
    const size_t sm = sizeof(unsigned long long) * (size_t)a.E * (a.BT / 64) +
                      sizeof(int) * (3 * (size_t)a.E + 1);
    hipLaunchKernelGGL(scatter_kernel, dim3(a.nblk), dim3(a.BT), sm, st, a);
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
