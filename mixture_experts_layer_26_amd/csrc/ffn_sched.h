// ffn_sched.h -- work list of the grouped expert GEMMs, built on the device.
//
// The rows of expert e are [offsets[e], offsets[e+1]) (data dependent, never
// copied to the host).  A work item is (expert, n-tile, m-tile); items are
// numbered expert-major, then n-tile, then m-tile, so the m-tiles that share
// a weight tile are neighbours.  Each persistent workgroup first turns the
// per-expert row counts into a prefix of m-tile counts in LDS, then walks
// its share of the items.
//
// XCD-aware split: MI355X dispatches workgroup i to accelerator die i % 8 and
// each die has its own L2.  The item range is cut into 8 contiguous chunks,
// one per die, and the workgroups of a die take that chunk's items round
// robin.  Items running at the same time on one die are therefore
// neighbours: the same expert's activation rows and the same weight tile
// are re-read from that die's L2 instead of HBM.
#pragma once

#include "moe_common.h"

namespace moe {

// m-tiles of an expert of `rows` rows: every BM-row block (kTilesAll); the
// whole 256-row blocks plus a remainder above 128 rows (kTilesFull, BM =
// 256); or one tile for a remainder of 1..128 rows (kTilesTail)
enum { kTilesAll = 0, kTilesFull = 1, kTilesTail = 2 };
__device__ __forceinline__ int tiles_of(int rows, int BM, int mode) {
    if (mode == kTilesFull) return (rows >> 8) + ((rows & 255) > 128 ? 1 : 0);
    if (mode == kTilesTail) return ((rows & 255) != 0 && (rows & 255) <= 128) ? 1 : 0;
    return (rows + BM - 1) / BM;
}

// mt_pre[e] = sum_{e' < e} tiles_of(rows(e')), mt_pre[E] = total m-tiles.
// Needs blockDim.x <= 1024, mt_pre of E+1 ints and tmp of 32 ints in LDS.
__device__ __forceinline__ int build_mtile_prefix(const int32_t* __restrict__ offsets, int E, int BM,
                                                  int* mt_pre, int* tmp, int mode = kTilesAll) {
    const int tid = threadIdx.x;
    const int per = (E + blockDim.x - 1) / blockDim.x;
    const int lo = tid * per;
    int local = 0;
    for (int e = lo; e < lo + per && e < E; ++e) {
        const int rows = offsets[e + 1] - offsets[e];
        local += tiles_of(rows, BM, mode);
    }
    const int incl = block_inclusive_scan(local, tmp);
    int run = incl - local;
    for (int e = lo; e < lo + per && e < E; ++e) {
        mt_pre[e] = run;
        const int rows = offsets[e + 1] - offsets[e];
        run += tiles_of(rows, BM, mode);
    }
    if (tid == blockDim.x - 1) mt_pre[E] = incl;
    __syncthreads();
    return mt_pre[E];
}

// s_poff[e] = sum over e' < e of the expert's rows rounded up to 16 (from
// s_off in LDS, visible to every thread); same scan as build_mtile_prefix.
__device__ __forceinline__ void build_padded_offsets(const int* s_off, int E, int* s_poff, int* tmp) {
    const int tid = threadIdx.x;
    const int per = (E + blockDim.x - 1) / blockDim.x;
    const int lo = tid * per;
    int local = 0;
    for (int e = lo; e < lo + per && e < E; ++e) local += (s_off[e + 1] - s_off[e] + 15) & ~15;
    const int incl = block_inclusive_scan(local, tmp);
    int run = incl - local;
    for (int e = lo; e < lo + per && e < E; ++e) {
        s_poff[e] = run;
        run += (s_off[e + 1] - s_off[e] + 15) & ~15;
    }
    if (tid == blockDim.x - 1) s_poff[E] = incl;
    __syncthreads();
}

struct WorkItem {
    int e, nt, mt;
};

// Largest e with mt_pre[e] * ntn <= item (that expert has >= 1 m-tile).
__device__ __forceinline__ WorkItem decode_item(const int* mt_pre, int E, int ntn, int64_t item) {
    int lo = 0, hi = E;
    while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if ((int64_t)mt_pre[mid] * ntn <= item) lo = mid;
        else hi = mid;
    }
    const int mte = mt_pre[lo + 1] - mt_pre[lo];
    const int64_t local = item - (int64_t)mt_pre[lo] * ntn;
    WorkItem w;
    w.e = lo;
    w.nt = (int)(local / mte);
    w.mt = (int)(local - (int64_t)w.nt * mte);
    return w;
}

struct ItemRange {
    int64_t first, end, step;
};

__device__ __forceinline__ ItemRange xcd_item_range(int64_t total) {
    const int P = gridDim.x;
    const int xcd = blockIdx.x % kXcds;
    const int slot = blockIdx.x / kXcds;
    const int nPx = (P - xcd + kXcds - 1) / kXcds;
    ItemRange r;
    const int64_t lo = total * xcd / kXcds;
    r.end = total * (xcd + 1) / kXcds;
    r.first = lo + slot;
    r.step = nPx;
    return r;
}

}  // namespace moe
