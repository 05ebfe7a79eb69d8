// lds_dma.h -- global -> LDS loads without VGPR staging, and the explicit
// waits and barriers that publish them (CDNA4).
//
// buffer_load_dwordx4 ... lds writes 16 bytes per lane to LDS at
// M0 + 16 * lane: one wave instruction fills 1 KiB.  The loads are issued as
// inline asm so that the compiler's wait insertion neither tracks them nor
// adds vmcnt(0) waits for them; every wait on them is explicit.  Vector
// memory loads return in order, so "s_waitcnt vmcnt(n)" means: every load
// of this wave except the n newest has landed.
#pragma once

#include "moe_common.h"

namespace moe {

typedef int i32x4_t __attribute__((ext_vector_type(4)));

// 16 bytes per lane from the buffer at byte offset voffset to lds + 16 * lane.
__device__ __forceinline__ void dma16(const i32x4_t& rsrc, const void* lds, int voffset) {
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds));
    asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(m0), "v"(voffset), "s"(rsrc) : "memory", "m0");
}

// Buffer descriptor: 48-bit base, stride 0, range in bytes, gfx9 data format.
// Offsets at or past the range read zeros and touch no memory.
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

// s_waitcnt immediate (gfx9 layout: vmcnt in bits 3:0 and 15:14, expcnt 6:4,
// lgkmcnt 11:8); expcnt is never waited on here
constexpr int waitcnt_imm(int vm, int lgkm) { return (vm & 15) | ((vm >> 4) << 14) | (7 << 4) | (lgkm << 8); }

// vmcnt(VM) lgkmcnt(0) then the workgroup barrier.  The wait goes through the
// builtin so the compiler's own wait insertion knows every LDS read has
// returned; the barrier is asm with a memory clobber so no LDS access moves
// across it, and the scheduling barriers keep arithmetic on its side.
template <int VM>
__device__ __forceinline__ void dma_barrier() {
    static_assert(VM >= 0 && VM < 64, "vmcnt range");
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(VM, 0));
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// K-contiguous tile rows of 64 bytes (32 bf16): logical 16-byte chunk c of
// row r sits at physical slot c ^ ((r >> 1) & 3), which puts the 16 rows one
// 16-lane group reads with ds_read_b128 (one chunk each) on distinct banks
// (measured conflict-free with SQ_LDS_BANK_CONFLICT on MI355X).
__device__ __forceinline__ int k64_swz(int r) { return (r >> 1) & 3; }
__device__ __forceinline__ int k64_slot(int r, int c) { return r * 4 + (c ^ k64_swz(r)); }

}  // namespace moe
