// Global -> LDS staging and prologue-load helpers shared by the decode kernels.
#pragma once

#include "rq_common.hpp"

namespace rq {

// ---- staging: the cache stream goes global -> LDS by DMA (global_load_lds_dwordx4), one
// 16-byte chunk per lane, without passing through registers.  The compiler does not
// track these LDS writes, so each wave waits for its own DMAs explicitly (vmcnt) before
// reading a staged pass; no other vector-memory instruction is issued inside the loop.
//
// The compiler inserts the wait states that the hardware requires between dependent
// instructions in front of its own instructions, not in front of inline assembly, so the
// statement carries them itself:
// * an LDS DMA that reads M0 right after a scalar write of M0 (the compiler's own move
//   of lds_addr into M0) needs 1 wait state;
// * FRESH: the base was just moved into scalar registers by a vector instruction
//   (v_readfirstlane, see uniform_ptr).  A vector-memory instruction that reads an SGPR
//   written by a VALU instruction needs 5 wait states; without them the DMA can take the
//   registers' previous contents as its address.
//
// The stream is read once per loop-step, so its loads carry the non-temporal hint (nt):
// the caches treat the lines as streaming, and the small data every loop-step reuses (the
// rotations, queries, split records) is less likely to be evicted by them.
// NT = false for a section that shares its cache lines with the next passes of its tile.
template <bool FRESH = false, bool NT = true>
__device__ __forceinline__ void dma16(uint32_t voff, const uint8_t* sbase, uint32_t lds_addr) {
    if constexpr (FRESH && NT)
        asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 nt" :: "v"(voff), "s"(sbase), "{m0}"(lds_addr) : "memory");
    else if constexpr (NT)
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt" :: "v"(voff), "s"(sbase), "{m0}"(lds_addr) : "memory");
    else if constexpr (FRESH)
        asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" :: "v"(voff), "s"(sbase), "{m0}"(lds_addr) : "memory");
    else
        asm volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" :: "v"(voff), "s"(sbase), "{m0}"(lds_addr) : "memory");
}

// copy BYTES (multiple of 16, at most 1024) from sbase + goff to LDS lds_addr
template <int BYTES, bool FRESH = false, bool NT = true>
__device__ __forceinline__ void stage(const uint8_t* sbase, uint32_t goff, uint32_t lds_addr, int lane) {
    static_assert(BYTES % 16 == 0 && BYTES <= 1024, "one DMA instruction per block");
    if (BYTES == 1024 || lane < BYTES / 16) dma16<FRESH, NT>(goff + 16u * lane, sbase, lds_addr);
}

// A wave-uniform pointer moved into scalar registers (the DMA takes its base there); a DMA
// that reads it must be issued with FRESH = true.
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
    const uint64_t u = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
    return (const uint8_t*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
    asm volatile("s_waitcnt vmcnt(%0)" :: "n"(N) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr_of(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Prologue loads go through inline asm as well: the compiler counts outstanding loads
// for its own waits and cannot see the stream DMAs issued after these, so its waits
// would also stall on the DMAs.  pin() orders every use of a loaded register after the
// explicit wait that follows the DMA issue.
__device__ __forceinline__ f32x4 gload16(const uint8_t* sbase, uint32_t voff) {
    f32x4 r;
    asm volatile("global_load_dwordx4 %0, %1, %2" : "=v"(r) : "v"(voff), "s"(sbase));
    return r;
}
__device__ __forceinline__ u32x2 gload8(const uint8_t* sbase, uint32_t voff) {
    u32x2 r;
    asm volatile("global_load_dwordx2 %0, %1, %2" : "=v"(r) : "v"(voff), "s"(sbase));
    return r;
}
template <class T>
__device__ __forceinline__ void pin(T& x) {
    asm volatile("" : "+v"(x));
}

// Sum each of N values over aligned groups of 2M consecutive lanes.  Reduce-scatter
// while values remain (lanes with bit M set keep the upper half), then plain
// butterflies; on return v[0] is the group sum of value `off`.
template <int CUR, int M, int N>
__device__ __forceinline__ void group_reduce_scatter(float (&v)[N], int lane, int& off) {
    if constexpr (M >= 1) {
        if constexpr (CUR > 1) {
            constexpr int half = CUR / 2;
#pragma unroll
            for (int i = 0; i < half; ++i) v[i] = rs_pair<M>(v[i], v[i + half]);
            if (lane & M) off += half;
            group_reduce_scatter<half, M / 2, N>(v, lane, off);
        } else {
            if constexpr (M == 16 || M == 32) {
                const int x = __float_as_int(v[0]);
                const auto r = (M == 16) ? __builtin_amdgcn_permlane16_swap(x, x, false, false)
                                         : __builtin_amdgcn_permlane32_swap(x, x, false, false);
                v[0] = __int_as_float((int)r[0]) + __int_as_float((int)r[1]);
            } else {
                v[0] += xpartner<M>(v[0]);
            }
            group_reduce_scatter<1, M / 2, N>(v, lane, off);
        }
    }
}

}  // namespace rq
