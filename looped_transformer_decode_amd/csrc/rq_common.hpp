// Internal definitions shared by the ResidualQuant HIP kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "rq.h"

namespace rq {

constexpr int kTile = 64;          // tokens per cache tile
constexpr int kMaxSplits = 64;     // split-K upper bound (sizes the workspace)
constexpr int kMaxLoops = 16;      // loops per anchor group
constexpr int kWave = 64;
constexpr int kStageDepth = 3;     // LDS ring slots per wave in the decode kernel (passes)

// Byte geometry of the packed cache, derived from rq_config on the host and passed
// to kernels by value.
struct Geom {
    int d, g, ba, br, L, n_groups, chained, hkv, hq, max_batch, max_ctx;
    int n_tiles;
    int a_row, m_row;                  // bytes per token row: anchor codes, meta
    int scale_rule;                    // 0: least-squares c, 1: norm-ratio c
    int rb[kMaxLoops];                 // residual code width of each local loop 0..L-2
    int64_t a_tile;                    // bytes per anchor tile
    int64_t r_pre[kMaxLoops];          // bytes of the residual tiles of local loops < l (one tile each)
    int64_t group_bytes, block_bytes, total;

    __host__ __device__ int rbits(int l) const { return rb[l]; }
    __host__ __device__ int rrow(int l) const { return d * rb[l] / 8; }                 // code bytes per token
    __host__ __device__ int64_t rtile(int l) const { return (int64_t)kTile * (rrow(l) + m_row + 2); }

    __host__ __device__ int64_t plane_offset(int b, int h, int x, int loop) const {
        const int k = loop / L, l = loop % L;
        return ((int64_t)(b * hkv + h) * 2 + x) * block_bytes + (int64_t)k * group_bytes +
               (int64_t)n_tiles * r_pre[l];
    }

    // Paged layout: a pool of physical blocks, each holding one 64-token tile of every (KV
    // head, K|V, anchor group, loop plane) as [head][K|V][group][residual planes..., anchor]
    // (g_tile bytes per (head, K|V, group)); bt[b * bt_stride + t] names the block of tile t
    // of row b.  bt == nullptr selects the contiguous layout above.
    const int32_t* bt;
    int bt_stride, n_blocks;
    int64_t g_tile, p_block;

    // byte offset of the tile of (h, x, loop) inside physical block blk
    __host__ __device__ int64_t paged_offset(int blk, int h, int x, int loop) const {
        const int k = loop / L, l = loop % L;
        return (int64_t)blk * p_block + ((int64_t)(h * 2 + x) * n_groups + k) * g_tile + r_pre[l];
    }

    // byte offset of tile `tile` of (b, h, x, loop) in either layout; a block id outside
    // [0, n_blocks) is clamped (the table is device data the host cannot check)
    __device__ int64_t tile_offset(int b, int h, int x, int loop, int tile) const {
        const int l = loop % L;
        if (bt == nullptr) return plane_offset(b, h, x, loop) + (int64_t)tile * (l == L - 1 ? a_tile : rtile(l));
        return paged_offset(block_id(b, tile), h, x, loop);
    }
    __device__ int block_id(int b, int tile) const {
        int blk = bt[(int64_t)b * bt_stride + tile];
        return blk < 0 ? 0 : (blk >= n_blocks ? n_blocks - 1 : blk);
    }
};

// Block id of a wave-uniform (row, tile) through the scalar cache: the decode kernels keep
// exact counts of their outstanding vector loads, which this load must not join.
__device__ __forceinline__ int block_id_scalar(const Geom& g, int b, int tile) {
    const int idx = __builtin_amdgcn_readfirstlane(b * g.bt_stride + tile);
    typedef const int32_t __attribute__((address_space(4)))* cptr;
    int blk = ((cptr)(uintptr_t)g.bt)[idx];
    blk = __builtin_amdgcn_readfirstlane(blk);
    return blk < 0 ? 0 : (blk >= g.n_blocks ? g.n_blocks - 1 : blk);
}

// Returns false if the configuration is outside the supported tuples.
bool make_geom(const rq_config* cfg, Geom* g);

// Workspace layout for split-K decode: per (batch row, query head, split) a record of
// acc_a[d] (anchor part, or the whole output of the BF16 kernel), acc_r[d] (residual part,
// before R_V^T), m (running max), l (denominator), 2 floats of padding; then one 32-bit
// arrival counter per (batch row, query head), which every call leaves at zero.
__host__ __device__ inline int partial_stride(int d) { return 2 * d + 4; }
inline size_t records_bytes(int max_batch, int hq, int d) {
    return (size_t)max_batch * hq * kMaxSplits * partial_stride(d) * sizeof(float);
}
inline size_t workspace_bytes(int max_batch, int hq, int d) {
    return records_bytes(max_batch, hq, d) + (((size_t)max_batch * hq * sizeof(uint32_t) + 255) & ~(size_t)255);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef double f64x2 __attribute__((ext_vector_type(2)));
typedef double f64x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- number formats

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// OCP FP8 E4M3FN byte -> float (finite patterns; 0x7F/0xFF are never stored by the pack).
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    float mag = (e == 0) ? (float)m * 0x1p-9f : __uint_as_float(((e + 120u) << 23) | (m << 20));
    return (b & 0x80u) ? -mag : mag;
}

// ---------------------------------------------------------------- block mapping

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2).
// Remap so that consecutive logical indices (the splits of one query head, and the
// query heads of one KV head) run on the same XCD.
__device__ __forceinline__ int xcd_logical_block(int bid, int nblocks) {
    constexpr int kXcd = 8;
    const int per = nblocks / kXcd, rem = nblocks % kXcd;
    const int xcd = bid % kXcd, local = bid / kXcd;
    return (xcd < rem) ? xcd * (per + 1) + local : rem * (per + 1) + (xcd - rem) * per + local;
}

// ---------------------------------------------------------------- cross-lane helpers

__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __shfl_xor(v, m, kWave); }

__device__ __forceinline__ double shfl_xor_d(double v, int m) {
    int2 p = *reinterpret_cast<int2*>(&v);
    p.x = __shfl_xor(p.x, m, kWave);
    p.y = __shfl_xor(p.y, m, kWave);
    return *reinterpret_cast<double*>(&p);
}

// ---------------------------------------------------------------- DPP reductions
// quad_perm patterns: [1,0,3,2] swaps neighbours, [2,3,0,1] swaps pairs.
constexpr int kDppQuadXor1 = 0xB1;
constexpr int kDppQuadXor2 = 0x4E;
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr3 = 0x113;
constexpr int kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

template <int CTRL, int ROWMASK = 0xF, int BANKMASK = 0xF>
__device__ __forceinline__ float dpp_f(float old, float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROWMASK,
                                                      BANKMASK, false));
}

constexpr int kDppRowHalfMirror = 0x141, kDppRowMirror = 0x140;

// Full-mask DPP read with zero for lanes whose source is outside the row (bound_ctrl):
// with no "old" operand the compiler can fold the move into the VALU op that uses it.
template <int CTRL>
__device__ __forceinline__ float dpp_z(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}


// Lane exchanges on the VALU instead of the LDS crossbar.  xshfl<M> returns the value of
// lane (lane ^ M): DPP quad permutes for M = 1, 2, row shifts for 4 and 8 (left for lanes
// with the bit clear, right for those with it set, so the source stays in its 16-lane
// row) and the gfx950 half swaps v_permlane16_swap / v_permlane32_swap for 16 and 32.
template <int M>
__device__ __forceinline__ int xshfl_i(int v) {
    if constexpr (M == 1) {
        return __builtin_amdgcn_mov_dpp(v, kDppQuadXor1, 0xF, 0xF, true);
    } else if constexpr (M == 2) {
        return __builtin_amdgcn_mov_dpp(v, kDppQuadXor2, 0xF, 0xF, true);
    } else if constexpr (M == 4 || M == 8) {
        const int up = __builtin_amdgcn_mov_dpp(v, 0x100 + M, 0xF, 0xF, true);   // row_shl: lane + M
        const int dn = __builtin_amdgcn_mov_dpp(v, 0x110 + M, 0xF, 0xF, true);   // row_shr: lane - M
        return (threadIdx.x & M) ? dn : up;
    } else if constexpr (M == 16) {
        const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
        return (int)((threadIdx.x & 16) ? r[0] : r[1]);
    } else {
        static_assert(M == 32, "lane xor mask 1, 2, 4, 8, 16 or 32");
        const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
        return (int)((threadIdx.x & 32) ? r[0] : r[1]);
    }
}
template <int M>
__device__ __forceinline__ float xshfl(float v) {
    return __int_as_float(xshfl_i<M>(__float_as_int(v)));
}

// One pair of a reduce-scatter step over lane bit M: with a = element i and b = element
// i + half of the lane's values, a lane with bit M clear returns a + (partner's a) and a
// lane with bit M set returns b + (partner's b), the partner being lane ^ M.  DPP row
// shifts (and quad permutes) read the partner for each half in one instruction; the
// gfx950 half swaps exchange the two halves between partners in one instruction, so at
// 16 and 32 every lane just adds the pair it receives.
template <int M>
__device__ __forceinline__ float rs_pair(float a, float b) {
    if constexpr (M == 16 || M == 32) {
        const int ia = __float_as_int(a), ib = __float_as_int(b);
        const auto r = (M == 16) ? __builtin_amdgcn_permlane16_swap(ia, ib, false, false)
                                 : __builtin_amdgcn_permlane32_swap(ia, ib, false, false);
        return __int_as_float((int)r[0]) + __int_as_float((int)r[1]);
    } else if constexpr (M == 4 || M == 8) {
        const float lo = a + dpp_z<0x100 + M>(a);         // row_shl: lane + M
        const float hi = b + dpp_z<0x110 + M>(b);         // row_shr: lane - M
        return (threadIdx.x & M) ? hi : lo;
    } else {
        static_assert(M == 1 || M == 2, "lane bit 1, 2, 4, 8, 16 or 32");
        constexpr int P = M == 1 ? kDppQuadXor1 : kDppQuadXor2;
        const float lo = a + dpp_z<P>(a);
        const float hi = b + dpp_z<P>(b);
        return (threadIdx.x & M) ? hi : lo;
    }
}

// Partner exchange for butterflies: the value of lane (lane ^ P(M)), where P(M) = M except
// P(4) = 7 and P(8) = 15, the DPP half-row and row mirrors (one instruction each).  P(M)
// has bit M set and no bit above it, so a butterfly over bits taken from high to low
// (a reduce-scatter that splits on bit M) pairs lanes that agree on every bit already
// taken; and from low to high (an all-reduce) the extra low bits only move the source
// inside a group whose values are already equal.
template <int M>
__device__ __forceinline__ float xpartner(float v) {
    if constexpr (M == 4) return dpp_z<kDppRowHalfMirror>(v);
    else if constexpr (M == 8) return dpp_z<kDppRowMirror>(v);
    else return xshfl<M>(v);
}

// All-reduce over aligned groups of N lanes (N a power of two up to 64); every lane gets
// the result.  At 16 and 32 the half swap hands each lane both halves' values at once.
template <int N, int M = 1, class Op>
__device__ __forceinline__ float group_reduce(float v, Op op) {
    if constexpr (M >= N) {
        return v;
    } else if constexpr (M == 16 || M == 32) {
        const int x = __float_as_int(v);
        const auto r = (M == 16) ? __builtin_amdgcn_permlane16_swap(x, x, false, false)
                                 : __builtin_amdgcn_permlane32_swap(x, x, false, false);
        return group_reduce<N, 2 * M>(op(__int_as_float((int)r[0]), __int_as_float((int)r[1])), op);
    } else {
        return group_reduce<N, 2 * M>(op(v, xpartner<M>(v)), op);
    }
}
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    return group_reduce<N>(v, [](float a, float b) { return a + b; });
}
template <int N>
__device__ __forceinline__ float group_max(float v) {
    return group_reduce<N>(v, [](float a, float b) { return fmaxf(a, b); });
}
// Integer sums are exact in float up to 2^24, which bounds every digit sum here.
template <int N>
__device__ __forceinline__ int group_sum_i(int v) {
    return (int)group_sum<N>((float)v);
}

// Sum over aligned groups of N = 1, 2 or 4 lanes; every lane of the group gets the sum.
template <int N>
__device__ __forceinline__ float group_sum_dpp(float v) {
    if constexpr (N >= 2) v += dpp_z<kDppQuadXor1>(v);
    if constexpr (N >= 4) v += dpp_z<kDppQuadXor2>(v);
    static_assert(N <= 4, "group of at most 4 lanes");
    return v;
}

// Online softmax keeps a running reference m and weights p = exp(s - m).  The reference
// only has to bound the scores well enough that p cannot overflow, so it is raised only
// when a score exceeds it by more than this slack (natural-log units; p <= e^8).
constexpr float kRescaleSlack = 8.0f;

// Two waves that share a SIMD (wave w and w + NW/2 of one workgroup, or two workgroups
// on one CU) advance at different rates because the older one wins every tie in issue.
// The younger one gets the higher priority on every other step and the lower one in
// between, so the pair advances at about the same rate.  Wave-uniform arguments.
__device__ __forceinline__ void prio_alternate(bool younger, int step) {
    if (!younger) __builtin_amdgcn_s_setprio(1);
    else if (step % 2 == 0) __builtin_amdgcn_s_setprio(2);
    else __builtin_amdgcn_s_setprio(0);
}

// A grid of at most two workgroups per CU is dispatched one per CU first, so block b and
// block b + n_cu share a CU and the second is the younger one (it loses ties in issue to
// the first).  False when that pairing does not hold (one workgroup per CU, or more than
// two rounds), where no side is favoured.
__device__ __forceinline__ bool younger_on_cu(int n_cu) {
    return n_cu > 0 && (int)gridDim.x > n_cu && (int)gridDim.x <= 2 * n_cu && (int)blockIdx.x >= n_cu;
}

// True in every lane if any lane of the wave has pred set.
__device__ __forceinline__ bool wave_any(bool pred) { return __builtin_amdgcn_ballot_w64(pred) != 0; }

// Maximum over the 64 lanes of the wave, returned as a wave-uniform value.
__device__ __forceinline__ float wave_max_uniform(float v) {
    v = fmaxf(v, dpp_f<kDppRowShr1>(v, v));
    v = fmaxf(v, dpp_f<kDppRowShr2>(v, v));
    v = fmaxf(v, dpp_f<kDppRowShr3>(v, v));
    v = fmaxf(v, dpp_f<kDppRowShr4, 0xF, 0xE>(v, v));
    v = fmaxf(v, dpp_f<kDppRowShr8, 0xF, 0xC>(v, v));
    v = fmaxf(v, dpp_f<kDppRowBcast15, 0xA>(v, v));
    v = fmaxf(v, dpp_f<kDppRowBcast31, 0xC>(v, v));
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

}  // namespace rq
