// The group quantizer shared by the pack kernels and the W4A4 quantizers, in float64:
// offset z = largest E4M3 value <= group min; scale s = smallest E4M3 value >= 2^-9
// with z + n s >= group max (n = 2^bits - 1); code = round-half-even((x - z) / s) in
// [0, n].  n s has at most 8 significant bits and z + n s is a multiple of 2^-9 below
// 2^13, so the covering test is exact; the candidate scale from an approximate quotient
// is off by at most one grid step and is corrected by that test.  The code divides
// exactly as a float64 reference does.  The float64 lane reductions the quantizers use for
// group extremes and dot products live here too.
#pragma once

#include "rq_common.hpp"
#include "rq_fp8.hpp"

namespace rq {

// Cross-lane steps on float64 values (DPP inside a 16-lane row, lane swaps across rows).

template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    const uint64_t u = (uint64_t)__double_as_longlong(v);
    const int lo = __builtin_amdgcn_update_dpp((int)(uint32_t)u, (int)(uint32_t)u, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp((int)(uint32_t)(u >> 32), (int)(uint32_t)(u >> 32), CTRL, 0xF,
                                               0xF, false);
    return __longlong_as_double((long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo));
}

// reduction over aligned groups of NL lanes (a power of two up to 64); every lane of the
// group gets the same value (both lanes of a pair combine the same two operands)
template <int NL, int M = 1, class Op>
__device__ __forceinline__ double lanes_reduce(double v, Op op) {
    if constexpr (M >= NL) {
        return v;
    } else if constexpr (M == 16 || M == 32) {
        const uint64_t u = (uint64_t)__double_as_longlong(v);
        const int lo = (int)(uint32_t)u, hi = (int)(uint32_t)(u >> 32);
        const auto rl = (M == 16) ? __builtin_amdgcn_permlane16_swap(lo, lo, false, false)
                                  : __builtin_amdgcn_permlane32_swap(lo, lo, false, false);
        const auto rh = (M == 16) ? __builtin_amdgcn_permlane16_swap(hi, hi, false, false)
                                  : __builtin_amdgcn_permlane32_swap(hi, hi, false, false);
        const double p = __longlong_as_double((long long)(((uint64_t)(uint32_t)rh[0] << 32) | (uint32_t)rl[0]));
        const double q = __longlong_as_double((long long)(((uint64_t)(uint32_t)rh[1] << 32) | (uint32_t)rl[1]));
        return lanes_reduce<NL, 2 * M>(op(p, q), op);
    } else {
        constexpr int CTRL = M == 1 ? kDppQuadXor1 : M == 2 ? kDppQuadXor2 : M == 4 ? kDppRowHalfMirror : kDppRowMirror;
        return lanes_reduce<NL, 2 * M>(op(v, dpp_d<CTRL>(v)), op);
    }
}

struct QOut {
    uint32_t code, zb, sb;
    double z, s;
};

// offset and scale of a group with minimum lo and maximum hi (code left unset)
__device__ __forceinline__ QOut group_params(double lo, double hi, int bits) {
    const double n = (double)((1 << bits) - 1);
    QOut o;
    o.zb = e4m3_floor_byte(lo);
    o.z = e4m3_value(o.zb);
    const double need = fmin(fmax((hi - o.z) * (bits == 4 ? 1.0 / 15.0 : 1.0 / 3.0), 0x1p-9), 448.0);
    uint32_t sb = e4m3_up_byte(need);
    if (sb > 1u && o.z + n * e4m3_value(sb - 1u) >= hi) --sb;
    if (sb < 0x7Eu && o.z + n * e4m3_value(sb) < hi) ++sb;
    o.sb = sb;
    o.s = e4m3_value(sb);
    o.code = 0;
    return o;
}

__device__ __forceinline__ uint32_t group_code(double x, const QOut& o, int bits) {
    const double t = rint((x - o.z) / o.s);
    return (uint32_t)fmin(fmax(t, 0.0), (double)((1 << bits) - 1));
}

}  // namespace rq
