// The group quantizer shared by the pack kernels and the W4A4 quantizers, in float64:
// offset z = largest E4M3 value <= group min; scale s = smallest E4M3 value >= 2^-9
// with z + n s >= group max (n = 2^bits - 1); code = round-half-even((x - z) / s) in
// [0, n].  n s has at most 8 significant bits and z + n s is a multiple of 2^-9 below
// 2^13, so the covering test is exact; the candidate scale from an approximate quotient
// is off by at most one grid step and is corrected by that test.  The code divides
// exactly as a float64 reference does.
#pragma once

#include "rq_fp8.hpp"

namespace rq {

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
