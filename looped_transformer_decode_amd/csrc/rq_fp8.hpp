// FP8 E4M3FN bytes and BF16 rounding of float64 values, for the pack kernels (and, being
// host-callable, for checking on the CPU).  OCP FP8 E4M3FN: sign, 4 exponent bits with
// bias 7, 3 mantissa bits, subnormals m * 2^-9, largest finite magnitude 448, no
// infinities (0x7F / 0xFF are NaN and are never produced here).  Exact: power-of-two
// scalings, floor/ceil and compares only.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace rq {

// value of an E4M3 byte (finite patterns; bit 7 is the sign)
__host__ __device__ __forceinline__ double e4m3_value(uint32_t b) {
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    const double mag = e == 0 ? (double)m * 0x1p-9 : ldexp((double)(8u + m), (int)e - 10);
    return (b & 0x80u) ? -mag : mag;
}

// byte of the largest grid value <= a, for 0 <= a (values above 448 give 448)
__host__ __device__ __forceinline__ uint32_t e4m3_down_byte(double a) {
    if (a >= 448.0) return 0x7Eu;
    if (a < 0x1p-6) return (uint32_t)floor(a * 512.0);          // subnormals: m * 2^-9
    const int e = ilogb(a);                                      // 2^e <= a < 2^(e+1)
    return ((uint32_t)(e + 7) << 3) | ((uint32_t)floor(ldexp(a, 3 - e)) - 8u);
}

// byte of the smallest grid value >= a, for 0 <= a (values above 448 give 448)
__host__ __device__ __forceinline__ uint32_t e4m3_up_byte(double a) {
    if (a >= 448.0) return 0x7Eu;
    if (a <= 0x1p-6) return (uint32_t)ceil(a * 512.0);           // 8 is the byte of 2^-6
    const int e = ilogb(a);
    return ((uint32_t)(e + 7) << 3) + ((uint32_t)ceil(ldexp(a, 3 - e)) - 8u);   // 8 carries
}

// byte of the largest grid value <= v; below -448 (outside the format) the offset
// saturates at -448, so a group whose minimum lies there keeps finite metadata and its
// lowest codes clamp at 0.
__host__ __device__ __forceinline__ uint32_t e4m3_floor_byte(double v) {
    if (v < -448.0) return 0xFEu;
    return v >= 0.0 ? e4m3_down_byte(v) : (0x80u | e4m3_up_byte(-v));
}

// BF16 round-to-nearest-even of a float64 value, in one rounding step.
__host__ __device__ __forceinline__ double bf16_round(double v) {
    if (v == 0.0) return 0.0;
    int e = ilogb(v);
    if (e < -126) e = -126;
    return ldexp(rint(ldexp(v, 7 - e)), e - 7);
}

}  // namespace rq
