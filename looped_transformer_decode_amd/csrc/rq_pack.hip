// rq_pack: quantize finished tokens of one anchor group into the packed cache.
//
// ResidualQuant explainer, paragraph on the master print: the last loop is the INT4
// anchor, each earlier loop stores residual = KV(loop) - c * anchor with a per-vector
// least-squares c, rotated before 2-bit quantization; paragraph "Which print is the
// master": the current token stays BF16 until its final loop and is quantized only
// then (this kernel is that drain step).  Group quantizer with FP8 offset and scale:
// "Worked example" of the same page and the arXiv digest's Figure 1 caption (g = 32).
//
// All arithmetic is float64 so that the integer decisions (codes, FP8 metadata, BF16
// rounding of c) are taken exactly like a float64 reference would take them.
#include "rq_args.hpp"

namespace rq {


// ---- FP8 E4M3FN on the float64 grid (exact: every step is a power-of-two scaling,
// floor/ceil or a comparison)

// largest grid value <= a, for 0 <= a (values above 448 give 448)
__device__ inline double e4m3_down_mag(double a) {
    if (a >= 448.0) return 448.0;
    if (a < 0x1p-6) return floor(a * 512.0) * 0x1p-9;        // subnormal spacing 2^-9
    const int e = ilogb(a);                                    // 2^e <= a < 2^(e+1)
    const double q = ldexp(1.0, e - 3);                        // 3 mantissa bits
    return floor(a / q) * q;
}

// smallest grid value >= a, for 0 <= a <= 448
__device__ inline double e4m3_up_mag(double a) {
    if (a <= 0x1p-6) return ceil(a * 512.0) * 0x1p-9;
    const int e = ilogb(a);
    const double q = ldexp(1.0, e - 3);
    return ceil(a / q) * q;
}

__device__ inline double e4m3_floor(double v) {
    return v >= 0.0 ? e4m3_down_mag(v) : -e4m3_up_mag(fmin(-v, 448.0));
}

__device__ inline uint32_t e4m3_bits(double v) {          // v on the grid
    const uint32_t sign = v < 0.0 ? 0x80u : 0u;
    const double a = fabs(v);
    if (a == 0.0) return 0u;
    if (a < 0x1p-6) return sign | (uint32_t)(a * 512.0);
    const int e = ilogb(a);
    const uint32_t man = (uint32_t)(a * ldexp(1.0, 3 - e)) - 8u;
    return sign | ((uint32_t)(e + 7) << 3) | man;
}

__device__ inline double e4m3_pos_value(uint32_t b) {     // 0 < b <= 0x7E
    const uint32_t e = (b >> 3) & 15u, m = b & 7u;
    return e == 0 ? m * 0x1p-9 : ldexp(1.0 + m * 0.125, (int)e - 7);
}

// BF16 round-to-nearest-even of a float64 value, in one rounding step.
__device__ inline double bf16_round(double v) {
    if (v == 0.0) return 0.0;
    int e = ilogb(v);
    if (e < -126) e = -126;
    const double q = ldexp(1.0, e - 7);
    return rint(v / q) * q;
}

struct QOut {
    uint32_t code;
    double z, s;
    uint32_t zb, sb;
};

// Group quantizer: every lane holds one channel; groups are `g` consecutive lanes.
__device__ inline QOut quantize_lane(double x, int bits, int g) {
    double lo = x, hi = x;
    for (int off = g >> 1; off >= 1; off >>= 1) {
        lo = fmin(lo, shfl_xor_d(lo, off));
        hi = fmax(hi, shfl_xor_d(hi, off));
    }
    QOut o;
    const double n = (double)((1 << bits) - 1);
    o.z = e4m3_floor(lo);
    // smallest scale s >= 2^-9 on the grid with z + n*s >= hi (the sum is exact)
    double need = (hi - o.z) / n;
    if (need < 0x1p-9) need = 0x1p-9;
    uint32_t sb = e4m3_bits(e4m3_up_mag(fmin(need, 448.0)));
    while (sb > 1u && o.z + n * e4m3_pos_value(sb - 1u) >= hi) --sb;
    while (sb < 0x7Eu && o.z + n * e4m3_pos_value(sb) < hi) ++sb;
    o.s = e4m3_pos_value(sb);
    o.sb = sb;
    o.zb = e4m3_bits(o.z);
    double t = rint((x - o.z) / o.s);
    t = fmin(fmax(t, 0.0), n);
    o.code = (uint32_t)t;
    return o;
}

// Sums over the D threads of the workgroup of N values per thread (float64).
template <int D, int N>
__device__ inline void block_sum_vec(double (&v)[N], double (*red)[N]) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1)
#pragma unroll
        for (int k = 0; k < N; ++k) v[k] += shfl_xor_d(v[k], off);
    constexpr int W = D / 64;
    if constexpr (W > 1) {
        const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
        __syncthreads();
        if (lane == 0)
#pragma unroll
            for (int k = 0; k < N; ++k) red[w][k] = v[k];
        __syncthreads();
#pragma unroll
        for (int k = 0; k < N; ++k) {
            double s = 0.0;
#pragma unroll
            for (int i = 0; i < W; ++i) s += red[i][k];
            v[k] = s;
        }
    }
}

// Pack `bits`-wide codes of consecutive lanes into 32-bit words and store them.
__device__ inline void store_codes(uint8_t* row, uint32_t code, int bits) {
    const int per = 32 / bits;
    const int i = threadIdx.x;
    uint32_t v = code << ((i % per) * bits);
    for (int off = 1; off < per; off <<= 1) v |= (uint32_t)__shfl_xor((int)v, off, kWave);
    if (i % per == 0) reinterpret_cast<uint32_t*>(row)[i / per] = v;
}

__device__ inline void store_meta(uint8_t* row, const QOut& q, int g) {
    const int i = threadIdx.x;
    if (i % g == 0) reinterpret_cast<uint16_t*>(row)[i / g] = (uint16_t)(q.zb | (q.sb << 8));
}

__device__ inline void store_c(uint8_t* cblk, int jj, double c) {
    if (threadIdx.x == 0) {
        const uint32_t cb = __float_as_uint((float)c) >> 16;    // c is a BF16 value
        reinterpret_cast<uint16_t*>(cblk)[jj] = (uint16_t)cb;
    }
}

// One workgroup per (token range, batch row, KV head, K|V); thread i owns channel i and
// keeps row i of R in registers for all tokens of the range.
template <int D>
__global__ __launch_bounds__(D) void rq_pack_kernel(PackArgs a) {
    const Geom& G = a.geo;
    const int i = threadIdx.x;
    int wg = blockIdx.x;
    const int x = wg & 1;
    wg >>= 1;
    const int h = wg % G.hkv;
    wg /= G.hkv;
    const int b = wg % a.batch;
    const int t0 = (wg / a.batch) * a.tokens_per_wg;
    const int t1 = min(t0 + a.tokens_per_wg, a.n_tokens);
    const int L = G.L;
    const int loop0 = a.group_idx * L;
    const float* R = a.rot + (int64_t)(h * 2 + x) * D * D;

    __shared__ double sh_y[kMaxLoops][D];
    __shared__ double red[D / 64][kMaxLoops];

    float rrow[D];                                     // row i of R: r_i = sum_k R[i][k] y_k
    {
        const float4* rp = reinterpret_cast<const float4*>(R + (int64_t)i * D);
#pragma unroll
        for (int k4 = 0; k4 < D / 4; ++k4) {
            const float4 v = rp[k4];
            rrow[4 * k4] = v.x;
            rrow[4 * k4 + 1] = v.y;
            rrow[4 * k4 + 2] = v.z;
            rrow[4 * k4 + 3] = v.w;
        }
    }
    uint8_t* a_plane = a.cache + G.plane_offset(b, h, x, loop0 + L - 1);

    for (int t = t0; t < t1; ++t) {
        const int slot = a.pos[b] + t;
        if (slot < 0 || slot >= G.max_ctx) continue;   // same for the whole workgroup
        const int tile = slot / kTile, jj = slot % kTile;

        double xv[kMaxLoops];
        const uint16_t* src = a.pending + t * a.st[0] + b * a.st[1] + x * a.st[3] + h * a.st[4] + i;
#pragma unroll
        for (int l = 0; l < kMaxLoops; ++l)
            if (l < L) xv[l] = (double)bf16_to_f32(src[l * a.st[2]]);

        // anchor: the group's last loop
        const QOut qa = quantize_lane(xv[L - 1], G.ba, G.g);
        {
            uint8_t* p = a_plane + tile * G.a_tile;
            store_codes(p + jj * G.a_row, qa.code, G.ba);
            store_meta(p + kTile * G.a_row + jj * G.m_row, qa, G.g);
        }
        const double a_hat = qa.z + qa.code * qa.s;      // dequantized anchor (exact)

        if (!G.chained) {
            // all loops reference a_hat: one reduction for every <x_l, a> and <a, a>
            double sums[kMaxLoops];
#pragma unroll
            for (int l = 0; l < kMaxLoops; ++l) sums[l] = (l < L - 1) ? xv[l] * a_hat : 0.0;
            sums[kMaxLoops - 1] = a_hat * a_hat;
            block_sum_vec<D, kMaxLoops>(sums, red);
            const double den = sums[kMaxLoops - 1];
            double cs[kMaxLoops];
#pragma unroll
            for (int l = 0; l < kMaxLoops - 1; ++l) {
                if (l < L - 1) {
                    cs[l] = bf16_round(den > 0.0 ? sums[l] / den : 0.0);
                    sh_y[l][i] = xv[l] - cs[l] * a_hat;
                }
            }
            __syncthreads();
#pragma unroll
            for (int l = 0; l < kMaxLoops - 1; ++l) {
                if (l < L - 1) {
                    double r = 0.0;
#pragma unroll
                    for (int k = 0; k < D; ++k) r += (double)rrow[k] * sh_y[l][k];
                    const QOut qr = quantize_lane(r, G.br, G.g);
                    uint8_t* p = a.cache + G.plane_offset(b, h, x, loop0 + l) + tile * G.r_tile;
                    store_codes(p + jj * G.r_row, qr.code, G.br);
                    store_meta(p + kTile * G.r_row + jj * G.m_row, qr, G.g);
                    store_c(p + kTile * (G.r_row + G.m_row), jj, cs[l]);
                }
            }
            __syncthreads();                              // sh_y is reused by the next token
        } else {
            // loop l references the rebuilt loop l+1 (the anchor closes the chain)
            double ref = a_hat;
            for (int l = L - 2; l >= 0; --l) {
                double s2[2] = {xv[l] * ref, ref * ref};
                block_sum_vec<D, 2>(s2, reinterpret_cast<double(*)[2]>(&red[0][0]));
                const double c = bf16_round(s2[1] > 0.0 ? s2[0] / s2[1] : 0.0);
                sh_y[0][i] = xv[l] - c * ref;
                __syncthreads();
                double r = 0.0;
#pragma unroll
                for (int k = 0; k < D; ++k) r += (double)rrow[k] * sh_y[0][k];
                const QOut qr = quantize_lane(r, G.br, G.g);
                uint8_t* p = a.cache + G.plane_offset(b, h, x, loop0 + l) + tile * G.r_tile;
                store_codes(p + jj * G.r_row, qr.code, G.br);
                store_meta(p + kTile * G.r_row + jj * G.m_row, qr, G.g);
                store_c(p + kTile * (G.r_row + G.m_row), jj, c);
                // R^T r_hat: thread i takes column i of R (coalesced across threads)
                sh_y[1][i] = qr.z + qr.code * qr.s;
                __syncthreads();
                double tcol = 0.0;
#pragma unroll 16
                for (int k = 0; k < D; ++k) tcol += (double)R[(int64_t)k * D + i] * sh_y[1][k];
                ref = c * ref + tcol;
                __syncthreads();
            }
        }
    }
}

hipError_t launch_pack(const PackArgs& a, hipStream_t stream) {
    if (!a.cache || !a.pending || !a.pos || !a.rot || a.batch < 1 || a.n_tokens < 1 || a.tokens_per_wg < 1)
        return hipErrorInvalidValue;
    const int nwg = (a.n_tokens + a.tokens_per_wg - 1) / a.tokens_per_wg * a.batch * a.geo.hkv * 2;
    if (a.geo.d == 128)
        hipLaunchKernelGGL(rq_pack_kernel<128>, dim3(nwg), dim3(128), 0, stream, a);
    else
        hipLaunchKernelGGL(rq_pack_kernel<64>, dim3(nwg), dim3(64), 0, stream, a);
    return hipGetLastError();
}

}  // namespace rq
