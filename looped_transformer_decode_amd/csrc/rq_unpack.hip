// rq_unpack_debug: rebuild one loop's K/V vectors from the packed cache, in float32.
//
// A checking aid for the cache layout: the decode kernel never materialises these
// vectors.  ResidualQuant explainer, paragraph on the master print: a loop's KV is
// c * anchor + residual with the residual stored in the rotated basis, so the rebuilt
// vector is c * a_hat + R^T r_hat; paragraph "Which print is the master": a chained loop
// l is rebuilt from the rebuilt loop l+1 instead of the anchor.  Dequantization of a
// group: offset z plus code times scale s ("Worked example" of the same page).
#include "rq_args.hpp"

namespace rq {

struct UnpackArgs {
    Geom geo;
    const uint8_t* cache;
    const float* rot;
    float* out;                 // [batch][hkv][2][t1 - t0][d]
    int loop, t0, t1, batch;
};

constexpr int kUnpackTokens = 8;    // token slots per workgroup

// Dequantized value of channel i of token row `jj` in a plane tile: codes of `bits`
// per channel, then the metadata rows (E4M3 offset, E4M3 scale per group).
__device__ __forceinline__ float dequant(const uint8_t* tile, int row_bytes, int bits, const Geom& G, int jj,
                                         int i) {
    const uint32_t* codes = reinterpret_cast<const uint32_t*>(tile + (int64_t)jj * row_bytes);
    const int per = 32 / bits;
    const uint32_t code = (codes[i / per] >> ((i % per) * bits)) & ((1u << bits) - 1u);
    const uint8_t* meta = tile + (int64_t)kTile * row_bytes + (int64_t)jj * G.m_row + 2 * (i / G.g);
    return e4m3_to_f32(meta[0]) + (float)code * e4m3_to_f32(meta[1]);
}

// One workgroup of d threads per (row, KV head, K|V, kUnpackTokens token slots);
// thread i owns channel i.
__global__ __launch_bounds__(128) void rq_unpack_kernel(UnpackArgs a) {
    const Geom& G = a.geo;
    const int D = G.d, L = G.L, i = threadIdx.x;
    int wg = blockIdx.x;
    const int n_chunks = (a.t1 - a.t0 + kUnpackTokens - 1) / kUnpackTokens;
    const int chunk = wg % n_chunks;
    wg /= n_chunks;
    const int x = wg % 2;
    wg /= 2;
    const int h = wg % G.hkv;
    const int b = wg / G.hkv;
    const int grp = a.loop / L, lloc = a.loop % L;
    const int aloop = grp * L + L - 1;
    const float* R = a.rot + (int64_t)(2 * h + x) * D * D;
    __shared__ float r_hat[128];

    const int nt = a.t1 - a.t0;
    for (int k = 0; k < kUnpackTokens; ++k) {
        const int t = chunk * kUnpackTokens + k;
        if (t >= nt) break;                            // same for the whole workgroup
        const int slot = a.t0 + t, tile = slot / kTile, jj = slot % kTile;
        float v = dequant(a.cache + G.tile_offset(b, h, x, aloop, tile), G.a_row, G.ba, G, jj, i);
        // residual loops from the one nearest the anchor down to `lloc` (shared: only `lloc`;
        // the anchor loop has none)
        const int first = lloc == L - 1 ? -1 : (G.chained ? L - 2 : lloc);
        for (int l = first; l >= lloc; --l) {
            const uint8_t* rt = a.cache + G.tile_offset(b, h, x, grp * L + l, tile);
            const float rh = dequant(rt, G.rrow(l), G.rbits(l), G, jj, i);
            const uint16_t cb = *reinterpret_cast<const uint16_t*>(rt + (int64_t)kTile * (G.rrow(l) + G.m_row) + 2 * jj);
            __syncthreads();                           // r_hat is reused
            r_hat[i] = rh;
            __syncthreads();
            float rt_r = 0.f;                          // (R^T r_hat)_i = sum_k R[k][i] r_hat[k]
            for (int kk = 0; kk < D; ++kk) rt_r += R[(int64_t)kk * D + i] * r_hat[kk];
            v = bf16_to_f32(cb) * v + rt_r;
        }
        a.out[((((int64_t)b * G.hkv + h) * 2 + x) * nt + t) * D + i] = v;
    }
}

}  // namespace rq

using namespace rq;

extern "C" rq_status rq_unpack_debug(const rq_config* cfg, const void* cache, int32_t loop, const float* rot,
                                     int32_t t0, int32_t t1, int32_t batch, float* out, hipStream_t stream) {
    Geom g;
    if (cfg == nullptr) return RQ_ERR_INVALID_ARG;
    if (!make_geom(cfg, &g)) return RQ_ERR_UNSUPPORTED;
    if (!cache || !rot || !out) return RQ_ERR_INVALID_ARG;
    if (batch < 1 || batch > g.max_batch) return RQ_ERR_INVALID_ARG;
    if (loop < 0 || loop >= g.L * g.n_groups) return RQ_ERR_INVALID_ARG;
    if (t0 < 0 || t1 <= t0 || t1 > g.max_ctx) return RQ_ERR_INVALID_ARG;
    if ((reinterpret_cast<uintptr_t>(cache) & 15u) || (reinterpret_cast<uintptr_t>(rot) & 15u) ||
        (reinterpret_cast<uintptr_t>(out) & 15u))
        return RQ_ERR_MISALIGNED;
    const int64_t n_chunks = (t1 - t0 + kUnpackTokens - 1) / kUnpackTokens;
    const int64_t nwg = n_chunks * batch * g.hkv * 2;
    if (nwg > 0x7FFFFFFFLL) return RQ_ERR_INVALID_ARG;
    UnpackArgs a;
    a.geo = g;
    a.cache = static_cast<const uint8_t*>(cache);
    a.rot = rot;
    a.out = out;
    a.loop = loop;
    a.t0 = t0;
    a.t1 = t1;
    a.batch = batch;
    hipLaunchKernelGGL(rq_unpack_kernel, dim3((unsigned)nwg), dim3(g.d), 0, stream, a);
    return hipGetLastError() == hipSuccess ? RQ_OK : RQ_ERR_HIP;
}
