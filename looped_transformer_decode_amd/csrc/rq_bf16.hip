// rq_bf16_decode_attention: split-K flash-decoding over an uncompressed BF16 KV cache.
//
// This is the baseline the arXiv digest's throughput paragraph (section 5.3) measures
// ResidualQuant against: BF16 decode attention over each loop's own K/V.  It uses the
// same lane mapping, online softmax, split-K merge and current-token handling as the
// ResidualQuant kernel, so the two differ only in what they read per token.
#include "rq_args.hpp"
#include "rq_splitk.hpp"

namespace rq {


template <int D, bool QBF16>
__global__ __launch_bounds__(kThreads) void rq_bf16_decode_kernel(Bf16Args a) {
    constexpr int LPT = D / 32;
    constexpr int SLOTS = kWave / LPT;
    constexpr int PPT = kTile / SLOTS;
    const int nwg = gridDim.x;
    const int lb = xcd_logical_block(blockIdx.x, nwg);
    const int split = lb % a.n_splits;
    const int bh = lb / a.n_splits;
    const int hq = bh % a.hq;
    const int b = bh / a.hq;
    const int gqa = a.hq / a.hkv;
    const int h = hq / gqa;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int chunk = lane % LPT, slot = lane / LPT;

    __shared__ float sq[D];
    __shared__ EpilogueSmem<D> sm;

    int n = a.ctx_len[b];
    n = n < 0 ? 0 : (n > a.ctx_bound ? a.ctx_bound : n);
    const int n_tiles = (n + kTile - 1) / kTile;
    const int t_begin = split * a.tiles_per_split;
    const int t_end = min(n_tiles, t_begin + a.tiles_per_split);

    for (int i = threadIdx.x; i < D; i += kThreads) {
        if constexpr (QBF16)
            sq[i] = bf16_to_f32(reinterpret_cast<const uint16_t*>(a.q)[(int64_t)bh * D + i]);
        else
            sq[i] = reinterpret_cast<const float*>(a.q)[(int64_t)bh * D + i];
    }
    __syncthreads();
    float qr[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) qr[i] = sq[32 * chunk + i];

    const int64_t base = ((int64_t)b * a.hkv + h) * a.t_cap * D;
    const uint16_t* K = a.k + base;
    const uint16_t* V = a.v + base;

    float acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = 0.f;
    float m_run = -INFINITY, l_lane = 0.f;

    for (int tile = t_begin + w; tile < t_end; tile += kWaves) {
#pragma unroll 1
        for (int p = 0; p < PPT; ++p) {
            const int j = tile * kTile + p * SLOTS + slot;
            const bool valid = j < n;
            const int jl = valid ? j : 0;             // never read past the cache for tail slots
            const uint4* kp = reinterpret_cast<const uint4*>(K + (int64_t)jl * D + 32 * chunk);
            float part = 0.f;
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
                const uint4 kw = kp[c4];
                const uint32_t ws[4] = {kw.x, kw.y, kw.z, kw.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    part += qr[8 * c4 + 2 * e] * bf16lo(ws[e]);
                    part += qr[8 * c4 + 2 * e + 1] * bf16hi(ws[e]);
                }
            }
            float score = chunk_sum<LPT>(part) * a.sm_scale;
            score = valid ? score : -INFINITY;
            const float pmax = slot_max<LPT>(score);
            if (pmax > m_run) {
                const float f = __expf(m_run - pmax);
#pragma unroll
                for (int i = 0; i < 32; ++i) acc[i] *= f;
                l_lane *= f;
                m_run = pmax;
            }
            const float pw = valid ? __expf(score - m_run) : 0.f;
            l_lane += pw;
            const uint4* vp = reinterpret_cast<const uint4*>(V + (int64_t)jl * D + 32 * chunk);
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
                const uint4 vw = vp[c4];
                const uint32_t ws[4] = {vw.x, vw.y, vw.z, vw.w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    acc[8 * c4 + 2 * e] += pw * bf16lo(ws[e]);
                    acc[8 * c4 + 2 * e + 1] += pw * bf16hi(ws[e]);
                }
            }
        }
    }

    float* recs = a.partials + (int64_t)bh * kMaxSplits * partial_stride(D);
    const bool last = splitk_epilogue<D, 32>(acc, m_run, l_lane, recs + (int64_t)split * partial_stride(D),
                                            a.counters + bh, a.n_splits, sm);
    if (!last) return;

    const uint16_t* kc = a.k_cur + ((int64_t)b * a.hkv + h) * D;
    const uint16_t* vc = a.v_cur + ((int64_t)b * a.hkv + h) * D;
    float pc = 0.f;
    for (int i = threadIdx.x; i < D; i += kThreads) pc += sq[i] * bf16_to_f32(kc[i]);
    const float s_cur = block_reduce_sum<kThreads>(pc, sm.red) * a.sm_scale;
    const MergeOut mo = splitk_merge_weights<D>(recs, a.n_splits, s_cur, sm);
    if (threadIdx.x < D) {
        const int i = threadIdx.x;
        float o = 0.f;
        for (int s = 0; s < a.n_splits; ++s) o += sm.wsplit[s] * recs[(int64_t)s * partial_stride(D) + i];
        o += mo.p_cur * bf16_to_f32(vc[i]);
        a.out[(int64_t)bh * D + i] = o / mo.denom;
        if (a.append && hq % gqa == 0 && n < a.t_cap) {
            a.k[base + (int64_t)n * D + i] = kc[i];
            a.v[base + (int64_t)n * D + i] = vc[i];
        }
    }
    if (threadIdx.x == 0) a.counters[bh] = 0u;
}

hipError_t launch_bf16(const Bf16Args& a, int d, bool qbf16, hipStream_t st) {
    const dim3 grid(a.batch * a.hq * a.n_splits);
    if (d == 128) {
        if (qbf16) hipLaunchKernelGGL((rq_bf16_decode_kernel<128, true>), grid, dim3(kThreads), 0, st, a);
        else hipLaunchKernelGGL((rq_bf16_decode_kernel<128, false>), grid, dim3(kThreads), 0, st, a);
    } else if (d == 64) {
        if (qbf16) hipLaunchKernelGGL((rq_bf16_decode_kernel<64, true>), grid, dim3(kThreads), 0, st, a);
        else hipLaunchKernelGGL((rq_bf16_decode_kernel<64, false>), grid, dim3(kThreads), 0, st, a);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace rq
