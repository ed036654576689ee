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
    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int split = lb % a.n_splits;
    const int bh = lb / a.n_splits;
    const int hq = bh % a.hq;
    const int b = bh / a.hq;
    const int h = hq / (a.hq / a.hkv);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int chunk = lane % LPT, slot = lane / LPT;
    const bool younger = younger_on_cu(a.n_cu);
    if (younger) __builtin_amdgcn_s_setprio(2);
    else __builtin_amdgcn_s_setprio(1);

    __shared__ float sq[D];
    __shared__ SplitSmem<D> sm;

    int n = a.ctx_len[b];
    n = n < 0 ? 0 : (n > a.ctx_bound ? a.ctx_bound : n);
    const int n_tiles = (n + kTile - 1) / kTile;
    const int t_begin = split * a.tiles_per_split;
    const int t_end = min(n_tiles, t_begin + a.tiles_per_split);
    const int first = t_begin + w;
    const int my_tiles = first < t_end ? (t_end - first + kWaves - 1) / kWaves : 0;
    const int n_it = my_tiles * PPT;

    const int64_t base = ((int64_t)b * a.hkv + h) * a.t_cap * D;
    const uint16_t* K = a.k + base;
    const uint16_t* V = a.v + base;

    struct F { u32x4 k[4], v[4]; };
    auto load = [&](F& f, int it) {
        const int j = (first + kWaves * (it / PPT)) * kTile + (it % PPT) * SLOTS + slot;
        const int jl = j < n ? j : 0;             // tail slots of the last tile read token 0
        const u32x4* kp = reinterpret_cast<const u32x4*>(K + (int64_t)jl * D + 32 * chunk);
        const u32x4* vp = reinterpret_cast<const u32x4*>(V + (int64_t)jl * D + 32 * chunk);
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            f.k[c] = kp[c];
            f.v[c] = vp[c];
        }
    };
    F fa, fb;
    if (n_it > 0) load(fa, 0);

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

    float acc[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) acc[i] = 0.f;
    float m_run = -INFINITY, l_lane = 0.f;

    auto compute = [&](const F& f, int it) {
        const int j = (first + kWaves * (it / PPT)) * kTile + (it % PPT) * SLOTS + slot;
        const bool valid = j < n;
        float part = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t ws[4] = {f.k[c].x, f.k[c].y, f.k[c].z, f.k[c].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                part += qr[8 * c + 2 * e] * bf16lo(ws[e]);
                part += qr[8 * c + 2 * e + 1] * bf16hi(ws[e]);
            }
        }
        float score = group_sum_dpp<LPT>(part) * a.sm_scale;
        score = valid ? score : -INFINITY;
        if (wave_any(score > m_run + kRescaleSlack)) {      // rare: raise the reference
            const float m_new = wave_max_uniform(score);
            const float fs = __expf(m_run - m_new);
#pragma unroll
            for (int i = 0; i < 32; ++i) acc[i] *= fs;
            l_lane *= fs;
            m_run = m_new;
        }
        const float pw = valid ? __expf(score - m_run) : 0.f;
        l_lane += pw;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t ws[4] = {f.v[c].x, f.v[c].y, f.v[c].z, f.v[c].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[8 * c + 2 * e] += pw * bf16lo(ws[e]);
                acc[8 * c + 2 * e + 1] += pw * bf16hi(ws[e]);
            }
        }
    };

    for (int it = 0; it < n_it; it += 2) {
        if (it % PPT == 0) prio_alternate(younger, it / PPT);
        if (it + 1 < n_it) load(fb, it + 1);
        compute(fa, it);
        if (it + 1 < n_it) {
            if (it + 2 < n_it) load(fa, it + 2);
            compute(fb, it + 1);
        }
    }

    __builtin_amdgcn_s_setprio(3);
    const float2 ml = splitk_merge_waves<D, 32>(acc, m_run, l_lane, sm);
    splitk_finish<D, false>(a.mg, bh, split, sm.sum, ml, sq, sm);
}

hipError_t launch_bf16(const Bf16Args& a, int d, bool qbf16, hipStream_t st) {
    if (!a.k || !a.v || !a.q || !a.ctx_len || !a.mg.partials || !a.mg.arrivals || !a.mg.k_cur || !a.mg.v_cur ||
        !a.mg.out || a.batch < 1 || a.n_splits < 1 || a.n_splits > kMaxSplits || a.mg.n_splits != a.n_splits ||
        a.t_cap < 1)
        return hipErrorInvalidValue;
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
