// rq_bf16_decode_attention: split-K flash-decoding over an uncompressed BF16 KV cache.
//
// This is the baseline the arXiv digest's throughput paragraph (section 5.3) measures
// ResidualQuant against: BF16 decode attention over each loop's own K/V.  It uses the
// same lane mapping, LDS DMA staging of the stream (non-temporal), online softmax, split-K
// merge and current-token handling as the ResidualQuant kernel, so the two differ only in
// what they read per token.
#include "rq_args.hpp"
#include "rq_splitk.hpp"
#include "rq_stage.hpp"

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
    // passes: full tiles, except that only the globally last tile can be partial
    int n_it = my_tiles * PPT;
    if (my_tiles > 0 && first + kWaves * (my_tiles - 1) == n_tiles - 1) {
        const int rem = n - (n_tiles - 1) * kTile;                 // 1..64 tokens in the last tile
        n_it -= PPT - (rem + SLOTS - 1) / SLOTS;
    }

    const int64_t base = ((int64_t)b * a.hkv + h) * a.t_cap * D;
    const uint8_t* Kb = reinterpret_cast<const uint8_t*>(a.k + base);
    const uint8_t* Vb = reinterpret_cast<const uint8_t*>(a.v + base);

    // ---- streaming: a pass (SLOTS consecutive tokens, 4 KB of K and 4 KB of V) goes
    // global -> LDS by 1 KB DMAs, each contiguous in memory and non-temporal, into a
    // 2-slot ring per wave; the lanes then read their (token, 32-channel chunk) from LDS.
    // A lane whose 16 bytes lie past t_cap reads the pass's first token instead (always
    // below ctx_len), so every DMA stays inside the row's cache and every wave issues the
    // same number of them (the explicit vmcnt counts depend on it).
    constexpr int PB = SLOTS * D * 2;                  // bytes of one pass of K (or V)
    constexpr int NC = PB / 1024;                      // 1 KB DMAs per pass of K (or V)
    constexpr int NDMA = 2 * NC;
    constexpr int NB = 2;
    static_assert(PB % 1024 == 0 && (NB - 1) * NDMA <= 63, "pass layout");
    __shared__ __attribute__((aligned(16))) uint8_t ring[kWaves][NB][2][PB];
    const uint32_t ring_base = __builtin_amdgcn_readfirstlane(lds_addr_of(&ring[w][0][0][0]));
    auto issue = [&](int it) {
        const int j0 = (first + kWaves * (it / PPT)) * kTile + (it % PPT) * SLOTS;
        const uint8_t* kp = uniform_ptr(Kb + (int64_t)j0 * (2 * D));
        const uint8_t* vp = uniform_ptr(Vb + (int64_t)j0 * (2 * D));
        const uint32_t dst = ring_base + (uint32_t)(it % NB) * 2 * PB;
#pragma unroll
        for (int m = 0; m < NC; ++m) {
            const int tok = j0 + (m * 1024 + 16 * lane) / (2 * D);
            const uint32_t voff = tok < a.t_cap ? (uint32_t)(m * 1024 + 16 * lane) : (uint32_t)((16 * lane) % (2 * D));
            dma16<true>(voff, kp, dst + m * 1024);
            dma16<true>(voff, vp, dst + PB + m * 1024);
        }
    };
    if (n_it > 0) issue(0);

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

    auto compute = [&](int it) {
        const int j = (first + kWaves * (it / PPT)) * kTile + (it % PPT) * SLOTS + slot;
        const bool valid = j < n;
        const int row = valid ? slot : 0;          // masked slots read the pass's first token
        const uint8_t* kr = &ring[w][it % NB][0][0] + row * (2 * D) + chunk * 64;
        const uint8_t* vr = &ring[w][it % NB][1][0] + row * (2 * D) + chunk * 64;
        u32x4 fk[4], fv[4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            fk[c] = reinterpret_cast<const u32x4*>(kr)[c];
            fv[c] = reinterpret_cast<const u32x4*>(vr)[c];
        }
        float part = 0.f;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const uint32_t ws[4] = {fk[c].x, fk[c].y, fk[c].z, fk[c].w};
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
            const uint32_t ws[4] = {fv[c].x, fv[c].y, fv[c].z, fv[c].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                acc[8 * c + 2 * e] += pw * bf16lo(ws[e]);
                acc[8 * c + 2 * e + 1] += pw * bf16hi(ws[e]);
            }
        }
    };

    for (int it = 0; it < n_it; ++it) {
        if (it % PPT == 0) prio_alternate(younger, it / PPT);
        if (it + 1 < n_it) {
            issue(it + 1);
            wait_vm<NDMA>();                       // pass `it` has landed, pass it + 1 in flight
        } else {
            wait_vm<0>();
        }
        compute(it);
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
