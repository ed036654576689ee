// Split-K merge of a whole query group: the last workgroup of a (batch row, KV head) merges
// the split records of its G query heads at once (used by the grouped-query decode kernels).
#pragma once

#include "rq_args.hpp"
#include "rq_splitk.hpp"

namespace rq {

// Merge of the split records of the G query heads bh0 .. bh0+G-1 (one KV head) by the last
// workgroup, all heads at once: NT/G threads per head, thread i of a head owns channel i.
// Same arithmetic as the one-head merge (splitk_merge_last); R_V is read once for the group.
template <int D, int NT, int G, bool RES>
__device__ __forceinline__ void merge_group(const MergeArgs& g, int bh0, const float (*sq)[D], float* scr) {
    constexpr int TPH = NT / G;                           // threads per head (128 or 256)
    constexpr int PS = 2 * D + 4;
    static_assert(TPH >= D && TPH % kWave == 0, "one thread per channel");
    const int tid = threadIdx.x, q = tid / TPH, i = tid % TPH;
    const int lane = tid & 63;
    const int bh = bh0 + q;
    const int hq = bh % g.hq, b = bh / g.hq, h = hq / G;
    const int S = g.n_splits;
    const float* recs = g.partials + (int64_t)bh * g.rec_splits * PS;
    float* s_red = scr;                                   // [NT / 64]
    float* s_w = s_red + NT / kWave;                      // [G][kMaxSplits]
    float* s_sc = s_w + G * kMaxSplits;                   // [G][4]: m, l_tot, p_cur
    float* s_r = s_sc + 4 * G;                            // [G][D] merged residual parts
    float* s_p = s_r + G * D;                             // [4][G][D] partial R_V^T products
    const bool ch = i < D;
    const int64_t kvo = ((int64_t)b * g.hkv + h) * D;
    uint32_t kc = 0, vc = 0;
    if (ch) {
        kc = g.k_cur[kvo + i];
        vc = g.v_cur[kvo + i];
    }
    float ms = -INFINITY, ls = 0.f;
    if (i < S) {
        ms = ld_agent(recs + (int64_t)i * PS + 2 * D);
        ls = ld_agent(recs + (int64_t)i * PS + 2 * D + 1);
    }
    constexpr int CH = 8;
    float pa[CH], pr[CH];
    auto load_chunk = [&](int s0) {
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            const bool ok = ch && s0 + k < S;
            pa[k] = ok ? ld_agent(recs + (int64_t)(s0 + k) * PS + i) : 0.f;
            pr[k] = (ok && RES) ? ld_agent(recs + (int64_t)(s0 + k) * PS + D + i) : 0.f;
        }
    };
    load_chunk(0);
    // R_V^T: thread (q, i) takes rows [32 q', 32 q' + 32) of column i for every head, q' = q
    // for G = 4 (rows [64 q', ...) for G = 2)
    constexpr int RR = D / G;
    float rv[RES ? RR : 1];
    if constexpr (RES) {
        if (ch) {
            const float* Rv = g.rot + (int64_t)(2 * h + 1) * D * D + (int64_t)(q * RR) * D + i;
#pragma unroll
            for (int k = 0; k < RR; ++k) rv[k] = Rv[(int64_t)k * D];
        }
    }
    float qk = ch ? sq[q][i] * bf16_to_f32(kc) : 0.f;
    qk = wave_sum<kWave>(qk);
    if (lane == 0) s_red[tid / kWave] = qk;
    __syncthreads();
    if (i < kWave) {                                      // first wave of each head
        float s_cur = 0.f;
#pragma unroll
        for (int k = 0; k < TPH / kWave; ++k) s_cur += s_red[q * (TPH / kWave) + k];
        s_cur *= g.sm_scale;
        const float mx = group_max<kWave>((ls > 0.f) ? ms : -INFINITY);
        const float m_f = fmaxf(mx, s_cur);
        const float ws = (ls > 0.f) ? __expf(ms - m_f) : 0.f;
        s_w[q * kMaxSplits + i] = ws;
        const float lt = wave_sum<kWave>(ws * ls);
        if (i == 0) {
            s_sc[4 * q] = m_f;
            s_sc[4 * q + 1] = lt;
            s_sc[4 * q + 2] = __expf(s_cur - m_f);
        }
    }
    __syncthreads();
    float acc_a = 0.f, acc_r = 0.f;
    for (int s0 = 0; s0 < S; s0 += CH) {
        if (s0 > 0) load_chunk(s0);
#pragma unroll
        for (int k = 0; k < CH; ++k) {
            if (s0 + k < S) {
                acc_a += s_w[q * kMaxSplits + s0 + k] * pa[k];
                acc_r += s_w[q * kMaxSplits + s0 + k] * pr[k];
            }
        }
    }
    float o_r = 0.f;
    if constexpr (RES) {
        if (ch) s_r[q * D + i] = acc_r;
        __syncthreads();
        if (ch) {
#pragma unroll
            for (int qq = 0; qq < G; ++qq) {
                float t = 0.f;
#pragma unroll
                for (int k = 0; k < RR; ++k) t += rv[k] * s_r[qq * D + q * RR + k];
                s_p[(q * G + qq) * D + i] = t;
            }
        }
        __syncthreads();
        if (ch) {
#pragma unroll
            for (int p = 0; p < G; ++p) o_r += s_p[(p * G + q) * D + i];
        }
    }
    if (ch) {
        const float p_cur = s_sc[4 * q + 2];
        g.out[(int64_t)bh * D + i] = (acc_a + o_r + p_cur * bf16_to_f32(vc)) / (s_sc[4 * q + 1] + p_cur);
        if (q == 0) {
            if (g.pending != nullptr) {
                uint16_t* pd = g.pending + (((int64_t)b * g.L + g.lloc) * 2 * g.hkv + h) * D + i;
                pd[0] = (uint16_t)kc;
                pd[(int64_t)g.hkv * D] = (uint16_t)vc;
            }
            if (g.k_app != nullptr) {                     // BF16 baseline: append at slot ctx_len[b]
                int n = g.ctx_len[b];
                n = n < 0 ? 0 : (n > g.ctx_bound ? g.ctx_bound : n);
                if (n < g.t_cap) {
                    const int64_t off = (((int64_t)b * g.hkv + h) * g.t_cap + n) * D + i;
                    g.k_app[off] = (uint16_t)kc;
                    g.v_app[off] = (uint16_t)vc;
                }
            }
        }
    }
}


}  // namespace rq
