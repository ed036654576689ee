// Split-K flash-decoding skeleton shared by the ResidualQuant and the BF16 decode kernels.
//
// Lane mapping inside a 64-lane wave: lane = slot * LPT + chunk, where chunk selects 32
// consecutive channels (LPT = d/32 lanes per token) and slot selects one of 64/LPT tokens
// processed per pass.  Each lane keeps partial output sums for its 32 channels; at the end
// of a split they are reduced over slots (reduce-scatter) and merged across the waves of
// the workgroup in LDS.  Each workgroup then publishes one record per split (unnormalised
// output o, running max m, denominator l) and counts its arrival; the last workgroup of a
// (batch row, query head) merges the records, adds the current token and writes the output.
#pragma once

#include "rq_args.hpp"

namespace rq {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;

// One step of the reduce-scatter over lane bit M; CUR values are still live.
template <int CUR, int M, int N>
__device__ __forceinline__ void reduce_scatter_step(float (&v)[N], int lane, int& off) {
    if constexpr (M < kWave) {
        constexpr int half = CUR / 2;
#pragma unroll
        for (int i = 0; i < half; ++i) v[i] = rs_pair<M>(v[i], v[i + half]);
        if (lane & M) off += half;
        reduce_scatter_step<half, 2 * M, N>(v, lane, off);
    }
}

// Reduce-scatter over the slot bits of the lane index.  On return lane holds in
// v[0 .. N*LPT/64) the slot-sums of the values with indices [off, off + N*LPT/64).
template <int N, int LPT>
__device__ __forceinline__ int slot_reduce_scatter(float (&v)[N], int lane) {
    int off = 0;
    reduce_scatter_step<N, LPT, N>(v, lane, off);
    return off;
}

template <int LPT, int M = LPT>
__device__ __forceinline__ float slot_sum(float v) {
    if constexpr (M < kWave) return slot_sum<LPT, 2 * M>(v + xshfl<M>(v));
    else return v;
}

// LDS of the split epilogue.
template <int D>
struct SplitSmem {
    float acc[kWaves][2 * D];   // per wave: [chunk][NV] values after the reduce-scatter
    float sum[2 * D];           // merged: acc_a[D], acc_r[D]
    float m[kWaves];
    float l[kWaves];
};

// Merge the per-wave states of the workgroup.  On return (after a barrier) sm.sum holds
// the anchor part in [0, D) and, for NV = 64, the residual part in [D, 2D), all scaled to
// the workgroup maximum; the returned pair is (m_wg, l_wg).
template <int D, int NV>
__device__ __forceinline__ float2 splitk_merge_waves(float (&v)[NV], float m_w, float l_lane,
                                                     SplitSmem<D>& sm) {
    constexpr int LPT = D / 32;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int chunk = lane % LPT;
    const float l_w = slot_sum<LPT>(l_lane);
    const int off = slot_reduce_scatter<NV, LPT>(v, lane);
    constexpr int KEEP = NV * LPT / kWave;
    if (lane == 0) {
        sm.m[w] = m_w;
        sm.l[w] = l_w;
    }
    __syncthreads();
    float m_wg = -INFINITY;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) m_wg = fmaxf(m_wg, sm.m[i]);
    float sc[kWaves], l_wg = 0.f;
#pragma unroll
    for (int i = 0; i < kWaves; ++i) {
        sc[i] = (sm.m[i] == -INFINITY) ? 0.f : __expf(sm.m[i] - m_wg);
        l_wg += sc[i] * sm.l[i];
    }
#pragma unroll
    for (int k = 0; k < KEEP; ++k) sm.acc[w][chunk * NV + off + k] = v[k] * sc[w];
    __syncthreads();
    for (int t = threadIdx.x; t < NV * LPT; t += kThreads) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) s += sm.acc[i][t];
        const int c = t / NV, idx = t % NV;
        sm.sum[(idx >= 32 ? D : 0) + 32 * c + (idx & 31)] = s;
    }
    __syncthreads();
    return make_float2(m_wg, l_wg);
}

// ---- publishing split records and the merge by the last workgroup
//
// Records and arrival counters are accessed with relaxed agent-scope atomic loads, stores
// and adds, each of which is coherent across the XCDs by itself, so no L2 writeback or
// invalidate is needed.  Every thread waits for its own record stores (vmcnt) before the
// barrier that precedes the arrival count; the workgroup that brings the count to
// n_splits reads the records only after that, and puts the counter back to zero.

__device__ __forceinline__ void st_agent(float* p, float v) {
    __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float* p) {
    return __uint_as_float(__hip_atomic_load(const_cast<uint32_t*>(reinterpret_cast<const uint32_t*>(p)),
                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

template <int N>
__device__ __forceinline__ float wave_sum(float v) {
    return group_sum<N>(v);
}

// Store this split's record (sum: LDS values acc_a[D], then acc_r[D] when RES; ml = (m, l)).
template <int D, bool RES, int NT = kThreads>
__device__ __forceinline__ void splitk_publish(const MergeArgs& g, int bh, int split, const float* sum, float2 ml) {
    constexpr int NVAL = RES ? 2 * D : D;
    constexpr int PS = 2 * D + 4;
    float* rec = g.partials + ((int64_t)bh * g.rec_splits + split) * PS;
    for (int t = threadIdx.x; t < NVAL; t += NT) st_agent(rec + t, sum[t]);
    if (threadIdx.x == 0) {
        st_agent(rec + 2 * D, ml.x);
        st_agent(rec + 2 * D + 1, ml.y);
    }
}

// After every thread's records are stored, count this workgroup's arrival on counter
// `slot`.  Returns true (in every thread) for the workgroup that arrives last; it also puts
// the counter back to zero.
__device__ __forceinline__ bool splitk_arrive(const MergeArgs& g, int slot) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __shared__ int s_last;
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t old = __hip_atomic_fetch_add(g.arrivals + slot, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int last = old == (uint32_t)(g.n_splits - 1);
        if (last) __hip_atomic_store(g.arrivals + slot, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = last;
    }
    __syncthreads();
    return s_last != 0;
}

// Merge of the records of (batch row, query head) bh by the last workgroup:
//   out = (sum_s w_s acc_a_s + R_V^T sum_s w_s acc_r_s + p_cur v_cur) / (sum_s w_s l_s + p_cur)
// with w_s = exp(m_s - m), p_cur = exp(s_cur - m), m = max(max_s m_s, s_cur); the current
// token goes into the pending buffer (or the BF16 cache) for the first query head of its
// KV head.  qf: LDS float32 query; scr: LDS scratch of at least NT/64 + kMaxSplits + 4 + D +
// NT floats (NT: threads of the workgroup).
template <int D, bool RES, int NT = kThreads>
__device__ __forceinline__ void splitk_merge_last(const MergeArgs& g, int bh, const float* qf, float* scr) {
    constexpr int NW = NT / kWave;
    constexpr int NVAL = RES ? 2 * D : D;
    constexpr int PS = 2 * D + 4;
    static_assert(kMaxSplits <= kWave, "one lane per split record");
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    const float* recs = g.partials + (int64_t)bh * g.rec_splits * PS;
    const int S = g.n_splits;
    const int hq = bh % g.hq, b = bh / g.hq;
    const int gqa = g.hq / g.hkv, h = hq / gqa;
    float* s_red = scr;                 // [NW]
    float* s_w = scr + NW;              // [kMaxSplits]
    float* s_sc = s_w + kMaxSplits;     // m, l_tot, p_cur
    float* s_r = s_sc + 4;              // [D] merged residual part
    float* s_p = s_r + D;               // [NT / D][D] partial R_V^T products
    // every load that does not depend on the merge weights goes out first
    const int64_t kvo = ((int64_t)b * g.hkv + h) * D;
    uint32_t kc = 0, vc = 0;
    if (tid < D) {
        kc = g.k_cur[kvo + tid];
        vc = g.v_cur[kvo + tid];
    }
    float ms = -INFINITY, ls = 0.f;
    if (tid < S) {
        ms = ld_agent(recs + (int64_t)tid * PS + 2 * D);
        ls = ld_agent(recs + (int64_t)tid * PS + 2 * D + 1);
    }
    constexpr int CH = 8;
    float pv[CH];
    auto load_chunk = [&](int s0) {
#pragma unroll
        for (int k = 0; k < CH; ++k)
            pv[k] = (tid < NVAL && s0 + k < S) ? ld_agent(recs + (int64_t)(s0 + k) * PS + tid) : 0.f;
    };
    load_chunk(0);
    constexpr int RP = NT / D;                 // parts of the R_V^T product
    constexpr int RROWS = D / RP;
    float rv[RES ? RROWS : 1];
    if constexpr (RES) {
        // column tid % D of R_V, rows of part tid / D: coalesced across the threads
        const float* Rv = g.rot + (int64_t)(2 * h + 1) * D * D + (int64_t)(tid / D) * RROWS * D + tid % D;
#pragma unroll
        for (int k = 0; k < RROWS; ++k) rv[k] = Rv[(int64_t)k * D];
    }
    // score of the current token
    float qk = tid < D ? qf[tid] * bf16_to_f32(kc) : 0.f;
    qk = wave_sum<kWave>(qk);
    if (lane == 0) s_red[w] = qk;
    __syncthreads();
    if (w == 0) {
        float s_cur = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i) s_cur += s_red[i];
        s_cur *= g.sm_scale;
        const float mx = group_max<kWave>((ls > 0.f) ? ms : -INFINITY);
        const float m_f = fmaxf(mx, s_cur);
        const float ws = (ls > 0.f) ? __expf(ms - m_f) : 0.f;
        if (lane < kMaxSplits) s_w[lane] = ws;
        const float lt = wave_sum<kWave>(ws * ls);
        if (lane == 0) {
            s_sc[0] = m_f;
            s_sc[1] = lt;
            s_sc[2] = __expf(s_cur - m_f);
        }
    }
    __syncthreads();
    float acc = 0.f;
    for (int s0 = 0; s0 < S; s0 += CH) {
        if (s0 > 0) load_chunk(s0);
#pragma unroll
        for (int k = 0; k < CH; ++k)
            if (s0 + k < S) acc += s_w[s0 + k] * pv[k];
    }
    float o = 0.f;
    if constexpr (RES) {
        if (tid >= D && tid < 2 * D) s_r[tid - D] = acc;
        __syncthreads();
        float pr = 0.f;
        const int r0 = (tid / D) * RROWS;
#pragma unroll
        for (int k = 0; k < RROWS; ++k) pr += rv[k] * s_r[r0 + k];
        s_p[tid] = pr;
        __syncthreads();
        if (tid < D) {
#pragma unroll
            for (int p = 0; p < RP; ++p) o += s_p[p * D + tid];
        }
    }
    if (tid < D) {
        const float p_cur = s_sc[2];
        o = (acc + o + p_cur * bf16_to_f32(vc)) / (s_sc[1] + p_cur);
        g.out[(int64_t)bh * D + tid] = o;
        if (hq % gqa == 0) {
            if (g.pending != nullptr) {
                uint16_t* pd = g.pending + (((int64_t)b * g.L + g.lloc) * 2 * g.hkv + h) * D + tid;
                pd[0] = (uint16_t)kc;
                pd[(int64_t)g.hkv * D] = (uint16_t)vc;
            }
            if (g.k_app != nullptr) {
                int n = g.ctx_len[b];
                n = n < 0 ? 0 : (n > g.ctx_bound ? g.ctx_bound : n);
                if (n < g.t_cap) {
                    const int64_t off = (((int64_t)b * g.hkv + h) * g.t_cap + n) * D + tid;
                    g.k_app[off] = (uint16_t)kc;
                    g.v_app[off] = (uint16_t)vc;
                }
            }
        }
    }
}

// One query head per workgroup: publish, count, and merge if last.
template <int D, bool RES>
__device__ __forceinline__ void splitk_finish(const MergeArgs& g, int bh, int split, const float* sum, float2 ml,
                                              const float* qf, SplitSmem<D>& sm) {
    static_assert(kWaves + kMaxSplits + 4 + D + kThreads <= kWaves * 2 * D, "merge scratch fits SplitSmem::acc");
    splitk_publish<D, RES>(g, bh, split, sum, ml);
    if (!splitk_arrive(g, bh)) return;
    splitk_merge_last<D, RES>(g, bh, qf, &sm.acc[0][0]);
}

}  // namespace rq
