// Split-K flash-decoding skeleton shared by the ResidualQuant and the BF16 decode kernels.
//
// Lane mapping inside a 64-lane wave: lane = slot * LPT + chunk, where chunk selects 32
// consecutive channels (LPT = d/32 lanes per token) and slot selects one of 64/LPT tokens
// processed per pass.  Each lane keeps partial output sums for its 32 channels; at the end
// of a split they are reduced over slots (reduce-scatter), merged across the 4 waves of
// the workgroup in LDS, and written as one partial record.  The last workgroup of a
// (batch row, query head) to arrive merges all partial records (log-sum-exp), adds the
// current token and writes the output.
#pragma once

#include "rq_common.hpp"

namespace rq {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * kWave;

// One step of the reduce-scatter over lane bit M; CUR values are still live.
template <int CUR, int M, int N>
__device__ __forceinline__ void reduce_scatter_step(float (&v)[N], int lane, int& off) {
    if constexpr (M < kWave) {
        constexpr int half = CUR / 2;
        const bool upper = (lane & M) != 0;
#pragma unroll
        for (int i = 0; i < half; ++i) {
            const float send = upper ? v[i] : v[i + half];
            const float keep = upper ? v[i + half] : v[i];
            v[i] = keep + shfl_xor_f(send, M);
        }
        if (upper) off += half;
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

template <int LPT>
__device__ __forceinline__ float slot_sum(float v) {
#pragma unroll
    for (int m = LPT; m < kWave; m <<= 1) v += shfl_xor_f(v, m);
    return v;
}

template <int LPT>
__device__ __forceinline__ float slot_max(float v) {
#pragma unroll
    for (int m = LPT; m < kWave; m <<= 1) v = fmaxf(v, shfl_xor_f(v, m));
    return v;
}

template <int LPT>
__device__ __forceinline__ float chunk_sum(float v) {
#pragma unroll
    for (int m = 1; m < LPT; m <<= 1) v += shfl_xor_f(v, m);
    return v;
}

template <int NT>
__device__ __forceinline__ float block_reduce_sum(float v, float* red) {
    for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_f(v, m);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) s += red[i];
    return s;
}

template <int NT>
__device__ __forceinline__ float block_reduce_max(float v, float* red) {
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor_f(v, m));
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    float s = -INFINITY;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) s = fmaxf(s, red[i]);
    return s;
}

// LDS used by the epilogue.
template <int D>
struct EpilogueSmem {
    float acc[kWaves][2 * D];   // per wave: chunk-major [chunk][NV] values after reduce-scatter
    float m[kWaves];
    float l[kWaves];
    float red[kWaves];
    float wsplit[kMaxSplits];
    float vec[D];
    int last;
};

// Per-wave state -> partial record of this split, then arrival counting.
// NV = values per lane (32 = acc_a only, 64 = acc_a then acc_r).  Returns true in the
// workgroup that arrived last for its (row, query head).
template <int D, int NV>
__device__ __forceinline__ bool splitk_epilogue(float (&v)[NV], float m_w, float l_lane, float* rec,
                                uint32_t* counter, int n_splits, EpilogueSmem<D>& sm) {
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
    const float sc = (m_w == -INFINITY) ? 0.f : __expf(m_w - m_wg);
#pragma unroll
    for (int k = 0; k < KEEP; ++k) sm.acc[w][chunk * NV + off + k] = v[k] * sc;
    __syncthreads();
    for (int t = threadIdx.x; t < NV * LPT; t += kThreads) {
        float s = 0.f;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) s += sm.acc[i][t];
        const int c = t / NV, idx = t % NV;
        // record layout: acc_a[D], acc_r[D], m, l
        const int ch = 32 * c + (idx & 31);
        rec[(idx >= 32 ? D : 0) + ch] = s;
    }
    if (threadIdx.x == 0) {
        float l_wg = 0.f;
#pragma unroll
        for (int i = 0; i < kWaves; ++i) {
            const float si = (sm.m[i] == -INFINITY) ? 0.f : __expf(sm.m[i] - m_wg);
            l_wg += si * sm.l[i];
        }
        rec[2 * D] = m_wg;
        rec[2 * D + 1] = l_wg;
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        const uint32_t prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        sm.last = (prev == (uint32_t)(n_splits - 1)) ? 1 : 0;
    }
    __syncthreads();
    const bool last = sm.last != 0;
    if (last) __threadfence();
    return last;
}

// Merge the partial records of one (row, query head).  On return (all threads):
// sm.wsplit[s] = weight of split s, and the returned values describe the merged
// softmax: m_f (max including the current token), scale of the current token and the
// total denominator.
struct MergeOut {
    float p_cur;
    float denom;
};

template <int D>
__device__ __forceinline__ MergeOut splitk_merge_weights(const float* recs, int n_splits, float s_cur,
                                         EpilogueSmem<D>& sm) {
    const int stride = partial_stride(D);
    float mloc = -INFINITY;
    for (int s = threadIdx.x; s < n_splits; s += kThreads) {
        const float* r = recs + (int64_t)s * stride;
        if (r[2 * D + 1] > 0.f) mloc = fmaxf(mloc, r[2 * D]);
    }
    float m_f = block_reduce_max<kThreads>(mloc, sm.red);
    m_f = fmaxf(m_f, s_cur);
    float lloc = 0.f;
    for (int s = threadIdx.x; s < n_splits; s += kThreads) {
        const float* r = recs + (int64_t)s * stride;
        const float l = r[2 * D + 1];
        const float ws = (l > 0.f) ? __expf(r[2 * D] - m_f) : 0.f;
        sm.wsplit[s] = ws;
        lloc += ws * l;
    }
    const float ltot = block_reduce_sum<kThreads>(lloc, sm.red);   // contains __syncthreads
    MergeOut o;
    o.p_cur = __expf(s_cur - m_f);
    o.denom = ltot + o.p_cur;
    return o;
}

}  // namespace rq
