// Split-K flash-decoding skeleton shared by the ResidualQuant and the BF16 decode kernels.
//
// Lane mapping inside a 64-lane wave: lane = slot * LPT + chunk, where chunk selects 32
// consecutive channels (LPT = d/32 lanes per token) and slot selects one of 64/LPT tokens
// processed per pass.  Each lane keeps partial output sums for its 32 channels; at the end
// of a split they are reduced over slots (reduce-scatter) and merged across the waves of
// the workgroup in LDS.  The split kernel writes one partial record per split
// (unnormalised output o[d], running max m, denominator l); a second, small kernel merges
// the records of each (batch row, query head) and adds the current token.  The kernel
// boundary orders the two, so no device-scope fence is needed inside the split kernel
// (on gfx950 such a fence writes back and invalidates the whole L2 of the XCD).
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

}  // namespace rq
