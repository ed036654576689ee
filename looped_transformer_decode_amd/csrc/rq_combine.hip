// Merge of split-K partial records (log-sum-exp) plus the current token.
//
// Explainer, paragraph "Which print is the master": the current token is not quantized
// until its final loop has run, so at every loop it enters attention from the BF16
// pending values; this kernel adds it as the last attention entry and, for the
// ResidualQuant path, stores it into the pending buffer that rq_quantize_token drains.
#include "rq_args.hpp"

namespace rq {

template <int NT>
__device__ __forceinline__ float cb_sum(float v, float* red) {
    for (int m = 32; m >= 1; m >>= 1) v += shfl_xor_f(v, m);
    if constexpr (NT == 64) return v;
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
__device__ __forceinline__ float cb_max(float v, float* red) {
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor_f(v, m));
    if constexpr (NT == 64) return v;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[w] = v;
    __syncthreads();
    float s = -INFINITY;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) s = fmaxf(s, red[i]);
    return s;
}

// one workgroup of D threads per (batch row, query head); thread i owns channel i.
// RES: the records carry a residual part acc_r that still has to be rotated back, once
// per head: o = sum_s w_s acc_a_s + R_V^T (sum_s w_s acc_r_s) + p_cur v_cur.
template <int D, bool QBF16, bool RES>
__global__ __launch_bounds__(D) void rq_combine_kernel(CombineArgs a) {
    static_assert(D >= kMaxSplits, "one thread per split record");
    const int bh = blockIdx.x;
    const int hq = bh % a.hq, b = bh / a.hq;
    const int gqa = a.hq / a.hkv;
    const int h = hq / gqa;
    const int i = threadIdx.x;
    __shared__ float red[D / 64 > 0 ? D / 64 : 1];
    __shared__ float wsplit[kMaxSplits];
    __shared__ float rvec[RES ? D : 1];

    const float qv = QBF16 ? bf16_to_f32(reinterpret_cast<const uint16_t*>(a.q)[(int64_t)bh * D + i])
                           : reinterpret_cast<const float*>(a.q)[(int64_t)bh * D + i];
    const int64_t kvo = ((int64_t)b * a.hkv + h) * D + i;
    const uint16_t kc = a.k_cur[kvo], vc = a.v_cur[kvo];
    const float s_cur = cb_sum<D>(qv * bf16_to_f32(kc), red) * a.sm_scale;

    const float* recs = a.partials + (int64_t)bh * kMaxSplits * partial_stride(D);
    float ms = -INFINITY, ls = 0.f;
    if (i < a.n_splits) {
        ms = recs[(int64_t)i * partial_stride(D) + 2 * D];
        ls = recs[(int64_t)i * partial_stride(D) + 2 * D + 1];
    }
    const float m_f = fmaxf(cb_max<D>(ls > 0.f ? ms : -INFINITY, red), s_cur);
    const float wsv = (ls > 0.f) ? __expf(ms - m_f) : 0.f;
    if (i < kMaxSplits) wsplit[i] = wsv;
    const float ltot = cb_sum<D>(wsv * ls, red);
    __syncthreads();
    float o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
    float r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
    const float* r = recs + i;
    const int64_t ps = partial_stride(D);
    int s = 0;
    for (; s + 4 <= a.n_splits; s += 4) {
        o0 += wsplit[s] * r[s * ps];
        o1 += wsplit[s + 1] * r[(s + 1) * ps];
        o2 += wsplit[s + 2] * r[(s + 2) * ps];
        o3 += wsplit[s + 3] * r[(s + 3) * ps];
        if constexpr (RES) {
            r0 += wsplit[s] * r[s * ps + D];
            r1 += wsplit[s + 1] * r[(s + 1) * ps + D];
            r2 += wsplit[s + 2] * r[(s + 2) * ps + D];
            r3 += wsplit[s + 3] * r[(s + 3) * ps + D];
        }
    }
    for (; s < a.n_splits; ++s) {
        o0 += wsplit[s] * r[s * ps];
        if constexpr (RES) r0 += wsplit[s] * r[s * ps + D];
    }
    float o_acc = (o0 + o1) + (o2 + o3);
    if constexpr (RES) {
        rvec[i] = (r0 + r1) + (r2 + r3);
        __syncthreads();
        // column i of R_V: R_V[k][i], coalesced across threads; all loads in flight together
        const float* rv = a.rot_v + (int64_t)h * 2 * D * D + i;
        float rk[D];
#pragma unroll
        for (int k = 0; k < D; ++k) rk[k] = rv[(int64_t)k * D];
        float t0 = 0.f, t1 = 0.f;
#pragma unroll
        for (int k = 0; k < D; k += 2) {
            t0 += rk[k] * rvec[k];
            t1 += rk[k + 1] * rvec[k + 1];
        }
        o_acc += t0 + t1;
    }
    const float p_cur = __expf(s_cur - m_f);
    const float o = (o_acc + p_cur * bf16_to_f32(vc)) / (ltot + p_cur);
    a.out[(int64_t)bh * D + i] = o;
    if (hq % gqa == 0) {
        if (a.pending != nullptr) {
            uint16_t* pd = a.pending + (((int64_t)b * a.L + a.lloc) * 2 * a.hkv + h) * D + i;
            pd[0] = kc;
            pd[(int64_t)a.hkv * D] = vc;
        }
        if (a.k_app != nullptr) {
            int n = a.ctx_len[b];
            n = n < 0 ? 0 : (n > a.ctx_bound ? a.ctx_bound : n);
            if (n < a.t_cap) {
                const int64_t off = (((int64_t)b * a.hkv + h) * a.t_cap + n) * D + i;
                a.k_app[off] = kc;
                a.v_app[off] = vc;
            }
        }
    }
}

template <int D, bool QB>
static void launch_c(const CombineArgs& a, dim3 grid, hipStream_t st) {
    if (a.rot_v) hipLaunchKernelGGL((rq_combine_kernel<D, QB, true>), grid, dim3(D), 0, st, a);
    else hipLaunchKernelGGL((rq_combine_kernel<D, QB, false>), grid, dim3(D), 0, st, a);
}

hipError_t launch_combine(const CombineArgs& a, int d, bool qbf16, int batch, hipStream_t st) {
    if (!a.partials || !a.q || !a.k_cur || !a.v_cur || !a.out || batch < 1 || a.n_splits < 1 ||
        a.n_splits > kMaxSplits || (a.k_app && (!a.v_app || !a.ctx_len)))
        return hipErrorInvalidValue;
    const dim3 grid(batch * a.hq);
    if (d == 128) {
        if (qbf16) launch_c<128, true>(a, grid, st);
        else launch_c<128, false>(a, grid, st);
    } else if (d == 64) {
        if (qbf16) launch_c<64, true>(a, grid, st);
        else launch_c<64, false>(a, grid, st);
    } else {
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace rq
