// rq_decode_attention: split-K flash-decoding over the packed ResidualQuant cache.
//
// ResidualQuant explainer, paragraph on the master print: attention rebuilds each loop's
// KV as c * anchor + residual tile by tile on chip, never writing it back to HBM;
// paragraph "Which print is the master": a shared anchor costs two reads per loop
// (anchor + own residual), a chained layout reads the anchor plus every residual
// between the loop and the anchor, and the current token is still BF16.
//
// The rebuilt key of token j at loop l is  k_j = C_j a_j + R^T sum_k gamma_jk r_jk
// (shared: C = c_l, one residual with gamma = 1; chained: C = prod_{m=l}^{L-2} c_m,
// gamma_k = prod_{m=l}^{k-1} c_m).  Since R is orthogonal and fixed per (KV head, K|V):
//   q . k_j = C_j (q . a_j) + sum_k gamma_jk (R_K q) . r_jk
// and with a = z + s * code per group,  q . a = sum_groups (z * sum(q) + s * sum(q * code)).
// Values: o = (sum_j p_j C_j a_j + R_V^T sum_j p_j sum_k gamma_jk r_jk + p_cur v_cur) / sum p,
// so the kernel accumulates the anchor part and the residual part separately and
// applies R_V^T once per output in the final merge.
#include "rq_args.hpp"
#include "rq_splitk.hpp"

namespace rq {


template <int BITS, int NW>
__device__ __forceinline__ float code_f(const uint32_t (&w)[NW], int idx) {
    constexpr uint32_t mask = (1u << BITS) - 1u;
    return (float)((w[(idx * BITS) >> 5] >> ((idx * BITS) & 31)) & mask);
}

template <int NB>
__device__ __forceinline__ void load_words(uint32_t (&w)[NB / 4], const uint8_t* p) {
    if constexpr (NB == 16) {
        const uint4 v = *reinterpret_cast<const uint4*>(p);
        w[0] = v.x; w[1] = v.y; w[2] = v.z; w[3] = v.w;
    } else {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        w[0] = v.x; w[1] = v.y;
    }
}

// metadata of this lane's GPL groups: byte pairs (z, s)
template <int GPL>
__device__ __forceinline__ uint32_t load_meta(const uint8_t* p) {
    if constexpr (GPL == 1) return *reinterpret_cast<const uint16_t*>(p);
    else return *reinterpret_cast<const uint32_t*>(p);
}

// Raw bytes of one token-pass for one lane: K and V words of the anchor plane and of the
// NR residual planes, with their metadata and coefficients.
template <int AW, int NR>
struct Frame {
    uint32_t ka[AW], kam, va[AW], vam;
    uint32_t kr[NR][2], krm[NR], kc[NR];
    uint32_t vr[NR][2], vrm[NR], vc[NR];
};

// D: head dim; GS: group size; BA: anchor bits; NRES: residual planes read (0 = anchor loop).
template <int D, int GS, int BA, int NRES, bool QBF16>
__global__ __launch_bounds__(kThreads) void rq_decode_kernel(DecodeArgs a) {
    constexpr int LPT = D / 32;            // lanes per token
    constexpr int SLOTS = kWave / LPT;     // tokens per pass
    constexpr int PPT = kTile / SLOTS;     // passes per tile
    constexpr int GPL = 32 / GS;           // quantization groups per lane
    constexpr int AB = 32 * BA / 8;        // anchor code bytes per lane
    constexpr int AW = AB / 4;
    constexpr int NR = NRES ? NRES : 1;
    constexpr int NV = NRES ? 64 : 32;

    const Geom& G = a.geo;
    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int split = lb % a.n_splits;
    const int bh = lb / a.n_splits;        // b * Hq + hq
    const int hq = bh % G.hq;
    const int b = bh / G.hq;
    const int h = hq / (G.hq / G.hkv);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int chunk = lane % LPT, slot = lane / LPT;

    __shared__ float sq[D];
    __shared__ float su[D];
    __shared__ SplitSmem<D> sm;

    int n = a.ctx_len[b];
    n = n < 0 ? 0 : (n > a.ctx_bound ? a.ctx_bound : n);
    const int n_tiles = (n + kTile - 1) / kTile;
    const int t_begin = split * a.tiles_per_split;
    const int t_end = min(n_tiles, t_begin + a.tiles_per_split);
    const int first = t_begin + w;
    const int my_tiles = first < t_end ? (t_end - first + kWaves - 1) / kWaves : 0;
    const int n_it = my_tiles * PPT;

    // ---- plane bases
    const int L = G.L;
    const int aloop = (a.loop / L) * L + L - 1;
    const uint8_t* aK = a.cache + G.plane_offset(b, h, 0, aloop);
    const uint8_t* aV = a.cache + G.plane_offset(b, h, 1, aloop);
    const uint8_t* rK[NR];
    const uint8_t* rV[NR];
#pragma unroll
    for (int k = 0; k < NR; ++k) {
        rK[k] = a.cache + G.plane_offset(b, h, 0, a.loop + k);
        rV[k] = a.cache + G.plane_offset(b, h, 1, a.loop + k);
    }
    const int a_meta = kTile * G.a_row;
    const int r_meta = kTile * G.r_row;
    const int r_cblk = kTile * (G.r_row + G.m_row);

    auto load = [&](Frame<AW, NR>& f, int it) {
        const int tile = first + kWaves * (it / PPT);
        const int jj = (it % PPT) * SLOTS + slot;
        const int64_t ta = (int64_t)tile * G.a_tile + jj * G.a_row + chunk * AB;
        const int64_t tm = (int64_t)tile * G.a_tile + a_meta + jj * G.m_row + chunk * GPL * 2;
        load_words<AB>(f.ka, aK + ta);
        load_words<AB>(f.va, aV + ta);
        f.kam = load_meta<GPL>(aK + tm);
        f.vam = load_meta<GPL>(aV + tm);
        if constexpr (NRES > 0) {
            const int64_t tr = (int64_t)tile * G.r_tile;
#pragma unroll
            for (int k = 0; k < NRES; ++k) {
                load_words<8>(f.kr[k], rK[k] + tr + jj * G.r_row + chunk * 8);
                load_words<8>(f.vr[k], rV[k] + tr + jj * G.r_row + chunk * 8);
                f.krm[k] = load_meta<GPL>(rK[k] + tr + r_meta + jj * G.m_row + chunk * GPL * 2);
                f.vrm[k] = load_meta<GPL>(rV[k] + tr + r_meta + jj * G.m_row + chunk * GPL * 2);
                f.kc[k] = *reinterpret_cast<const uint16_t*>(rK[k] + tr + r_cblk + jj * 2);
                f.vc[k] = *reinterpret_cast<const uint16_t*>(rV[k] + tr + r_cblk + jj * 2);
            }
        }
    };

    Frame<AW, NR> fa, fb;
    if (n_it > 0) load(fa, 0);

    // ---- prologue (overlaps the first loads): q and u = R_K q
    for (int i = threadIdx.x; i < D; i += kThreads) {
        float qv;
        if constexpr (QBF16)
            qv = bf16_to_f32(reinterpret_cast<const uint16_t*>(a.q)[(int64_t)bh * D + i]);
        else
            qv = reinterpret_cast<const float*>(a.q)[(int64_t)bh * D + i];
        sq[i] = qv;
    }
    __syncthreads();
    if constexpr (NRES > 0) {
        const float* RK = a.rot + (int64_t)(h * 2 + 0) * D * D;
        constexpr int TPR = kThreads / D;          // threads per row
        constexpr int COLS = D / TPR;
        const int row = threadIdx.x / TPR, part = threadIdx.x % TPR;
        const float4* rr = reinterpret_cast<const float4*>(RK + (int64_t)row * D + part * COLS);
        float acc = 0.f;
#pragma unroll
        for (int k4 = 0; k4 < COLS / 4; ++k4) {
            const float4 r4 = rr[k4];
            const int c0 = part * COLS + 4 * k4;
            acc += r4.x * sq[c0] + r4.y * sq[c0 + 1] + r4.z * sq[c0 + 2] + r4.w * sq[c0 + 3];
        }
#pragma unroll
        for (int m = 1; m < TPR; m <<= 1) acc += shfl_xor_f(acc, m);
        if (part == 0) su[row] = acc;
        __syncthreads();
    }
    float qr[32], ur[NRES ? 32 : 1], Qg[GPL], Ug[GPL];
#pragma unroll
    for (int i = 0; i < 32; ++i) qr[i] = sq[32 * chunk + i];
    if constexpr (NRES > 0) {
#pragma unroll
        for (int i = 0; i < 32; ++i) ur[i] = su[32 * chunk + i];
    }
#pragma unroll
    for (int gg = 0; gg < GPL; ++gg) {
        float s1 = 0.f, s2 = 0.f;
#pragma unroll
        for (int i = 0; i < GS; ++i) {
            s1 += qr[gg * GS + i];
            if constexpr (NRES > 0) s2 += ur[gg * GS + i];
        }
        Qg[gg] = s1;
        Ug[gg] = s2;
    }

    float accA[32], accR[NRES ? 32 : 1], offA[GPL], offR[GPL];
#pragma unroll
    for (int i = 0; i < 32; ++i) accA[i] = 0.f;
#pragma unroll
    for (int i = 0; i < (NRES ? 32 : 1); ++i) accR[i] = 0.f;
#pragma unroll
    for (int gg = 0; gg < GPL; ++gg) offA[gg] = offR[gg] = 0.f;
    float m_run = -INFINITY, l_lane = 0.f;
    const float sm_scale = a.sm_scale;

    auto compute = [&](const Frame<AW, NR>& f, int it) {
        const int tile = first + kWaves * (it / PPT);
        const int jj = (it % PPT) * SLOTS + slot;
        const bool valid = tile * kTile + jj < n;
        // ---------------- keys
        float part_a = 0.f;
#pragma unroll
        for (int gg = 0; gg < GPL; ++gg) {
            const float z = e4m3_to_f32((f.kam >> (16 * gg)) & 0xFF);
            const float s = e4m3_to_f32((f.kam >> (16 * gg + 8)) & 0xFF);
            float dot = 0.f;
#pragma unroll
            for (int i = 0; i < GS; ++i) dot += qr[gg * GS + i] * code_f<BA>(f.ka, gg * GS + i);
            part_a += z * Qg[gg] + s * dot;
        }
        float coef = 1.f, part_r = 0.f;
#pragma unroll
        for (int k = 0; k < NRES; ++k) {
            float pr = 0.f;
#pragma unroll
            for (int gg = 0; gg < GPL; ++gg) {
                const float z = e4m3_to_f32((f.krm[k] >> (16 * gg)) & 0xFF);
                const float s = e4m3_to_f32((f.krm[k] >> (16 * gg + 8)) & 0xFF);
                float dot = 0.f;
#pragma unroll
                for (int i = 0; i < GS; ++i) dot += ur[gg * GS + i] * code_f<2>(f.kr[k], gg * GS + i);
                pr += z * Ug[gg] + s * dot;
            }
            part_r += coef * pr;
            coef *= valid ? bf16_to_f32(f.kc[k]) : 0.f;
        }
        float score = chunk_sum<LPT>(coef * part_a + part_r) * sm_scale;
        score = valid ? score : -INFINITY;
        const float pmax = slot_max<LPT>(score);
        if (pmax > m_run) {                         // uniform across the wave
            const float fs = __expf(m_run - pmax);
#pragma unroll
            for (int i = 0; i < 32; ++i) accA[i] *= fs;
#pragma unroll
            for (int i = 0; i < (NRES ? 32 : 1); ++i) accR[i] *= fs;
#pragma unroll
            for (int gg = 0; gg < GPL; ++gg) { offA[gg] *= fs; offR[gg] *= fs; }
            l_lane *= fs;
            m_run = pmax;
        }
        const float pw = valid ? __expf(score - m_run) : 0.f;
        l_lane += pw;
        // ---------------- values
        float wv = pw;
#pragma unroll
        for (int k = 0; k < NRES; ++k) {
#pragma unroll
            for (int gg = 0; gg < GPL; ++gg) {
                const float z = e4m3_to_f32((f.vrm[k] >> (16 * gg)) & 0xFF);
                const float s = e4m3_to_f32((f.vrm[k] >> (16 * gg + 8)) & 0xFF);
                offR[gg] += wv * z;
                const float ws = wv * s;
#pragma unroll
                for (int i = 0; i < GS; ++i) accR[gg * GS + i] += ws * code_f<2>(f.vr[k], gg * GS + i);
            }
            wv *= valid ? bf16_to_f32(f.vc[k]) : 0.f;
        }
#pragma unroll
        for (int gg = 0; gg < GPL; ++gg) {
            const float z = e4m3_to_f32((f.vam >> (16 * gg)) & 0xFF);
            const float s = e4m3_to_f32((f.vam >> (16 * gg + 8)) & 0xFF);
            offA[gg] += wv * z;
            const float ws = wv * s;
#pragma unroll
            for (int i = 0; i < GS; ++i) accA[gg * GS + i] += ws * code_f<BA>(f.va, gg * GS + i);
        }
    };

    // ---- main loop, two frames in flight
    for (int it = 0; it < n_it; it += 2) {
        if (it + 1 < n_it) load(fb, it + 1);
        compute(fa, it);
        if (it + 1 < n_it) {
            if (it + 2 < n_it) load(fa, it + 2);
            compute(fb, it + 1);
        }
    }

    // ---- fold group offsets, merge the waves, apply R_V^T to the residual part
    float v[NV];
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = accA[i] + offA[i / GS];
    if constexpr (NRES > 0) {
#pragma unroll
        for (int i = 0; i < 32; ++i) v[32 + i] = accR[i] + offR[i / GS];
    }
    const float2 ml = splitk_merge_waves<D, NV>(v, m_run, l_lane, sm);
    float* rec = a.partials + ((int64_t)bh * kMaxSplits + split) * partial_stride(D);
    if constexpr (NRES > 0) {
        // o_i = A_i + sum_k R_V[k][i] * Rr_k ; TPR threads per output, k split in parts
        const float* RV = a.rot + (int64_t)(h * 2 + 1) * D * D;
        constexpr int PARTS = kThreads / D;
        constexpr int KP = D / PARTS;
        const int i = threadIdx.x % D, part = threadIdx.x / D;
        float t0 = 0.f, t1 = 0.f;
#pragma unroll 8
        for (int k = part * KP; k < (part + 1) * KP; k += 2) {
            t0 += RV[(int64_t)k * D + i] * sm.sum[D + k];
            t1 += RV[(int64_t)(k + 1) * D + i] * sm.sum[D + k + 1];
        }
        sm.acc[part][i] = t0 + t1;                 // wave scratch is free again
        __syncthreads();
        if (threadIdx.x < D) {
            float o = sm.sum[i];
#pragma unroll
            for (int p = 0; p < PARTS; ++p) o += sm.acc[p][i];
            rec[i] = o;
        }
    } else {
        if (threadIdx.x < D) rec[threadIdx.x] = sm.sum[threadIdx.x];
    }
    if (threadIdx.x == 0) {
        rec[D] = ml.x;
        rec[D + 1] = ml.y;
    }
}

template <int D, int GS, int BA, bool QB>
static hipError_t launch_nres(const DecodeArgs& a, int nres, dim3 grid, hipStream_t st) {
    switch (nres) {
        case 0: hipLaunchKernelGGL((rq_decode_kernel<D, GS, BA, 0, QB>), grid, dim3(kThreads), 0, st, a); break;
        case 1: hipLaunchKernelGGL((rq_decode_kernel<D, GS, BA, 1, QB>), grid, dim3(kThreads), 0, st, a); break;
        case 2: hipLaunchKernelGGL((rq_decode_kernel<D, GS, BA, 2, QB>), grid, dim3(kThreads), 0, st, a); break;
        case 3: hipLaunchKernelGGL((rq_decode_kernel<D, GS, BA, 3, QB>), grid, dim3(kThreads), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int D, int GS, int BA>
static hipError_t launch_q(const DecodeArgs& a, int nres, bool qbf16, dim3 grid, hipStream_t st) {
    return qbf16 ? launch_nres<D, GS, BA, true>(a, nres, grid, st)
                 : launch_nres<D, GS, BA, false>(a, nres, grid, st);
}

hipError_t launch_decode(const DecodeArgs& a, int nres, bool qbf16, hipStream_t st) {
    if (!a.cache || !a.q || !a.ctx_len || !a.rot || !a.partials || a.batch < 1 || a.n_splits < 1 ||
        a.n_splits > kMaxSplits)
        return hipErrorInvalidValue;
    const dim3 grid(a.batch * a.geo.hq * a.n_splits);
    const int d = a.geo.d, g = a.geo.g, ba = a.geo.ba;
    if (d == 128 && g == 32 && ba == 4) return launch_q<128, 32, 4>(a, nres, qbf16, grid, st);
    if (d == 128 && g == 16 && ba == 2) return launch_q<128, 16, 2>(a, nres, qbf16, grid, st);
    if (d == 128 && g == 16 && ba == 4) return launch_q<128, 16, 4>(a, nres, qbf16, grid, st);
    if (d == 128 && g == 32 && ba == 2) return launch_q<128, 32, 2>(a, nres, qbf16, grid, st);
    if (d == 64 && g == 32 && ba == 4) return launch_q<64, 32, 4>(a, nres, qbf16, grid, st);
    if (d == 64 && g == 16 && ba == 4) return launch_q<64, 16, 4>(a, nres, qbf16, grid, st);
    if (d == 64 && g == 32 && ba == 2) return launch_q<64, 32, 2>(a, nres, qbf16, grid, st);
    if (d == 64 && g == 16 && ba == 2) return launch_q<64, 16, 2>(a, nres, qbf16, grid, st);
    return hipErrorInvalidValue;
}

}  // namespace rq
