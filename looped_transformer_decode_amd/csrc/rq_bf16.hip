// rq_bf16_decode_attention: split-K flash-decoding over an uncompressed BF16 KV cache.
//
// This is the baseline the arXiv digest's throughput paragraph (section 5.3) measures
// ResidualQuant against: BF16 decode attention over each loop's own K/V.  It uses the
// same lane mapping, LDS DMA staging of the stream (non-temporal), online softmax, split-K
// merge and current-token handling as the ResidualQuant kernel, so the two differ only in
// what they read per token.
#include "rq_args.hpp"
#include "rq_merge_group.hpp"
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

// ---- grouped queries: one workgroup of 8 waves per (batch row, KV head, split) serves the
// G query heads of the KV head, so every K/V tile is read from HBM once for the group (the
// digest's BF16 FlashAttention baseline reads each tile once per group as well).  A token
// costs 2 d multiply-adds per query against 4 d bytes read, 2 per byte at G = 4, well inside
// the vector units' budget at the HBM rate, so this stays on the VALU in float32.
// Staging as in the one-query kernel (16-token passes of K and V by 1 KB DMAs into a 2-slot
// ring per wave); the compute takes a pass in 4 steps of 4 tokens, lane = (token, 8-channel
// chunk), and every lane keeps the G queries' running sums of its 8 channels.
namespace bgqa {
constexpr int D = 128, NW = 8, NT = NW * kWave;
constexpr int PT = 16;                      // tokens per staged pass
constexpr int CPL = 8;                      // channels per lane
constexpr int LPT = D / CPL;                // lanes per token (16: one DPP row)
constexpr int TPS = kWave / LPT;            // tokens per compute step (4)
constexpr int PB = PT * D * 2;              // bytes of one pass of K (or V): 4 KB
constexpr int NC = PB / 1024;               // 1 KB DMAs per pass of K (or V)
constexpr int NDMA = 2 * NC;
}  // namespace bgqa

template <int G, bool QBF16>
__global__ __launch_bounds__(bgqa::NT) void rq_bf16_decode_gqa_kernel(Bf16Args a) {
    using namespace bgqa;
    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int split = lb % a.n_splits;
    const int bk = lb / a.n_splits;                   // b * hkv + h
    const int h = bk % a.hkv, b = bk / a.hkv;
    const int bh0 = b * a.hq + h * G;                 // first query head of the group
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int c = lane % LPT, tt = lane / LPT;        // 8-channel chunk, token of the step

    __shared__ float sq[G][D];
    __shared__ float s_m[NW][G], s_l[NW][G];
    __shared__ __attribute__((aligned(16))) uint8_t ring[NW][2][2][PB];   // also the epilogue's scratch

    int n = a.ctx_len[b];
    n = n < 0 ? 0 : (n > a.ctx_bound ? a.ctx_bound : n);
    const int n_tiles = (n + kTile - 1) / kTile;
    const int t_begin = split * a.tiles_per_split;
    const int t_end = min(n_tiles, t_begin + a.tiles_per_split);
    // 16-token passes of this split, dealt to the waves round-robin
    const int p0 = t_begin * (kTile / PT), p1 = min(t_end * (kTile / PT), (n + PT - 1) / PT);
    const int first = p0 + w;
    const int n_it = first < p1 ? (p1 - first + NW - 1) / NW : 0;

    const int64_t base = ((int64_t)b * a.hkv + h) * a.t_cap * D;
    const uint8_t* Kb = reinterpret_cast<const uint8_t*>(a.k + base);
    const uint8_t* Vb = reinterpret_cast<const uint8_t*>(a.v + base);
    const uint32_t ring_base = __builtin_amdgcn_readfirstlane(lds_addr_of(&ring[w][0][0][0]));
    // a lane whose 16 bytes lie past t_cap reads the pass's first token instead (always below
    // ctx_len), so every DMA stays inside the row's cache and every wave issues as many
    auto issue = [&](int it) {
        const int j0 = (first + NW * it) * PT;
        const uint8_t* kp = uniform_ptr(Kb + (int64_t)j0 * (2 * D));
        const uint8_t* vp = uniform_ptr(Vb + (int64_t)j0 * (2 * D));
        const uint32_t dst = ring_base + (uint32_t)(it % 2) * 2 * PB;
#pragma unroll
        for (int m = 0; m < NC; ++m) {
            const int tok = j0 + (m * 1024 + 16 * lane) / (2 * D);
            const uint32_t voff = tok < a.t_cap ? (uint32_t)(m * 1024 + 16 * lane) : (uint32_t)((16 * lane) % (2 * D));
            dma16<true>(voff, kp, dst + m * 1024);
            dma16<true>(voff, vp, dst + PB + m * 1024);
        }
    };
    if (n_it > 0) issue(0);

    for (int i = threadIdx.x; i < G * D; i += NT) {
        const int64_t qi = (int64_t)bh0 * D + i;      // the G heads of the group are consecutive
        if constexpr (QBF16) sq[i / D][i % D] = bf16_to_f32(reinterpret_cast<const uint16_t*>(a.q)[qi]);
        else sq[i / D][i % D] = reinterpret_cast<const float*>(a.q)[qi];
    }
    __syncthreads();
    float qr[G][CPL], acc[G][CPL], m_run[G], l_lane[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            qr[g][i] = sq[g][CPL * c + i];
            acc[g][i] = 0.f;
        }
        m_run[g] = -INFINITY;
        l_lane[g] = 0.f;
    }
    const bool younger = w >= NW / 2;                  // waves w and w + 4 share a SIMD

    auto step = [&](int it, int s) {
        const int jj = s * TPS + tt;                   // token of the pass
        const bool valid = (first + NW * it) * PT + jj < n;
        const int row = valid ? jj : 0;                // masked lanes read the pass's first token
        const uint8_t* kr = &ring[w][it % 2][0][0] + row * (2 * D) + c * 16;
        const uint8_t* vr = &ring[w][it % 2][1][0] + row * (2 * D) + c * 16;
        const u32x4 k4 = *reinterpret_cast<const u32x4*>(kr);
        const u32x4 v4 = *reinterpret_cast<const u32x4*>(vr);
        const float kf[CPL] = {bf16lo(k4.x), bf16hi(k4.x), bf16lo(k4.y), bf16hi(k4.y),
                               bf16lo(k4.z), bf16hi(k4.z), bf16lo(k4.w), bf16hi(k4.w)};
        const float vf[CPL] = {bf16lo(v4.x), bf16hi(v4.x), bf16lo(v4.y), bf16hi(v4.y),
                               bf16lo(v4.z), bf16hi(v4.z), bf16lo(v4.w), bf16hi(v4.w)};
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float part = 0.f;
#pragma unroll
            for (int i = 0; i < CPL; ++i) part = fmaf(qr[g][i], kf[i], part);
            float score = group_sum<LPT>(part) * a.sm_scale;     // every lane of the token's row
            score = valid ? score : -INFINITY;
            if (wave_any(score > m_run[g] + kRescaleSlack)) {    // rare: raise the reference
                const float m_new = fmaxf(m_run[g], wave_max_uniform(score));
                const float fs = m_run[g] == -INFINITY ? 0.f : __expf(m_run[g] - m_new);
#pragma unroll
                for (int i = 0; i < CPL; ++i) acc[g][i] *= fs;
                l_lane[g] *= fs;
                m_run[g] = m_new;
            }
            const float p = valid ? __expf(score - m_run[g]) : 0.f;
            if (c == 0) l_lane[g] += p;                           // one lane per token counts it
#pragma unroll
            for (int i = 0; i < CPL; ++i) acc[g][i] = fmaf(p, vf[i], acc[g][i]);
        }
    };

    for (int it = 0; it < n_it; ++it) {
        prio_alternate(younger, it);
        if (it + 1 < n_it) {
            issue(it + 1);
            wait_vm<NDMA>();                       // pass `it` has landed, pass it + 1 in flight
        } else {
            wait_vm<0>();
        }
#pragma unroll
        for (int s = 0; s < PT / TPS; ++s) step(it, s);
    }

    // ---- epilogue: per wave and query, sums over the 4 token rows; then over the waves in LDS
    __builtin_amdgcn_s_setprio(3);
    __syncthreads();                               // every wave is done with its ring
    float* scr = reinterpret_cast<float*>(&ring[0][0][0][0]);   // [NW][G][D], then the merge's scratch
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const float lw = group_sum<kWave>(l_lane[g]);
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
            float v = acc[g][i];
            v += xshfl<16>(v);
            v += xshfl<32>(v);
            acc[g][i] = v;
        }
        if (tt == 0) {
#pragma unroll
            for (int i = 0; i < CPL; ++i) scr[(w * G + g) * D + CPL * c + i] = acc[g][i];
        }
        if (lane == 0) {
            s_m[w][g] = m_run[g];
            s_l[w][g] = lw;
        }
    }
    __syncthreads();
    // publish the G records (the waves scaled to the workgroup maximum), then count the arrival
    for (int idx = threadIdx.x; idx < G * D; idx += NT) {
        const int q = idx / D, ch = idx % D;
        float m_q = -INFINITY;
#pragma unroll
        for (int i = 0; i < NW; ++i) m_q = fmaxf(m_q, s_m[i][q]);
        float v = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i)
            if (s_m[i][q] != -INFINITY) v += __expf(s_m[i][q] - m_q) * scr[(i * G + q) * D + ch];
        st_agent(a.mg.partials + ((int64_t)(bh0 + q) * a.mg.rec_splits + split) * (2 * D + 4) + ch, v);
    }
    if (threadIdx.x < G) {
        const int q = threadIdx.x;
        float m_q = -INFINITY, l_q = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i) m_q = fmaxf(m_q, s_m[i][q]);
#pragma unroll
        for (int i = 0; i < NW; ++i)
            if (s_m[i][q] != -INFINITY) l_q += __expf(s_m[i][q] - m_q) * s_l[i][q];
        float* rec = a.mg.partials + ((int64_t)(bh0 + q) * a.mg.rec_splits + split) * (2 * D + 4);
        st_agent(rec + 2 * D, m_q);
        st_agent(rec + 2 * D + 1, l_q);
    }
    if (!splitk_arrive(a.mg, bh0)) return;
    __syncthreads();                               // scr is reused by the merge
    merge_group<D, NT, G, false>(a.mg, bh0, sq, scr);
}

bool bf16_gqa_supported(int d, int hq, int hkv) {
    const int g = hq / hkv;
    return d == bgqa::D && (g == 2 || g == 4);
}

hipError_t launch_bf16_gqa(const Bf16Args& a, bool qbf16, hipStream_t st) {
    if (!a.k || !a.v || !a.q || !a.ctx_len || !a.mg.partials || !a.mg.arrivals || !a.mg.k_cur || !a.mg.v_cur ||
        !a.mg.out || a.batch < 1 || a.n_splits < 1 || a.n_splits > kMaxSplits || a.mg.n_splits != a.n_splits ||
        a.mg.rec_splits < a.n_splits || a.t_cap < 1 || !bf16_gqa_supported(bgqa::D, a.hq, a.hkv))
        return hipErrorInvalidValue;
    const dim3 grid(a.batch * a.hkv * a.n_splits), block(bgqa::NT);
    const int g = a.hq / a.hkv;
    if (g == 4) {
        if (qbf16) hipLaunchKernelGGL((rq_bf16_decode_gqa_kernel<4, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((rq_bf16_decode_gqa_kernel<4, false>), grid, block, 0, st, a);
    } else {
        if (qbf16) hipLaunchKernelGGL((rq_bf16_decode_gqa_kernel<2, true>), grid, block, 0, st, a);
        else hipLaunchKernelGGL((rq_bf16_decode_gqa_kernel<2, false>), grid, block, 0, st, a);
    }
    return hipGetLastError();
}

hipError_t launch_bf16(const Bf16Args& a, int d, bool qbf16, hipStream_t st) {
    if (!a.k || !a.v || !a.q || !a.ctx_len || !a.mg.partials || !a.mg.arrivals || !a.mg.k_cur || !a.mg.v_cur ||
        !a.mg.out || a.batch < 1 || a.n_splits < 1 || a.n_splits > kMaxSplits || a.mg.n_splits != a.n_splits ||
        a.mg.rec_splits < a.n_splits || a.t_cap < 1)
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
