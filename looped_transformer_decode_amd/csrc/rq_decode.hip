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
// so the kernel accumulates the anchor part and the residual part separately; the last
// workgroup of each (batch row, query head) merges the splits and applies R_V^T once.
#include "rq_args.hpp"
#include "rq_splitk.hpp"
#include "rq_stage.hpp"

namespace rq {


// ---- keys: exact integer dot products on the packed codes
//
// q is written per quantization group as 24-bit fixed point Q_i = rint(q_i / delta),
// delta = 2^(e-21) with 2^e <= max|q_i|, split into six balanced base-16 digits d_k in
// [-8, 7] (Q = sum_k 16^k d_k).  u = R_K q multiplies the residual codes (2-bit, or 4-bit
// in the uniform INT4 setting) and uses 16-bit fixed point, delta = 2^(e-13), four digits
// in the digit layout of its code width.  A digit word holds the
// digits of the 8 channels whose codes share one 32-bit code word, at the same nibble
// positions, so v_dot8_i32_i4 multiplies codes by digits without unpacking: 4-bit codes
// are first offset to signed c - 8 (xor 0x8 per nibble; the offset is added back as
// 8 * sum Q), 2-bit codes are split into even/odd channels (c in 0..3 fits a signed nibble).
// sum_i q_i c_i = delta * sum_k 16^k dot_k (+ 8 delta sum Q for 4-bit codes).

__device__ __forceinline__ int sdot8(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot8((int)a, (int)b, c, false);
}

// nibble words of a lane's 32 channels: 4 of them, in digit-word order
template <int BITS>
__device__ __forceinline__ void code_nibbles(uint32_t (&nib)[4], const uint32_t* w) {
    if constexpr (BITS == 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) nib[k] = w[k] ^ 0x88888888u;
    } else {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            nib[2 * k] = w[k] & 0x33333333u;
            nib[2 * k + 1] = (w[k] >> 2) & 0x33333333u;
        }
    }
}

// sum_k 16^k dot_k over the nibble words [w0, w0 + NW) of one group, ND = 6 or 4 digits
template <int NW, int ND>
__device__ __forceinline__ float digit_dot(const uint32_t (&nib)[4], const uint32_t (&dg)[ND][4], int w0) {
    int acc[ND];
#pragma unroll
    for (int k = 0; k < ND; ++k) acc[k] = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int k = 0; k < ND; ++k) acc[k] = sdot8(nib[w0 + w], dg[k][w0 + w], acc[k]);
    if constexpr (ND == 6) {
        const int t0 = acc[0] + (acc[1] << 4) + (acc[2] << 8);
        const int t1 = acc[3] + (acc[4] << 4) + (acc[5] << 8);
        return (float)t0 + 4096.f * (float)t1;
    } else {
        const int t0 = acc[0] + (acc[1] << 4);
        const int t1 = acc[2] + (acc[3] << 4);
        return (float)t0 + 256.f * (float)t1;
    }
}

// ---- values: FP16 magic numbers
//
// OR-ing a code into the mantissa of FP16 1024.0 (0x6400) gives 1024 + m*c exactly, where
// m = 2^(bit position) of the code inside the half; v_fma_mix_f32 then accumulates
// w * (1024 + m c) in fp32.  Per channel: sum_j w_j c_j = (acc - 1024 * sum_j w_j) / m.
__device__ __forceinline__ void fma_pair(float& a0, float& a1, uint32_t pk, float w) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 h = __builtin_bit_cast(h2, pk);
    a0 = fmaf((float)h.x, w, a0);
    a1 = fmaf((float)h.y, w, a1);
}

constexpr uint32_t kMagic = 0x64006400u;

// (x & mask) | magic in one v_and_or_b32 (mask as a scalar operand, magic in a register)
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t magic) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(magic));
    return r;
}

// 4-bit word: channels 0..7 of the word at nibbles 0..7
__device__ __forceinline__ void v_acc4(float* acc, uint32_t w, float wt, uint32_t mg) {
    const uint32_t w8 = w >> 8;
    fma_pair(acc[0], acc[4], and_or(w, 0x000F000Fu, mg), wt);
    fma_pair(acc[1], acc[5], and_or(w, 0x00F000F0u, mg), wt);
    fma_pair(acc[2], acc[6], and_or(w8, 0x000F000Fu, mg), wt);
    fma_pair(acc[3], acc[7], and_or(w8, 0x00F000F0u, mg), wt);
}
__host__ __device__ constexpr float mult4(int ch) { return (ch & 1) ? 16.f : 1.f; }

// 2-bit word: channels 0..15 of the word at bits 2c
__device__ __forceinline__ void v_acc2(float* acc, uint32_t w, float wt, uint32_t mg) {
    const uint32_t w10 = w >> 10;
    fma_pair(acc[0], acc[8], and_or(w, 0x00030003u, mg), wt);
    fma_pair(acc[1], acc[9], and_or(w, 0x000C000Cu, mg), wt);
    fma_pair(acc[2], acc[10], and_or(w, 0x00300030u, mg), wt);
    fma_pair(acc[3], acc[11], and_or(w, 0x00C000C0u, mg), wt);
    fma_pair(acc[4], acc[12], and_or(w, 0x03000300u, mg), wt);
    fma_pair(acc[5], acc[13], and_or(w10, 0x00030003u, mg), wt);
    fma_pair(acc[6], acc[14], and_or(w10, 0x000C000Cu, mg), wt);
    fma_pair(acc[7], acc[15], and_or(w10, 0x00300030u, mg), wt);
}
__host__ __device__ constexpr float mult2(int ch) {
    return (float)(1 << (2 * ((ch & 7) < 5 ? (ch & 7) : (ch & 7) - 5)));
}

template <int BITS>
__device__ __forceinline__ void v_acc(float* acc, const uint32_t* w, float wt, int g0, int ng, uint32_t mg) {
    // accumulate the channels of code words [g0, g0 + ng)
    if constexpr (BITS == 4) {
        for (int k = g0; k < g0 + ng; ++k) v_acc4(acc + 8 * k, w[k], wt, mg);
    } else {
        for (int k = g0; k < g0 + ng; ++k) v_acc2(acc + 16 * k, w[k], wt, mg);
    }
}

template <int BITS>
__host__ __device__ constexpr float inv_mult(int ch) {
    return BITS == 4 ? 1.f / mult4(ch % 8) : 1.f / mult2(ch % 16);
}

__device__ __forceinline__ float fp8(uint32_t word, int byte) {
    switch (byte) {
        case 0: return __builtin_amdgcn_cvt_f32_fp8((int)word, 0);
        case 1: return __builtin_amdgcn_cvt_f32_fp8((int)word, 1);
        case 2: return __builtin_amdgcn_cvt_f32_fp8((int)word, 2);
        default: return __builtin_amdgcn_cvt_f32_fp8((int)word, 3);
    }
}

// D: head dim; GS: group size; BA: anchor bits; BR: residual bits; NRES: residual planes
// read (0 = anchor loop); PAGED: tiles addressed through the block table (G.bt).
template <int D, int GS, int BA, int BR, int NRES, bool QBF16, bool PAGED>
__global__ __launch_bounds__(kThreads) void rq_decode_kernel(DecodeArgs a) {
    constexpr int LPT = D / 32;            // lanes per token
    constexpr int SLOTS = kWave / LPT;     // tokens per pass
    constexpr int PPT = kTile / SLOTS;     // passes per tile
    constexpr int GPL = 32 / GS;           // quantization groups per lane
    constexpr int AB = 32 * BA / 8;        // anchor code bytes per lane
    constexpr int AW = AB / 4;             // anchor code words per lane
    constexpr int RW = BR;                 // residual code words per lane (32 channels)
    constexpr int NR = NRES ? NRES : 1;
    constexpr int NV = NRES ? 64 : 32;
    constexpr int NG = D / GS;             // groups per head vector
    // bytes of one pass (SLOTS tokens) per block; each block is one DMA instruction
    constexpr int AC = SLOTS * D * BA / 8;         // anchor codes
    constexpr int AM = SLOTS * 2 * D / GS;         // FP8 offset/scale pairs
    constexpr int RC = SLOTS * D * BR / 8;         // residual codes
    constexpr int CC = SLOTS * 2;                  // BF16 coefficients
    constexpr int PASS = 2 * (AC + AM + NRES * (RC + AM + CC));
    constexpr int NDMA = 2 * (2 + 3 * NRES);       // DMA instructions per pass
    // ring slots per wave: the loads of NB - 1 passes in flight must fit the 6-bit vmcnt
    constexpr int NB = (kStageDepth - 1) * NDMA <= 63 ? kStageDepth : 1 + 63 / NDMA;

    const Geom& G = a.geo;
    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int split = lb % a.n_splits;
    const int bh = lb / a.n_splits;        // b * Hq + hq
    const int hq = bh % G.hq;
    const int b = bh / G.hq;
    const int h = hq / (G.hq / G.hkv);
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int chunk = lane % LPT, slot = lane / LPT;
    const bool younger = younger_on_cu(a.n_cu);
    if (younger) __builtin_amdgcn_s_setprio(2);        // it also fetches its prologue second
    else __builtin_amdgcn_s_setprio(1);

    __shared__ SplitSmem<D> sm;
    __shared__ __attribute__((aligned(16))) uint8_t ring[kWaves][NB][PASS];
    __shared__ float sv[2][D];                         // q and u = R_K q
    __shared__ uint32_t s_dig[10 * (D / 8)];           // digit words: q [6][D/8], u [4][D/8]
    __shared__ float s_f[6][NG];                       // delta_q, corr_q, sum_q, delta_u, sum_u, corr_u

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
    // the residual planes a loop-step reads all have BR-bit codes (the host picks the
    // instantiation from the loop's width; chained layouts have one width)
    const int a_meta = kTile * G.a_row;
    const int r_meta = kTile * (D * BR / 8);
    const int r_cblk = kTile * (D * BR / 8 + G.m_row);

    // Paged layout: the block of each of this wave's tiles is read through the scalar cache
    // one tile ahead (the first one here, at the top of the prologue).
    constexpr bool paged = PAGED;
    int blk_cur = 0, blk_nxt = 0;
    if (paged && my_tiles > 0) blk_nxt = block_id_scalar(G, b, first);

    // Stage pass `it` (SLOTS consecutive tokens of one tile) of every plane into ring slot
    // it % NB of this wave.  LDS slot layout: K then V, each [anchor codes][anchor meta]
    // then per residual plane [codes][meta][c].
    const uint32_t ring_base = __builtin_amdgcn_readfirstlane(lds_addr_of(&ring[w][0][0]));
    auto issue = [&](int it) {
        const uint32_t tile = first + kWaves * (it / PPT);
        const uint32_t p = it % PPT;
        uint32_t dst = ring_base + (uint32_t)(it % NB) * PASS;
        if (paged && p == 0) {
            blk_cur = blk_nxt;
            if (it / PPT + 1 < my_tiles) blk_nxt = block_id_scalar(G, b, (int)tile + kWaves);
        }
        const uint32_t ta = paged ? 0u : tile * (uint32_t)G.a_tile;
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const uint8_t* ap = paged ? uniform_ptr(a.cache + G.paged_offset(blk_cur, h, x, aloop)) : (x ? aV : aK);
            stage<AC, PAGED>(ap, ta + p * AC, dst, lane);
            stage<AM, PAGED>(ap, ta + a_meta + p * AM, dst + AC, lane);
            dst += AC + AM;
            if constexpr (NRES > 0) {
                const uint32_t tr = paged ? 0u : tile * (uint32_t)(kTile * (D * BR / 8 + G.m_row + 2));
#pragma unroll
                for (int k = 0; k < NRES; ++k) {
                    const uint8_t* rp =
                        paged ? uniform_ptr(a.cache + G.paged_offset(blk_cur, h, x, a.loop + k)) : (x ? rV[k] : rK[k]);
                    stage<RC, PAGED>(rp, tr + p * RC, dst, lane);
                    stage<AM, PAGED>(rp, tr + r_meta + p * AM, dst + RC, lane);
                    stage<CC, PAGED, false>(rp, tr + r_cblk + p * CC, dst + RC + AM, lane);   // line shared by the tile's passes
                    dst += RC + AM + CC;
                }
            }
        }
    };
    // wait until pass `it` has landed while `ahead` later passes stay in flight
    static_assert((NB - 1) * NDMA <= 63, "vmcnt holds at most 63 outstanding loads");
    auto wait_pass = [&](int ahead) {
        if constexpr (NB >= 5) {
            if (ahead >= 4) { wait_vm<4 * NDMA>(); return; }
        }
        if constexpr (NB >= 4) {
            if (ahead >= 3) { wait_vm<3 * NDMA>(); return; }
        }
        if constexpr (NB >= 3) {
            if (ahead >= 2) { wait_vm<2 * NDMA>(); return; }
        }
        if (ahead >= 1) wait_vm<NDMA>();
        else wait_vm<0>();
    };
    // ---- prologue.  R_K and q are loaded first, coalesced: load k of thread t holds row
    // k * RPL + t / C4, columns [4 * (t % C4), 4 * (t % C4) + 4) of R_K, and the thread's
    // q segment covers the same columns.  The stream DMAs of the first passes are issued
    // behind them; vector loads return in order, so waiting until only those DMAs are
    // outstanding leaves them in flight while u = R_K q and the digits are computed.
    constexpr int C4 = D / 4;                          // 16-byte columns per row
    constexpr int RPL = kThreads / C4;                 // rows covered by one load
    constexpr int RL = NRES ? D / RPL : 1;             // R_K loads per thread
    const int c4 = threadIdx.x % C4;
    f32x4 rq4[RL];
    f32x4 q4f;
    u32x2 q4b;
    {
        const uint8_t* qb = static_cast<const uint8_t*>(a.q) + (int64_t)bh * D * (QBF16 ? 2 : 4);
        if constexpr (QBF16) q4b = gload8(qb, (uint32_t)c4 * 8u);
        else q4f = gload16(qb, (uint32_t)c4 * 16u);
        if constexpr (NRES > 0) {
            const uint8_t* rb = reinterpret_cast<const uint8_t*>(a.rot + (int64_t)(h * 2) * D * D);
#pragma unroll
            for (int k = 0; k < RL; ++k) rq4[k] = gload16(rb, (uint32_t)(k * kThreads + threadIdx.x) * 16u);
        }
    }
    const int n_pre = min(NB - 1, n_it);
    for (int k = 0; k < n_pre; ++k) issue(k);
    wait_pass(n_pre);
    if constexpr (QBF16) {
        pin(q4b);
        q4f = f32x4{bf16lo(q4b.x), bf16hi(q4b.x), bf16lo(q4b.y), bf16hi(q4b.y)};
    } else {
        pin(q4f);
    }
    if (threadIdx.x < C4) {
#pragma unroll
        for (int e = 0; e < 4; ++e) sv[0][4 * c4 + e] = q4f[e];
    }
    if constexpr (NRES > 0) {
        float pr[RL];
#pragma unroll
        for (int k = 0; k < RL; ++k) {
            pin(rq4[k]);
            pr[k] = rq4[k].x * q4f.x + rq4[k].y * q4f.y + rq4[k].z * q4f.z + rq4[k].w * q4f.w;
        }
        int off = 0;
        group_reduce_scatter<RL, C4 / 2, RL>(pr, lane, off);
        sv[1][off * RPL + threadIdx.x / C4] = pr[0];
    }
    __syncthreads();
    // fixed-point digits (see the comment above digit_dot): q in the anchor-code layout,
    // u in the 2-bit layout
    if (threadIdx.x < (NRES ? 2 : 1) * D) {
        const int which = threadIdx.x / D, i = threadIdx.x % D;
        const float val = sv[which][i];
        const bool four = which ? (BR == 4) : (BA == 4);
        const float amax = group_max<GS>(fabsf(val));
        const float vsum = group_sum<GS>(val);
        const int e = amax > 0.f ? ilogbf(amax) : 0;
        const int fb = which ? 13 : 21;                    // |Q| <= 2^(fb + 1)
        int Q = (int)rintf(val * ldexpf(1.f, fb - e));     // exact power-of-two scaling
        const int qsum = group_sum_i<GS>(Q);
        const int shift = four ? 4 * (i % 8) : 4 * ((i % 16) / 2);
        const int widx = four ? i / 8 : (i / 16) * 2 + (i & 1);
        const int nd = which ? 4 : 6;
        const int base = which ? 6 * (D / 8) : 0;
        // the 8 channels of a digit word sit in 8 lanes of this wave (consecutive ones for
        // 4-bit codes, one parity of a 16-lane row for 2-bit codes) with disjoint nibbles:
        // OR them over the lane exchanges, and the first lane of the group stores the word
        const bool lead = four ? (i % 8) == 0 : (i % 16) < 2;
#pragma unroll
        for (int k = 0; k < 6; ++k) {
            if (k < nd) {
                const int d = ((Q + 8) & 15) - 8;
                Q = (Q - d) >> 4;
                int word = (d & 15) << shift;
                if (four) {
                    word |= xshfl_i<1>(word);
                    word |= xshfl_i<2>(word);
                    word |= xshfl_i<4>(word);
                } else {
                    word |= xshfl_i<2>(word);
                    word |= xshfl_i<4>(word);
                    word |= xshfl_i<8>(word);
                }
                if (lead) s_dig[base + k * (D / 8) + widx] = (uint32_t)word;
            }
        }
        if (i % GS == 0) {
            const int gi = i / GS;
            if (which == 0) {
                s_f[0][gi] = ldexpf(1.f, e - fb);
                s_f[1][gi] = four ? 8.f * (float)qsum : 0.f;
                s_f[2][gi] = vsum;
            } else {
                s_f[3][gi] = ldexpf(1.f, e - fb);
                s_f[4][gi] = vsum;
                s_f[5][gi] = four ? 8.f * (float)qsum : 0.f;
            }
        }
    }
    __syncthreads();
    uint32_t dq[6][4], du[4][4];
    float dlq[GPL], crq[GPL], Qg[GPL], dlu[GPL], Ug[GPL], cru[GPL];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
#pragma unroll
        for (int k = 0; k < 6; ++k) dq[k][x] = s_dig[k * (D / 8) + 4 * chunk + x];
#pragma unroll
        for (int k = 0; k < 4; ++k) du[k][x] = NRES ? s_dig[6 * (D / 8) + k * (D / 8) + 4 * chunk + x] : 0u;
    }
#pragma unroll
    for (int gg = 0; gg < GPL; ++gg) {
        const int gi = chunk * GPL + gg;
        dlq[gg] = s_f[0][gi];
        crq[gg] = s_f[1][gi];
        Qg[gg] = s_f[2][gi];
        dlu[gg] = NRES ? s_f[3][gi] : 0.f;
        Ug[gg] = NRES ? s_f[4][gi] : 0.f;
        cru[gg] = (NRES && BR == 4) ? s_f[5][gi] : 0.f;
    }

    float accA[32], accR[NRES ? 32 : 1], wA[GPL], wR[GPL], zA[GPL], zR[GPL];
#pragma unroll
    for (int i = 0; i < 32; ++i) accA[i] = 0.f;
#pragma unroll
    for (int i = 0; i < (NRES ? 32 : 1); ++i) accR[i] = 0.f;
#pragma unroll
    for (int gg = 0; gg < GPL; ++gg) wA[gg] = wR[gg] = zA[gg] = zR[gg] = 0.f;
    float m_run = -INFINITY, l_lane = 0.f;
    const float sm_scale = a.sm_scale;
    constexpr int DW = 4 / GPL;            // digit/nibble words per group
    const uint32_t magic = kMagic;

    auto compute = [&](int it) {
        const int tile = first + kWaves * (it / PPT);
        const int jj = (it % PPT) * SLOTS + slot;
        const bool valid = tile * kTile + jj < n;
        const int row = valid ? slot : 0;          // tail slots read the pass's first (valid) token
        const uint8_t* sp = &ring[w][it % NB][0];
        // lane's words: anchor codes, metadata (GPL pairs), per residual plane codes/meta/c
        uint32_t ka[AW], va[AW], kr[NR][RW], vr[NR][RW], krm[NR], vrm[NR], kc[NR], vc[NR];
        uint32_t kam, vam;
        {
            const uint8_t* kp = sp;
            const uint8_t* vp = sp + (PASS / 2);
#pragma unroll
            for (int q4 = 0; q4 < AW; ++q4) {
                ka[q4] = reinterpret_cast<const uint32_t*>(kp + row * (AC / SLOTS) + chunk * AB)[q4];
                va[q4] = reinterpret_cast<const uint32_t*>(vp + row * (AC / SLOTS) + chunk * AB)[q4];
            }
            if constexpr (GPL == 1) {
                kam = *reinterpret_cast<const uint16_t*>(kp + AC + row * (AM / SLOTS) + chunk * 2);
                vam = *reinterpret_cast<const uint16_t*>(vp + AC + row * (AM / SLOTS) + chunk * 2);
            } else {
                kam = *reinterpret_cast<const uint32_t*>(kp + AC + row * (AM / SLOTS) + chunk * 4);
                vam = *reinterpret_cast<const uint32_t*>(vp + AC + row * (AM / SLOTS) + chunk * 4);
            }
#pragma unroll
            for (int k = 0; k < NRES; ++k) {
                const int o = AC + AM + k * (RC + AM + CC);
#pragma unroll
                for (int q4 = 0; q4 < RW; ++q4) {
                    kr[k][q4] = reinterpret_cast<const uint32_t*>(kp + o + row * (RC / SLOTS) + chunk * 4 * RW)[q4];
                    vr[k][q4] = reinterpret_cast<const uint32_t*>(vp + o + row * (RC / SLOTS) + chunk * 4 * RW)[q4];
                }
                if constexpr (GPL == 1) {
                    krm[k] = *reinterpret_cast<const uint16_t*>(kp + o + RC + row * (AM / SLOTS) + chunk * 2);
                    vrm[k] = *reinterpret_cast<const uint16_t*>(vp + o + RC + row * (AM / SLOTS) + chunk * 2);
                } else {
                    krm[k] = *reinterpret_cast<const uint32_t*>(kp + o + RC + row * (AM / SLOTS) + chunk * 4);
                    vrm[k] = *reinterpret_cast<const uint32_t*>(vp + o + RC + row * (AM / SLOTS) + chunk * 4);
                }
                kc[k] = *reinterpret_cast<const uint16_t*>(kp + o + RC + AM + row * 2);
                vc[k] = *reinterpret_cast<const uint16_t*>(vp + o + RC + AM + row * 2);
            }
        }
        // ---------------- keys
        float part_a = 0.f;
        {
            uint32_t nib[4];
            code_nibbles<BA>(nib, ka);
#pragma unroll
            for (int gg = 0; gg < GPL; ++gg) {
                const float dot = dlq[gg] * (digit_dot<DW, 6>(nib, dq, gg * DW) + crq[gg]);
                part_a += fp8(kam, 2 * gg) * Qg[gg] + fp8(kam, 2 * gg + 1) * dot;
            }
        }
        float coef = 1.f, part_r = 0.f;
#pragma unroll
        for (int k = 0; k < NRES; ++k) {
            uint32_t nib[4];
            code_nibbles<BR>(nib, kr[k]);
            float pr = 0.f;
#pragma unroll
            for (int gg = 0; gg < GPL; ++gg) {
                const float dot = dlu[gg] * (digit_dot<DW, 4>(nib, du, gg * DW) + cru[gg]);
                pr += fp8(krm[k], 2 * gg) * Ug[gg] + fp8(krm[k], 2 * gg + 1) * dot;
            }
            part_r += coef * pr;
            coef *= bf16_to_f32(kc[k]);
        }
        float score = group_sum_dpp<LPT>(coef * part_a + part_r) * sm_scale;
        score = valid ? score : -INFINITY;
        if (wave_any(score > m_run + kRescaleSlack)) {      // rare: raise the reference
            const float m_new = wave_max_uniform(score);
            const float fs = __expf(m_run - m_new);
#pragma unroll
            for (int i = 0; i < 32; ++i) accA[i] *= fs;
#pragma unroll
            for (int i = 0; i < (NRES ? 32 : 1); ++i) accR[i] *= fs;
#pragma unroll
            for (int gg = 0; gg < GPL; ++gg) {
                wA[gg] *= fs;
                wR[gg] *= fs;
                zA[gg] *= fs;
                zR[gg] *= fs;
            }
            l_lane *= fs;
            m_run = m_new;
        }
        const float pw = valid ? __expf(score - m_run) : 0.f;
        l_lane += pw;
        // ---------------- values
        float wv = pw;
#pragma unroll
        for (int k = 0; k < NRES; ++k) {
#pragma unroll
            for (int gg = 0; gg < GPL; ++gg) {
                const float ws = wv * fp8(vrm[k], 2 * gg + 1);
                zR[gg] += wv * fp8(vrm[k], 2 * gg);
                wR[gg] += ws;
                v_acc<BR>(accR, vr[k], ws, gg * RW / GPL, RW / GPL, magic);
            }
            wv *= bf16_to_f32(vc[k]);
        }
#pragma unroll
        for (int gg = 0; gg < GPL; ++gg) {
            const float ws = wv * fp8(vam, 2 * gg + 1);
            zA[gg] += wv * fp8(vam, 2 * gg);
            wA[gg] += ws;
            v_acc<BA>(accA, va, ws, gg * AW / GPL, AW / GPL, magic);
        }
    };

    // ---- main loop: NB-1 passes in flight while one is computed from LDS
    for (int it = 0; it < n_it; ++it) {
        if (it % PPT == 0) prio_alternate(younger, it / PPT);
        if (it + NB - 1 < n_it) issue(it + NB - 1);
        wait_pass(min(NB - 1, n_it - 1 - it));
        compute(it);
    }

    // ---- undo the FP16 magic offsets, merge the waves; the last split applies R_V^T
    float v[NV];
#pragma unroll
    for (int i = 0; i < 32; ++i)
        v[i] = (accA[i] - 1024.f * wA[i / GS]) * inv_mult<BA>(i) + zA[i / GS];
    if constexpr (NRES > 0) {
#pragma unroll
        for (int i = 0; i < 32; ++i)
            v[32 + i] = (accR[i] - 1024.f * wR[i / GS]) * inv_mult<BR>(i) + zR[i / GS];
    }
    __builtin_amdgcn_s_setprio(3);                // the merge is on the critical path
    const float2 ml = splitk_merge_waves<D, NV>(v, m_run, l_lane, sm);
    splitk_finish<D, (NRES > 0)>(a.mg, bh, split, sm.sum, ml, sv[0], sm);
}

template <int D, int GS, int BA, bool QB, bool PG>
static hipError_t launch_nres(const DecodeArgs& a, int nres, dim3 grid, hipStream_t st) {
    // the anchor loop (nres 0) reads no residual plane: one instantiation for both widths
    if (nres >= 1 && a.geo.rbits(a.loop % a.geo.L) == 4) {
        if (nres == 1) {
            hipLaunchKernelGGL((rq_decode_kernel<D, GS, BA, 4, 1, QB, PG>), grid, dim3(kThreads), 0, st, a);
            return hipGetLastError();
        }
        if (nres != 0) return hipErrorInvalidValue;  // 4-bit residuals: shared anchor only
    }
    switch (nres) {
        case 0: hipLaunchKernelGGL((rq_decode_kernel<D, GS, BA, 2, 0, QB, PG>), grid, dim3(kThreads), 0, st, a); break;
        case 1: hipLaunchKernelGGL((rq_decode_kernel<D, GS, BA, 2, 1, QB, PG>), grid, dim3(kThreads), 0, st, a); break;
        case 2: hipLaunchKernelGGL((rq_decode_kernel<D, GS, BA, 2, 2, QB, PG>), grid, dim3(kThreads), 0, st, a); break;
        case 3: hipLaunchKernelGGL((rq_decode_kernel<D, GS, BA, 2, 3, QB, PG>), grid, dim3(kThreads), 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <int D, int GS, int BA>
static hipError_t launch_q(const DecodeArgs& a, int nres, bool qbf16, dim3 grid, hipStream_t st) {
    if (a.geo.bt != nullptr)
        return qbf16 ? launch_nres<D, GS, BA, true, true>(a, nres, grid, st)
                     : launch_nres<D, GS, BA, false, true>(a, nres, grid, st);
    return qbf16 ? launch_nres<D, GS, BA, true, false>(a, nres, grid, st)
                 : launch_nres<D, GS, BA, false, false>(a, nres, grid, st);
}

hipError_t launch_decode(const DecodeArgs& a, int nres, bool qbf16, hipStream_t st) {
    if (!a.cache || !a.q || !a.rot || !a.ctx_len || !a.mg.partials || !a.mg.arrivals || !a.mg.k_cur ||
        !a.mg.v_cur || !a.mg.out || !a.mg.rot || a.batch < 1 || a.n_splits < 1 || a.n_splits > kMaxSplits ||
        a.mg.n_splits != a.n_splits || a.mg.rec_splits < a.n_splits)
        return hipErrorInvalidValue;
    if (gqa_supported(a.geo, a.loop, nres)) return launch_decode_gqa(a, nres, qbf16, st);
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
