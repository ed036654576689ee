// rq_decode_attention for grouped-query attention: one workgroup per (batch row, KV head,
// split) serves all G query heads of the KV head, so every packed tile is read from HBM
// once and dequantized once for the group (arXiv digest: Huginn-3.5B runs 32 query heads
// on 8 KV heads; explainer, paragraph on the master print: rebuild on chip only).
//
// With G queries sharing a tile the work per byte is G times that of one query, so the
// products run on the matrix cores (v_mfma_f32_16x16x32_f16) on exact small integers:
//  * keys: D[(q, g)][token] = sum_{c in group g} (q_c / m_c) * (m_c * code_c), where m_c is
//    the power of two at which a code sits inside its FP16 magic number (1024 + m_c code),
//    so B is the exact integer m_c * code after subtracting 1024.  A holds q (or
//    u = R_K q for the residual plane) split into two FP16 terms (hi + lo, 22 significant
//    bits) and is block-diagonal over the 4 channel groups, so one 16x16 result holds
//    the 4 group dot products of 4 queries for 16 tokens.  The score is then
//    sum_g z_g sum(q over g) + s_g D_g per plane, as in the one-query kernel.
//  * values: D[q][channel] += sum_t (w_qt / m_t) (m_t code_tc), K = 32 tokens, with
//    w = p c s_a (anchor) or p s_r (residual).  The token-major codes are turned into
//    the channel-major B operand by the LDS transpose read ds_read_b64_tr_b4, which
//    gives each lane one 4-bit column of 16 rows (rows = 8-byte chunks named by the
//    16 lanes of its group).  The weights go through LDS as FP16 in the same K order
//    (the anchor weight as hi + lo terms, the residual weight as one term); the group
//    offsets z accumulate separately in float32.
// The split-K merge is the same as the one-query kernel's, run for each query head.
#include "rq_args.hpp"
#include "rq_merge_group.hpp"
#include "rq_splitk.hpp"
#include "rq_stage.hpp"

namespace rq {
namespace gqa {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));
typedef int v2i __attribute__((ext_vector_type(2)));

constexpr int D = 128, GS = 32, NG = D / GS;     // head dim, group size, groups
constexpr int BT = 32;                           // tokens per block (a wave's unit of work)
constexpr int AROW = D / 2, RROW = D / 4, MROW = 2 * NG;   // bytes per token row
constexpr int AC = BT * AROW, AM = BT * MROW, RC = BT * RROW, RM = BT * MROW, CC = BT * 2;
constexpr int NB = 2;                            // ring slots (blocks) per wave
constexpr int NW = 8, NT = NW * kWave;           // waves and threads per workgroup (one per CU)
constexpr uint32_t kMagic2 = 0x64006400u;
// The value weights p c s_a and p s_r (p = exp(score - reference)) are rounded to FP16 for
// the matrix cores, whose largest finite value is 65504.  With the reference raised whenever
// a score exceeds it by more than 4, p <= e^4 < 54.6.  s_r <= 448, and |c| s_a <= 0.16 |x|
// (|c| <= |x| / |a_hat| by Cauchy-Schwarz; s_a <= 1.125 * (2 + 1/8) max|a_hat| / 15, the
// offset lying at most an eighth below the group minimum), at most 810 for d = 128 inputs in
// the E4M3 range: every weight stays below 44,300.  A larger slack would let p reach e^8 and
// the anchor weights overflow once |c| s_a exceeds 22; a smaller one pushes more weights of
// tokens that still matter into FP16's subnormal range.
constexpr float kSlack = 4.0f;

__device__ __forceinline__ uint32_t gload4(const uint8_t* sbase, uint32_t voff) {
    uint32_t r;
    asm volatile("global_load_dword %0, %1, %2" : "=v"(r) : "v"(voff), "s"(sbase));
    return r;
}

// (x & mask) | magic, then minus 1024 in both halves: the exact integers m * code
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(kMagic2));
    return r;
}
__device__ __forceinline__ uint32_t unmagic(uint32_t r) {
    const h2 v = __builtin_bit_cast(h2, r) - (h2){(_Float16)1024.0f, (_Float16)1024.0f};
    return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ h8 pack_h8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    const u4 v = {a, b, c, d};
    return __builtin_bit_cast(h8, v);
}

// 8 channels of a 4-bit code word -> K order [0,4,1,5,2,6,3,7], weights [1,1,16,16,1,1,16,16]
__device__ __forceinline__ h8 b_from_nibbles(uint32_t w) {
    const uint32_t w8 = w >> 8;
    return pack_h8(unmagic(and_or(w, 0x000F000Fu)), unmagic(and_or(w, 0x00F000F0u)),
                   unmagic(and_or(w8, 0x000F000Fu)), unmagic(and_or(w8, 0x00F000F0u)));
}
// 8 channels of a 2-bit code word (bits 0-7 and 16-23 after the caller's shift) -> K order
// [0,8,1,9,2,10,3,11] (+4 for the shifted half), weights [1,1,4,4,16,16,64,64]
__device__ __forceinline__ h8 b_from_crumbs(uint32_t w) {
    return pack_h8(unmagic(and_or(w, 0x00030003u)), unmagic(and_or(w, 0x000C000Cu)),
                   unmagic(and_or(w, 0x00300030u)), unmagic(and_or(w, 0x00C000C0u)));
}

// key operands keep the magic offset: D = 1024 sum(A) + sum(q code); the constant is removed
// per (query, group) in the score
__device__ __forceinline__ h8 b_magic_nibbles(uint32_t w) {
    const uint32_t w8 = w >> 8;
    return pack_h8(and_or(w, 0x000F000Fu), and_or(w, 0x00F000F0u), and_or(w8, 0x000F000Fu), and_or(w8, 0x00F000F0u));
}
__device__ __forceinline__ h8 b_magic_crumbs(uint32_t w) {
    return pack_h8(and_or(w, 0x00030003u), and_or(w, 0x000C000Cu), and_or(w, 0x00300030u), and_or(w, 0x00C000C0u));
}

__device__ __forceinline__ float fp8(uint32_t word, int byte) {
    switch (byte) {
        case 0: return __builtin_amdgcn_cvt_f32_fp8((int)word, 0);
        case 1: return __builtin_amdgcn_cvt_f32_fp8((int)word, 1);
        case 2: return __builtin_amdgcn_cvt_f32_fp8((int)word, 2);
        default: return __builtin_amdgcn_cvt_f32_fp8((int)word, 3);
    }
}

__device__ __forceinline__ f32x4 mfma(h8 a, h8 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// over the 16 lanes of a DPP row (one query in the score layout)
__device__ __forceinline__ float row_max16(float v) {
    v = fmaxf(v, dpp<0xB1>(v));
    v = fmaxf(v, dpp<0x4E>(v));
    v = fmaxf(v, dpp<0x141>(v));
    v = fmaxf(v, dpp<0x140>(v));
    return v;
}
__device__ __forceinline__ float row_sum16(float v) {
    v += dpp<0xB1>(v);
    v += dpp<0x4E>(v);
    v += dpp<0x141>(v);
    v += dpp<0x140>(v);
    return v;
}

// LDS of one workgroup
template <int G, int NRES>
struct Smem {
    static constexpr int PASS = 2 * (AC + AM + NRES * (RC + RM + CC));
    uint8_t ring[NW][NB][PASS];                          // also the epilogue's scratch
    _Float16 wbuf[NW][3][NG][G][BT];                     // value weights in MFMA K order: anchor hi, anchor lo, residual
    h8 akey[4][NG][kWave];                               // key A operands: q hi, q lo, u hi, u lo
    float sq[G][D];                                      // queries (float32)
    float su[G][D];                                      // u = R_K q
    float qsum[2][G][NG];                                // group sums of q and of u
    float koff[2][G][NG];                                // 1024 * sum of the key A values
    float mw[NW][G], lw[NW][G];
};

// token position in the value K order and its FP16 magic weight
__device__ __forceinline__ int vpos(int t) {
    const int e = t & 7;
    return 8 * (t >> 3) + 2 * (e & 3) + (e >> 2);
}

template <int G, int NRES, bool QBF16, bool PAGED>
__global__ __launch_bounds__(NT) void rq_decode_gqa_kernel(DecodeArgs a) {
    static_assert(G == 2 || G == 4, "2 or 4 query heads per KV head");
    constexpr int PASS = Smem<G, NRES>::PASS;
    constexpr int NDMA = 2 * (3 + 3 * NRES);             // DMA instructions per block
    constexpr int RES_OFF = AC + AM;                      // residual section inside a plane
    constexpr int PLANE = PASS / 2;
    __shared__ Smem<G, NRES> sm;

    const Geom& Gm = a.geo;
    const int lb = xcd_logical_block(blockIdx.x, gridDim.x);
    const int split = lb % a.n_splits;
    const int bk = lb / a.n_splits;                      // b * Hkv + h
    const int h = bk % Gm.hkv, b = bk / Gm.hkv;
    const int bh0 = b * Gm.hq + h * G;                   // first query head of the group
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int l16 = lane & 15, kg = lane >> 4;

    int n = a.ctx_len[b];
    n = n < 0 ? 0 : (n > a.ctx_bound ? a.ctx_bound : n);
    const int n_tiles = (n + kTile - 1) / kTile;
    const int t_begin = split * a.tiles_per_split;
    const int t_end = min(n_tiles, t_begin + a.tiles_per_split);
    // blocks of this split, dealt to the waves round-robin
    const int blk0 = 2 * t_begin, blk1 = min(2 * t_end, (n + BT - 1) / BT);
    const int first = blk0 + w;
    const int n_it = first < blk1 ? (blk1 - first + NW - 1) / NW : 0;

    const int L = Gm.L;
    const int aloop = (a.loop / L) * L + L - 1;
    const uint8_t* aK = a.cache + Gm.plane_offset(b, h, 0, aloop);
    const uint8_t* aV = a.cache + Gm.plane_offset(b, h, 1, aloop);
    const uint8_t* rK = a.cache + Gm.plane_offset(b, h, 0, a.loop);
    const uint8_t* rV = a.cache + Gm.plane_offset(b, h, 1, a.loop);
    const uint32_t a_meta = kTile * AROW, r_meta = kTile * RROW, r_cblk = kTile * (RROW + MROW);

    // Paged layout: the physical block of each block's tile is read through the scalar cache
    // one block ahead (the first one here, at the top of the prologue).
    int pblk_cur = 0, pblk_nxt = 0;
    if constexpr (PAGED) {
        if (n_it > 0) pblk_nxt = block_id_scalar(Gm, b, first >> 1);
    }

    const uint32_t ring_base = __builtin_amdgcn_readfirstlane(lds_addr_of(&sm.ring[w][0][0]));
    // The residual code rows land swizzled: the 16-byte chunk j of token t at slot
    // j ^ ((t >> 2) & 1) of its 32-byte row, so that a read of one chunk column over 16
    // tokens (the key words, the transposed value reads) spreads over the LDS banks.  Each
    // DMA lane fetches the chunk its slot holds.
    const uint32_t r_swz = 16u * ((lane & ~1u) | ((lane & 1u) ^ ((lane >> 3) & 1u)));
    const uint32_t hr = (l16 >> 2) & 1;                  // the swizzle of the lane's tokens
    auto issue = [&](int it) {
        const uint32_t blk = first + NW * it;
        const uint32_t tile = blk >> 1, hb = blk & 1;
        uint32_t dst = ring_base + (uint32_t)(it % NB) * PASS;
        if constexpr (PAGED) {
            pblk_cur = pblk_nxt;
            if (it + 1 < n_it) pblk_nxt = block_id_scalar(Gm, b, (int)((blk + NW) >> 1));
        }
        const uint32_t ta = PAGED ? 0u : tile * (uint32_t)Gm.a_tile, tr = PAGED ? 0u : tile * (uint32_t)Gm.rtile(a.loop % L);
#pragma unroll
        for (int x = 0; x < 2; ++x) {
            const uint8_t* ap = PAGED ? uniform_ptr(a.cache + Gm.paged_offset(pblk_cur, h, x, aloop)) : (x ? aV : aK);
            stage<1024, PAGED>(ap, ta + hb * AC, dst, lane);
            stage<1024, PAGED>(ap, ta + hb * AC + 1024, dst + 1024, lane);
            stage<AM, PAGED>(ap, ta + a_meta + hb * AM, dst + AC, lane);
            if constexpr (NRES > 0) {
                const uint8_t* rp = PAGED ? uniform_ptr(a.cache + Gm.paged_offset(pblk_cur, h, x, a.loop)) : (x ? rV : rK);
                static_assert(RC == 1024, "one DMA per block of residual rows");
                dma16<PAGED, true>(tr + hb * RC + r_swz, rp, dst + RES_OFF);
                stage<RM, PAGED>(rp, tr + r_meta + hb * RM, dst + RES_OFF + RC, lane);
                stage<CC, PAGED, false>(rp, tr + r_cblk + hb * CC, dst + RES_OFF + RC + RM, lane);   // line shared by the tile's two blocks
            }
            dst += PLANE;
        }
    };
    static_assert((NB - 1) * NDMA <= 63, "vmcnt");
    auto wait_pass = [&](int ahead) {
        if (ahead >= 1) wait_vm<NDMA>();
        else wait_vm<0>();
    };

    // ---- prologue: q of the G heads and R_K (residual loops), loaded before the first DMAs
    constexpr int C4 = D / 4, RPL = NT / C4, RL = D / RPL;         // 32, 16, 8
    const int c4 = threadIdx.x % C4;
    f32x4 rq4[NRES ? RL : 1];
    u4 qraw[G];
    {
        const int64_t qrow = (int64_t)bh0 * D;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if constexpr (QBF16) {
                const uint8_t* qb = static_cast<const uint8_t*>(a.q) + (qrow + g * D) * 2;
                qraw[g] = u4{gload4(qb, (uint32_t)c4 * 8u), gload4(qb, (uint32_t)c4 * 8u + 4u), 0u, 0u};
            } else {
                const uint8_t* qb = static_cast<const uint8_t*>(a.q) + (qrow + g * D) * 4;
                qraw[g] = __builtin_bit_cast(u4, gload16(qb, (uint32_t)c4 * 16u));
            }
        }
        if constexpr (NRES > 0) {
            const uint8_t* rb = reinterpret_cast<const uint8_t*>(a.rot + (int64_t)(h * 2) * D * D);
#pragma unroll
            for (int k = 0; k < RL; ++k) rq4[k] = gload16(rb, (uint32_t)(k * NT + threadIdx.x) * 16u);
        }
    }
    const int n_pre = min(NB - 1, n_it);
    for (int k = 0; k < n_pre; ++k) issue(k);
    wait_pass(n_pre);
    f32x4 qf[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        pin(qraw[g]);
        if constexpr (QBF16) {
            qf[g] = f32x4{bf16lo(qraw[g].x), bf16hi(qraw[g].x), bf16lo(qraw[g].y), bf16hi(qraw[g].y)};
        } else {
            qf[g] = __builtin_bit_cast(f32x4, qraw[g]);
        }
        if (threadIdx.x < C4) {
#pragma unroll
            for (int e = 0; e < 4; ++e) sm.sq[g][4 * c4 + e] = qf[g][e];
        }
    }
    if constexpr (NRES > 0) {
        // u_g = R_K q_g: partial dots of the thread's 16 rows, summed over the 32 lanes of a row
        float pr[RL * G];
#pragma unroll
        for (int k = 0; k < RL; ++k) {
            pin(rq4[k]);
#pragma unroll
            for (int g = 0; g < G; ++g)
                pr[k * G + g] = rq4[k].x * qf[g].x + rq4[k].y * qf[g].y + rq4[k].z * qf[g].z + rq4[k].w * qf[g].w;
        }
        int off = 0;
        group_reduce_scatter<RL * G, C4 / 2, RL * G>(pr, lane, off);
        // the lane now holds the 32-lane sums of values [off, off + RL*G/32); with fewer values
        // than lanes (G = 2) it holds one, which its butterfly partners hold as well
        constexpr int KEEP = RL * G / 32 > 0 ? RL * G / 32 : 1;
#pragma unroll
        for (int i = 0; i < KEEP; ++i) {
            const int v = off + i, k = v / G, g = v % G;
            sm.su[g][k * RPL + threadIdx.x / C4] = pr[i];
        }
    }
    __syncthreads();
    // group sums of q and u (for the offsets z), one thread per (plane, query, group), on the
    // upper waves (the lower four build the key operands below at the same time)
    if (threadIdx.x >= NT - 2 * G * NG) {
        const int tq = threadIdx.x - (NT - 2 * G * NG);
        const int pl = tq / (G * NG), g = (tq / NG) % G, gi = tq % NG;
        const float* src = pl ? sm.su[g] : sm.sq[g];
        float s = 0.f, off = 0.f;
        if (pl == 0 || NRES > 0) {
            for (int c = 0; c < GS; ++c) {
                const float v = src[GS * gi + c];
                s += v;
                // the key A value of channel c, as the MFMA sees it (FP16 hi + lo)
                const float a = pl ? ldexpf(v, -2 * (c & 3)) : ((c & 1) ? v * 0.0625f : v);
                const _Float16 hi = (_Float16)a;
                off += (float)hi + (float)(_Float16)(a - (float)hi);
            }
        }
        sm.qsum[pl][g][gi] = s;
        sm.koff[pl][g][gi] = 1024.f * off;
    }
    // A operands of the key products, shared by the waves: lane (m = 4 qh + g', kg) holds
    // row m, K elements 8 kg .. 8 kg + 7 of channel group gi, nonzero only where g' == gi.
    // Thread t < 4 * 64 builds kind t / 64 (q hi, q lo, u hi, u lo) for lane t % 64.
    if (threadIdx.x < 4 * kWave) {
        const int kind = threadIdx.x / kWave, L = threadIdx.x % kWave;
        const int ll = L & 15, lk = L >> 4, qh_a = ll >> 2, ga = ll & 3;
        h8 frag;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            float v;
            if (kind < 2) {
                const int e = (k >> 1) + 4 * (k & 1);                      // [0,4,1,5,2,6,3,7]
                const float m = (k & 2) ? (1.f / 16.f) : 1.f;              // [1,1,16,16,...]^-1
                v = qh_a < G ? sm.sq[qh_a][GS * ga + 8 * lk + e] * m : 0.f;
            } else {
                const int e = (k >> 1) + 8 * (k & 1) + 4 * (lk & 1);       // [0,8,1,9,...] (+4)
                const float m = k < 2 ? 1.f : (k < 4 ? 0.25f : (k < 6 ? 1.f / 16.f : 1.f / 64.f));
                v = (NRES > 0 && qh_a < G) ? sm.su[qh_a][GS * ga + 16 * (lk >> 1) + e] * m : 0.f;
            }
            const _Float16 hi = (_Float16)v;
            frag[k] = (kind & 1) ? (_Float16)(v - (float)hi) : hi;
        }
        const h8 z8 = {};
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) sm.akey[kind][gi][L] = gi == ga ? frag : z8;
    }
    __syncthreads();
    // score-layout lane: token l16 of a 16-token round, query kg
    const int qs = kg;
    const bool q_ok = qs < G;
    float Qs[NG], Us[NG], Ca[NG], Cu[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        Qs[gi] = q_ok ? sm.qsum[0][qs][gi] : 0.f;
        Us[gi] = q_ok ? sm.qsum[1][qs][gi] : 0.f;
        Ca[gi] = q_ok ? sm.koff[0][qs][gi] : 0.f;
        Cu[gi] = q_ok ? sm.koff[1][qs][gi] : 0.f;
    }

    // value accumulators: 8 anchor N-blocks (16 channels each) and 8 residual N-blocks
    f32x4 va[8], vr[NRES ? 8 : 1];
#pragma unroll
    for (int i = 0; i < 8; ++i) va[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < (NRES ? 8 : 1); ++i) vr[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float zA[NG], zR[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) zA[gi] = zR[gi] = 0.f;
    float m_run = -INFINITY, l_lane = 0.f;
    const float sm_scale = a.sm_scale;

    for (int it = 0; it < n_it; ++it) {
        if (it % 2 == 0) prio_alternate(w >= NW / 2, it / 2);
        if (it + NB - 1 < n_it) issue(it + NB - 1);
        wait_pass(min(NB - 1, n_it - 1 - it));
        const uint8_t* sp = &sm.ring[w][it % NB][0];
        const uint8_t* vp = sp + PLANE;
        const int blk = first + NW * it;
        const int tok0 = blk * BT;

        // ---- keys: scores of both 16-token rounds first (independent work the compiler can
        // interleave), then one rescale check for the 32 tokens, then the weights
        float sc[2];
        bool vl[2];
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int t = 16 * r + l16;                   // token of this lane's B column
            f32x4 da = {0.f, 0.f, 0.f, 0.f}, dr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const uint32_t wa = *reinterpret_cast<const uint32_t*>(sp + t * AROW + (4 * gi + kg) * 4);
                const h8 bq = b_magic_nibbles(wa);
                da = mfma(sm.akey[0][gi][lane], bq, da);
                da = mfma(sm.akey[1][gi][lane], bq, da);
                if constexpr (NRES > 0) {
                    uint32_t wr = *reinterpret_cast<const uint32_t*>(sp + RES_OFF + t * RROW + 16 * ((gi >> 1) ^ hr) +
                                                                      4 * ((2 * gi + (kg >> 1)) & 3));
                    wr = (kg & 1) ? (wr >> 8) : wr;
                    const h8 bu = b_magic_crumbs(wr);
                    dr = mfma(sm.akey[3][gi][lane], bu, mfma(sm.akey[2][gi][lane], bu, dr));
                }
            }
            // score of (token t, query qs): this lane holds the 4 group products in da / dr
            const uint2 am = *reinterpret_cast<const uint2*>(sp + AC + t * MROW);
            float part_a = 0.f;
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const uint32_t mw = gi < 2 ? am.x : am.y;
                part_a += fp8(mw, 2 * (gi & 1)) * Qs[gi] + fp8(mw, 2 * (gi & 1) + 1) * (da[gi] - Ca[gi]);
            }
            float coef = 1.f, part_r = 0.f;
            if constexpr (NRES > 0) {
                const uint2 rm = *reinterpret_cast<const uint2*>(sp + RES_OFF + RC + t * MROW);
#pragma unroll
                for (int gi = 0; gi < NG; ++gi) {
                    const uint32_t mw = gi < 2 ? rm.x : rm.y;
                    part_r += fp8(mw, 2 * (gi & 1)) * Us[gi] + fp8(mw, 2 * (gi & 1) + 1) * (dr[gi] - Cu[gi]);
                }
                coef = bf16_to_f32(*reinterpret_cast<const uint16_t*>(sp + RES_OFF + RC + RM + t * 2));
            }
            vl[r] = q_ok && (tok0 + t < n);
            const float score = (coef * part_a + part_r) * sm_scale;
            sc[r] = vl[r] ? score : -INFINITY;
        }
        const float smax = fmaxf(sc[0], sc[1]);
        if (wave_any(smax > m_run + kSlack)) {            // rare: raise the reference of each query
            const float m_new = fmaxf(m_run, row_max16(smax));
            const float fs = m_run == -INFINITY ? 0.f : __expf(m_run - m_new);
            float fq[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) fq[q] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(fs), 16 * q));
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int q = 0; q < 4; ++q) va[i][q] *= fq[q];
            if constexpr (NRES > 0) {
#pragma unroll
                for (int i = 0; i < 8; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q) vr[i][q] *= fq[q];
            }
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                zA[gi] *= fs;
                zR[gi] *= fs;
            }
            l_lane *= fs;
            m_run = m_new;
        }
        // ---- softmax weights of both rounds
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int t = 16 * r + l16;
            const bool valid = vl[r];
            const float p = valid ? __expf(sc[r] - m_run) : 0.f;
            l_lane += p;
            // value weights from the V plane's metadata and coefficient: anchor p c s_a,
            // residual p s_r (zero for masked tokens), and the offsets
            // a masked token's metadata and coefficient read as zero (its bytes may be anything,
            // NaN patterns included), so with p = 0 every product below is an exact zero
            uint2 vam = *reinterpret_cast<const uint2*>(vp + AC + t * MROW);
            uint2 vrm = {0u, 0u};
            float vcoef = 1.f;
            if constexpr (NRES > 0) {
                vrm = *reinterpret_cast<const uint2*>(vp + RES_OFF + RC + t * MROW);
                vcoef = bf16_to_f32(*reinterpret_cast<const uint16_t*>(vp + RES_OFF + RC + RM + t * 2));
            }
            if (!valid) {
                vam = uint2{0u, 0u};
                vrm = uint2{0u, 0u};
                vcoef = 0.f;
            }
            const int pos = vpos(t);
            const float mult = (t & 1) ? (1.f / 16.f) : 1.f;
            const float pc = p * vcoef;
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                const uint32_t mw = gi < 2 ? vam.x : vam.y;
                const float za = fp8(mw, 2 * (gi & 1)), sa = fp8(mw, 2 * (gi & 1) + 1);
                zA[gi] += pc * za;
                const float wa = pc * sa * mult;
                // the anchor weight as two FP16 terms (about 22 significant bits): the anchor part
                // carries most of the output, so its weights get the second term
                const _Float16 wa_hi = (_Float16)wa;
                if (q_ok) {
                    sm.wbuf[w][0][gi][qs][pos] = wa_hi;
                    sm.wbuf[w][1][gi][qs][pos] = (_Float16)(wa - (float)wa_hi);
                }
                if constexpr (NRES > 0) {
                    const uint32_t rw = gi < 2 ? vrm.x : vrm.y;
                    const float zr = fp8(rw, 2 * (gi & 1)), sr = fp8(rw, 2 * (gi & 1) + 1);
                    zR[gi] += p * zr;
                    const float wr = p * sr * mult;
                    if (q_ok) sm.wbuf[w][2][gi][qs][pos] = (_Float16)wr;
                }
            }
        }

        // ---- values: K = the 32 tokens of the block, N = 16 channels per product
        // A: lane (m = query, kg) reads the 8 weights of tokens 8kg.. in K order.  Rows m >= G
        // hold a copy of row m mod G: their results are never read (the epilogue takes rows
        // 0..G-1), and a real row costs no zero fill in the loop.
        const int mrow = l16 & (G - 1);
        h8 wa8[NG], wl8[NG], wr8[NG];
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            wa8[gi] = *reinterpret_cast<const h8*>(&sm.wbuf[w][0][gi][mrow][8 * kg]);
            wl8[gi] = *reinterpret_cast<const h8*>(&sm.wbuf[w][1][gi][mrow][8 * kg]);
            if constexpr (NRES > 0) wr8[gi] = *reinterpret_cast<const h8*>(&sm.wbuf[w][2][gi][mrow][8 * kg]);
        }
        // transpose reads: lane l16 of group kg names row (token 8kg + l16 % 8, chunk c0 + l16 / 8)
        typedef __attribute__((address_space(3))) v2i* lp;
        const uint32_t vbase = lds_addr_of(vp);
#pragma unroll
        for (int nb2 = 0; nb2 < NG; ++nb2) {              // anchor: 16-channel chunks 2nb2, 2nb2+1
            const uint32_t addr = vbase + (8 * kg + (l16 & 7)) * AROW + (2 * nb2 + (l16 >> 3)) * 8;
            const v2i tv = __builtin_amdgcn_ds_read_tr4_b64_v2i32((lp)(uintptr_t)addr);
            const h8 bx = b_from_nibbles((uint32_t)tv.x), by = b_from_nibbles((uint32_t)tv.y);
            va[2 * nb2] = mfma(wl8[nb2], bx, mfma(wa8[nb2], bx, va[2 * nb2]));
            va[2 * nb2 + 1] = mfma(wl8[nb2], by, mfma(wa8[nb2], by, va[2 * nb2 + 1]));
        }
        if constexpr (NRES > 0) {
#pragma unroll
            for (int cp = 0; cp < 2; ++cp) {               // residual: 32-channel chunks 2cp, 2cp+1
                const uint32_t addr = vbase + RES_OFF + (8 * kg + (l16 & 7)) * RROW + 16 * (cp ^ hr) + 8 * (l16 >> 3);
                const v2i tv = __builtin_amdgcn_ds_read_tr4_b64_v2i32((lp)(uintptr_t)addr);
#pragma unroll
                for (int hw = 0; hw < 2; ++hw) {
                    const uint32_t wd = hw ? (uint32_t)tv.y : (uint32_t)tv.x;
                    const int chunk = 2 * cp + hw;
                    // even channels 2j: crumbs at bits 0-1 of each nibble; odd: bits 2-3 (x4)
                    const uint32_t w8 = wd >> 8;
                    const h8 be = pack_h8(unmagic(and_or(wd, 0x00030003u)), unmagic(and_or(wd, 0x00300030u)),
                                          unmagic(and_or(w8, 0x00030003u)), unmagic(and_or(w8, 0x00300030u)));
                    const h8 bo = pack_h8(unmagic(and_or(wd, 0x000C000Cu)), unmagic(and_or(wd, 0x00C000C0u)),
                                          unmagic(and_or(w8, 0x000C000Cu)), unmagic(and_or(w8, 0x00C000C0u)));
                    vr[2 * chunk] = mfma(wr8[chunk], be, vr[2 * chunk]);
                    vr[2 * chunk + 1] = mfma(wr8[chunk], bo, vr[2 * chunk + 1]);
                }
            }
        }
    }

    // ---- epilogue: per-query sums of the wave, merged over the waves in LDS
    __builtin_amdgcn_s_setprio(3);
    // offsets and denominators of the lane's query, summed over its 16 tokens
    const float l_q = row_sum16(l_lane);
    float zAq[NG], zRq[NG];
#pragma unroll
    for (int gi = 0; gi < NG; ++gi) {
        zAq[gi] = row_sum16(zA[gi]);
        zRq[gi] = row_sum16(zR[gi]);
    }
    __syncthreads();                                      // ring is free: every DMA has landed
    float* scr = reinterpret_cast<float*>(&sm.ring[0][0][0]);   // [NW][G][2D]
    static_assert((NW * G * 2 * D + NW * 2 * G * NG) * sizeof(float) <= sizeof(sm.ring), "epilogue scratch");
    if (l16 == 0 && q_ok) {
        sm.mw[w][qs] = m_run;
        sm.lw[w][qs] = l_q;
    }
    // offsets per (query, group) to LDS first (lane 0 of each query row)
    float* zsc = scr + NW * G * 2 * D;                    // [NW][2][G][NG] after the values
    if (l16 == 0 && q_ok) {
#pragma unroll
        for (int gi = 0; gi < NG; ++gi) {
            zsc[((w * 2 + 0) * G + qs) * NG + gi] = zAq[gi];
            zsc[((w * 2 + 1) * G + qs) * NG + gi] = zRq[gi];
        }
    }
    __syncthreads();
    // workgroup maximum per query, and this wave's scale towards it (the denominators are
    // only needed by the threads that publish them, below)
    float sc_w[G], m_wg[G];
#pragma unroll
    for (int q = 0; q < G; ++q) {
        m_wg[q] = -INFINITY;
#pragma unroll
        for (int i = 0; i < NW; ++i) m_wg[q] = fmaxf(m_wg[q], sm.mw[i][q]);
        const float mw = sm.mw[w][q];
        sc_w[q] = mw == -INFINITY ? 0.f : __expf(mw - m_wg[q]);
    }
    // values of lanes 0..15 (rows = queries) -> scr[w][q][channel], plus the offsets
    if (kg == 0) {
        // every offset first: the stores below go to the same array, and reads placed
        // after them would each wait for the store before
        float za[G][NG], zr[G][NG];
#pragma unroll
        for (int q = 0; q < G; ++q) {
#pragma unroll
            for (int gi = 0; gi < NG; ++gi) {
                za[q][gi] = zsc[((w * 2 + 0) * G + q) * NG + gi];
                zr[q][gi] = NRES > 0 ? zsc[((w * 2 + 1) * G + q) * NG + gi] : 0.f;
            }
        }
#pragma unroll
        for (int q = 0; q < G; ++q) {
            float* dst = scr + ((w * G) + q) * 2 * D;
#pragma unroll
            for (int nb = 0; nb < 8; ++nb) {
                const int c = 16 * nb + l16;                  // channel group c / GS = 16 nb / GS
                dst[c] = (va[nb][q] + za[q][16 * nb / GS]) * sc_w[q];
            }
            if constexpr (NRES > 0) {
#pragma unroll
                for (int nb = 0; nb < 8; ++nb) {
                    const int chunk = nb >> 1, par = nb & 1;
                    const int c = GS * chunk + 2 * l16 + par;
                    const float v = par ? vr[nb][q] * 0.25f : vr[nb][q];
                    dst[D + c] = (v + zr[q][chunk]) * sc_w[q];
                }
            }
        }
    }
    __syncthreads();
    // publish the G records (sums over the waves), then count the arrival
    constexpr int NV = NRES ? 2 * D : D;
    for (int idx = threadIdx.x; idx < G * NV; idx += NT) {
        const int q = idx / NV, c = idx % NV;
        float v = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i) v += scr[((i * G) + q) * 2 * D + c];
        st_agent(a.mg.partials + ((int64_t)(bh0 + q) * a.mg.rec_splits + split) * (2 * D + 4) + c, v);
    }
    if (threadIdx.x < G) {
        const int q = threadIdx.x;
        float m_q = -INFINITY, l_q = 0.f;
#pragma unroll
        for (int i = 0; i < NW; ++i) m_q = fmaxf(m_q, sm.mw[i][q]);
#pragma unroll
        for (int i = 0; i < NW; ++i)
            if (sm.mw[i][q] != -INFINITY) l_q += __expf(sm.mw[i][q] - m_q) * sm.lw[i][q];
        float* rec = a.mg.partials + ((int64_t)(bh0 + q) * a.mg.rec_splits + split) * (2 * D + 4);
        st_agent(rec + 2 * D, m_q);
        st_agent(rec + 2 * D + 1, l_q);
    }
    if (!splitk_arrive(a.mg, bh0)) return;
    merge_group<D, NT, G, (NRES > 0)>(a.mg, bh0, sm.sq, reinterpret_cast<float*>(&sm.ring[0][0][0]));
}

template <int G, int NRES>
static hipError_t launch_q(const DecodeArgs& a, bool qbf16, dim3 grid, hipStream_t st) {
    if (a.geo.bt != nullptr) {
        if (qbf16) hipLaunchKernelGGL((rq_decode_gqa_kernel<G, NRES, true, true>), grid, dim3(NT), 0, st, a);
        else hipLaunchKernelGGL((rq_decode_gqa_kernel<G, NRES, false, true>), grid, dim3(NT), 0, st, a);
    } else {
        if (qbf16) hipLaunchKernelGGL((rq_decode_gqa_kernel<G, NRES, true, false>), grid, dim3(NT), 0, st, a);
        else hipLaunchKernelGGL((rq_decode_gqa_kernel<G, NRES, false, false>), grid, dim3(NT), 0, st, a);
    }
    return hipGetLastError();
}

}  // namespace gqa

bool gqa_supported(const Geom& g, int loop, int nres) {
    const int gq = g.hq / g.hkv;
    return g.d == gqa::D && g.g == gqa::GS && g.ba == 4 && (nres == 0 || g.rbits(loop % g.L) == 2) && nres <= 1 &&
           (gq == 2 || gq == 4);
}

hipError_t launch_decode_gqa(const DecodeArgs& a, int nres, bool qbf16, hipStream_t st) {
    if (!gqa_supported(a.geo, a.loop, nres) || !a.cache || !a.q || !a.rot || !a.ctx_len || !a.mg.partials ||
        !a.mg.arrivals || !a.mg.k_cur || !a.mg.v_cur || !a.mg.out || a.batch < 1 || a.n_splits < 1 ||
        a.n_splits > kMaxSplits || a.mg.n_splits != a.n_splits || a.mg.rec_splits < a.n_splits)
        return hipErrorInvalidValue;
    const int gq = a.geo.hq / a.geo.hkv;
    const dim3 grid(a.batch * a.geo.hkv * a.n_splits);
    if (gq == 4) return nres ? gqa::launch_q<4, 1>(a, qbf16, grid, st) : gqa::launch_q<4, 0>(a, qbf16, grid, st);
    return nres ? gqa::launch_q<2, 1>(a, qbf16, grid, st) : gqa::launch_q<2, 0>(a, qbf16, grid, st);
}

}  // namespace rq
