// rq_pack: quantize finished tokens of one anchor group into the packed cache.
//
// ResidualQuant explainer, paragraph on the master print: the last loop is the INT4
// anchor, each earlier loop stores residual = KV(loop) - c * anchor with a per-vector
// least-squares c, rotated before 2-bit quantization; paragraph "Which print is the
// master": the current token stays BF16 until its final loop and is quantized only
// then (this kernel is that drain step).  Group quantizer with FP8 offset and scale:
// "Worked example" of the same page and the arXiv digest's Figure 1 caption (g = 32).
//
// All arithmetic is float64 so that the integer decisions (codes, FP8 metadata, BF16
// rounding of c) are taken exactly like a float64 reference would take them.  A token
// is a chain of short dependent steps, so the kernel is written for latency: group
// reductions use DPP inside a 16-lane row, E4M3 rounding uses exponent arithmetic
// instead of division, and the residual loops are rotated and quantized side by side.
#include "rq_args.hpp"
#include "rq_fp8.hpp"
#include "rq_quant.hpp"

namespace rq {


// min / max over aligned groups of NL = 16, 32 or 64 lanes, result in every lane
template <int NL>
__device__ __forceinline__ double group_min(double v) {
    return lanes_reduce<NL>(v, [](double p, double q) { return fmin(p, q); });
}
template <int NL>
__device__ __forceinline__ double group_max(double v) {
    return lanes_reduce<NL>(v, [](double p, double q) { return fmax(p, q); });
}

// the two threads of a channel hold halves of a sum: both get the whole (a + b == b + a)
__device__ __forceinline__ double pair_sum(double v) { return v + dpp_d<kDppQuadXor1>(v); }

// ---- the group quantizer (two lanes per channel, groups of G consecutive channels);
// QOut, group_params, group_code and lanes_reduce are in rq_quant.hpp

template <int G>
__device__ __forceinline__ QOut quantize_lane(double x, int bits) {
    QOut o = group_params(group_min<2 * G>(x), group_max<2 * G>(x), bits);
    o.code = group_code(x, o, bits);
    return o;
}

// ---- stores (two lanes per channel: thread t holds channel t / 2)

// Pack `bits`-wide codes of consecutive channels into 32-bit words and store them.
__device__ __forceinline__ void store_codes(uint8_t* row, uint32_t code, int bits) {
    const int per = 32 / bits;                          // channels per word
    const int t = threadIdx.x, ch = t >> 1;
    uint32_t v = (t & 1) ? 0u : code << ((ch % per) * bits);
    for (int off = 2; off < 2 * per; off <<= 1) v |= (uint32_t)__shfl_xor((int)v, off, kWave);
    if ((t & (2 * per - 1)) == 0) reinterpret_cast<uint32_t*>(row)[ch / per] = v;
}

__device__ __forceinline__ void store_meta(uint8_t* row, const QOut& q, int g) {
    const int t = threadIdx.x;
    if ((t & 1) == 0 && (t >> 1) % g == 0) reinterpret_cast<uint16_t*>(row)[(t >> 1) / g] = (uint16_t)(q.zb | (q.sb << 8));
}

__device__ __forceinline__ void store_c(uint8_t* cblk, int jj, double c) {
    if (threadIdx.x == 0) {
        const uint32_t cb = __float_as_uint((float)c) >> 16;    // c is a BF16 value
        reinterpret_cast<uint16_t*>(cblk)[jj] = (uint16_t)cb;
    }
}

// Sum over the channels of N float64 values per channel (each given by both threads of
// the channel): DPP and half swaps inside each wave, then the wave sums through LDS,
// added in a fixed order.  Every thread gets the sums.
template <int NT, int N>
__device__ __forceinline__ void block_sum(double (&v)[N], double (*red)[NT / 64]) {
    const auto add = [](double p, double q) { return p + q; };
#pragma unroll
    for (int k = 0; k < N; ++k) v[k] = lanes_reduce<64>((threadIdx.x & 1) ? 0.0 : v[k], add);
    __syncthreads();                                    // red is reused
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
        for (int k = 0; k < N; ++k) red[k][threadIdx.x >> 6] = v[k];
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < N; ++k) {
        double s = 0.0;
#pragma unroll
        for (int r = 0; r < NT / 64; ++r) s += red[k][r];
        v[k] = s;
    }
}

// The float64 copy of an R element is made where it is used: the empty asm keeps the
// compiler from hoisting 2 * D registers of converted R out of the token loop.
__device__ __forceinline__ double r_elem(float r) {
    asm volatile("" : "+v"(r));
    return (double)r;
}

// r_l = sum_k R[i][k] y_l[k] for LR vectors y_l in LDS: this thread holds half of row i
// of R (columns [H p, H p + H), H = D / 2) and the pair of threads adds its halves.  Each
// R element is converted once and used by every vector.
template <int D, int LR>
__device__ __forceinline__ void rotate_rows(const float (&rhalf)[D / 2], const double (*y)[D], int p,
                                            double (&r)[LR]) {
    constexpr int H = D / 2;
    double r0[LR], r1[LR];
#pragma unroll
    for (int l = 0; l < LR; ++l) r0[l] = r1[l] = 0.0;
#pragma unroll
    for (int k = 0; k < H; k += 2) {
        // the empty asm with a memory clobber bounds how far ahead the LDS reads of y are
        // scheduled, which would otherwise keep most of y in registers
        if (k % 8 == 0) asm volatile("" ::: "memory");
        const double ra = r_elem(rhalf[k]), rb = r_elem(rhalf[k + 1]);
#pragma unroll
        for (int l = 0; l < LR; ++l) {
            r0[l] = fma(ra, y[l][H * p + k], r0[l]);
            r1[l] = fma(rb, y[l][H * p + k + 1], r1[l]);
        }
    }
#pragma unroll
    for (int l = 0; l < LR; ++l) r[l] = pair_sum(r0[l] + r1[l]);
}

// All LR residual loops, rotated three at a time (register pressure).
template <int D, int LR, int L0 = 0>
__device__ __forceinline__ void rotate_all(const float (&rhalf)[D / 2], const double (*y)[D], int p,
                                           double (&r)[LR]) {
    if constexpr (L0 < LR) {
        constexpr int NB = (LR - L0) < 3 ? (LR - L0) : 3;
        double rb[NB];
        rotate_rows<D, NB>(rhalf, y + L0, p, rb);
#pragma unroll
        for (int l = 0; l < NB; ++l) r[L0 + l] = rb[l];
        rotate_all<D, LR, L0 + NB>(rhalf, y, p, r);
    }
}

// One workgroup of 2 D threads per (token range, batch row, KV head, K|V): threads 2i
// and 2i+1 own channel i and keep the two halves of row i of R in registers for all
// tokens of the range.  LR = L - 1 residual loops.
// SPLIT (shared anchor only): one residual loop per workgroup, selected by the block index;
// every workgroup of a token quantizes the anchor, the one of loop 0 stores it.  This
// shortens the chain of a single token (rotation and residual quantizer of one loop).  A
// SPLIT kernel takes the loop count from the configuration (LR is unused), so one
// instantiation serves every group length.
// The coefficient follows the configuration's rule: least squares <x, ref>/<ref, ref> or
// the norm ratio sqrt(<x, x>/<ref, ref>), both rounded to BF16.
// The SPLIT kernel is held to three waves per SIMD (144 VGPRs, no spills): at batch 16 its
// 1536 workgroups then run in two rounds instead of three (per-step pack 25 -> 22 us); four
// or more waves per SIMD spill and are slower.
template <int D, int G, int LR, bool SPLIT>
__global__ __launch_bounds__(2 * D) __attribute__((amdgpu_waves_per_eu(SPLIT ? 3 : 1))) void rq_pack_kernel(PackArgs a) {
    const int LRr = SPLIT ? a.geo.L - 1 : LR;         // residual loops of the group
    const int L = LRr + 1;
    constexpr int NL = SPLIT ? 1 : LR;                 // residual loops of this workgroup
    constexpr int NT = 2 * D;
    constexpr int H = D / 2;
    const Geom& Gm = a.geo;
    const int i = threadIdx.x >> 1, p = threadIdx.x & 1;
    int wg = blockIdx.x;
    int lsel = 0;
    if constexpr (SPLIT) {
        lsel = wg % LRr;
        wg /= LRr;
    }
    const int x = wg & 1;
    wg >>= 1;
    const int h = wg % Gm.hkv;
    wg /= Gm.hkv;
    const int b = wg % a.batch;
    const int t0 = (wg / a.batch) * a.tokens_per_wg;
    const int t1 = min(t0 + a.tokens_per_wg, a.n_tokens);
    const int loop0 = a.group_idx * L;
    const float* R = a.rot + (int64_t)(h * 2 + x) * D * D;
    const bool norm_ratio = Gm.scale_rule == 1;

    __shared__ double sh_y[NL > 1 ? NL : 2][D];
    __shared__ double red[NL + 1 > 2 ? NL + 1 : 2][NT / 64];

    float rhalf[H];                                    // R[i][H p + k]
    {
        const float4* rp = reinterpret_cast<const float4*>(R + (int64_t)i * D + H * p);
#pragma unroll
        for (int k4 = 0; k4 < H / 4; ++k4) {
            const float4 v = rp[k4];
            rhalf[4 * k4] = v.x;
            rhalf[4 * k4 + 1] = v.y;
            rhalf[4 * k4 + 2] = v.z;
            rhalf[4 * k4 + 3] = v.w;
        }
    }
    for (int t = t0; t < t1; ++t) {
        const int slot = a.pos[b] + t;
        if (slot < 0 || slot >= Gm.max_ctx) continue;  // same for the whole workgroup
        const int tile = slot / kTile, jj = slot % kTile;

        // xv[0..NL): the residual loops of this workgroup; xv[NL]: the anchor (the group's last loop)
        double xv[NL + 1];
        const uint16_t* src = a.pending + t * a.st[0] + b * a.st[1] + x * a.st[3] + h * a.st[4] + i;
#pragma unroll
        for (int l = 0; l < NL; ++l) xv[l] = (double)bf16_to_f32(src[(int64_t)(SPLIT ? lsel : l) * a.st[2]]);
        xv[NL] = (double)bf16_to_f32(src[(int64_t)(L - 1) * a.st[2]]);

        const QOut qa = quantize_lane<G>(xv[NL], Gm.ba);
        if (!SPLIT || lsel == 0) {
            uint8_t* pl = a.cache + Gm.tile_offset(b, h, x, loop0 + L - 1, tile);
            store_codes(pl + jj * Gm.a_row, qa.code, Gm.ba);
            store_meta(pl + kTile * Gm.a_row + jj * Gm.m_row, qa, Gm.g);
        }
        const double a_hat = qa.z + qa.code * qa.s;      // dequantized anchor (exact)

        if (!Gm.chained) {
            // every loop l < L-1 references a_hat: one reduction gives all <x_l, a> and
            // <a, a>; the loops are rotated together and then quantized side by side
            double sums[NL + 1];
#pragma unroll
            for (int l = 0; l < NL; ++l) sums[l] = xv[l] * (norm_ratio ? xv[l] : a_hat);
            sums[NL] = a_hat * a_hat;
            block_sum<NT, NL + 1>(sums, red);
            double cs[NL];
#pragma unroll
            for (int l = 0; l < NL; ++l) {
                const double q = sums[l] / sums[NL];
                cs[l] = bf16_round(sums[NL] > 0.0 ? (norm_ratio ? sqrt(q) : q) : 0.0);
                if (p == 0) sh_y[l][i] = xv[l] - cs[l] * a_hat;
            }
            __syncthreads();
            double rl[NL];
            rotate_all<D, NL>(rhalf, sh_y, p, rl);
            QOut qr[NL];
#pragma unroll
            for (int l = 0; l < NL; ++l) qr[l] = quantize_lane<G>(rl[l], Gm.rbits(SPLIT ? lsel : l));
#pragma unroll
            for (int l = 0; l < NL; ++l) {
                const int ll = SPLIT ? lsel : l;         // local loop of this residual
                uint8_t* pl = a.cache + Gm.tile_offset(b, h, x, loop0 + ll, tile);
                store_codes(pl + jj * Gm.rrow(ll), qr[l].code, Gm.rbits(ll));
                store_meta(pl + kTile * Gm.rrow(ll) + jj * Gm.m_row, qr[l], Gm.g);
                store_c(pl + kTile * (Gm.rrow(ll) + Gm.m_row), jj, cs[l]);
            }
            __syncthreads();                              // sh_y is reused by the next token
        } else if constexpr (!SPLIT) {
            // loop l references the rebuilt loop l+1 (the anchor closes the chain)
            double ref = a_hat;
            for (int l = L - 2; l >= 0; --l) {
                double s2[2] = {xv[l] * (norm_ratio ? xv[l] : ref), ref * ref};
                block_sum<NT, 2>(s2, red);
                const double q = s2[0] / s2[1];
                const double c = bf16_round(s2[1] > 0.0 ? (norm_ratio ? sqrt(q) : q) : 0.0);
                if (p == 0) sh_y[0][i] = xv[l] - c * ref;
                __syncthreads();
                double rl[1];
                rotate_rows<D, 1>(rhalf, sh_y, p, rl);
                const QOut qr = quantize_lane<G>(rl[0], Gm.rbits(l));
                uint8_t* pl = a.cache + Gm.tile_offset(b, h, x, loop0 + l, tile);
                store_codes(pl + jj * Gm.rrow(l), qr.code, Gm.rbits(l));
                store_meta(pl + kTile * Gm.rrow(l) + jj * Gm.m_row, qr, Gm.g);
                store_c(pl + kTile * (Gm.rrow(l) + Gm.m_row), jj, c);
                // R^T r_hat: the thread pair of channel i takes column i of R, rows
                // [H p, H p + H) each (coalesced across the pairs)
                if (p == 0) sh_y[1][i] = qr.z + qr.code * qr.s;
                __syncthreads();
                double c0 = 0.0, c1 = 0.0;
#pragma unroll 16
                for (int k = 0; k < H; k += 2) {
                    const int row = H * p + k;
                    c0 = fma(r_elem(R[(int64_t)row * D + i]), sh_y[1][row], c0);
                    c1 = fma(r_elem(R[(int64_t)(row + 1) * D + i]), sh_y[1][row + 1], c1);
                }
                ref = c * ref + pair_sum(c0 + c1);
                __syncthreads();
            }
        }
    }
}

// ---- per-step drain with R in LDS: every residual loop of one token per workgroup
//
// The kernel above holds half a row of R per thread in registers, which allows at most
// three of its workgroups per CU.  Here one workgroup of 2 D threads per (token, batch row,
// KV head, K|V) stages R in LDS (66 KB at d = 128, so two workgroups per CU) and takes every
// residual loop of the group (quantized side by side, rotated one loop at a time): the
// Ouro-sized drain at batch 16 is 512 workgroups, one round on 256 CUs, where one loop per
// workgroup needs 1536.  The anchor quantizer, the c reductions, the rotation (the same two
// chains per half row, the pair adding its halves) and the quantizers are the float64 steps
// of the kernel above in the same order, so the bytes it writes are identical.
// R rows are padded to d + 4 floats, so the 8 channels of a 16-lane group of a 128-bit LDS
// read start in 8 different 4-bank groups (the two halves of a channel share one: a two-way
// conflict on the R reads, which are a third of the rotation's LDS reads).
template <int D>
__device__ __forceinline__ int rlds_slot(int row, int c4) { return row * ((D + 4) / 4) + c4; }

// r = sum_k R[i][k] y[k] with R in LDS: the same two chains per half row and the same order as
// rotate_rows.  One base address per operand, so every read takes its step as an immediate
// offset.
template <int D>
__device__ __forceinline__ double rotate_row_lds(const f32x4* rs, int i, const double* y, int p) {
    constexpr int H = D / 2;
    const f32x4* rrow = rs + rlds_slot<D>(i, p * (H / 4));
    const double* yb = y + H * p;
    double r0 = 0.0, r1 = 0.0;
#pragma unroll
    for (int k = 0; k < H; k += 4) {
        if (k % 16 == 0) __builtin_amdgcn_sched_barrier(0);
        const f32x4 rv = rrow[k / 4];
        r0 = fma((double)rv.x, yb[k], r0);
        r1 = fma((double)rv.y, yb[k + 1], r1);
        r0 = fma((double)rv.z, yb[k + 2], r0);
        r1 = fma((double)rv.w, yb[k + 3], r1);
    }
    return pair_sum(r0 + r1);
}

template <int D, int G, int LR>
__global__ __launch_bounds__(2 * D) __attribute__((amdgpu_waves_per_eu(2))) void rq_drain_kernel(PackArgs a) {
    constexpr int NT = 2 * D;
    constexpr int NR = D * D / 4 / NT;                // float4 of R per thread
    const Geom& Gm = a.geo;
    const int L = LR + 1;
    const int i = threadIdx.x >> 1, p = threadIdx.x & 1;
    int wg = blockIdx.x;
    const int x = wg & 1;
    wg >>= 1;
    const int h = wg % Gm.hkv;
    wg /= Gm.hkv;
    const int b = wg % a.batch;
    const int t = wg / a.batch;
    const int slot = a.pos[b] + t;
    if (t >= a.n_tokens || slot < 0 || slot >= Gm.max_ctx) return;   // the whole workgroup
    const int tile = slot / kTile, jj = slot % kTile;
    const int loop0 = a.group_idx * L;
    const bool norm_ratio = Gm.scale_rule == 1;

    __shared__ f32x4 rs[D * (D + 4) / 4];
    __shared__ double sh_y[LR][D];
    __shared__ double red[LR + 1][NT / 64];

    // every global load first: R (landed in LDS after the anchor quantizer), the loops' inputs
    const f32x4* R4 = reinterpret_cast<const f32x4*>(a.rot + (int64_t)(h * 2 + x) * D * D);
    f32x4 rv[NR];
#pragma unroll
    for (int e = 0; e < NR; ++e) rv[e] = R4[threadIdx.x + e * NT];
    double xv[LR + 1];                                 // residual loops, then the anchor
    const uint16_t* src = a.pending + t * a.st[0] + b * a.st[1] + x * a.st[3] + h * a.st[4] + i;
#pragma unroll
    for (int l = 0; l <= LR; ++l) xv[l] = (double)bf16_to_f32(src[(int64_t)l * a.st[2]]);

    const QOut qa = quantize_lane<G>(xv[LR], Gm.ba);
    {
        uint8_t* pl = a.cache + Gm.tile_offset(b, h, x, loop0 + L - 1, tile);
        store_codes(pl + jj * Gm.a_row, qa.code, Gm.ba);
        store_meta(pl + kTile * Gm.a_row + jj * Gm.m_row, qa, Gm.g);
    }
    const double a_hat = qa.z + qa.code * qa.s;
#pragma unroll
    for (int e = 0; e < NR; ++e) {
        const int idx = threadIdx.x + e * NT;
        rs[rlds_slot<D>(idx / (D / 4), idx % (D / 4))] = rv[e];
    }

    double sums[LR + 1];
#pragma unroll
    for (int l = 0; l < LR; ++l) sums[l] = xv[l] * (norm_ratio ? xv[l] : a_hat);
    sums[LR] = a_hat * a_hat;
    block_sum<NT, LR + 1>(sums, red);                  // its barriers also publish rs
    double cs[LR];
#pragma unroll
    for (int l = 0; l < LR; ++l) {
        const double q = sums[l] / sums[LR];
        cs[l] = bf16_round(sums[LR] > 0.0 ? (norm_ratio ? sqrt(q) : q) : 0.0);
        if (p == 0) sh_y[l][i] = xv[l] - cs[l] * a_hat;
    }
    __syncthreads();
    // one loop at a time: with the loops side by side the scheduler hoists every LDS read of
    // the rotation and spills
    double rl[LR];
#pragma unroll
    for (int l = 0; l < LR; ++l) {
        __builtin_amdgcn_sched_barrier(0);
        rl[l] = rotate_row_lds<D>(rs, i, sh_y[l], p);
    }
    QOut qr[LR];
#pragma unroll
    for (int l = 0; l < LR; ++l) qr[l] = quantize_lane<G>(rl[l], Gm.rbits(l));
#pragma unroll
    for (int l = 0; l < LR; ++l) {
        uint8_t* pl = a.cache + Gm.tile_offset(b, h, x, loop0 + l, tile);
        store_codes(pl + jj * Gm.rrow(l), qr[l].code, Gm.rbits(l));
        store_meta(pl + kTile * Gm.rrow(l) + jj * Gm.m_row, qr[l], Gm.g);
        store_c(pl + kTile * (Gm.rrow(l) + Gm.m_row), jj, cs[l]);
    }
}

// ---- bulk pack: many tokens of one (row, KV head, K|V) per workgroup
//
// For a prefilled context the token-at-a-time chain above leaves the chip idle.  Here a
// workgroup takes kBulkTokens tokens: the quantizers and the c dot products run one token
// per wave (lane = D/64 consecutive channels), and the rotations of all residual loops of
// all its tokens form one product R Y (D x D times D x (tokens x loops)) on the float64
// matrix cores.  Same float64 arithmetic and the same decisions as the kernel above; only
// the order of the additions inside the dot products differs.
constexpr int kBulkTokens = 16;
// threads per workgroup: 8 waves at D = 128 (one 16-row tile of R each), two workgroups per CU
template <int D>
constexpr int bulk_threads() { return D == 128 ? 512 : 256; }

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
}

// OR over aligned groups of NL <= 16 lanes
template <int NL, int M = 1>
__device__ __forceinline__ uint32_t lanes_or(uint32_t v) {
    static_assert(NL <= 16, "within a DPP row");
    if constexpr (M >= NL) {
        return v;
    } else {
        constexpr int CTRL = M == 1 ? kDppQuadXor1 : M == 2 ? kDppQuadXor2 : M == 4 ? kDppRowHalfMirror : kDppRowMirror;
        return lanes_or<NL, 2 * M>(v | dpp_u<CTRL>(v));
    }
}

// Quantize the CPL channels of this lane (channels CPL*lane + c) of S tokens at once (one
// wave holds S tokens; their chains are independent, so the compiler interleaves them) with
// groups of G channels; store codes and metadata into token row jj[t] of tile[t] where
// store[t]; return the dequantized values.
template <int G, int CPL, int BITS, int S>
__device__ __forceinline__ void quantize_rows(const double (&x)[S][CPL], double (&xhat)[S][CPL], uint8_t* const (&tile)[S],
                                              int row_bytes, int m_row, const int (&jj)[S], const bool (&store)[S],
                                              int lane) {
    constexpr int GL = G / CPL;                       // lanes per group
    constexpr int PER = 32 / BITS;                    // channels per code word
    double lo[S], hi[S];
#pragma unroll
    for (int t = 0; t < S; ++t) {
        lo[t] = hi[t] = x[t][0];
#pragma unroll
        for (int c = 1; c < CPL; ++c) {
            lo[t] = fmin(lo[t], x[t][c]);
            hi[t] = fmax(hi[t], x[t][c]);
        }
    }
#pragma unroll
    for (int t = 0; t < S; ++t) {
        lo[t] = lanes_reduce<GL>(lo[t], [](double p, double q) { return fmin(p, q); });
        hi[t] = lanes_reduce<GL>(hi[t], [](double p, double q) { return fmax(p, q); });
    }
    QOut o[S];
    uint32_t word[S];
#pragma unroll
    for (int t = 0; t < S; ++t) {
        o[t] = group_params(lo[t], hi[t], BITS);
        word[t] = 0;
#pragma unroll
        for (int c = 0; c < CPL; ++c) {
            const uint32_t code = group_code(x[t][c], o[t], BITS);
            xhat[t][c] = o[t].z + (double)code * o[t].s;
            word[t] |= code << (((CPL * lane + c) % PER) * BITS);
        }
    }
#pragma unroll
    for (int t = 0; t < S; ++t) word[t] = lanes_or<PER / CPL>(word[t]);
#pragma unroll
    for (int t = 0; t < S; ++t) {
        if (store[t]) {
            if ((CPL * lane) % PER == 0)
                reinterpret_cast<uint32_t*>(tile[t] + (int64_t)jj[t] * row_bytes)[(CPL * lane) / PER] = word[t];
            if ((CPL * lane) % G == 0)
                reinterpret_cast<uint16_t*>(tile[t] + (int64_t)kTile * row_bytes + (int64_t)jj[t] * m_row)[(CPL * lane) / G] =
                    (uint16_t)(o[t].zb | (o[t].sb << 8));
        }
    }
}

// LB = min(L - 1, 3) residual loops per product; the loop count itself comes from the
// configuration, so one instantiation serves every group length of at least LB + 1.
template <int D, int G, int LB>
__global__ __launch_bounds__(bulk_threads<D>()) __attribute__((amdgpu_waves_per_eu(D == 128 ? 4 : 3))) void rq_pack_bulk_kernel(PackArgs a) {
    constexpr int kBulkThreads = bulk_threads<D>();
    constexpr int TK = kBulkTokens, NW = kBulkThreads / kWave;
    constexpr int CPL = D / kWave;                    // channels per lane
    constexpr int NCOL = TK * LB;                     // columns of Y: (token, loop)
    static_assert(D / 16 == NW && TK % NW == 0, "one 16-row tile of R per wave, tokens per wave");
    constexpr int YS = D + 2;                         // padded LDS row of Y (doubles)
    const Geom& Gm = a.geo;
    const int LR = Gm.L - 1, L = Gm.L;
    const bool norm_ratio = Gm.scale_rule == 1;
    int wg = blockIdx.x;
    const int x = wg & 1;
    wg >>= 1;
    const int h = wg % Gm.hkv;
    wg /= Gm.hkv;
    const int b = wg % a.batch;
    const int t0 = (wg / a.batch) * TK;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int loop0 = a.group_idx * L;

    __shared__ __attribute__((aligned(16))) double yt[NCOL][YS];   // Y, then R Y: [column][channel]
    __shared__ double ah[TK][D];                                   // dequantized anchors
    __shared__ double aa[TK];                                      // <a_hat, a_hat>
    __shared__ uint16_t xs[LB][TK][D];                             // BF16 inputs of the loops at hand

    // The A operand of the rotation product: this lane's part of the 16 rows of R that its wave
    // multiplies (row 16 w + lane % 16, channels (D/4) (lane / 16) ..), read from global memory
    // (L2) right before each product and never staged in LDS: that leaves room for two
    // workgroups per CU (79 KB of LDS, 94 VGPRs), whose latency-bound phases overlap.
    const int i16 = lane & 15, kq = lane >> 4;
    const f32x4* rp = reinterpret_cast<const f32x4*>(a.rot + (int64_t)(h * 2 + x) * D * D +
                                                     (int64_t)(16 * w + i16) * D + (D / 4) * kq);

    const int p0 = a.pos[b] + t0;
    auto valid = [&](int tok) {
        const int slot = p0 + tok;
        return t0 + tok < a.n_tokens && slot >= 0 && slot < Gm.max_ctx;
    };
    // Stage the BF16 inputs of loops [l0, l0 + nl) of every token in xs (all loads in flight
    // together); tokens that are not packed read as zero.
    constexpr int PE = TK * D / kBulkThreads;         // elements per thread and loop
    auto stage_x = [&](int l0, int nl) {
        uint16_t v[LB][PE];
#pragma unroll
        for (int li = 0; li < LB; ++li) {
#pragma unroll
            for (int e = 0; e < PE; ++e) {
                const int idx = e * kBulkThreads + threadIdx.x, i = idx % D, tok = idx / D;
                v[li][e] = (li < nl && valid(tok))
                               ? a.pending[(int64_t)(t0 + tok) * a.st[0] + (int64_t)b * a.st[1] +
                                           (int64_t)(l0 + li) * a.st[2] + (int64_t)x * a.st[3] +
                                           (int64_t)h * a.st[4] + i]
                               : (uint16_t)0;
            }
        }
#pragma unroll
        for (int li = 0; li < LB; ++li)
#pragma unroll
            for (int e = 0; e < PE; ++e) {
                const int idx = e * kBulkThreads + threadIdx.x;
                xs[li][idx / D][idx % D] = v[li][e];
            }
    };
    auto load_x = [&](int li, int tok, double (&v)[CPL]) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) v[c] = (double)bf16_to_f32(xs[li][tok][CPL * lane + c]);
    };
    const auto add = [](double p, double q) { return p + q; };

    // the S = TK / NW tokens of this wave (tokens t NW + w), taken SB at a time side by side
    constexpr int S = TK / NW, SB = S < 2 ? S : 2;
    int jjs[S], tiles[S];
    bool oks[S];
#pragma unroll
    for (int t = 0; t < S; ++t) {
        const int tok = t * NW + w;
        oks[t] = valid(tok);                          // wave-uniform
        const int slot = oks[t] ? p0 + tok : 0;
        tiles[t] = slot / kTile;
        jjs[t] = slot % kTile;
    }

    // ---- anchors, SB of the wave's tokens side by side
    stage_x(L - 1, 1);
    __syncthreads();
#pragma unroll
    for (int tb = 0; tb < S; tb += SB) {
        double xa[SB][CPL], xh[SB][CPL];
        uint8_t* pl[SB];
        int jb[SB];
        bool ob[SB];
#pragma unroll
        for (int u = 0; u < SB; ++u) {
            load_x(0, (tb + u) * NW + w, xa[u]);
            pl[u] = a.cache + Gm.tile_offset(b, h, x, loop0 + L - 1, tiles[tb + u]);
            jb[u] = jjs[tb + u];
            ob[u] = oks[tb + u];
        }
        if (Gm.ba == 4) quantize_rows<G, CPL, 4, SB>(xa, xh, pl, Gm.a_row, Gm.m_row, jb, ob, lane);
        else quantize_rows<G, CPL, 2, SB>(xa, xh, pl, Gm.a_row, Gm.m_row, jb, ob, lane);
        double ss[SB];
#pragma unroll
        for (int u = 0; u < SB; ++u) {
            ss[u] = 0.0;
#pragma unroll
            for (int c = 0; c < CPL; ++c) {
                ss[u] = fma(xh[u][c], xh[u][c], ss[u]);
                ah[(tb + u) * NW + w][CPL * lane + c] = xh[u][c];
            }
        }
#pragma unroll
        for (int u = 0; u < SB; ++u) ss[u] = lanes_reduce<kWave>(ss[u], add);
        if (lane == 0) {
#pragma unroll
            for (int u = 0; u < SB; ++u) aa[(tb + u) * NW + w] = ss[u];
        }
    }

    for (int lb0 = 0; lb0 < LR; lb0 += LB) {
        // ---- c and y = x - c a_hat of the loops [lb0, lb0 + LB), one token per wave
        __syncthreads();                              // ah and aa written; xs and yt free
        stage_x(lb0, LB < LR - lb0 ? LB : LR - lb0);
        __syncthreads();
        {
            // the dot products of SB tokens' loops first, then their reductions side by side;
            // the inputs are read again from LDS for y, rather than held in registers
            const auto lok = [&](int t, int li) { return oks[t] && lb0 + li < LR; };
#pragma unroll
            for (int tb = 0; tb < S; tb += SB) {
                double dot[SB][LB];
#pragma unroll
                for (int u = 0; u < SB; ++u) {
                    const int tok = (tb + u) * NW + w;
                    double xh[CPL];
#pragma unroll
                    for (int c = 0; c < CPL; ++c) xh[c] = ah[tok][CPL * lane + c];
#pragma unroll
                    for (int li = 0; li < LB; ++li) {
                        double xl[CPL];
                        load_x(li, tok, xl);
                        dot[u][li] = 0.0;
#pragma unroll
                        for (int c = 0; c < CPL; ++c) dot[u][li] = fma(xl[c], norm_ratio ? xl[c] : xh[c], dot[u][li]);
                        if (!lok(tb + u, li)) dot[u][li] = 0.0;
                    }
                }
#pragma unroll
                for (int u = 0; u < SB; ++u)
#pragma unroll
                    for (int li = 0; li < LB; ++li) dot[u][li] = lanes_reduce<kWave>(dot[u][li], add);
#pragma unroll
                for (int u = 0; u < SB; ++u) {
                    const int t = tb + u, tok = t * NW + w;
                    const double na = aa[tok];
                    double xh[CPL];
#pragma unroll
                    for (int c = 0; c < CPL; ++c) xh[c] = ah[tok][CPL * lane + c];
#pragma unroll
                    for (int li = 0; li < LB; ++li) {
                        const int l = lb0 + li;
                        const double qn = dot[u][li] / na;
                        const double cl = bf16_round(na > 0.0 ? (norm_ratio ? sqrt(qn) : qn) : 0.0);
                        if (lok(t, li) && lane == 0) {
                            uint8_t* pl = a.cache + Gm.tile_offset(b, h, x, loop0 + l, tiles[t]);
                            reinterpret_cast<uint16_t*>(pl + (int64_t)kTile * (Gm.rrow(l) + Gm.m_row))[jjs[t]] =
                                (uint16_t)(__float_as_uint((float)cl) >> 16);
                        }
                        double xl[CPL];
                        load_x(li, tok, xl);
#pragma unroll
                        for (int c = 0; c < CPL; ++c)
                            yt[tok * LB + li][CPL * lane + c] = (lok(t, li) ? xl[c] : 0.0) - cl * xh[c];
                    }
                }
            }
        }
        __syncthreads();
        // ---- r = R y for every column on the matrix cores (v_mfma_f64_16x16x4_f64): wave w
        // takes the 16 rows 16 w .. of R and every 16-column tile of Y.  The sum over the
        // channels is split over the four K slots of the product, slot kq taking channels
        // (D/4) kq + s at step s, so that each lane reads its R row and its Y column as
        // contiguous runs (R loaded into registers, Y from LDS).  Lane layout (measured with
        // an in-bounds probe): A[i][k] in lane i + 16 k, B[k][j] in lane j + 16 k, D[i][j] in
        // lane j + 16 (i % 4), element i / 4.
        {
            f32x4 ra[D / 16];
#pragma unroll
            for (int q = 0; q < D / 16; ++q) ra[q] = rp[q];
            f64x4 acc[LB];
#pragma unroll
            for (int c = 0; c < LB; ++c) acc[c] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int q = 0; q < D / 16; ++q) {
                const f32x4 rv = ra[q];
#pragma unroll
                for (int c = 0; c < LB; ++c) {
                    const double* yb = &yt[16 * c + i16][(D / 4) * kq + 4 * q];
                    const f64x2 y01 = *reinterpret_cast<const f64x2*>(yb);
                    const f64x2 y23 = *reinterpret_cast<const f64x2*>(yb + 2);
                    acc[c] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)rv.x, y01.x, acc[c], 0, 0, 0);
                    acc[c] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)rv.y, y01.y, acc[c], 0, 0, 0);
                    acc[c] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)rv.z, y23.x, acc[c], 0, 0, 0);
                    acc[c] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)rv.w, y23.y, acc[c], 0, 0, 0);
                }
            }
            __syncthreads();                          // every wave has read Y
#pragma unroll
            for (int c = 0; c < LB; ++c)
#pragma unroll
                for (int e = 0; e < 4; ++e) yt[16 * c + i16][16 * w + 4 * e + kq] = acc[c][e];
        }
        __syncthreads();
        // ---- residual codes, SB of the wave's tokens side by side
#pragma unroll
        for (int li = 0; li < LB; ++li) {
            const int l = lb0 + li;
            const int lq = l < LR ? l : 0;                // a loop past the group's last is not stored
#pragma unroll
            for (int tb = 0; tb < S; tb += SB) {
                double r[SB][CPL], rh[SB][CPL];
                uint8_t* pl[SB];
                int jb[SB];
                bool st[SB];
#pragma unroll
                for (int u = 0; u < SB; ++u) {
#pragma unroll
                    for (int c = 0; c < CPL; ++c) r[u][c] = yt[((tb + u) * NW + w) * LB + li][CPL * lane + c];
                    pl[u] = a.cache + Gm.tile_offset(b, h, x, loop0 + lq, tiles[tb + u]);
                    jb[u] = jjs[tb + u];
                    st[u] = oks[tb + u] && l < LR;
                }
                if (Gm.rbits(lq) == 4) quantize_rows<G, CPL, 4, SB>(r, rh, pl, Gm.rrow(lq), Gm.m_row, jb, st, lane);
                else quantize_rows<G, CPL, 2, SB>(r, rh, pl, Gm.rrow(lq), Gm.m_row, jb, st, lane);
            }
        }
    }
}

// ---- bulk pack of the chained layout: many tokens per workgroup
//
// Chained: loop l is stored against the rebuilt loop l + 1 (the anchor closes the chain), so
// the loops run one after the other, each with two products on the float64 matrix cores over
// the workgroup's 16 tokens: r = R y, then the rebuilt loop c ref + R^T r_hat, which is the
// next loop's reference.  The coefficient and quantizer phases run one token per wave as in
// the kernel above.  Same float64 steps and decisions as the token-at-a-time kernel; only the
// order of the additions inside the products differs.
template <int D, int G>
__global__ __launch_bounds__(bulk_threads<D>()) __attribute__((amdgpu_waves_per_eu(D == 128 ? 4 : 3)))
void rq_pack_bulk_chained_kernel(PackArgs a) {
    constexpr int kBulkThreads = bulk_threads<D>();
    constexpr int TK = kBulkTokens, NW = kBulkThreads / kWave;
    constexpr int CPL = D / kWave;                    // channels per lane
    static_assert(D / 16 == NW && TK % NW == 0, "one 16-row tile of R per wave, tokens per wave");
    constexpr int YS = D + 2;                         // padded LDS row of Y (doubles)
    const Geom& Gm = a.geo;
    const int L = Gm.L;
    const bool norm_ratio = Gm.scale_rule == 1;
    int wg = blockIdx.x;
    const int x = wg & 1;
    wg >>= 1;
    const int h = wg % Gm.hkv;
    wg /= Gm.hkv;
    const int b = wg % a.batch;
    const int t0 = (wg / a.batch) * TK;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int loop0 = a.group_idx * L;

    __shared__ __attribute__((aligned(16))) double yt[TK][YS];     // y, then R y, then r_hat: [token][channel]
    __shared__ double ref[TK][D];                                  // reference of the loop at hand
    __shared__ double cs[TK];                                      // its coefficient per token
    __shared__ uint16_t xs[TK][D];                                 // BF16 inputs of the loop at hand

    // A operands: rows 16 w + lane % 16 of R (channels (D/4) (lane / 16) + s, contiguous) for
    // r = R y, and the same rows of R^T (R[(D/4) (lane / 16) + s][16 w + lane % 16], one
    // float per step) for R^T r_hat, both read from L2 right before their product
    const int i16 = lane & 15, kq = lane >> 4;
    const float* Rm = a.rot + (int64_t)(h * 2 + x) * D * D;
    const f32x4* rp = reinterpret_cast<const f32x4*>(Rm + (int64_t)(16 * w + i16) * D + (D / 4) * kq);
    const float* rtp = Rm + (int64_t)((D / 4) * kq) * D + 16 * w + i16;

    const int p0 = a.pos[b] + t0;
    auto valid = [&](int tok) {
        const int slot = p0 + tok;
        return t0 + tok < a.n_tokens && slot >= 0 && slot < Gm.max_ctx;
    };
    constexpr int PE = TK * D / kBulkThreads;         // elements per thread
    auto stage_x = [&](int l) {
        uint16_t v[PE];
#pragma unroll
        for (int e = 0; e < PE; ++e) {
            const int idx = e * kBulkThreads + threadIdx.x, i = idx % D, tok = idx / D;
            v[e] = valid(tok) ? a.pending[(int64_t)(t0 + tok) * a.st[0] + (int64_t)b * a.st[1] + (int64_t)l * a.st[2] +
                                          (int64_t)x * a.st[3] + (int64_t)h * a.st[4] + i]
                              : (uint16_t)0;
        }
#pragma unroll
        for (int e = 0; e < PE; ++e) {
            const int idx = e * kBulkThreads + threadIdx.x;
            xs[idx / D][idx % D] = v[e];
        }
    };
    auto load_x = [&](int tok, double (&v)[CPL]) {
#pragma unroll
        for (int c = 0; c < CPL; ++c) v[c] = (double)bf16_to_f32(xs[tok][CPL * lane + c]);
    };
    const auto add = [](double p, double q) { return p + q; };
    // one 16 x 16 output tile per wave: D[i][j] = sum_k A[i][k] Y[k][j] with B from yt
    auto product = [&](const auto& a_of) {
        f64x4 acc = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int q = 0; q < D / 16; ++q) {
            const double* yb = &yt[i16][(D / 4) * kq + 4 * q];
            const f64x2 y01 = *reinterpret_cast<const f64x2*>(yb);
            const f64x2 y23 = *reinterpret_cast<const f64x2*>(yb + 2);
            acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a_of(4 * q), y01.x, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a_of(4 * q + 1), y01.y, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a_of(4 * q + 2), y23.x, acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a_of(4 * q + 3), y23.y, acc, 0, 0, 0);
        }
        return acc;
    };

    constexpr int S = TK / NW, SB = S < 2 ? S : 2;
    int jjs[S], tiles[S];
    bool oks[S];
#pragma unroll
    for (int t = 0; t < S; ++t) {
        const int tok = t * NW + w;
        oks[t] = valid(tok);
        const int slot = oks[t] ? p0 + tok : 0;
        tiles[t] = slot / kTile;
        jjs[t] = slot % kTile;
    }

    // ---- anchors: the first reference
    stage_x(L - 1);
    __syncthreads();
#pragma unroll
    for (int tb = 0; tb < S; tb += SB) {
        double xa[SB][CPL], xh[SB][CPL];
        uint8_t* pl[SB];
        int jb[SB];
        bool ob[SB];
#pragma unroll
        for (int u = 0; u < SB; ++u) {
            load_x((tb + u) * NW + w, xa[u]);
            pl[u] = a.cache + Gm.tile_offset(b, h, x, loop0 + L - 1, tiles[tb + u]);
            jb[u] = jjs[tb + u];
            ob[u] = oks[tb + u];
        }
        if (Gm.ba == 4) quantize_rows<G, CPL, 4, SB>(xa, xh, pl, Gm.a_row, Gm.m_row, jb, ob, lane);
        else quantize_rows<G, CPL, 2, SB>(xa, xh, pl, Gm.a_row, Gm.m_row, jb, ob, lane);
#pragma unroll
        for (int u = 0; u < SB; ++u)
#pragma unroll
            for (int c = 0; c < CPL; ++c) ref[(tb + u) * NW + w][CPL * lane + c] = xh[u][c];
    }

    for (int l = L - 2; l >= 0; --l) {
        __syncthreads();                              // ref written; xs and yt free
        stage_x(l);
        __syncthreads();
        // ---- c and y = x - c ref
#pragma unroll
        for (int tb = 0; tb < S; tb += SB) {
            double dot[SB], nn[SB];
#pragma unroll
            for (int u = 0; u < SB; ++u) {
                const int tok = (tb + u) * NW + w;
                double xl[CPL];
                load_x(tok, xl);
                dot[u] = nn[u] = 0.0;
#pragma unroll
                for (int c = 0; c < CPL; ++c) {
                    const double rf = ref[tok][CPL * lane + c];
                    dot[u] = fma(xl[c], norm_ratio ? xl[c] : rf, dot[u]);
                    nn[u] = fma(rf, rf, nn[u]);
                }
            }
#pragma unroll
            for (int u = 0; u < SB; ++u) {
                dot[u] = lanes_reduce<kWave>(dot[u], add);
                nn[u] = lanes_reduce<kWave>(nn[u], add);
            }
#pragma unroll
            for (int u = 0; u < SB; ++u) {
                const int t = tb + u, tok = t * NW + w;
                const double qn = dot[u] / nn[u];
                const double cl = bf16_round(nn[u] > 0.0 ? (norm_ratio ? sqrt(qn) : qn) : 0.0);
                if (lane == 0) {
                    cs[tok] = cl;
                    if (oks[t]) {
                        uint8_t* pl = a.cache + Gm.tile_offset(b, h, x, loop0 + l, tiles[t]);
                        reinterpret_cast<uint16_t*>(pl + (int64_t)kTile * (Gm.rrow(l) + Gm.m_row))[jjs[t]] =
                            (uint16_t)(__float_as_uint((float)cl) >> 16);
                    }
                }
                double xl[CPL];
                load_x(tok, xl);
#pragma unroll
                for (int c = 0; c < CPL; ++c) yt[tok][CPL * lane + c] = xl[c] - cl * ref[tok][CPL * lane + c];
            }
        }
        __syncthreads();
        // ---- r = R y (R is read again each loop: held across the loops it would spill)
        {
            const f32x4* rpl = rp;
            asm volatile("" : "+v"(rpl));
            f32x4 ra[D / 16];
#pragma unroll
            for (int q = 0; q < D / 16; ++q) ra[q] = rpl[q];
            const f64x4 acc = product([&](int s) { return (double)ra[s / 4][s % 4]; });
            __syncthreads();                          // every wave has read y
#pragma unroll
            for (int e = 0; e < 4; ++e) yt[i16][16 * w + 4 * e + kq] = acc[e];
        }
        __syncthreads();
        // ---- residual codes; r_hat replaces r in yt (each wave its own tokens' rows)
#pragma unroll
        for (int tb = 0; tb < S; tb += SB) {
            double r[SB][CPL], rh[SB][CPL];
            uint8_t* pl[SB];
            int jb[SB];
            bool st[SB];
#pragma unroll
            for (int u = 0; u < SB; ++u) {
#pragma unroll
                for (int c = 0; c < CPL; ++c) r[u][c] = yt[(tb + u) * NW + w][CPL * lane + c];
                pl[u] = a.cache + Gm.tile_offset(b, h, x, loop0 + l, tiles[tb + u]);
                jb[u] = jjs[tb + u];
                st[u] = oks[tb + u];
            }
            if (Gm.rbits(l) == 4) quantize_rows<G, CPL, 4, SB>(r, rh, pl, Gm.rrow(l), Gm.m_row, jb, st, lane);
            else quantize_rows<G, CPL, 2, SB>(r, rh, pl, Gm.rrow(l), Gm.m_row, jb, st, lane);
#pragma unroll
            for (int u = 0; u < SB; ++u)
#pragma unroll
                for (int c = 0; c < CPL; ++c) yt[(tb + u) * NW + w][CPL * lane + c] = rh[u][c];
        }
        if (l == 0) break;                            // no later loop needs the rebuilt loop 0
        __syncthreads();
        // ---- the next reference: c ref + R^T r_hat
        {
            const float* rtl = rtp;
            asm volatile("" : "+v"(rtl));
            float rt[D / 4];
#pragma unroll
            for (int s = 0; s < D / 4; ++s) rt[s] = rtl[(int64_t)s * D];
            const f64x4 acc = product([&](int s) { return (double)rt[s]; });
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                double& rf = ref[i16][16 * w + 4 * e + kq];
                rf = cs[i16] * rf + acc[e];
            }
        }
    }
}

template <int D, int G>
static hipError_t launch_bulk_chained(const PackArgs& a, int nwg, hipStream_t stream) {
    const int LR = a.geo.L - 1;
    if (LR < 1 || LR > kMaxLoops - 1) return hipErrorInvalidValue;
    hipLaunchKernelGGL((rq_pack_bulk_chained_kernel<D, G>), dim3(nwg), dim3(bulk_threads<D>()), 0, stream, a);
    return hipGetLastError();
}

template <int D, int G>
static hipError_t launch_bulk(const PackArgs& a, int nwg, hipStream_t stream) {
    constexpr int kBulkThreads = bulk_threads<D>();
    const int LR = a.geo.L - 1;
    if (LR < 1 || LR > kMaxLoops - 1) return hipErrorInvalidValue;
    switch (LR < 3 ? LR : 3) {
        case 1: hipLaunchKernelGGL((rq_pack_bulk_kernel<D, G, 1>), dim3(nwg), dim3(kBulkThreads), 0, stream, a); break;
        case 2: hipLaunchKernelGGL((rq_pack_bulk_kernel<D, G, 2>), dim3(nwg), dim3(kBulkThreads), 0, stream, a); break;
        default: hipLaunchKernelGGL((rq_pack_bulk_kernel<D, G, 3>), dim3(nwg), dim3(kBulkThreads), 0, stream, a); break;
    }
    return hipGetLastError();
}

// SPLIT: one instantiation (the loop count is read at run time); otherwise one per loop count
template <int D, int G, bool SPLIT>
static hipError_t launch_dgs(const PackArgs& a, int nwg, hipStream_t stream) {
    const int LR = a.geo.L - 1;
    if (LR < 1 || LR > kMaxLoops - 1) return hipErrorInvalidValue;
    if constexpr (SPLIT) {
        hipLaunchKernelGGL((rq_pack_kernel<D, G, 1, true>), dim3(nwg * LR), dim3(2 * D), 0, stream, a);
        return hipGetLastError();
    }
    const dim3 grid(nwg);
    switch (LR) {
        case 1: hipLaunchKernelGGL((rq_pack_kernel<D, G, 1, false>), grid, dim3(2 * D), 0, stream, a); break;
        case 2: hipLaunchKernelGGL((rq_pack_kernel<D, G, 2, false>), grid, dim3(2 * D), 0, stream, a); break;
        case 3: hipLaunchKernelGGL((rq_pack_kernel<D, G, 3, false>), grid, dim3(2 * D), 0, stream, a); break;
        case 4: hipLaunchKernelGGL((rq_pack_kernel<D, G, 4, false>), grid, dim3(2 * D), 0, stream, a); break;
        case 5: hipLaunchKernelGGL((rq_pack_kernel<D, G, 5, false>), grid, dim3(2 * D), 0, stream, a); break;
        case 6: hipLaunchKernelGGL((rq_pack_kernel<D, G, 6, false>), grid, dim3(2 * D), 0, stream, a); break;
        case 7: hipLaunchKernelGGL((rq_pack_kernel<D, G, 7, false>), grid, dim3(2 * D), 0, stream, a); break;
        default: return hipErrorInvalidValue;           // longer groups take the SPLIT kernel
    }
    return hipGetLastError();
}

// every residual loop of one token per workgroup with R in LDS (shared anchor, up to 8 loops)
template <int D, int G>
static hipError_t launch_drain(const PackArgs& a, int nwg, hipStream_t stream) {
    const dim3 grid(nwg), block(2 * D);
    switch (a.geo.L - 1) {
        case 1: hipLaunchKernelGGL((rq_drain_kernel<D, G, 1>), grid, block, 0, stream, a); break;
        case 2: hipLaunchKernelGGL((rq_drain_kernel<D, G, 2>), grid, block, 0, stream, a); break;
        case 3: hipLaunchKernelGGL((rq_drain_kernel<D, G, 3>), grid, block, 0, stream, a); break;
        case 4: hipLaunchKernelGGL((rq_drain_kernel<D, G, 4>), grid, block, 0, stream, a); break;
        case 5: hipLaunchKernelGGL((rq_drain_kernel<D, G, 5>), grid, block, 0, stream, a); break;
        case 6: hipLaunchKernelGGL((rq_drain_kernel<D, G, 6>), grid, block, 0, stream, a); break;
        case 7: hipLaunchKernelGGL((rq_drain_kernel<D, G, 7>), grid, block, 0, stream, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// A few tokens with a shared anchor (the per-step drain), one token per workgroup.  One residual
// loop per workgroup has the shortest chain (10.4 us for the Ouro-sized drain at batch 4, against
// 12.9 us with every loop and R in LDS) while its workgroups fit one round at three per CU; past
// that the kernel with R in LDS runs (batch 16: 16.8 us in one round, against 21.5 us in two).
template <int D, int G>
static hipError_t launch_dg(const PackArgs& a, int nwg, hipStream_t stream) {
    if (!a.geo.chained && a.tokens_per_wg == 1) {
        const int64_t split_wgs = (int64_t)nwg * (a.geo.L - 1);
        if (a.geo.L <= 8 && split_wgs > 3LL * (a.n_cu > 0 ? a.n_cu : 256)) return launch_drain<D, G>(a, nwg, stream);
        return launch_dgs<D, G, true>(a, nwg, stream);
    }
    return launch_dgs<D, G, false>(a, nwg, stream);
}

template <int D>
static hipError_t launch_d(const PackArgs& a, int nwg, hipStream_t stream) {
    return a.geo.g == 32 ? launch_dg<D, 32>(a, nwg, stream) : launch_dg<D, 16>(a, nwg, stream);
}

hipError_t launch_pack(const PackArgs& a, hipStream_t stream) {
    if (!a.cache || !a.pending || !a.pos || !a.rot || a.batch < 1 || a.n_tokens < 1 || a.tokens_per_wg < 1 ||
        (a.geo.g != 16 && a.geo.g != 32) || (a.geo.d != 64 && a.geo.d != 128))
        return hipErrorInvalidValue;
    if (a.n_tokens >= kBulkTokens) {
        const int nwg = (a.n_tokens + kBulkTokens - 1) / kBulkTokens * a.batch * a.geo.hkv * 2;
        if (a.geo.chained) {
            if (a.geo.d == 128)
                return a.geo.g == 32 ? launch_bulk_chained<128, 32>(a, nwg, stream) : launch_bulk_chained<128, 16>(a, nwg, stream);
            return a.geo.g == 32 ? launch_bulk_chained<64, 32>(a, nwg, stream) : launch_bulk_chained<64, 16>(a, nwg, stream);
        }
        if (a.geo.d == 128) return a.geo.g == 32 ? launch_bulk<128, 32>(a, nwg, stream) : launch_bulk<128, 16>(a, nwg, stream);
        return a.geo.g == 32 ? launch_bulk<64, 32>(a, nwg, stream) : launch_bulk<64, 16>(a, nwg, stream);
    }
    const int nwg = (a.n_tokens + a.tokens_per_wg - 1) / a.tokens_per_wg * a.batch * a.geo.hkv * 2;
    return a.geo.d == 128 ? launch_d<128>(a, nwg, stream) : launch_d<64>(a, nwg, stream);
}

}  // namespace rq
