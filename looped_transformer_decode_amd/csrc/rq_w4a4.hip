// W4A4 linear layer of a looped block with cross-loop residual activations (arXiv digest,
// scope paragraph after the results: the residual-reconstruction principle carries over
// to W4A4 activation quantization).  Three kernels:
//  * weight quantizer (offline): 4-bit group codes of W or of W R^T (rotation folded
//    into a second weight copy), written in the tile layout the GEMM streams;
//  * activation quantizer (per loop): the anchor loop's activations as 4-bit groups, or
//    a later loop's BF16 least-squares coefficient c and its 4-bit quantized rotated
//    residual r = R (x - c a_hat); float64 arithmetic, so codes match a float64
//    reference except at inexact near-ties;
//  * GEMM: y = W_hat x_hat on the matrix cores for up to 16 tokens.  Per group of 32
//    channels, sum_k (z_w + s_w q_w)(z_x + s_x q_x) = sum (s_x q_x)(s_w q_w) + z_x sum s_w q_w
//    + z_w X with X = sum_k x_hat_k.  The FP16 operands s q are exact (an E4M3 scale has 4
//    significant bits, a code 4), so the first two terms are products of exact FP16 values
//    accumulated in float32 by v_mfma_f32_16x16x32_f16 (one product per group); the
//    z_w X terms of all groups of a wave form one more product with X split into two FP16
//    terms.  Residual loops add c y0, the anchor loop's product kept by the caller.
#include "rq_args.hpp"
#include "rq_quant.hpp"

namespace rq {
namespace w4 {

typedef _Float16 h8 __attribute__((ext_vector_type(8)));
typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef uint32_t u4 __attribute__((ext_vector_type(4)));

constexpr int GS = 32;          // channels per group
constexpr int RB = 128;         // channels per rotation block (and per weight quad)
constexpr int TN = 16;          // weight rows per tile
constexpr int QB = 1024 + 128;  // bytes per (row tile, group quad) block
constexpr uint32_t kMagic2 = 0x64006400u;

__device__ __forceinline__ int act_row_bytes(int k) { return k / 2 + k / 16; }

// ---------------------------------------------------------------- weight quantizer

struct WArgs {
    const uint16_t* w;
    int64_t ldw;
    const float* rot;
    uint8_t* out;
    int k, n;
};

// grid (N / 16 row tiles, K / 128 quads), 256 threads: the 16 x 128 block of W (or of
// W R^T) in float64, then 64 threads quantize one (row, group) each.
template <bool ROT>
__global__ __launch_bounds__(256) void quantize_weights_kernel(WArgs a) {
    __shared__ double v[TN][RB];
    __shared__ double src[ROT ? TN : 1][ROT ? RB : 1];
    __shared__ float rt[ROT ? RB : 1][ROT ? RB : 1];      // rt[c][j] = R[j][c]
    const int t = threadIdx.x, nt = blockIdx.x, qd = blockIdx.y;
    for (int e = t; e < TN * RB; e += 256) {
        const int i = e / RB, c = e % RB;
        const double w = (double)bf16_to_f32(a.w[(int64_t)(nt * TN + i) * a.ldw + qd * RB + c]);
        if constexpr (ROT) src[i][c] = w;
        else v[i][c] = w;
    }
    if constexpr (ROT) {
        for (int e = t; e < RB * RB; e += 256) rt[e % RB][e / RB] = a.rot[e];
        __syncthreads();
        // (W R^T)[i][j] = sum_c W[i][c] R[j][c]
        const int i = t / 16, j0 = (t % 16) * 8;
        for (int j = j0; j < j0 + 8; ++j) {
            double acc = 0.0;
            for (int c = 0; c < RB; ++c) acc = fma(src[i][c], (double)rt[c][j], acc);
            v[i][j] = acc;
        }
    }
    __syncthreads();
    if (t < TN * 4) {
        const int i = t / 4, j = t % 4;
        const double* g = &v[i][GS * j];
        double lo = g[0], hi = g[0];
        for (int c = 1; c < GS; ++c) {
            lo = fmin(lo, g[c]);
            hi = fmax(hi, g[c]);
        }
        const QOut q = group_params(lo, hi, 4);
        uint8_t* blk = a.out + ((size_t)nt * (a.k / RB) + qd) * QB;
        for (int kg = 0; kg < 4; ++kg) {
            uint32_t word = 0;
            for (int e = 0; e < 8; ++e) word |= group_code(g[8 * kg + e], q, 4) << (4 * e);
            reinterpret_cast<uint32_t*>(blk + 16 * (16 * kg + i))[j] = word;
        }
        reinterpret_cast<uint16_t*>(blk + 1024)[4 * i + j] = (uint16_t)(q.zb | (q.sb << 8));
    }
}

// ---------------------------------------------------------------- activation quantizer

struct AArgs {
    const uint16_t* x;
    int64_t ldx;
    const uint8_t* anchor;      // 4-bit anchor rows (read by residual loops)
    uint8_t* act;               // this loop's 4-bit rows (the anchor rows at the anchor loop)
    uint8_t* act2;              // optional second copy of the rows (or null)
    const float* rot;
    float* c;                   // [M] coefficient used (1 at the anchor loop)
    float* c2;                  // optional second copy of c (or null)
    float* xsum;                // [M][K/32] sum of the group's dequantized values
    int k, m;
};

constexpr int TQ = 1;           // tokens per activation-quantizer workgroup
constexpr int TM = 16;          // tokens per GEMM workgroup (one MFMA tile of rows)
constexpr int kMaxTokens = 64;
constexpr int kMaxK = 16384;    // input channels

// Sums over the 256 threads of two values in a fixed order, both reduced side by side (every
// thread gets the results): DPP and lane swaps inside each wave, then the 4 wave sums in order.
__device__ __forceinline__ void block_sum256(double (&u)[TQ], double (&v)[TQ], double (*red)[4]) {
    const auto add = [](double p, double q) { return p + q; };
#pragma unroll
    for (int q = 0; q < TQ; ++q) {
        u[q] = lanes_reduce<kWave>(u[q], add);
        v[q] = lanes_reduce<kWave>(v[q], add);
    }
    if ((threadIdx.x & 63) == 0) {
#pragma unroll
        for (int q = 0; q < TQ; ++q) {
            red[2 * q][threadIdx.x >> 6] = u[q];
            red[2 * q + 1][threadIdx.x >> 6] = v[q];
        }
    }
    __syncthreads();
#pragma unroll
    for (int q = 0; q < TQ; ++q) {
        u[q] = ((red[2 * q][0] + red[2 * q][1]) + red[2 * q][2]) + red[2 * q][3];
        v[q] = ((red[2 * q + 1][0] + red[2 * q + 1][1]) + red[2 * q + 1][2]) + red[2 * q + 1][3];
    }
    __syncthreads();
}

// grid (K / 128 channel blocks, M tokens), 256 threads.  Each workgroup quantizes the 4
// groups of its channel block for its token; at a residual loop it first forms the token's
// coefficient c from the whole row (every block computes the same sums in the same order,
// so every block gets the same c) and rotates its block of the residual (two threads per
// output, 64 float64 products each).  The quantizer runs 16 threads per group, two values
// each.
template <bool RES, int CST>
__global__ __launch_bounds__(256) void quantize_act_kernel(AArgs a) {
    constexpr int GMAX = kMaxK / GS;
    __shared__ double ys[TQ][RB];               // the block's values (x, or x - c a_hat)
    __shared__ double rs[RES ? TQ : 1][RES ? RB : 1];          // the rotated residual
    __shared__ double za[RES ? TQ : 1][RES ? GMAX : 1];        // anchor offsets and scales
    __shared__ double sa[RES ? TQ : 1][RES ? GMAX : 1];
    __shared__ double red[2 * TQ][4];
    __shared__ uint32_t cw[TQ][RB / 8];         // the block's code words
    const int t = threadIdx.x, b = blockIdx.x, m0 = blockIdx.y * TQ, K = a.k, G = K / GS;
    const int rowb = act_row_bytes(K);
    const int nq = min(TQ, a.m - m0);           // tokens of this workgroup
    // every global load first, all in flight together: R, the anchor metadata, the row
    // chunks for c (8 channels per step), and the block's own values
    constexpr int RV = RES ? RB / 2 / 4 : 1;                     // float4 of R per thread: half a row
    constexpr int CSTEP = RES ? CST : 1;                         // row steps of 2048 channels per token
    float4 rv[RV];
    uint32_t mbv[RES ? 2 : 1];
    uint4 xc[TQ][CSTEP];
    uint32_t cc[TQ][CSTEP];
    uint32_t xb[1], cb[1];
    if constexpr (RES) {
        // thread t takes row t / 2 of R, columns 64 (t % 2) .. 64 (t % 2) + 63
#pragma unroll
        for (int k = 0; k < RV; ++k) rv[k] = reinterpret_cast<const float4*>(a.rot + RB * (t / 2) + 64 * (t & 1))[k];
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int e = t + 256 * k, q = e / G, g = e % G;
            mbv[k] = (e < TQ * G && q < nq)
                         ? reinterpret_cast<const uint16_t*>(a.anchor + (size_t)(m0 + q) * rowb + K / 2)[g] : 0u;
        }
#pragma unroll
        for (int q = 0; q < TQ; ++q) {
            const int mq = m0 + min(q, nq - 1);
#pragma unroll
            for (int st = 0; st < CSTEP; ++st) {
                const int e0 = min(8 * t + 2048 * st, K - 8);
                xc[q][st] = *reinterpret_cast<const uint4*>(a.x + (int64_t)mq * a.ldx + e0);
                cc[q][st] = *reinterpret_cast<const uint32_t*>(a.anchor + (size_t)mq * rowb + e0 / 2);
            }
        }
    }
    {
        const int ch = RB * b + (t % RB);                  // threads t < 128 use their value
        xb[0] = a.x[(int64_t)m0 * a.ldx + ch];
        cb[0] = RES ? a.anchor[(size_t)m0 * rowb + ch / 2] : 0u;
    }

    double c[TQ];
#pragma unroll
    for (int q = 0; q < TQ; ++q) c[q] = 1.0;
    if constexpr (RES) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            const int e = t + 256 * k;
            if (e < TQ * G) {
                za[e / G][e % G] = e4m3_value(mbv[k] & 0xFFu);
                sa[e / G][e % G] = e4m3_value(mbv[k] >> 8);
            }
        }
        __syncthreads();
        // c = <x, a_hat> / <a_hat, a_hat> over the whole row
        double num[TQ], den[TQ];
#pragma unroll
        for (int q = 0; q < TQ; ++q) {
            num[q] = den[q] = 0.0;
#pragma unroll
            for (int st = 0; st < CSTEP; ++st) {
                const int e0 = 8 * t + 2048 * st;
                if (q < nq && e0 < K) {
                    const double z = za[q][e0 / GS], sc = sa[q][e0 / GS];
                    const uint32_t xw[4] = {xc[q][st].x, xc[q][st].y, xc[q][st].z, xc[q][st].w};
#pragma unroll
                    for (int k = 0; k < 8; ++k) {
                        const double ah = z + (double)((cc[q][st] >> (4 * k)) & 15u) * sc;
                        const double xk = (double)(k & 1 ? bf16hi(xw[k / 2]) : bf16lo(xw[k / 2]));
                        num[q] = fma(xk, ah, num[q]);
                        den[q] = fma(ah, ah, den[q]);
                    }
                }
            }
        }
        block_sum256(num, den, red);
#pragma unroll
        for (int q = 0; q < TQ; ++q) c[q] = bf16_round(den[q] > 0.0 ? num[q] / den[q] : 0.0);
    }
    // the block's values: x, or x - c a_hat
    if (t < RB) {
        const int ch = RB * b + t;
        double v = (double)bf16_to_f32(xb[0]);
        if constexpr (RES) {
            const uint32_t code = (cb[0] >> (4 * (ch & 1))) & 15u;
            v -= c[0] * (za[0][ch / GS] + (double)code * sa[0][ch / GS]);
        }
        ys[0][t] = v;
    }
    __syncthreads();
    const double (*src)[RB] = ys;
    if constexpr (RES) {
        // r_j = sum_i R[j][i] y_i: threads 2 j and 2 j + 1 take i < 64 and i >= 64 (the R values
        // already in their registers), each as 4 partial sums over i mod 4 (independent
        // chains); the halves are added by both threads (a + b == b + a), the partial sums in
        // a fixed order
        const int j = t / 2, h = t & 1;
        double p[4] = {0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int k = 0; k < RV; ++k) {
            const int i = 64 * h + 4 * k;
            p[0] = fma((double)rv[k].x, ys[0][i], p[0]);
            p[1] = fma((double)rv[k].y, ys[0][i + 1], p[1]);
            p[2] = fma((double)rv[k].z, ys[0][i + 2], p[2]);
            p[3] = fma((double)rv[k].w, ys[0][i + 3], p[3]);
        }
        double r = (p[0] + p[1]) + (p[2] + p[3]);
        r += dpp_d<kDppQuadXor1>(r);
        if (h == 0) rs[0][j] = r;
        __syncthreads();
        src = rs;
    }
    // quantize: group (t / 16) = (token q, group jg of the block), values 2u, 2u + 1 (u = t % 16)
    if (t < TQ * 64) {
        const int grp = t / 16, u = t % 16, q = grp / 4, jg = grp % 4;
        const double v0 = src[q][GS * jg + 2 * u], v1 = src[q][GS * jg + 2 * u + 1];
        const double lo = lanes_reduce<16>(fmin(v0, v1), [](double p, double q) { return fmin(p, q); });
        const double hi = lanes_reduce<16>(fmax(v0, v1), [](double p, double q) { return fmax(p, q); });
        const QOut qo = group_params(lo, hi, 4);
        const uint32_t c0 = group_code(v0, qo, 4), c1 = group_code(v1, qo, 4);
        const double sum = lanes_reduce<16>((qo.z + (double)c0 * qo.s) + (qo.z + (double)c1 * qo.s),
                                            [](double p, double q) { return p + q; });
        // byte u of the group's 16 code bytes; four neighbouring lanes form one word
        uint32_t byte = (c0 | (c1 << 4)) << (8 * (u & 3));
        byte |= (uint32_t)xshfl_i<1>((int)byte);
        byte |= (uint32_t)xshfl_i<2>((int)byte);
        if ((u & 3) == 0) cw[q][4 * jg + u / 4] = byte;
        if (u == 0 && q < nq) {
            const int g = 4 * b + jg, m = m0 + q;
            const uint16_t mb = (uint16_t)(qo.zb | (qo.sb << 8));
            reinterpret_cast<uint16_t*>(a.act + (size_t)m * rowb + K / 2)[g] = mb;
            if (a.act2) reinterpret_cast<uint16_t*>(a.act2 + (size_t)m * rowb + K / 2)[g] = mb;
            a.xsum[(size_t)m * G + g] = (float)sum;
        }
    }
    __syncthreads();
    if (t < TQ * 16 && t / 16 < nq) {
        const int q = t / 16, wd = t % 16, m = m0 + q;
        reinterpret_cast<uint32_t*>(a.act + (size_t)m * rowb + 64 * b)[wd] = cw[q][wd];
        if (a.act2) reinterpret_cast<uint32_t*>(a.act2 + (size_t)m * rowb + 64 * b)[wd] = cw[q][wd];
    }
    if (b == 0 && t < nq) {
        a.c[m0 + t] = (float)c[t];
        if (a.c2) a.c2[m0 + t] = (float)c[t];
    }
}

// ---------------------------------------------------------------- GEMM

struct GArgs {
    const uint8_t* w;           // weight tiles
    const uint8_t* act;         // 4-bit activation rows
    const float* xsum;          // [M][K/32]
    const float* c;             // [M]
    const float* y0_in;         // residual loops: the anchor product
    float* y0_out;              // anchor loop: the product kept for the group's later loops
    float* y;                   // [M][N]
    float* part;                // split K: [splits][M][N] partial sums (the epilogue then runs apart), else null
    int m, n, k;
};

__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(kMagic2));
    return r;
}

// (offset, scale) of a group from its two E4M3 bytes, as exact FP16 values
__device__ __forceinline__ h2 meta_h2(uint32_t mb) { return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(mb, 1.0f, false); }

// 8 channels (nibble e = channel e) of a code word times the group scale s, in the MFMA K
// order [0,4,1,5,2,6,3,7].  Each channel pair is moved to bits 4..7 and 20..23 and OR-ed
// into FP16 1024, giving 1024 + 16 q; one fused multiply-add (1024 + 16 q)(s / 16) - 64 s
// then yields q s exactly (q s has at most 8 significant bits and lies in [2^-9, 6720];
// s / 16 and 64 s <= 28672 are exact FP16 values).  sv = (s/16, s/16), cv = (-64 s, -64 s).
__device__ __forceinline__ h8 scaled_codes(uint32_t w, h2 sv, h2 cv) {
    const h2 p0 = __builtin_elementwise_fma(__builtin_bit_cast(h2, and_or(w << 4, 0x00F000F0u)), sv, cv);
    const h2 p1 = __builtin_elementwise_fma(__builtin_bit_cast(h2, and_or(w, 0x00F000F0u)), sv, cv);
    const h2 p2 = __builtin_elementwise_fma(__builtin_bit_cast(h2, and_or(w >> 4, 0x00F000F0u)), sv, cv);
    const h2 p3 = __builtin_elementwise_fma(__builtin_bit_cast(h2, and_or(w >> 8, 0x00F000F0u)), sv, cv);
    return (h8){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}
__device__ __forceinline__ h2 sv_of(_Float16 s) { return (h2){s, s} * (h2){(_Float16)0.0625f, (_Float16)0.0625f}; }
__device__ __forceinline__ h2 cv_of(_Float16 s) { return (h2){s, s} * (h2){(_Float16)-64.0f, (_Float16)-64.0f}; }

__device__ __forceinline__ f32x4 mfma(h8 a, h8 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

// A workgroup of NW waves (NW * GW * 32 = K channels; wave w covers the GW groups
// [w GW, (w + 1) GW)) builds the activation operands once and then walks over steps of NTW
// 16-row tiles (step blockIdx.x, + gridDim.x, ...), loading the next step's weights into a
// second register buffer while it multiplies the current one; the waves' products of a
// step are summed in LDS (two buffers, one barrier per step).  MFMA operands: A row = token
// (lane l16), B column = output row of the tile (lane l16), K = the 32 channels of a group.
// MASK: a general K.  The workgroups of split blockIdx.z take the NW NQ quads from quad
// blockIdx.z NW NQ on; a wave's quads past the row are read at the last quad (in bounds) and
// multiplied by zero activation operands.
template <int GW, int NW, int NTW, bool RES, bool MASK>
__global__ __launch_bounds__(NW * 64) void gemm_kernel(GArgs g) {
    constexpr int NQ = GW / 4;                  // weight quads per wave
    // this workgroup's tile of up to 16 tokens (blockIdx.y): the arguments shifted to its rows
    GArgs a = g;
    {
        const int m0 = TM * blockIdx.y;
        a.m = min(TM, g.m - m0);
        a.act += (size_t)m0 * act_row_bytes(g.k);
        a.xsum += (size_t)m0 * (g.k / GS);
        a.c += m0;
        if (a.y0_in) a.y0_in += (size_t)m0 * g.n;
        if (a.y0_out) a.y0_out += (size_t)m0 * g.n;
        a.y += (size_t)m0 * g.n;
        if (a.part) a.part += ((size_t)blockIdx.z * g.m + m0) * g.n;
    }
    static_assert(GW % 4 == 0 && GW <= 16, "groups per wave");
    __shared__ f32x4 red[2][NTW][NW][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l16 = lane & 15, kg = lane >> 4;
    const int tiles = a.n / TN, K = a.k, G = K / GS;
    const int pairs = (tiles + NTW - 1) / NTW;
    const int KQ = K / RB;                      // quads of a row
    const int wq0 = (MASK ? (int)blockIdx.z * NW * NQ : 0) + w * NQ;   // first quad of this wave
    const auto quad = [&](int q) { return MASK ? min(wq0 + q, KQ - 1) : wq0 + q; };
    const auto grp = [&](int gl) { return MASK ? min(4 * wq0 + gl, G - 1) : 4 * wq0 + gl; };
    const auto gvalid = [&](int gl) { return !MASK || 4 * wq0 + gl < G; };

    // the weights of pair p: row l16 of each tile, quarter kg, 4 groups per quad (a missing
    // second tile reads the first again)
    auto load_w = [&](int p, u4 (&wc)[NTW][NQ], uint2 (&wm)[NTW][NQ]) {
        const int nt0 = NTW * p;
        const bool two = nt0 + 1 < tiles;
#pragma unroll
        for (int u = 0; u < NTW; ++u) {
            const uint8_t* wt = a.w + (size_t)(two ? nt0 + u : nt0) * KQ * QB;
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
                const uint8_t* wq = wt + (size_t)quad(q) * QB;
                wc[u][q] = *reinterpret_cast<const u4*>(wq + 16 * (16 * kg + l16));
                wm[u][q] = *reinterpret_cast<const uint2*>(wq + 1024 + 8 * l16);
            }
        }
    };
    u4 wcA[NTW][NQ], wcB[NTW][NQ];
    uint2 wmA[NTW][NQ], wmB[NTW][NQ];
    int p = blockIdx.x;                         // the grid never exceeds the pair count
    load_w(p, wcA, wmA);

    // activation operands of token l16; lanes past the last token read the last token's
    // row (every load unconditional, so all are in flight together) and zero it
    const bool mok = l16 < a.m;
    const int rowb = act_row_bytes(K);
    const int mrow = mok ? l16 : a.m - 1;
    const uint8_t* arow = a.act + (size_t)mrow * rowb;
    uint32_t aw[GW], am[GW];
#pragma unroll
    for (int gl = 0; gl < GW; ++gl) {
        aw[gl] = *reinterpret_cast<const uint32_t*>(arow + 16 * grp(gl) + 4 * kg);
        am[gl] = reinterpret_cast<const uint16_t*>(arow + K / 2)[grp(gl)];
    }
    float xq[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) xq[j] = a.xsum[(size_t)mrow * G + grp(min(4 * kg + j, GW - 1))];
    // s_x q_x as exact FP16 operands; z_x kept as one packed pair per group and broadcast
    // into the 8-wide operand at each use (fewer registers than holding the operands)
    h8 a1[GW];
    uint32_t zx2[GW];
#pragma unroll
    for (int gl = 0; gl < GW; ++gl) {
        const bool ok = mok && gvalid(gl);
        const h2 zs = meta_h2(ok ? am[gl] : 0u);
        a1[gl] = scaled_codes(ok ? aw[gl] : 0u, sv_of(zs.y), cv_of(zs.y));
        zx2[gl] = __builtin_bit_cast(uint32_t, (h2){zs.x, zs.x});
    }
    // z_w X terms: K' position 8 kg + e <-> local group 4 kg + e / 2, FP16 hi (e even) / lo
    // (e odd) of X / 32 on the token side, 32 z_w on the weight side (powers of two: exact)
    h8 ax;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int gl = 4 * kg + e / 2;
        const float xv = (gl < GW && mok && gvalid(gl)) ? xq[e / 2] * (1.f / 32.f) : 0.f;
        const _Float16 hi = (_Float16)xv;
        ax[e] = (e & 1) ? (_Float16)(xv - (float)hi) : hi;
    }

    // one pair: products, the waves' sums in LDS buffer `it & 1`, waves 0 and 1 store a tile each
    auto pair = [&](int p, int it, const u4 (&wc)[NTW][NQ], const uint2 (&wm)[NTW][NQ]) {
        const int nt0 = NTW * p;
        const bool two = nt0 + 1 < tiles;
        const bool storer = w < NTW && (w == 0 || two);
        float ce[4] = {0.f, 0.f, 0.f, 0.f}, y0e[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (RES) {
            if (storer && !a.part) {
                const int n = (nt0 + w) * TN + l16;
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = min(4 * kg + r, a.m - 1);
                    ce[r] = a.c[m];
                    y0e[r] = a.y0_in[(size_t)m * a.n + n];
                }
            }
        }
#pragma unroll
        for (int u = 0; u < NTW; ++u) {
            h8 bx;
            {
                // the lane's quarter kg holds the offsets of the wave's quad kg
                uint2 mq = wm[u][0];
#pragma unroll
                for (int q = 1; q < NQ; ++q)
                    if (q == kg) mq = wm[u][q];
#pragma unroll
                for (int jp = 0; jp < 2; ++jp) {
                    const uint32_t word = jp ? mq.y : mq.x;
                    const h2 m0 = meta_h2(word & 0xFFFFu), m1 = meta_h2(word >> 16);
                    const _Float16 z0 = kg < NQ ? m0.x * (_Float16)32.0f : (_Float16)0.0f;
                    const _Float16 z1 = kg < NQ ? m1.x * (_Float16)32.0f : (_Float16)0.0f;
                    bx[4 * jp + 0] = z0;
                    bx[4 * jp + 1] = z0;
                    bx[4 * jp + 2] = z1;
                    bx[4 * jp + 3] = z1;
                }
            }
            f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int q = 0; q < NQ; ++q) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t mb = ((j < 2) ? wm[u][q].x : wm[u][q].y) >> (16 * (j & 1));
                    const _Float16 sw = meta_h2(mb & 0xFFFFu).y;
                    const h8 b = scaled_codes(wc[u][q][j], sv_of(sw), cv_of(sw));
                    const uint32_t zz = zx2[4 * q + j];
                    acc = mfma(a1[4 * q + j], b, acc);
                    acc = mfma(__builtin_bit_cast(h8, (u4){zz, zz, zz, zz}), b, acc);
                }
            }
            red[it & 1][u][w][lane] = mfma(ax, bx, acc);
        }
        __syncthreads();
        if (storer) {
            f32x4 v = red[it & 1][w][0][lane];
#pragma unroll
            for (int i = 1; i < NW; ++i) v += red[it & 1][w][i][lane];
            const int n = (nt0 + w) * TN + l16;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * kg + r;
                if (m < a.m) {
                    const size_t o = (size_t)m * a.n + n;
                    if (a.part) {
                        a.part[o] = v[r];
                    } else if constexpr (RES) {
                        a.y[o] = ce[r] * y0e[r] + v[r];
                    } else {
                        a.y[o] = v[r];
                        if (a.y0_out) a.y0_out[o] = v[r];
                    }
                }
            }
        }
    };

    // ping-pong over the workgroup's pairs: multiply with one buffer while the other loads
    for (int it = 0;; it += 2) {
        const int pb = p + gridDim.x;
        if (pb < pairs) load_w(pb, wcB, wmB);
        pair(p, it, wcA, wmA);
        if (pb >= pairs) break;
        const int pa = pb + gridDim.x;
        if (pa < pairs) load_w(pa, wcA, wmA);
        pair(pb, it + 1, wcB, wmB);
        if (pa >= pairs) break;
        p = pa;
    }
}

static int w4_cu_count() {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) !=
                                                 hipSuccess || n <= 0)
        n = 256;
    return n;
}

// two tiles per step while the registers allow (they share the activation operands), one
// at K >= 3072.  More than 16 tokens: one row of workgroups per 16-token tile (each reads
// the weights; the tiles after the first mostly from the Infinity Cache), about one
// workgroup per CU in all.  A general K: `splits` slices of up to 4096 channels
// (blockIdx.z), whose partial products a second kernel adds in order.
template <int GW, int NW, bool MASK>
static void launch_gemm(const GArgs& g, bool res, int splits, hipStream_t st) {
    constexpr int NTW = GW <= 8 ? 2 : 1;
    const int steps = (g.n / TN + NTW - 1) / NTW;
    const int tiles_m = (g.m + TM - 1) / TM;
    const int cus = w4_cu_count();
    const int per_tile = cus / (tiles_m * splits) > 0 ? cus / (tiles_m * splits) : 1;
    const dim3 grid(steps < per_tile ? steps : per_tile, tiles_m, splits);
    if (res) hipLaunchKernelGGL((gemm_kernel<GW, NW, NTW, true, MASK>), grid, dim3(NW * 64), 0, st, g);
    else hipLaunchKernelGGL((gemm_kernel<GW, NW, NTW, false, MASK>), grid, dim3(NW * 64), 0, st, g);
}

// the split-K epilogue: y = c y0 + sum of the splits' partial products (in split order) at a
// residual loop, y = y0 = the sum at the anchor loop
template <bool RES>
__global__ __launch_bounds__(256) void splitk_epilogue_kernel(GArgs g, int splits) {
    const int64_t total = (int64_t)g.m * g.n;
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= total) return;
    float v = 0.f;
    for (int s = 0; s < splits; ++s) v += g.part[s * total + i];
    if constexpr (RES) {
        g.y[i] = g.c[i / g.n] * g.y0_in[i] + v;
    } else {
        g.y[i] = v;
        if (g.y0_out) g.y0_out[i] = v;
    }
}

// channels per split of a general K
constexpr int kSplitK = 4096;
inline int splits_of(int k) { return (k + kSplitK - 1) / kSplitK; }
inline bool fast_k(int k) { return k == 1024 || k == 2048 || k == 3072 || k == 4096; }

}  // namespace w4

static bool w4_cfg_ok(const rq_w4a4_config* cfg) {
    if (!cfg) return false;
    const int k = cfg->in_features;
    return k >= w4::RB && k <= w4::kMaxK && k % w4::RB == 0 && cfg->out_features > 0 &&
           cfg->out_features % w4::TN == 0 && cfg->max_tokens >= 1 && cfg->max_tokens <= w4::kMaxTokens;
}
static bool w4_aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
static size_t w4_round256(size_t b) { return (b + 255) & ~(size_t)255; }

}  // namespace rq

using namespace rq;

extern "C" {

size_t rq_w4_weight_bytes(const rq_w4a4_config* cfg) {
    if (!w4_cfg_ok(cfg)) return 0;
    return (size_t)cfg->out_features * cfg->in_features / 2 + (size_t)cfg->out_features * cfg->in_features / 16;
}

size_t rq_w4a4_act_bytes(const rq_w4a4_config* cfg) {
    if (!w4_cfg_ok(cfg)) return 0;
    return (size_t)cfg->max_tokens * (cfg->in_features / 2 + cfg->in_features / 16);
}

// workspace: X [max_tokens][K/32], c [max_tokens], activation rows, and with a split K the
// partial products [splits][max_tokens][N]
static size_t w4_part_offset(const rq_w4a4_config* cfg) {
    const size_t m = cfg->max_tokens, k = cfg->in_features;
    return w4_round256(m * (k / w4::GS) * sizeof(float)) + w4_round256(m * sizeof(float)) +
           w4_round256(rq_w4a4_act_bytes(cfg));
}

size_t rq_w4a4_workspace_bytes(const rq_w4a4_config* cfg) {
    if (!w4_cfg_ok(cfg)) return 0;
    const int k = cfg->in_features, splits = w4::fast_k(k) ? 1 : w4::splits_of(k);
    const size_t part = splits > 1 ? w4_round256((size_t)splits * cfg->max_tokens * cfg->out_features * sizeof(float)) : 0;
    return w4_part_offset(cfg) + part;
}

rq_status rq_w4_quantize_weights(const rq_w4a4_config* cfg, const uint16_t* w, int64_t w_stride, const float* rot,
                                 void* out, hipStream_t stream) {
    if (!w4_cfg_ok(cfg) || !w || !out || w_stride < cfg->in_features) return RQ_ERR_INVALID_ARG;
    if (!w4_aligned16(out) || (rot && !w4_aligned16(rot)) || (reinterpret_cast<uintptr_t>(w) & 1u))
        return RQ_ERR_MISALIGNED;
    w4::WArgs a{w, w_stride, rot, static_cast<uint8_t*>(out), cfg->in_features, cfg->out_features};
    const dim3 grid(cfg->out_features / w4::TN, cfg->in_features / w4::RB);
    if (rot) hipLaunchKernelGGL((w4::quantize_weights_kernel<true>), grid, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((w4::quantize_weights_kernel<false>), grid, dim3(256), 0, stream, a);
    return hipGetLastError() == hipSuccess ? RQ_OK : RQ_ERR_HIP;
}

rq_status rq_w4a4_linear(const rq_w4a4_config* cfg, const void* weights, const uint16_t* x, int64_t x_stride,
                         int32_t loop_local, void* anchor, void* act, const float* rot, float* c_out, float* y0,
                         float* y, int32_t n_tokens, void* workspace, size_t workspace_bytes, hipStream_t stream) {
    if (!w4_cfg_ok(cfg) || !weights || !x || !anchor || !y0 || !y || loop_local < 0 || n_tokens < 1 ||
        n_tokens > cfg->max_tokens || x_stride < cfg->in_features || (loop_local > 0 && !rot))
        return RQ_ERR_INVALID_ARG;
    if (!w4_aligned16(weights) || !w4_aligned16(anchor) || (act && !w4_aligned16(act)) ||
        (rot && !w4_aligned16(rot)) || !w4_aligned16(x) || (x_stride % 8) != 0 ||
        (reinterpret_cast<uintptr_t>(y) & 3u) || (reinterpret_cast<uintptr_t>(y0) & 3u))
        return RQ_ERR_MISALIGNED;
    if (!workspace || workspace_bytes < rq_w4a4_workspace_bytes(cfg) || !w4_aligned16(workspace))
        return RQ_ERR_WORKSPACE;
    const int k = cfg->in_features, m = n_tokens;
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    float* xsum = reinterpret_cast<float*>(ws);
    float* cbuf = reinterpret_cast<float*>(ws + w4_round256((size_t)cfg->max_tokens * (k / w4::GS) * sizeof(float)));
    uint8_t* act_ws = reinterpret_cast<uint8_t*>(cbuf) + w4_round256((size_t)cfg->max_tokens * sizeof(float));
    const bool res = loop_local > 0;
    uint8_t* act_rows = res ? (act ? static_cast<uint8_t*>(act) : act_ws) : static_cast<uint8_t*>(anchor);

    uint8_t* act2 = (!res && act && act != anchor) ? static_cast<uint8_t*>(act) : nullptr;
    w4::AArgs qa{x, x_stride, static_cast<const uint8_t*>(anchor), act_rows, act2, rot, cbuf, c_out, xsum, k, m};
    const dim3 qgrid(k / w4::RB, (m + w4::TQ - 1) / w4::TQ);
    // row steps of 2048 channels for the c sums
    if (res) {
        if (k <= 2048) hipLaunchKernelGGL((w4::quantize_act_kernel<true, 1>), qgrid, dim3(256), 0, stream, qa);
        else if (k <= 4096) hipLaunchKernelGGL((w4::quantize_act_kernel<true, 2>), qgrid, dim3(256), 0, stream, qa);
        else if (k <= 8192) hipLaunchKernelGGL((w4::quantize_act_kernel<true, 4>), qgrid, dim3(256), 0, stream, qa);
        else hipLaunchKernelGGL((w4::quantize_act_kernel<true, 8>), qgrid, dim3(256), 0, stream, qa);
    } else {
        hipLaunchKernelGGL((w4::quantize_act_kernel<false, 1>), qgrid, dim3(256), 0, stream, qa);
    }
    if (hipGetLastError() != hipSuccess) return RQ_ERR_HIP;

    w4::GArgs g{static_cast<const uint8_t*>(weights), act_rows, xsum, cbuf, y0, res ? nullptr : y0, y, nullptr, m,
                cfg->out_features, k};
    if (w4::fast_k(k)) {
        // 8 waves per workgroup, each covering K / 256 groups
        switch (k) {
            case 1024: w4::launch_gemm<4, 8, false>(g, res, 1, stream); break;
            case 2048: w4::launch_gemm<8, 8, false>(g, res, 1, stream); break;
            case 3072: w4::launch_gemm<12, 8, false>(g, res, 1, stream); break;
            default: w4::launch_gemm<16, 8, false>(g, res, 1, stream); break;
        }
        return hipGetLastError() == hipSuccess ? RQ_OK : RQ_ERR_HIP;
    }
    const int splits = w4::splits_of(k);
    if (splits > 1) g.part = reinterpret_cast<float*>(ws + w4_part_offset(cfg));
    w4::launch_gemm<16, 8, true>(g, res, splits, stream);
    if (hipGetLastError() != hipSuccess) return RQ_ERR_HIP;
    if (splits > 1) {
        const int64_t total = (int64_t)m * cfg->out_features;
        const dim3 egrid((unsigned)((total + 255) / 256));
        if (res) hipLaunchKernelGGL((w4::splitk_epilogue_kernel<true>), egrid, dim3(256), 0, stream, g, splits);
        else hipLaunchKernelGGL((w4::splitk_epilogue_kernel<false>), egrid, dim3(256), 0, stream, g, splits);
    }
    return hipGetLastError() == hipSuccess ? RQ_OK : RQ_ERR_HIP;
}

}  // extern "C"
