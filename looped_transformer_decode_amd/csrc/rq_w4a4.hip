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

constexpr int TQ = 4;           // tokens per activation-quantizer workgroup

// Sums over the 256 threads in a fixed order, TQ values per thread at once (every thread
// gets the results).
__device__ __forceinline__ void block_sum256(double (&v)[TQ], double (*red)[256]) {
#pragma unroll
    for (int q = 0; q < TQ; ++q) red[q][threadIdx.x] = v[q];
    __syncthreads();
    for (int s = 128; s > 0; s >>= 1) {
        if (threadIdx.x < s) {
#pragma unroll
            for (int q = 0; q < TQ; ++q) red[q][threadIdx.x] += red[q][threadIdx.x + s];
        }
        __syncthreads();
    }
#pragma unroll
    for (int q = 0; q < TQ; ++q) v[q] = red[q][0];
    __syncthreads();
}

// grid (K / 128 channel blocks, ceil(M / 4) token quads), 256 threads.  Each workgroup
// quantizes the 4 groups of its channel block for its 4 tokens; at a residual loop it
// first forms each token's coefficient c from the whole row (every block computes the
// same sums in the same order, so every block gets the same c) and rotates its block of
// the residual (two outputs per thread, 128 float64 products each).
template <bool RES>
__global__ __launch_bounds__(256) void quantize_act_kernel(AArgs a) {
    __shared__ double ys[TQ][RB];               // the block's values (x, or x - c a_hat)
    __shared__ double rs[RES ? TQ : 1][RES ? RB : 1];   // the rotated residual
    __shared__ float rt[RES ? RB : 1][RES ? RB : 1];    // rt[i][j] = R[j][i]
    __shared__ double red[RES ? TQ : 1][RES ? 256 : 1];
    const int t = threadIdx.x, b = blockIdx.x, m0 = blockIdx.y * TQ, K = a.k, G = K / GS;
    const int rowb = act_row_bytes(K);
    const int nq = min(TQ, a.m - m0);           // tokens of this workgroup
    double c[TQ];
#pragma unroll
    for (int q = 0; q < TQ; ++q) c[q] = 1.0;
    if constexpr (RES) {
        for (int e = t; e < RB * RB; e += 256) rt[e % RB][e / RB] = a.rot[e];
        // c = <x, a_hat> / <a_hat, a_hat> over the whole row
        double num[TQ], den[TQ];
#pragma unroll
        for (int q = 0; q < TQ; ++q) {
            num[q] = den[q] = 0.0;
            if (q < nq) {
                const uint16_t* xr = a.x + (int64_t)(m0 + q) * a.ldx;
                const uint8_t* arow = a.anchor + (size_t)(m0 + q) * rowb;
                for (int e = t; e < K; e += 256) {
                    const uint32_t code = (arow[e / 2] >> (4 * (e & 1))) & 15u;
                    const uint32_t mb = reinterpret_cast<const uint16_t*>(arow + K / 2)[e / GS];
                    const double ah = e4m3_value(mb & 0xFFu) + (double)code * e4m3_value(mb >> 8);
                    num[q] = fma((double)bf16_to_f32(xr[e]), ah, num[q]);
                    den[q] = fma(ah, ah, den[q]);
                }
            }
        }
        block_sum256(num, red);
        block_sum256(den, red);
#pragma unroll
        for (int q = 0; q < TQ; ++q) c[q] = bf16_round(den[q] > 0.0 ? num[q] / den[q] : 0.0);
    }
    // the block's values: x, or x - c a_hat
    for (int e = t; e < TQ * RB; e += 256) {
        const int q = e / RB, i = e % RB, ch = RB * b + i;
        double v = 0.0;
        if (q < nq) {
            v = (double)bf16_to_f32(a.x[(int64_t)(m0 + q) * a.ldx + ch]);
            if constexpr (RES) {
                const uint8_t* arow = a.anchor + (size_t)(m0 + q) * rowb;
                const uint32_t code = (arow[ch / 2] >> (4 * (ch & 1))) & 15u;
                const uint32_t mb = reinterpret_cast<const uint16_t*>(arow + K / 2)[ch / GS];
                v -= c[q] * (e4m3_value(mb & 0xFFu) + (double)code * e4m3_value(mb >> 8));
            }
        }
        ys[q][i] = v;
    }
    __syncthreads();
    const double (*src)[RB] = ys;
    if constexpr (RES) {
        // r_j = sum_i R[j][i] y_i: thread t -> token t / 64, outputs 2 (t % 64), 2 (t % 64) + 1
        const int q = t / 64, j = 2 * (t % 64);
        double r0 = 0.0, r1 = 0.0;
        for (int i = 0; i < RB; ++i) {
            r0 = fma((double)rt[i][j], ys[q][i], r0);
            r1 = fma((double)rt[i][j + 1], ys[q][i], r1);
        }
        rs[q][j] = r0;
        rs[q][j + 1] = r1;
        __syncthreads();
        src = rs;
    }
    // quantize: thread t < 16 -> token t / 4, group t % 4 of the block
    if (t < TQ * 4 && t / 4 < nq) {
        const int q = t / 4, jg = t % 4, g = 4 * b + jg, m = m0 + q;
        const double* v = &src[q][GS * jg];
        double lo = v[0], hi = v[0];
        for (int e = 1; e < GS; ++e) {
            lo = fmin(lo, v[e]);
            hi = fmax(hi, v[e]);
        }
        const QOut qo = group_params(lo, hi, 4);
        uint8_t* row = a.act + (size_t)m * rowb;
        double sum = 0.0;
        for (int w = 0; w < 4; ++w) {
            uint32_t word = 0;
            for (int e = 0; e < 8; ++e) {
                const uint32_t code = group_code(v[8 * w + e], qo, 4);
                word |= code << (4 * e);
                sum += qo.z + (double)code * qo.s;
            }
            reinterpret_cast<uint32_t*>(row + 16 * g)[w] = word;
            if (a.act2) reinterpret_cast<uint32_t*>(a.act2 + (size_t)m * rowb + 16 * g)[w] = word;
        }
        const uint16_t mb = (uint16_t)(qo.zb | (qo.sb << 8));
        reinterpret_cast<uint16_t*>(row + K / 2)[g] = mb;
        if (a.act2) reinterpret_cast<uint16_t*>(a.act2 + (size_t)m * rowb + K / 2)[g] = mb;
        a.xsum[(size_t)m * G + g] = (float)sum;
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
    int m, n, k;
};

__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask) {
    uint32_t r;
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(kMagic2));
    return r;
}
// (1024 + v, 1024 + v') -> (v, v') exactly
__device__ __forceinline__ h2 unmagic(uint32_t r) {
    return __builtin_bit_cast(h2, r) - (h2){(_Float16)1024.0f, (_Float16)1024.0f};
}

// 8 channels (nibble e = channel e) of a code word times scale s, in the MFMA K order
// [0,4,1,5,2,6,3,7]; every value is exact in FP16 (4-bit code x 4-significant-bit E4M3
// scale, magnitude in [2^-9, 6720]).  Odd channel pairs come out of the mask as 16 q and
// are scaled by s / 16 (an exact power-of-two step, still a normal FP16 value).
__device__ __forceinline__ h8 scaled_codes(uint32_t w, _Float16 s) {
    const uint32_t w8 = w >> 8;
    const _Float16 s16 = s * (_Float16)0.0625f;
    const h2 p0 = unmagic(and_or(w, 0x000F000Fu)) * (h2){s, s};
    const h2 p1 = unmagic(and_or(w, 0x00F000F0u)) * (h2){s16, s16};
    const h2 p2 = unmagic(and_or(w8, 0x000F000Fu)) * (h2){s, s};
    const h2 p3 = unmagic(and_or(w8, 0x00F000F0u)) * (h2){s16, s16};
    return (h8){p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
}

__device__ __forceinline__ f32x4 mfma(h8 a, h8 b, f32x4 c) { return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0); }

// one workgroup (8 waves) per tile of 16 output rows; wave w covers the GW groups
// [w GW, (w + 1) GW) of the input channels, the waves' products are summed in LDS.
// MFMA operands: A row = token (lane l16), B column = output row of the tile (lane l16),
// K = the 32 channels of one group (8 per lane quarter kg).
template <int GW, bool RES>
__global__ __launch_bounds__(512) void gemm_kernel(GArgs a) {
    constexpr int NQ = GW / 4;                  // weight quads per wave
    static_assert(GW % 4 == 0 && GW <= 16, "groups per wave");
    __shared__ f32x4 red[8][64];
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, l16 = lane & 15, kg = lane >> 4;
    const int nt = blockIdx.x, K = a.k, G = K / GS;

    // weights of the wave's quads: row l16 of the tile, quarter kg, 4 groups per quad
    const uint8_t* wt = a.w + ((size_t)nt * (K / RB) + (size_t)w * NQ) * QB;
    u4 wc[NQ];
    uint2 wm[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
        wc[q] = *reinterpret_cast<const u4*>(wt + q * QB + 16 * (16 * kg + l16));
        wm[q] = *reinterpret_cast<const uint2*>(wt + q * QB + 1024 + 8 * l16);
    }

    // activation operands of token l16 (zero rows past the last token)
    const bool mok = l16 < a.m;
    const int rowb = act_row_bytes(K);
    const uint8_t* arow = a.act + (size_t)(mok ? l16 : 0) * rowb;
    h8 a1[GW], a2[GW];
#pragma unroll
    for (int gl = 0; gl < GW; ++gl) {
        const int g = w * GW + gl;
        const uint32_t word = mok ? *reinterpret_cast<const uint32_t*>(arow + 16 * g + 4 * kg) : 0u;
        const uint32_t mb = mok ? reinterpret_cast<const uint16_t*>(arow + K / 2)[g] : 0u;
        const _Float16 zx = (_Float16)e4m3_to_f32(mb & 0xFFu), sx = (_Float16)e4m3_to_f32(mb >> 8);
        a1[gl] = scaled_codes(word, sx);
        a2[gl] = (h8){zx, zx, zx, zx, zx, zx, zx, zx};
    }
    // z_w X terms: K' position 8 kg + e <-> local group 4 kg + e / 2, FP16 hi (e even) / lo
    // (e odd) of X / 32 on the token side, 32 z_w on the weight side (powers of two: exact)
    h8 ax = {}, bx = {};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int gl = 4 * kg + e / 2;
        if (gl < GW && mok) {
            const float xv = a.xsum[(size_t)l16 * G + w * GW + gl] * (1.f / 32.f);
            const _Float16 hi = (_Float16)xv;
            ax[e] = (e & 1) ? (_Float16)(xv - (float)hi) : hi;
        }
    }
    {
        // the lane's quarter kg holds the zero points of the wave's quad kg
        uint2 mq = {0u, 0u};
#pragma unroll
        for (int q = 0; q < NQ; ++q)
            if (q == kg) mq = wm[q];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int j = e / 2;
            const uint32_t mb = (j < 2 ? mq.x : mq.y) >> (16 * (j & 1));
            if (kg < NQ) bx[e] = (_Float16)(32.f * e4m3_to_f32(mb & 0xFFu));
        }
    }

    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint32_t mb = ((j < 2) ? wm[q].x : wm[q].y) >> (16 * (j & 1));
            const _Float16 sw = (_Float16)e4m3_to_f32((mb >> 8) & 0xFFu);
            const h8 b = scaled_codes(wc[q][j], sw);
            acc = mfma(a1[4 * q + j], b, acc);
            acc = mfma(a2[4 * q + j], b, acc);
        }
    }
    acc = mfma(ax, bx, acc);

    red[w][lane] = acc;
    __syncthreads();
    if (w == 0) {
        f32x4 v = red[0][lane];
#pragma unroll
        for (int i = 1; i < 8; ++i) v += red[i][lane];
        const int n = nt * TN + l16;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = 4 * kg + r;
            if (m < a.m) {
                const size_t o = (size_t)m * a.n + n;
                if constexpr (RES) {
                    a.y[o] = a.c[m] * a.y0_in[o] + v[r];
                } else {
                    a.y[o] = v[r];
                    if (a.y0_out) a.y0_out[o] = v[r];
                }
            }
        }
    }
}

template <int GW>
static void launch_gemm(const GArgs& g, bool res, hipStream_t st) {
    const dim3 grid(g.n / TN);
    if (res) hipLaunchKernelGGL((gemm_kernel<GW, true>), grid, dim3(512), 0, st, g);
    else hipLaunchKernelGGL((gemm_kernel<GW, false>), grid, dim3(512), 0, st, g);
}

}  // namespace w4

static bool w4_cfg_ok(const rq_w4a4_config* cfg) {
    if (!cfg) return false;
    const int k = cfg->in_features;
    return (k == 1024 || k == 2048 || k == 3072 || k == 4096) && cfg->out_features > 0 &&
           cfg->out_features % w4::TN == 0 && cfg->max_tokens >= 1 && cfg->max_tokens <= 16;
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

size_t rq_w4a4_workspace_bytes(const rq_w4a4_config* cfg) {
    if (!w4_cfg_ok(cfg)) return 0;
    const size_t m = cfg->max_tokens, k = cfg->in_features;
    return w4_round256(m * (k / w4::GS) * sizeof(float)) + w4_round256(m * sizeof(float)) +
           w4_round256(rq_w4a4_act_bytes(cfg));
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
        (rot && !w4_aligned16(rot)) || (reinterpret_cast<uintptr_t>(x) & 1u) ||
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
    if (res) hipLaunchKernelGGL((w4::quantize_act_kernel<true>), qgrid, dim3(256), 0, stream, qa);
    else hipLaunchKernelGGL((w4::quantize_act_kernel<false>), qgrid, dim3(256), 0, stream, qa);
    if (hipGetLastError() != hipSuccess) return RQ_ERR_HIP;

    w4::GArgs g{static_cast<const uint8_t*>(weights), act_rows, xsum, cbuf, y0, res ? nullptr : y0, y, m,
                cfg->out_features, k};
    switch (k / 256) {
        case 4: w4::launch_gemm<4>(g, res, stream); break;
        case 8: w4::launch_gemm<8>(g, res, stream); break;
        case 12: w4::launch_gemm<12>(g, res, stream); break;
        default: w4::launch_gemm<16>(g, res, stream); break;
    }
    return hipGetLastError() == hipSuccess ? RQ_OK : RQ_ERR_HIP;
}

}  // extern "C"
