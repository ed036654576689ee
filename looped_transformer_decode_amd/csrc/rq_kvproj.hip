// rq_kv_project: K and V of the current token at one loop, written where the decode step
// reads them.
//
// ResidualQuant explainer, paragraph "Which print is the master": every loop's K/V of the
// token being decoded stays BF16 in a temporary buffer until the anchor group's last loop
// has run; only then is the token quantized.  A looped Transformer runs the same layer in
// every loop, so loop l's K/V are that layer's projections of the loop's hidden state x:
// k = W_K x, v = W_V x.  This kernel computes them on the matrix cores and its epilogue
// rounds them once to BF16 and stores them both as the decode kernel's current-token
// inputs (k_cur, v_cur) and into the pending buffer slot of the loop, so no separate K/V
// tensor and no copy sit between the projection and the cache.
//
// Shape: M = batch rows (1..64, in tiles of 16), N = 2 * n_kv_heads * head_dim outputs,
// K = hidden.  With a handful of rows the product is a stream of the weights (N * hidden
// BF16 bytes), so the launch is laid out for memory parallelism: one workgroup of 8 waves
// per 16 output channels, each wave owning a contiguous eighth of `hidden` and issuing all
// of a round's loads (16 bytes per lane, up to 16 k-steps of 32) before its first product.
#include "rq_args.hpp"

namespace rq {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kPW = 8;      // waves per workgroup

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}

// float32 -> BF16, round to nearest, ties to even (finite inputs): add half a BF16 unit in
// the last place, minus one unless the kept part is odd, and truncate.
__device__ __forceinline__ uint16_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// Matrix-core operand layout of v_mfma_f32_16x16x32_bf16 (64 lanes, g = lane / 16):
//   A (16 x 32, rows = batch rows)      lane holds A[lane % 16][8g .. 8g+7]
//   B (32 x 16, columns = outputs)      lane holds B[8g .. 8g+7][lane % 16]
//   D (16 x 16 float32)                 lane holds D[4g + r][lane % 16], r = 0..3
// The k index is the same function of (g, element) in A and B, so A = 8 consecutive
// hidden channels of one row of x and B = the same 8 channels of one weight row: both are
// one 16-byte load.
// MT: tiles of 16 batch rows; KU: k-steps of 32 channels loaded per wave before its
// products (the launch picks the smallest power of two covering a wave's share of `hidden`,
// at most 16, so no load is spent on a k-step outside the share).  XC > 0 (one row tile):
// the batch rows of x are staged once per workgroup in LDS, XC 16-byte chunks per thread,
// instead of every wave loading its A operands from L2 (eight waves read the same rows).
template <int MT, int KU, int XC>
__global__ __launch_bounds__(kPW * 64) void rq_kv_project_kernel(KvProjArgs a) {
    static_assert(XC == 0 || MT == 1, "x is staged for one row tile only");
    __shared__ float red[kPW][MT][4][64];
    // staged rows, then one spare 16-byte slot that takes the stores of clamped chunks
    constexpr int kSpare = XC * kPW * 64 * 16 + 16 * 16;
    __shared__ __attribute__((aligned(16))) uint8_t xs[XC > 0 ? kSpare + 16 : 16];
    const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    const int col = lane & 15, g = lane >> 4;
    const int n0 = blockIdx.x * 16;
    const int ns = a.hidden / 32;                       // k-steps
    const int s0 = wv * ns / kPW, s1 = (wv + 1) * ns / kPW;
    const uint8_t* wrow = reinterpret_cast<const uint8_t*>(a.w + (int64_t)(n0 + col) * a.hidden) + g * 16;
    // staged row r starts at r * xrow bytes; the 16-byte pad moves each row four LDS banks on,
    // so the 16 rows of an A-operand read hit distinct banks
    const int xrow = 2 * a.hidden + 16;
    f32x4 acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m) acc[m] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Loads are unconditional (a k-step past the wave's range re-reads its last one, a row
    // past `batch` reads row 0) and the operands of those are zeroed after they land; a
    // scheduling barrier keeps every load of a round ahead of the first product, so one
    // round costs one memory latency instead of one per k-step.
    u32x4 xst[XC > 0 ? XC : 1];
    if constexpr (XC > 0) {
        const int per_row = a.hidden / 8, total = a.batch * per_row;
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            const int c = min((int)threadIdx.x + i * kPW * 64, total - 1);
            const int r = c / per_row, k8 = c - r * per_row;
            xst[i] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(a.x + (int64_t)r * a.x_stride) +
                                                     k8 * 16);
        }
    }
    u32x4 wb[KU];
    auto load_w = [&](int s, int nk) {
#pragma unroll
        for (int j = 0; j < KU; ++j)
            wb[j] = *reinterpret_cast<const u32x4*>(wrow + (int64_t)min(s + min(j, nk - 1), ns - 1) * 64);
    };
    // the first round's weights go out before the staging waits for x (a wave without a
    // share loads and ignores its clamped last k-step)
    load_w(s0, max(1, min(KU, s1 - s0)));
    if constexpr (XC > 0) {
        const int per_row = a.hidden / 8, total = a.batch * per_row;
#pragma unroll
        for (int i = 0; i < XC; ++i) {
            // unconditional store (a branch would let the compiler sink the load into it,
            // behind a wait for every weight load)
            const int c = (int)threadIdx.x + i * kPW * 64;
            const int r = c / per_row, k8 = c - r * per_row;
            *reinterpret_cast<u32x4*>(&xs[c < total ? r * xrow + k8 * 16 : kSpare]) = xst[i];
        }
        __syncthreads();
    }
    for (int s = s0; s < s1; s += KU) {
        const int nk = min(KU, s1 - s);
        if (s != s0) load_w(s, nk);
        u32x4 xb[MT][KU];
        if constexpr (XC == 0) {
#pragma unroll
            for (int m = 0; m < MT; ++m) {
                const int r = m * 16 + col;              // batch row of this lane's A operand
                const uint8_t* xr =
                    reinterpret_cast<const uint8_t*>(a.x + (int64_t)(r < a.batch ? r : 0) * a.x_stride) + g * 16;
#pragma unroll
                for (int j = 0; j < KU; ++j)
                    xb[m][j] = *reinterpret_cast<const u32x4*>(xr + (int64_t)(s + min(j, nk - 1)) * 64);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            const bool live = m * 16 + col < a.batch;
#pragma unroll
            for (int j = 0; j < KU; ++j) {
                u32x4 xa;
                if constexpr (XC > 0)
                    xa = *reinterpret_cast<const u32x4*>(&xs[(live ? col : 0) * xrow + (s + min(j, nk - 1)) * 64 + g * 16]);
                else
                    xa = xb[m][j];
                xa = (live && j < nk) ? xa : u32x4{0u, 0u, 0u, 0u};
                acc[m] = mfma_bf16(xa, wb[j], acc[m]);
            }
        }
    }

    // the 8 waves' partial sums, added in wave order
#pragma unroll
    for (int m = 0; m < MT; ++m)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wv][m][r][lane] = acc[m][r];
    __syncthreads();
    const int hd = a.hkv * a.d;
    for (int e = threadIdx.x; e < MT * 256; e += kPW * 64) {
        const int m = e >> 8, i = (e >> 4) & 15, j = e & 15;    // tile, row in tile, output in tile
        const int row = m * 16 + i;
        if (row >= a.batch) continue;
        const int src = 16 * (i >> 2) + j;
        float y = 0.f;
#pragma unroll
        for (int w = 0; w < kPW; ++w) y += red[w][m][i & 3][src];
        const uint16_t v = bf16_rne(y);
        const int n = n0 + j;
        const int x = n / hd, hc = n % hd;                        // K|V, then head * d + channel
        uint16_t* cur = x ? a.v_out : a.k_out;
        if (cur) cur[(int64_t)row * hd + hc] = v;
        if (a.pending) a.pending[((int64_t)(row * a.L + a.lloc) * 2 + x) * hd + hc] = v;
    }
}

template <int MT, int XC>
hipError_t launch_ku(const KvProjArgs& a, int ku, dim3 grid, dim3 block, hipStream_t st) {
    switch (ku) {
        case 1: hipLaunchKernelGGL((rq_kv_project_kernel<MT, 1, XC>), grid, block, 0, st, a); break;
        case 2: hipLaunchKernelGGL((rq_kv_project_kernel<MT, 2, XC>), grid, block, 0, st, a); break;
        case 4: hipLaunchKernelGGL((rq_kv_project_kernel<MT, 4, XC>), grid, block, 0, st, a); break;
        case 8: hipLaunchKernelGGL((rq_kv_project_kernel<MT, 8, XC>), grid, block, 0, st, a); break;
        default:
            if constexpr (MT < 4) hipLaunchKernelGGL((rq_kv_project_kernel<MT, 16, XC>), grid, block, 0, st, a);
            else return hipErrorInvalidValue;
            break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_kv_project(const KvProjArgs& a, hipStream_t st) {
    if (!a.x || !a.w || (!a.k_out && !a.v_out && !a.pending) || a.batch < 1 || a.batch > 64 || a.hidden < 32 ||
        a.hidden % 32 != 0 || a.x_stride < a.hidden || (2 * a.hkv * a.d) % 16 != 0)
        return hipErrorInvalidValue;
    const dim3 grid(2 * a.hkv * a.d / 16), block(kPW * 64);
    const int share = (a.hidden / 32 + kPW - 1) / kPW;          // k-steps of the widest wave
    const int ku = share <= 1 ? 1 : share <= 2 ? 2 : share <= 4 ? 4 : share <= 8 ? 8 : 16;
    const int mt = (a.batch + 15) / 16;
    if (mt == 1) {
        // x staged in LDS when its rows fit 16 chunks of 16 bytes per thread (<= 128 KB)
        const int chunks = (a.batch * (a.hidden / 8) + kPW * 64 - 1) / (kPW * 64);
        if (chunks <= 2) return launch_ku<1, 2>(a, ku, grid, block, st);
        if (chunks <= 8) return launch_ku<1, 8>(a, ku, grid, block, st);
        if (chunks <= 16) return launch_ku<1, 16>(a, ku, grid, block, st);
        return launch_ku<1, 0>(a, ku, grid, block, st);
    }
    if (mt == 2) return launch_ku<2, 0>(a, ku, grid, block, st);
    return launch_ku<4, 0>(a, ku < 16 ? ku : 8, grid, block, st);   // 4 row tiles: 8 k-steps per round at most
}

}  // namespace rq
