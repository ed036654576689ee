/*
 * rq.h - C ABI of the ResidualQuant decode library (librq.so), AMD MI355X (gfx950).
 *
 * ResidualQuant stores the KV cache of a looped Transformer per anchor group of
 * loops: the last loop of the group ("anchor") as INT4 codes, every earlier loop as
 * a 2-bit residual r = R (kv_l - c * anchor_hat) with one BF16 least-squares
 * coefficient c per key or value vector, a fixed orthogonal rotation R per
 * (KV head, K|V), and an FP8-E4M3 offset and scale per group of contiguous
 * channels.  Decode attention rebuilds c * anchor_hat + R^T r_hat on chip.
 *
 * Sources: "ResidualQuant ... cross-loop KV residual quantization" explainer
 * (learnaivisually.com): paragraph on the master print and overlays (anchor,
 * residual, c, rotation, on-chip rebuild), paragraph "Which print is the master"
 * (shared vs chained reads, BF16 pending token), "Worked example" (4-bit anchor,
 * 2-bit residuals, FP8 scale and offset, BF16 c); arXiv digest (ai4snews),
 * Figure 1 caption (g = 32) and the paragraph on Huginn-3.5B's 8 groups of 4 loops.
 *
 * Conventions for every entry point:
 *  - Pointers named "device" are device memory owned by the caller; the library
 *    never allocates, frees or synchronises, and only enqueues work on `stream`.
 *  - BF16 tensors are passed as their 16-bit patterns (uint16_t).
 *  - All argument checks run on the host before anything is launched; a failing
 *    check returns its status and enqueues nothing.  A launch failure returns
 *    RQ_ERR_HIP.  Values inside device buffers (ctx_len, pos) are not visible to
 *    the host: the kernels clamp them as documented instead.
 *  - Calls that share a workspace must not overlap in time (same stream is fine).
 */
#ifndef RQ_H_
#define RQ_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rq_status {
    RQ_OK = 0,
    RQ_ERR_INVALID_ARG = 1,   /* null pointer, size out of range, inconsistent shape */
    RQ_ERR_UNSUPPORTED = 2,   /* configuration tuple without a compiled kernel */
    RQ_ERR_MISALIGNED = 3,    /* device pointer not 16-byte aligned */
    RQ_ERR_WORKSPACE = 4,     /* workspace missing or smaller than required */
    RQ_ERR_HIP = 5            /* the HIP runtime reported an error at launch */
} rq_status;

/* Shape of one layer's compressed cache.  Supported tuples: head_dim 64 or 128;
 * group 16 or 32 (dividing head_dim); anchor_bits 4 or 2; resid_bits 2 or 4 (4 with a
 * shared anchor only); loops_per_group 2..16 (2..4 chained); n_groups >= 1; n_q_heads a
 * multiple (1..8) of n_kv_heads; scale_rule 0 or 1.  The digest's precision settings map
 * to (anchor_bits, resid_bits) = (4, 4) uniform INT4, (2, 2) uniform INT2 and (4, 2) the
 * mixed INT2/4; its appendix's larger loop groups to loops_per_group 8 or 16. */
typedef struct rq_config {
    int32_t head_dim;         /* d */
    int32_t group;            /* g: channels per quantization group */
    int32_t anchor_bits;      /* code width of the anchor (last) loop of a group */
    int32_t resid_bits;       /* code width of the residual loops */
    int32_t loops_per_group;  /* L: loops sharing one anchor; loop L-1 of the group is the anchor */
    int32_t n_groups;         /* anchor groups; total loops = L * n_groups */
    int32_t chained;          /* 0: every loop references the anchor; 1: loop l references rebuilt loop l+1 */
    int32_t n_kv_heads;
    int32_t n_q_heads;        /* query head hq reads KV head hq / (n_q_heads / n_kv_heads) */
    int32_t max_batch;
    int32_t max_ctx;          /* token slots per sequence; storage is rounded up to 64-token tiles */
    int32_t scale_rule;       /* coefficient c of a residual loop: 0 = least squares <x,ref>/<ref,ref>
                                 (explainer and digest), 1 = norm ratio ||x||/||ref|| (the digest's
                                 appendix alternative, read as the ratio of Euclidean norms) */
    int32_t resid_bits_loop[16]; /* residual code width of local loop l (0..L-2): 2 or 4, or 0 for
                                 resid_bits; entries from L-1 on must be 0.  Per-loop widths let
                                 the loops far from the anchor keep more bits than the near ones
                                 (commentary page, section "它压的根本不是 KV"); widths that differ
                                 need the shared anchor (chained = 0).  All zero: uniform. */
} rq_config;

/* Byte layout of the cache (one flat, 16-byte-aligned device buffer):
 * [batch][KV head][K|V] blocks; each block holds the n_groups*L planes in global loop
 * order (the anchor plane is the last of its group); each plane is ceil(max_ctx/64)
 * tiles of 64 tokens; a tile holds
 *   codes: 64 rows of d*bits/8 bytes, channel i at bit i*bits of its row (little-endian),
 *          bits being the plane's own width (anchor_bits, or the loop's residual width);
 *   meta : 64 rows of 2*(d/g) bytes: E4M3 offset then E4M3 scale of each channel group;
 *   c    : residual planes only, 64 BF16 coefficients.
 * At d=128, g=32, INT4/INT2 a token costs 72 B (anchor) + 42 B (each residual) per
 * KV head per K|V.  Returns 0 for an invalid or unsupported configuration. */
size_t rq_cache_bytes(const rq_config* cfg);

/* Bytes of workspace that rq_decode_attention needs for `cfg`: one split-K partial record
 * (unnormalised output, running max, denominator) per (batch row, query head, split), then
 * one arrival counter per (batch row, query head).  The caller allocates it and fills it
 * with zeros once before its first use; every call leaves the counters at zero again, so
 * the same workspace serves any number of later calls (and HIP graph replays) as long as
 * they do not overlap in time and nothing else writes to it.  A call whose kernel does not
 * run to its end (a device fault, which also leaves the HIP context unusable) may leave
 * counters above zero, and later calls on that workspace would then merge wrong records:
 * after any RQ_ERR_HIP or device error, fill the workspace with zeros again (or allocate a
 * new one in the new context) before the next call. */
size_t rq_workspace_bytes(const rq_config* cfg);

/* Shape of one loop's uncompressed BF16 cache for the baseline decode kernel. */
typedef struct rq_bf16_config {
    int32_t head_dim;         /* 64 or 128 */
    int32_t n_kv_heads;
    int32_t n_q_heads;        /* multiple of n_kv_heads */
    int32_t max_batch;
    int32_t t_cap;            /* token slots per sequence in k_cache/v_cache */
} rq_bf16_config;

/* Workspace bytes for rq_bf16_decode_attention (same contract as rq_workspace_bytes). */
size_t rq_bf16_workspace_bytes(const rq_bf16_config* cfg);

const char* rq_status_str(rq_status status);

/* rq_quantize_token - quantize finished tokens of one anchor group into the cache.
 * Explainer, "Which print is the master": a token's K/V stay BF16 in a temporary
 * buffer until the group's last loop has run, and are quantized only then.  For
 * each (token, batch row b, KV head, K|V) and the L loops x_0..x_{L-1} of group
 * `group_idx`:
 *   anchor  : x_{L-1} quantized per group of g channels at anchor_bits;
 *   loop l<L-1 (shared): c = BF16(<x_l,a>/<a,a>) with a the dequantized anchor
 *             (c = 0 if a = 0; BF16(||x_l||/||a||) with scale_rule 1),
 *             r = R (x_l - c a), r quantized per group at resid_bits;
 *   chained : same with a replaced by the rebuilt loop l+1 (c_{l+1} a' + R^T r_hat_{l+1}).
 * Quantizer: offset z = largest E4M3 value <= group min; scale s = smallest E4M3
 * value >= 2^-9 with z + (2^bits-1) s >= group max; code = round-half-even((x-z)/s)
 * clamped to [0, 2^bits-1].  All of this is computed in float64.
 *   cfg       : host pointer.
 *   cache     : device, rq_cache_bytes(cfg) bytes; written at the token slots only.
 *   pending   : device BF16 values of x, element (t, b, l, X, h, i) at
 *               t*st[0] + b*st[1] + l*st[2] + X*st[3] + h*st[4] + i (X: 0 = K, 1 = V).
 *   pending_strides : host array of 5 element strides, or NULL for the contiguous
 *               [n_tokens][batch][L][2][n_kv_heads][head_dim] layout.
 *   group_idx : anchor group 0..n_groups-1 the loops belong to.
 *   pos       : device int32[batch]; token t of row b goes to slot pos[b] + t.  Slots
 *               outside [0, max_ctx) are skipped (nothing is written).
 *   rot       : device float32 [n_kv_heads][2][head_dim][head_dim], row-major R.
 *   batch     : rows 1..max_batch;  n_tokens : tokens per row, >= 1.
 * Inputs must be finite.  E4M3 metadata holds offsets >= -448 and scales <= 448: a
 * group whose minimum lies below -448, or whose range needs a larger scale, gets the
 * offset -448 or the scale 448 and codes clamped to [0, 2^bits-1], so the cache stays
 * finite but those elements lose the scale/2 error bound. */
rq_status rq_quantize_token(const rq_config* cfg, void* cache, const uint16_t* pending,
                            const int64_t* pending_strides, int32_t group_idx,
                            const int32_t* pos, const float* rot, int32_t batch,
                            int32_t n_tokens, hipStream_t stream);

/* rq_decode_attention - one loop-step of fused decode attention over the packed cache.
 * Explainer, paragraph on the master print: each loop's KV is rebuilt as
 * c * anchor + residual tile by tile on chip and never written back; with a shared
 * anchor a loop reads two planes (anchor + its residual), chained loop l reads the
 * anchor and the residual planes l..L-2.  The kernel never rebuilds K/V explicitly:
 * score_j = C_j (q . a_j) + sum_k gamma_jk (R_K q) . r_jk and the output accumulates
 * sum p_j C_j a_j and sum p_j gamma_jk r_jk separately, applying R_V^T once per
 * (batch row, query head) when the split-K partial results are merged.  The current
 * token (not yet quantized) is the last attention entry, in BF16.
 * One kernel is enqueued: one workgroup per (row, query head, split); the last
 * workgroup of a (row, query head) to finish merges the splits.
 * For each batch row b and query head hq (KV head h = hq / (Hq/Hkv)):
 *   out[b][hq] = softmax over j in [0, ctx_len[b]) and the current token of
 *                sm_scale * q . k_j, applied to the rebuilt values v_j.
 *   cfg       : host pointer.   cache : device, as written by rq_quantize_token.
 *   loop      : global loop index 0..L*n_groups-1 (group = loop / L).
 *   q         : device [batch][n_q_heads][head_dim], float32 (q_is_bf16 = 0) or BF16 (1).
 *   k_cur, v_cur : device BF16 [batch][n_kv_heads][head_dim], the current token's K/V of this loop.
 *   pending   : device or NULL.  If set, k_cur/v_cur are also stored into the pending
 *               buffer [batch][L][2][n_kv_heads][head_dim] at local loop loop % L (the
 *               buffer rq_quantize_token later reads).
 *   ctx_len   : device int32[batch], tokens already in the cache (clamped to [0, ctx_bound]).
 *   ctx_bound : host upper bound of every ctx_len[b], 0..max_ctx; sizes the launch.
 *   rot       : device float32 [n_kv_heads][2][head_dim][head_dim].
 *   out       : device float32 [batch][n_q_heads][head_dim].
 *   workspace : device, >= rq_workspace_bytes(cfg) bytes, zero-filled before first use.
 *   n_splits  : split-K factor 1..64, or 0 to let the library choose.
 * Alignment: cache, q, k_cur, v_cur, pending, out, rot and workspace 16-byte aligned. */
rq_status rq_decode_attention(const rq_config* cfg, const void* cache, int32_t loop,
                              const void* q, int32_t q_is_bf16,
                              const uint16_t* k_cur, const uint16_t* v_cur, uint16_t* pending,
                              const int32_t* ctx_len, int32_t ctx_bound, const float* rot,
                              float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                              int32_t batch, int32_t n_splits, hipStream_t stream);

/* rq_decode_attention_noalloc - rq_decode_attention without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation).  Same arguments, same kernels and the same
 * results as rq_decode_attention, except that the split records and arrival counters live
 * in a static device array inside the library (about 4 MiB per GPU, held until the process
 * ends): room for the arrival counters of batch * n_q_heads <= 4096 (row, query head) pairs
 * and for 4 MiB of split records, i.e. batch * n_q_heads * splits * (2 * head_dim + 4) * 4
 * bytes.  With n_splits = 0 the split count is capped to what fits; an explicit n_splits
 * that does not fit, or more than 4096 pairs, returns RQ_ERR_WORKSPACE and launches nothing.
 * It calls no allocation routine.  The first call on a device looks up the array's address
 * (hipGetSymbolAddress) and enqueues a kernel on `stream` that zeroes the counters; every
 * call leaves them at zero.  All calls on one GPU share the array: calls that overlap in
 * time on one GPU (other streams, other threads) race and give wrong results. */
rq_status rq_decode_attention_noalloc(const rq_config* cfg, const void* cache, int32_t loop, const void* q,
                                      int32_t q_is_bf16, const uint16_t* k_cur, const uint16_t* v_cur,
                                      uint16_t* pending, const int32_t* ctx_len, int32_t ctx_bound,
                                      const float* rot, float sm_scale, float* out, int32_t batch,
                                      int32_t n_splits, hipStream_t stream);

/* rq_bf16_decode_attention - the same decode attention over an uncompressed BF16
 * cache (the baseline the arXiv digest's section 5.3 compares against: BF16
 * FlashAttention decode over each loop's own KV).  With head_dim 128 and 2 or 4 query
 * heads per KV head one workgroup serves the whole query group, so each K/V tile is read
 * once per group; otherwise one workgroup per query head.
 *   cfg       : host pointer.
 *   k_cache, v_cache : device BF16 [max_batch][n_kv_heads][t_cap][head_dim] of one loop.
 *   append    : if nonzero, k_cur/v_cur are also stored at slot ctx_len[b] (when < t_cap).
 *   ctx_bound : host upper bound of every ctx_len[b], 0..t_cap.
 *   workspace : >= rq_bf16_workspace_bytes(cfg) bytes, zero-filled before first use.
 * Other arguments as for rq_decode_attention. */
rq_status rq_bf16_decode_attention(const rq_bf16_config* cfg, uint16_t* k_cache, uint16_t* v_cache,
                                   const void* q, int32_t q_is_bf16,
                                   const uint16_t* k_cur, const uint16_t* v_cur, int32_t append,
                                   const int32_t* ctx_len, int32_t ctx_bound, float sm_scale,
                                   float* out, void* workspace, size_t workspace_bytes,
                                   int32_t batch, int32_t n_splits, hipStream_t stream);

/* rq_unpack_debug - rebuild loop `loop` of every (batch row, KV head, K|V) for the token
 * slots [t0, t1) in float32: the vectors decode attention attends to, which the decode
 * kernel itself never materialises (a checking aid for the cache layout).  Explainer,
 * paragraph on the master print (a loop's KV = c * anchor + residual, the residual
 * stored in the rotated basis) and "Which print is the master" (chained loops):
 *   anchor loop       : a_hat = z + code * s per channel group;
 *   shared loop l     : c_l * a_hat + R^T r_hat_l;
 *   chained loop l    : c_l * x_hat_{l+1} + R^T r_hat_l, with x_hat of the anchor loop = a_hat.
 * Dequantized values are exact in float32; the R^T products are float32 sums.
 *   cfg    : host pointer.   cache : device, as written by rq_quantize_token.
 *   loop   : global loop index 0..L*n_groups-1.
 *   rot    : device float32 [n_kv_heads][2][head_dim][head_dim].
 *   t0, t1 : slot range, 0 <= t0 < t1 <= max_ctx (slots never written hold whatever the
 *            cache held).
 *   out    : device float32 [batch][n_kv_heads][2][t1 - t0][head_dim], written fully.
 * Alignment: cache, rot and out 16-byte aligned. */
rq_status rq_unpack_debug(const rq_config* cfg, const void* cache, int32_t loop, const float* rot,
                          int32_t t0, int32_t t1, int32_t batch, float* out, hipStream_t stream);

/* Paged cache (vLLM-style block tables).  The same 64-token tiles live in a pool of
 * physical blocks shared by all sequences.  One block holds one tile of every
 * (KV head, K|V, anchor group, loop plane), laid out as [KV head][K|V][anchor group]
 * [residual planes of loops 0..L-2 (tile bytes each), then the anchor plane's tile].
 * Row b's logical tile t (token slots 64t..64t+63) lives in block
 * block_table[b * table_stride + t].  The table is device data, so the host cannot check
 * it: an entry outside [0, n_blocks) is clamped into range (giving wrong values, never an
 * out-of-bounds access).  Rows must not share a block they write.
 * The arguments not listed below are as for the contiguous entry points.
 *   pool         : device, n_blocks * rq_paged_block_bytes(cfg) bytes, 16-byte aligned.
 *   n_blocks     : physical blocks in the pool, >= 1.
 *   block_table  : device int32 [max_batch][table_stride], 4-byte aligned.
 *   table_stride : entries per row, >= ceil(max_ctx / 64).
 * Returns 0 bytes for an invalid or unsupported configuration. */
size_t rq_paged_block_bytes(const rq_config* cfg);

/* rq_quantize_token over a paged cache: same computation as rq_quantize_token; the tile
 * of slot pos[b] + t is found through the block table. */
rq_status rq_quantize_token_paged(const rq_config* cfg, void* pool, int32_t n_blocks,
                                  const int32_t* block_table, int32_t table_stride,
                                  const uint16_t* pending, const int64_t* pending_strides,
                                  int32_t group_idx, const int32_t* pos, const float* rot,
                                  int32_t batch, int32_t n_tokens, hipStream_t stream);

/* rq_decode_attention over a paged cache: same computation and results as
 * rq_decode_attention on a contiguous cache holding the same tiles. */
rq_status rq_decode_attention_paged(const rq_config* cfg, const void* pool, int32_t n_blocks,
                                    const int32_t* block_table, int32_t table_stride, int32_t loop,
                                    const void* q, int32_t q_is_bf16,
                                    const uint16_t* k_cur, const uint16_t* v_cur, uint16_t* pending,
                                    const int32_t* ctx_len, int32_t ctx_bound, const float* rot,
                                    float sm_scale, float* out, void* workspace, size_t workspace_bytes,
                                    int32_t batch, int32_t n_splits, hipStream_t stream);

/* rq_kv_project - K and V of the current token at one loop, stored where the decode step
 * reads them.  Explainer, paragraph "Which print is the master": each loop's K/V of the
 * token being decoded stay BF16 in a temporary buffer until the anchor group's last loop
 * has run.  A looped Transformer runs the same layer every loop, so loop `loop`'s K/V are
 * the layer's projections of that loop's hidden state:
 *   k[b][h][i] = BF16(sum_c W_K[h][i][c] x[b][c]),  v likewise with W_V,
 * rounded once to BF16 (half to even) from float32 sums of the exact products (the
 * matrix cores accumulate in float32; no bias, no positional rotation).
 *   cfg       : host pointer; n_kv_heads, head_dim, loops_per_group, n_groups, max_batch.
 *   x         : device BF16 [batch][x_stride], the first `hidden` of each row used.
 *   x_stride  : elements between rows, >= hidden, a multiple of 8.
 *   hidden    : model width, a multiple of 32 in [32, 65536].
 *   w_kv      : device BF16 [2][n_kv_heads][head_dim][hidden]: the K weight rows, then the V
 *               rows, each output channel's weights contiguous over `hidden`.
 *   loop      : global loop index 0..L*n_groups-1; the pending slot is loop % L.
 *   k_cur, v_cur : device BF16 [batch][n_kv_heads][head_dim] or NULL: the decode step's
 *               current-token inputs for this loop.
 *   pending   : device BF16 [batch][L][2][n_kv_heads][head_dim] or NULL: the slot of loop
 *               `loop % L` is written, the other slots are left alone.
 *               At least one of k_cur, v_cur, pending is set.
 *   batch     : rows 1..min(max_batch, 64) (more rows return RQ_ERR_UNSUPPORTED).
 * Alignment: x, w_kv and the outputs 16-byte aligned.  One kernel is enqueued. */
rq_status rq_kv_project(const rq_config* cfg, const uint16_t* x, int64_t x_stride, int32_t hidden,
                        const uint16_t* w_kv, int32_t loop, uint16_t* k_cur, uint16_t* v_cur,
                        uint16_t* pending, int32_t batch, hipStream_t stream);

/* ---- W4A4 linear layer with cross-loop residual activations --------------------------
 * arXiv digest (ai4snews), scope paragraph after the results: the authors carry the same
 * residual-reconstruction principle over to W4A4 activation quantization (the pages give
 * no scheme).  A looped block runs the same linear layer y = W x at every loop.  Weights
 * are 4-bit codes with the KV anchor's group quantizer (groups of 32 consecutive input
 * channels of one output row, FP8-E4M3 offset rounded down, smallest covering E4M3 scale,
 * codes rounded half to even).  In each group of loops the FIRST loop's activations are
 * the 4-bit anchor a_hat (at decode time an earlier loop's layer runs before any later
 * loop's activation exists) and its product y0 = W_hat a_hat is kept; every later loop
 * takes a BF16 least-squares coefficient c = <x, a_hat> / <a_hat, a_hat> and the 4-bit
 * quantized residual r = R (x - c a_hat) (one orthogonal 128 x 128 R applied to every block
 * of 128 input channels), and its output is y = c y0 + W_R_hat r_hat, where W_R_hat is the
 * 4-bit quantization of W R^T (the rotation folded into a second weight copy).
 *
 * Byte layouts.  Weights: rows in tiles of 16, input groups in quads of 4; per (row tile,
 * quad) 1024 code bytes then 128 metadata bytes, blocks ordered by row tile then quad.
 * The 16 code bytes at 16 (16 kg + i) hold for row i of the tile four little-endian words,
 * word j for group j of the quad, channels 8 kg .. 8 kg + 7 (channel 8 kg + e in bits 4 e);
 * metadata bytes 2 (4 i + j) and 2 (4 i + j) + 1 are that group's offset and scale.
 * Activations: one row per token of K/2 code bytes (channel 2 i in the low nibble of byte
 * i, 2 i + 1 in the high one) then K/16 metadata bytes (offset, scale per group). */
typedef struct rq_w4a4_config {
    int32_t in_features;      /* K: a multiple of 128 up to 16384 (1024, 2048, 3072 and 4096 take
                                 the fastest path; others run in slices of up to 4096 channels
                                 whose partial products a second kernel adds, which the
                                 workspace holds) */
    int32_t out_features;     /* N: a positive multiple of 16 */
    int32_t max_tokens;       /* tokens per call: 1..64 (the product runs in tiles of 16) */
} rq_w4a4_config;

/* Bytes of one packed weight matrix (N K / 2 + N K / 16), of max_tokens activation rows
 * (max_tokens (K/2 + K/16)), and of the workspace rq_w4a4_linear needs; 0 for an
 * unsupported configuration. */
size_t rq_w4_weight_bytes(const rq_w4a4_config* cfg);
size_t rq_w4a4_act_bytes(const rq_w4a4_config* cfg);
size_t rq_w4a4_workspace_bytes(const rq_w4a4_config* cfg);

/* rq_w4_quantize_weights - offline: pack W (rot NULL) or W R^T (rot set) as 4-bit groups in
 * the weight tile layout.  Float64 arithmetic: codes and metadata are those of a float64
 * reference except at inexact ties of the code rounding.
 *   w        : device BF16 [out_features][w_stride], the first in_features of each row used.
 *   rot      : device float32 [128][128] (row-major R) or NULL.
 *   out      : device, rq_w4_weight_bytes(cfg) bytes, 16-byte aligned.
 * One kernel is enqueued. */
rq_status rq_w4_quantize_weights(const rq_w4a4_config* cfg, const uint16_t* w, int64_t w_stride,
                                 const float* rot, void* out, hipStream_t stream);

/* rq_w4a4_linear - one loop of the layer for n_tokens tokens.
 *   weights    : packed W_hat at loop_local 0, packed W_R_hat at loop_local > 0.
 *   x          : device BF16 [n_tokens][x_stride] activations of this loop; 16-byte aligned,
 *                x_stride a multiple of 8.
 *   loop_local : position of the loop in its group; 0 is the anchor loop.
 *   anchor     : device activation rows [max_tokens]: written at loop_local 0 (the 4-bit
 *                anchor), read at loop_local > 0.  Keep it across the group's loops.
 *   act        : device activation rows of this loop (a copy of the anchor rows at loop 0,
 *                the residual rows otherwise) or NULL (then the workspace holds them).
 *   rot        : device float32 [128][128] R; required at loop_local > 0.
 *   c_out      : device float32 [n_tokens] coefficient used (1 at the anchor loop) or NULL.
 *   y0         : device float32 [n_tokens][out_features]: the anchor product, written at
 *                loop_local 0 and read at loop_local > 0 (y0 == y is allowed at loop 0).
 *   y          : device float32 [n_tokens][out_features] output.
 * Arithmetic: the quantizers in float64 (codes as a float64 reference except inexact
 * near-ties; c within one BF16 step), the product on the matrix cores from exact FP16
 * operands with float32 accumulation.  Alignment: weights, x, anchor, act, rot, workspace
 * 16-byte aligned; y, y0 4-byte aligned.  Two kernels are enqueued (three when K is above
 * 4096 and not 1024, 2048, 3072 or 4096). */
rq_status rq_w4a4_linear(const rq_w4a4_config* cfg, const void* weights, const uint16_t* x, int64_t x_stride,
                         int32_t loop_local, void* anchor, void* act, const float* rot, float* c_out,
                         float* y0, float* y, int32_t n_tokens, void* workspace, size_t workspace_bytes,
                         hipStream_t stream);

/* rq_stream_read - a measuring stick, not part of the method: read `bytes` of `buf`
 * with plain 16-byte loads (one contiguous slab per workgroup, XOR-folded into one word
 * per thread of `sink`).  Timed over the same buffers as the decode kernel it gives the
 * read rate a simple load loop reaches on the device, next to the datasheet peak.
 *   buf        : device, 16-byte aligned; bytes : a nonzero multiple of 16.
 *   sink       : device uint32 scratch of sink_words >= 1048576 words (contents unspecified). */
rq_status rq_stream_read(const void* buf, size_t bytes, uint32_t* sink, size_t sink_words,
                         hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* RQ_H_ */
