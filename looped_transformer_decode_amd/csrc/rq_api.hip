// C ABI of librq.so: argument validation on the host, then kernel launches.
#include <string.h>

#include <atomic>
#include <mutex>

#include "rq_args.hpp"

namespace rq {


bool make_geom(const rq_config* c, Geom* g) {
    if (c == nullptr) return false;
    const int d = c->head_dim, gs = c->group;
    if (d != 64 && d != 128) return false;
    if ((gs != 16 && gs != 32) || d % gs != 0) return false;
    if (c->anchor_bits != 4 && c->anchor_bits != 2) return false;
    if (c->resid_bits != 2 && c->resid_bits != 4) return false;
    if (c->loops_per_group < 2 || c->loops_per_group > kMaxLoops) return false;
    bool mixed = false;
    for (int l = 0; l < kMaxLoops; ++l) {
        const int w = c->resid_bits_loop[l];
        if (w != 0 && (l >= c->loops_per_group - 1 || (w != 2 && w != 4))) return false;
        if (w != 0 && w != c->resid_bits) mixed = true;
    }
    if (mixed && c->chained) return false;                      // chained decode reads one width
    if (c->n_groups < 1 || c->n_groups > 64) return false;
    if (c->chained != 0 && c->chained != 1) return false;
    if (c->chained && c->loops_per_group > 4) return false;     // kernels read at most 3 residual planes
    if (c->chained && c->resid_bits != 2) return false;
    if (c->scale_rule != 0 && c->scale_rule != 1) return false;
    if (c->n_kv_heads < 1 || c->n_q_heads < c->n_kv_heads || c->n_q_heads % c->n_kv_heads != 0) return false;
    if (c->n_q_heads / c->n_kv_heads > 8) return false;
    if (c->max_batch < 1 || c->max_ctx < 1 || c->max_ctx > (1 << 24)) return false;
    g->d = d;
    g->g = gs;
    g->ba = c->anchor_bits;
    g->br = c->resid_bits;
    g->L = c->loops_per_group;
    g->n_groups = c->n_groups;
    g->chained = c->chained;
    g->hkv = c->n_kv_heads;
    g->hq = c->n_q_heads;
    g->max_batch = c->max_batch;
    g->max_ctx = c->max_ctx;
    g->scale_rule = c->scale_rule;
    g->n_tiles = (c->max_ctx + kTile - 1) / kTile;
    g->a_row = d * g->ba / 8;
    g->m_row = 2 * (d / gs);
    g->a_tile = (int64_t)kTile * (g->a_row + g->m_row);
    int64_t pre = 0;
    for (int l = 0; l < kMaxLoops; ++l) {
        g->rb[l] = (l < g->L - 1) ? (c->resid_bits_loop[l] ? c->resid_bits_loop[l] : g->br) : 0;
        g->r_pre[l] = pre;
        if (l < g->L - 1) pre += g->rtile(l);
    }
    g->group_bytes = (int64_t)g->n_tiles * (g->a_tile + g->r_pre[g->L - 1]);
    g->block_bytes = (int64_t)g->n_groups * g->group_bytes;
    g->total = (int64_t)g->max_batch * g->hkv * 2 * g->block_bytes;
    g->bt = nullptr;
    g->bt_stride = 0;
    g->n_blocks = 0;
    g->g_tile = g->a_tile + g->r_pre[g->L - 1];
    g->p_block = (int64_t)g->hkv * 2 * g->n_groups * g->g_tile;
    return true;
}

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Compute units of the current device (queried once per device; 256 on MI355X).
static int device_cu_count() {
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

// Split-K factor: about two workgroups per CU (4 waves each) in flight, and at least four
// 64-token tiles per workgroup so that its prologue (queries, R_K q) and epilogue (wave
// merge, R_V^T) stay small next to its stream.
// rows = independent (batch row, head) units of the grid; target = workgroups wanted
static int auto_splits(int rows, int n_tiles, int target) {
    if (n_tiles <= 0) return 1;
    int s = (target + rows - 1) / rows;
    const int by_tiles = n_tiles / 4 > 0 ? n_tiles / 4 : 1;
    if (s > by_tiles) s = by_tiles;
    if (s > kMaxSplits) s = kMaxSplits;
    return s < 1 ? 1 : s;
}

// ---- scratch of the entry point that allocates nothing (rq_decode_attention_noalloc):
// one arrival counter per (batch row, query head) for up to kScratchPairs pairs, then the
// split records.  Each GPU holds its own copy until the process ends; its address comes
// from hipGetSymbolAddress once per device (the array's name is a host-side stand-in).
constexpr int64_t kScratchPairs = 4096;
constexpr int64_t kScratchCounterBytes = kScratchPairs * sizeof(uint32_t);
constexpr int64_t kScratchRecordBytes = (int64_t)4 << 20;

static __device__ __align__(256) uint8_t scratch[kScratchCounterBytes + kScratchRecordBytes];

__global__ void scratch_zero_kernel(uint32_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// Device address of the current device's scratch; nullptr on a HIP error.  The first call
// on a device looks the address up and enqueues a fill kernel on `stream` that zeroes the
// counters (every decode call leaves them at zero again); a fill kernel rather than a memset,
// so that a first call made under HIP graph capture records a kernel node.
static uint8_t* scratch_base(hipStream_t stream) {
    static std::mutex mu;
    static uint8_t* addr[64] = {};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (addr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
        const int n = (int)(kScratchCounterBytes / sizeof(uint32_t));
        hipLaunchKernelGGL(scratch_zero_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, static_cast<uint32_t*>(p), n);
        if (hipGetLastError() != hipSuccess) return nullptr;
        addr[dev] = static_cast<uint8_t*>(p);
    }
    return addr[dev];
}

}  // namespace rq

using namespace rq;

extern "C" {

size_t rq_cache_bytes(const rq_config* cfg) {
    Geom g;
    if (!make_geom(cfg, &g)) return 0;
    return (size_t)g.total;
}

size_t rq_workspace_bytes(const rq_config* cfg) {
    Geom g;
    if (!make_geom(cfg, &g)) return 0;
    return workspace_bytes(g.max_batch, g.hq, g.d);
}

static bool bf16_cfg_ok(const rq_bf16_config* c) {
    return c != nullptr && (c->head_dim == 64 || c->head_dim == 128) && c->n_kv_heads >= 1 &&
           c->n_q_heads >= c->n_kv_heads && c->n_q_heads % c->n_kv_heads == 0 && c->max_batch >= 1 &&
           c->t_cap >= 1 && c->t_cap <= (1 << 24);
}

size_t rq_bf16_workspace_bytes(const rq_bf16_config* cfg) {
    if (!bf16_cfg_ok(cfg)) return 0;
    return workspace_bytes(cfg->max_batch, cfg->n_q_heads, cfg->head_dim);
}

const char* rq_status_str(rq_status s) {
    switch (s) {
        case RQ_OK: return "ok";
        case RQ_ERR_INVALID_ARG: return "invalid argument";
        case RQ_ERR_UNSUPPORTED: return "unsupported configuration";
        case RQ_ERR_MISALIGNED: return "device pointer not 16-byte aligned";
        case RQ_ERR_WORKSPACE: return "workspace missing or too small";
        case RQ_ERR_HIP: return "HIP launch error";
    }
    return "unknown status";
}

// paging: bt == nullptr for the contiguous layout, else the block table (checked by the callers)
static rq_status quantize_impl(const rq_config* cfg, void* cache, const int32_t* bt, int32_t bt_stride,
                               int32_t n_blocks, const uint16_t* pending, const int64_t* pending_strides,
                               int32_t group_idx, const int32_t* pos, const float* rot, int32_t batch,
                               int32_t n_tokens, hipStream_t stream) {
    Geom g;
    if (cfg == nullptr) return RQ_ERR_INVALID_ARG;
    if (!make_geom(cfg, &g)) return RQ_ERR_UNSUPPORTED;
    g.bt = bt;
    g.bt_stride = bt_stride;
    g.n_blocks = n_blocks;
    if (!cache || !pending || !pos || !rot) return RQ_ERR_INVALID_ARG;
    if (batch < 1 || batch > g.max_batch || n_tokens < 1) return RQ_ERR_INVALID_ARG;
    if (group_idx < 0 || group_idx >= g.n_groups) return RQ_ERR_INVALID_ARG;
    if ((int64_t)n_tokens * batch * g.hkv * 2 > 0x7FFFFFFFLL) return RQ_ERR_INVALID_ARG;
    if (!aligned16(cache) || !aligned16(rot) || (reinterpret_cast<uintptr_t>(pending) & 1u))
        return RQ_ERR_MISALIGNED;
    PackArgs a;
    memset(&a, 0, sizeof(a));
    a.geo = g;
    a.cache = static_cast<uint8_t*>(cache);
    a.pending = pending;
    if (pending_strides) {
        for (int i = 0; i < 5; ++i) {
            if (pending_strides[i] < 0) return RQ_ERR_INVALID_ARG;
            a.st[i] = pending_strides[i];
        }
    } else {
        a.st[4] = g.d;
        a.st[3] = (int64_t)g.hkv * g.d;
        a.st[2] = 2 * a.st[3];
        a.st[1] = (int64_t)g.L * a.st[2];
        a.st[0] = (int64_t)batch * a.st[1];
    }
    a.pos = pos;
    a.rot = rot;
    a.group_idx = group_idx;
    a.batch = batch;
    a.n_tokens = n_tokens;
    // a few tokens: one per workgroup; groups longer than the per-loop-count instantiations
    // (L > 8, shared anchor) always take the one-loop-per-workgroup kernel below the bulk size
    a.tokens_per_wg = (n_tokens <= 8 || (!g.chained && g.L > 8)) ? 1 : 32;
    a.n_cu = device_cu_count();
    return launch_pack(a, stream) == hipSuccess ? RQ_OK : RQ_ERR_HIP;
}

// table_stride >= tiles of max_ctx, n_blocks >= 1, table 4-byte aligned
static rq_status paging_ok(const rq_config* cfg, int32_t n_blocks, const int32_t* table, int32_t table_stride) {
    Geom g;
    if (cfg == nullptr) return RQ_ERR_INVALID_ARG;
    if (!make_geom(cfg, &g)) return RQ_ERR_UNSUPPORTED;
    if (!table || n_blocks < 1 || table_stride < g.n_tiles) return RQ_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(table) & 3u) return RQ_ERR_MISALIGNED;
    if ((int64_t)g.max_batch * table_stride > 0x7FFFFFFFLL) return RQ_ERR_INVALID_ARG;
    return RQ_OK;
}

rq_status rq_quantize_token(const rq_config* cfg, void* cache, const uint16_t* pending,
                            const int64_t* pending_strides, int32_t group_idx, const int32_t* pos,
                            const float* rot, int32_t batch, int32_t n_tokens, hipStream_t stream) {
    return quantize_impl(cfg, cache, nullptr, 0, 0, pending, pending_strides, group_idx, pos, rot, batch, n_tokens,
                         stream);
}

size_t rq_paged_block_bytes(const rq_config* cfg) {
    Geom g;
    if (!make_geom(cfg, &g)) return 0;
    return (size_t)g.p_block;
}

rq_status rq_quantize_token_paged(const rq_config* cfg, void* pool, int32_t n_blocks, const int32_t* block_table,
                                  int32_t table_stride, const uint16_t* pending, const int64_t* pending_strides,
                                  int32_t group_idx, const int32_t* pos, const float* rot, int32_t batch,
                                  int32_t n_tokens, hipStream_t stream) {
    const rq_status st = paging_ok(cfg, n_blocks, block_table, table_stride);
    if (st != RQ_OK) return st;
    return quantize_impl(cfg, pool, block_table, table_stride, n_blocks, pending, pending_strides, group_idx, pos,
                         rot, batch, n_tokens, stream);
}

// Split records and arrival counters of one decode call: `rec_splits` records per (batch row,
// query head) at `partials`, one counter per pair at `arrivals` (zero between calls); the
// automatic split count is capped at rec_splits.
struct SplitStore {
    float* partials;
    uint32_t* arrivals;
    int rec_splits;
};

// Host checks of every decode argument except the split store.
static rq_status decode_check(const rq_config* cfg, Geom* g, const void* cache, int32_t loop, const void* q,
                              int32_t q_is_bf16, const uint16_t* k_cur, const uint16_t* v_cur,
                              const uint16_t* pending, const int32_t* ctx_len, int32_t ctx_bound,
                              const float* rot, float sm_scale, const float* out, int32_t batch,
                              int32_t n_splits) {
    if (cfg == nullptr) return RQ_ERR_INVALID_ARG;
    if (!make_geom(cfg, g)) return RQ_ERR_UNSUPPORTED;
    if (!cache || !q || !k_cur || !v_cur || !ctx_len || !rot || !out) return RQ_ERR_INVALID_ARG;
    if (batch < 1 || batch > g->max_batch) return RQ_ERR_INVALID_ARG;
    if (loop < 0 || loop >= g->L * g->n_groups) return RQ_ERR_INVALID_ARG;
    if (ctx_bound < 0 || ctx_bound > g->max_ctx) return RQ_ERR_INVALID_ARG;
    if (n_splits < 0 || n_splits > kMaxSplits) return RQ_ERR_INVALID_ARG;
    if (q_is_bf16 != 0 && q_is_bf16 != 1) return RQ_ERR_INVALID_ARG;
    if (!(sm_scale > 0.f) || sm_scale != sm_scale) return RQ_ERR_INVALID_ARG;
    if (!aligned16(cache) || !aligned16(q) || !aligned16(k_cur) || !aligned16(v_cur) || !aligned16(out) ||
        !aligned16(rot) || (pending && !aligned16(pending)))
        return RQ_ERR_MISALIGNED;
    return RQ_OK;
}

static rq_status decode_impl(const rq_config* cfg, const void* cache, const int32_t* bt, int32_t bt_stride,
                             int32_t n_blocks, int32_t loop, const void* q, int32_t q_is_bf16,
                             const uint16_t* k_cur, const uint16_t* v_cur, uint16_t* pending,
                             const int32_t* ctx_len, int32_t ctx_bound, const float* rot, float sm_scale,
                             float* out, const SplitStore& store, int32_t batch, int32_t n_splits,
                             hipStream_t stream) {
    Geom g;
    const rq_status chk = decode_check(cfg, &g, cache, loop, q, q_is_bf16, k_cur, v_cur, pending, ctx_len,
                                       ctx_bound, rot, sm_scale, out, batch, n_splits);
    if (chk != RQ_OK) return chk;
    g.bt = bt;
    g.bt_stride = bt_stride;
    g.n_blocks = n_blocks;
    if (n_splits > store.rec_splits) return RQ_ERR_WORKSPACE;
    const int lloc = loop % g.L;
    const int nres = (lloc == g.L - 1) ? 0 : (g.chained ? g.L - 1 - lloc : 1);
    const int n_tiles = (ctx_bound + kTile - 1) / kTile;
    // the grouped-query kernel runs one workgroup per KV head and split (one per CU)
    const bool grouped = gqa_supported(g, loop, nres);
    const int n_cu = device_cu_count();
    int S = n_splits ? n_splits
                     : (grouped ? auto_splits(batch * g.hkv, n_tiles, n_cu)
                                : auto_splits(batch * g.hq, n_tiles, 2 * n_cu));
    if (n_tiles > 0 && S > n_tiles) S = n_tiles;
    if (S > store.rec_splits) S = store.rec_splits;
    if (S < 1) S = 1;
    DecodeArgs a;
    memset(&a, 0, sizeof(a));
    a.geo = g;
    a.cache = static_cast<const uint8_t*>(cache);
    a.loop = loop;
    a.q = q;
    a.rot = rot;
    a.ctx_len = ctx_len;
    a.ctx_bound = ctx_bound;
    a.sm_scale = sm_scale;
    a.batch = batch;
    a.n_splits = S;
    a.tiles_per_split = n_tiles > 0 ? (n_tiles + S - 1) / S : 0;
    a.n_cu = n_cu;
    MergeArgs& m = a.mg;
    m.partials = store.partials;
    m.arrivals = store.arrivals;
    m.n_splits = S;
    m.rec_splits = store.rec_splits;
    m.hkv = g.hkv;
    m.hq = g.hq;
    m.sm_scale = sm_scale;
    m.k_cur = k_cur;
    m.v_cur = v_cur;
    m.out = out;
    m.pending = pending;
    m.L = g.L;
    m.lloc = lloc;
    m.rot = rot;
    return launch_decode(a, nres, q_is_bf16 != 0, stream) == hipSuccess ? RQ_OK : RQ_ERR_HIP;
}

// The caller's workspace: kMaxSplits records per (row, query head) of the configuration's
// capacity, then the counters.
static rq_status caller_store(const rq_config* cfg, void* workspace, size_t workspace_bytes_, SplitStore* st) {
    Geom g;
    if (cfg == nullptr) return RQ_ERR_INVALID_ARG;
    if (!make_geom(cfg, &g)) return RQ_ERR_UNSUPPORTED;
    if (workspace && !aligned16(workspace)) return RQ_ERR_MISALIGNED;
    if (!workspace || workspace_bytes_ < workspace_bytes(g.max_batch, g.hq, g.d)) return RQ_ERR_WORKSPACE;
    st->partials = static_cast<float*>(workspace);
    st->arrivals = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(workspace) + records_bytes(g.max_batch, g.hq, g.d));
    st->rec_splits = kMaxSplits;
    return RQ_OK;
}

rq_status rq_decode_attention(const rq_config* cfg, const void* cache, int32_t loop, const void* q,
                              int32_t q_is_bf16, const uint16_t* k_cur, const uint16_t* v_cur,
                              uint16_t* pending, const int32_t* ctx_len, int32_t ctx_bound,
                              const float* rot, float sm_scale, float* out, void* workspace,
                              size_t workspace_bytes_, int32_t batch, int32_t n_splits,
                              hipStream_t stream) {
    Geom g;
    const rq_status chk = decode_check(cfg, &g, cache, loop, q, q_is_bf16, k_cur, v_cur, pending, ctx_len,
                                       ctx_bound, rot, sm_scale, out, batch, n_splits);
    if (chk != RQ_OK) return chk;
    SplitStore st;
    const rq_status ws = caller_store(cfg, workspace, workspace_bytes_, &st);
    if (ws != RQ_OK) return ws;
    return decode_impl(cfg, cache, nullptr, 0, 0, loop, q, q_is_bf16, k_cur, v_cur, pending, ctx_len, ctx_bound, rot,
                       sm_scale, out, st, batch, n_splits, stream);
}

rq_status rq_decode_attention_noalloc(const rq_config* cfg, const void* cache, int32_t loop, const void* q,
                                      int32_t q_is_bf16, const uint16_t* k_cur, const uint16_t* v_cur,
                                      uint16_t* pending, const int32_t* ctx_len, int32_t ctx_bound,
                                      const float* rot, float sm_scale, float* out, int32_t batch,
                                      int32_t n_splits, hipStream_t stream) {
    Geom g;
    const rq_status chk = decode_check(cfg, &g, cache, loop, q, q_is_bf16, k_cur, v_cur, pending, ctx_len,
                                       ctx_bound, rot, sm_scale, out, batch, n_splits);
    if (chk != RQ_OK) return chk;
    // records of batch * n_q_heads pairs in the static array: as many splits as fit
    const int64_t pairs = (int64_t)batch * g.hq;
    const int64_t rec = (int64_t)partial_stride(g.d) * sizeof(float);
    const int64_t fit = pairs > kScratchPairs ? 0 : (int64_t)kScratchRecordBytes / (pairs * rec);
    if (fit < 1 || (n_splits > 0 && n_splits > fit)) return RQ_ERR_WORKSPACE;
    uint8_t* base = scratch_base(stream);
    if (base == nullptr) return RQ_ERR_HIP;
    SplitStore st;
    st.arrivals = reinterpret_cast<uint32_t*>(base);
    st.partials = reinterpret_cast<float*>(base + kScratchCounterBytes);
    st.rec_splits = (int)(fit < kMaxSplits ? fit : kMaxSplits);
    return decode_impl(cfg, cache, nullptr, 0, 0, loop, q, q_is_bf16, k_cur, v_cur, pending, ctx_len, ctx_bound, rot,
                       sm_scale, out, st, batch, n_splits, stream);
}

rq_status rq_decode_attention_paged(const rq_config* cfg, const void* pool, int32_t n_blocks,
                                    const int32_t* block_table, int32_t table_stride, int32_t loop, const void* q,
                                    int32_t q_is_bf16, const uint16_t* k_cur, const uint16_t* v_cur,
                                    uint16_t* pending, const int32_t* ctx_len, int32_t ctx_bound,
                                    const float* rot, float sm_scale, float* out, void* workspace,
                                    size_t workspace_bytes_, int32_t batch, int32_t n_splits,
                                    hipStream_t stream) {
    const rq_status st = paging_ok(cfg, n_blocks, block_table, table_stride);
    if (st != RQ_OK) return st;
    Geom g;
    const rq_status chk = decode_check(cfg, &g, pool, loop, q, q_is_bf16, k_cur, v_cur, pending, ctx_len,
                                       ctx_bound, rot, sm_scale, out, batch, n_splits);
    if (chk != RQ_OK) return chk;
    SplitStore ss;
    const rq_status ws = caller_store(cfg, workspace, workspace_bytes_, &ss);
    if (ws != RQ_OK) return ws;
    return decode_impl(cfg, pool, block_table, table_stride, n_blocks, loop, q, q_is_bf16, k_cur, v_cur, pending,
                       ctx_len, ctx_bound, rot, sm_scale, out, ss, batch, n_splits, stream);
}

rq_status rq_bf16_decode_attention(const rq_bf16_config* cfg, uint16_t* k_cache, uint16_t* v_cache,
                                   const void* q, int32_t q_is_bf16, const uint16_t* k_cur,
                                   const uint16_t* v_cur, int32_t append, const int32_t* ctx_len,
                                   int32_t ctx_bound, float sm_scale, float* out, void* workspace,
                                   size_t workspace_bytes_, int32_t batch, int32_t n_splits,
                                   hipStream_t stream) {
    if (cfg == nullptr) return RQ_ERR_INVALID_ARG;
    if (!bf16_cfg_ok(cfg)) return RQ_ERR_UNSUPPORTED;
    const int head_dim = cfg->head_dim, n_q_heads = cfg->n_q_heads;
    if (!k_cache || !v_cache || !q || !k_cur || !v_cur || !ctx_len || !out) return RQ_ERR_INVALID_ARG;
    if (batch < 1 || batch > cfg->max_batch || ctx_bound < 0 || ctx_bound > cfg->t_cap) return RQ_ERR_INVALID_ARG;
    if (n_splits < 0 || n_splits > kMaxSplits) return RQ_ERR_INVALID_ARG;
    if (q_is_bf16 != 0 && q_is_bf16 != 1) return RQ_ERR_INVALID_ARG;
    if (!(sm_scale > 0.f) || sm_scale != sm_scale) return RQ_ERR_INVALID_ARG;
    if (!aligned16(k_cache) || !aligned16(v_cache) || !aligned16(q) || !aligned16(k_cur) ||
        !aligned16(v_cur) || !aligned16(out) || (workspace && !aligned16(workspace)))
        return RQ_ERR_MISALIGNED;
    const size_t need = workspace_bytes(cfg->max_batch, n_q_heads, head_dim);
    if (!workspace || workspace_bytes_ < need) return RQ_ERR_WORKSPACE;
    const int n_tiles = (ctx_bound + kTile - 1) / kTile;
    const int n_cu = device_cu_count();
    // grouped queries: one workgroup of 8 waves per (row, KV head, split), one per CU
    const bool grouped = bf16_gqa_supported(head_dim, n_q_heads, cfg->n_kv_heads);
    int S = n_splits ? n_splits
                     : (grouped ? auto_splits(batch * cfg->n_kv_heads, n_tiles, n_cu)
                                : auto_splits(batch * n_q_heads, n_tiles, 2 * n_cu));
    if (n_tiles > 0 && S > n_tiles) S = n_tiles;
    if (S < 1) S = 1;
    Bf16Args a;
    memset(&a, 0, sizeof(a));
    a.k = k_cache;
    a.v = v_cache;
    a.t_cap = cfg->t_cap;
    a.hkv = cfg->n_kv_heads;
    a.hq = n_q_heads;
    a.q = q;
    a.ctx_len = ctx_len;
    a.ctx_bound = ctx_bound;
    a.sm_scale = sm_scale;
    a.batch = batch;
    a.n_splits = S;
    a.tiles_per_split = n_tiles > 0 ? (n_tiles + S - 1) / S : 0;
    a.n_cu = n_cu;
    MergeArgs& m = a.mg;
    m.partials = static_cast<float*>(workspace);
    m.arrivals = reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(workspace) +
                                             records_bytes(cfg->max_batch, n_q_heads, head_dim));
    m.n_splits = S;
    m.rec_splits = kMaxSplits;
    m.hkv = cfg->n_kv_heads;
    m.hq = n_q_heads;
    m.sm_scale = sm_scale;
    m.k_cur = k_cur;
    m.v_cur = v_cur;
    m.out = out;
    if (append) {
        m.k_app = k_cache;
        m.v_app = v_cache;
        m.t_cap = cfg->t_cap;
        m.ctx_len = ctx_len;
        m.ctx_bound = ctx_bound;
    }
    if (grouped) return launch_bf16_gqa(a, q_is_bf16 != 0, stream) == hipSuccess ? RQ_OK : RQ_ERR_HIP;
    return launch_bf16(a, head_dim, q_is_bf16 != 0, stream) == hipSuccess ? RQ_OK : RQ_ERR_HIP;
}

rq_status rq_kv_project(const rq_config* cfg, const uint16_t* x, int64_t x_stride, int32_t hidden,
                        const uint16_t* w_kv, int32_t loop, uint16_t* k_cur, uint16_t* v_cur, uint16_t* pending,
                        int32_t batch, hipStream_t stream) {
    Geom g;
    if (cfg == nullptr) return RQ_ERR_INVALID_ARG;
    if (!make_geom(cfg, &g)) return RQ_ERR_UNSUPPORTED;
    if (!x || !w_kv || (!k_cur && !v_cur && !pending)) return RQ_ERR_INVALID_ARG;
    if (batch < 1 || batch > g.max_batch || loop < 0 || loop >= g.L * g.n_groups) return RQ_ERR_INVALID_ARG;
    if (hidden < 32 || hidden > 65536 || hidden % 32 != 0 || x_stride < hidden || x_stride > (1LL << 30))
        return RQ_ERR_INVALID_ARG;
    if (batch > 64) return RQ_ERR_UNSUPPORTED;
    if (!aligned16(x) || !aligned16(w_kv) || (x_stride % 8) != 0 || (k_cur && !aligned16(k_cur)) ||
        (v_cur && !aligned16(v_cur)) || (pending && !aligned16(pending)))
        return RQ_ERR_MISALIGNED;
    KvProjArgs a;
    memset(&a, 0, sizeof(a));
    a.x = x;
    a.x_stride = x_stride;
    a.w = w_kv;
    a.hidden = hidden;
    a.batch = batch;
    a.hkv = g.hkv;
    a.d = g.d;
    a.L = g.L;
    a.lloc = loop % g.L;
    a.k_out = k_cur;
    a.v_out = v_cur;
    a.pending = pending;
    return launch_kv_project(a, stream) == hipSuccess ? RQ_OK : RQ_ERR_HIP;
}

}  // extern "C"
