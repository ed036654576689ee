// Kernel argument blocks (passed by value to the kernels).
#pragma once

#include "rq_common.hpp"

namespace rq {

struct PackArgs {
    Geom geo;
    uint8_t* cache;
    const uint16_t* pending;
    int64_t st[5];
    const int32_t* pos;
    const float* rot;
    int group_idx;
    int batch;
    int n_tokens;
    int tokens_per_wg;          // tokens handled by one workgroup (it keeps its row of R)
    int n_cu;                   // compute units of the device (choice of the drain kernel)
};

// The split-K merge that the last workgroup of each (batch row, query head) performs.
struct MergeArgs {
    float* partials;            // [batch * hq][rec_splits] records of partial_stride(d) floats
    uint32_t* arrivals;         // [batch * hq] arrival counters; zero between calls
    int n_splits;
    int rec_splits;             // records per (batch row, query head) in `partials` (>= n_splits)
    int hkv, hq;
    float sm_scale;
    const uint16_t* k_cur;      // [batch][hkv][d] BF16 current token of this loop
    const uint16_t* v_cur;
    float* out;                 // [batch][hq][d]
    uint16_t* pending;          // ResidualQuant: [batch][L][2][hkv][d] or null
    int L, lloc;
    const float* rot;           // ResidualQuant residual loops: R of (KV head h, V) at rot + (2h+1)*d*d
    uint16_t* k_app;            // BF16 baseline append target [batch][hkv][t_cap][d] or null
    uint16_t* v_app;
    int t_cap;
    const int32_t* ctx_len;
    int ctx_bound;
};

struct DecodeArgs {
    Geom geo;
    const uint8_t* cache;
    int loop;
    const void* q;              // [batch][hq][d], float32 or BF16
    const float* rot;           // [hkv][2][d][d]
    const int32_t* ctx_len;
    int ctx_bound;
    float sm_scale;
    int batch;
    int n_splits;
    int tiles_per_split;
    int n_cu;                   // compute units of the device (workgroup pairing on a CU)
    MergeArgs mg;
};

// BF16 baseline split kernel: K and V caches [batch][hkv][t_cap][d].
struct Bf16Args {
    const uint16_t* k;
    const uint16_t* v;
    int t_cap, hkv, hq;
    const void* q;
    const int32_t* ctx_len;
    int ctx_bound;
    float sm_scale;
    int batch;
    int n_splits;
    int tiles_per_split;
    int n_cu;
    MergeArgs mg;
};

// K/V projection of the current token: x [batch][hidden] (row stride x_stride elements),
// w [2][hkv][d][hidden]; outputs BF16 k_out/v_out [batch][hkv][d] and the pending slot
// [batch][L][2][hkv][d] at loop lloc (each output may be null, not all three).
struct KvProjArgs {
    const uint16_t* x;
    int64_t x_stride;
    const uint16_t* w;
    int hidden, batch, hkv, d, L, lloc;
    uint16_t* k_out;
    uint16_t* v_out;
    uint16_t* pending;
};

hipError_t launch_pack(const PackArgs& a, hipStream_t stream);
hipError_t launch_kv_project(const KvProjArgs& a, hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, int nres, bool qbf16, hipStream_t st);
// grouped-query kernel (several query heads per KV head read each tile once)
bool gqa_supported(const Geom& g, int loop, int nres);
hipError_t launch_decode_gqa(const DecodeArgs& a, int nres, bool qbf16, hipStream_t st);
hipError_t launch_bf16(const Bf16Args& a, int d, bool qbf16, hipStream_t st);
// grouped-query BF16 kernel (the G query heads of a KV head read each tile once)
bool bf16_gqa_supported(int d, int hq, int hkv);
hipError_t launch_bf16_gqa(const Bf16Args& a, bool qbf16, hipStream_t st);

}  // namespace rq
