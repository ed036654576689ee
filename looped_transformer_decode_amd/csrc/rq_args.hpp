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
    float* partials;
    int batch;
    int n_splits;
    int tiles_per_split;
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
    float* partials;
    int batch;
    int n_splits;
    int tiles_per_split;
};

// Merge of the split-K partial records of one loop-step, plus the current token.
struct CombineArgs {
    const float* partials;      // [batch * hq][kMaxSplits][d + 4]
    int n_splits;
    const void* q;
    const uint16_t* k_cur;      // [batch][hkv][d]
    const uint16_t* v_cur;
    int hkv, hq;
    float sm_scale;
    float* out;                 // [batch][hq][d]
    uint16_t* pending;          // ResidualQuant: [batch][L][2][hkv][d] or null
    int L, lloc;
    const float* rot_v;         // ResidualQuant residual loops: R_V of KV head h at rot_v + h*2*d*d, else null
    uint16_t* k_app;            // BF16 baseline append target [batch][hkv][t_cap][d] or null
    uint16_t* v_app;
    int t_cap;
    const int32_t* ctx_len;
    int ctx_bound;
};

hipError_t launch_pack(const PackArgs& a, hipStream_t stream);
hipError_t launch_combine(const CombineArgs& a, int d, bool qbf16, int batch, hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, int nres, bool qbf16, hipStream_t st);
hipError_t launch_bf16(const Bf16Args& a, int d, bool qbf16, hipStream_t st);

}  // namespace rq
