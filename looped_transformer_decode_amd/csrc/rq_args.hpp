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
};

struct DecodeArgs {
    Geom geo;
    const uint8_t* cache;
    int loop;
    const void* q;
    const uint16_t* k_cur;
    const uint16_t* v_cur;
    uint16_t* pending;
    const int32_t* ctx_len;
    int ctx_bound;
    const float* rot;
    float sm_scale;
    float* out;
    float* partials;
    uint32_t* counters;
    int batch;
    int n_splits;
    int tiles_per_split;
};

struct Bf16Args {
    uint16_t* k;
    uint16_t* v;
    int t_cap, hkv, hq;
    const void* q;
    const uint16_t* k_cur;
    const uint16_t* v_cur;
    int append;
    const int32_t* ctx_len;
    int ctx_bound;
    float sm_scale;
    float* out;
    float* partials;
    uint32_t* counters;
    int batch;
    int n_splits;
    int tiles_per_split;
};

hipError_t launch_pack(const PackArgs& a, hipStream_t stream);
hipError_t launch_decode(const DecodeArgs& a, int nres, bool qbf16, hipStream_t st);
hipError_t launch_bf16(const Bf16Args& a, int d, bool qbf16, hipStream_t st);

}  // namespace rq
