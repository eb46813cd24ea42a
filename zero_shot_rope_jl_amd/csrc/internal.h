// Host-side launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace jl {

struct PrefillParams {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* lse;
    const TableHeader* table;
    const float2* TF;   // (cos, sin)(n theta_i) rows, n < coverage
    int64_t B, L, Hq, Hkv;
    int R;              // Hq / Hkv
    int BQ;             // query positions per workgroup (256 / R)
    int n_qtiles;
    int64_t w0;
    int64_t G;
    float sm_scale_log2;  // sm_scale * log2(e)
    double rope_base;
    int head_dim;
};

struct DecodeParams {
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* lse;
    float* ws;
    const TableHeader* table;
    const float2* TF;   // (cos, sin)(n theta_i) rows, n < coverage
    int64_t B, L, Lmax, Hq, Hkv;
    int R;
    int n_split;        // workgroups per (batch, KV head)
    int wave_chunk;     // consecutive keys per wave (multiple of 32)
    int64_t w0;
    int64_t G;
    float sm_scale_log2;
    double rope_base;
    int head_dim;
};

// Decode split plan: at most kDecodeMaxSplits workgroups of 4 waves per
// (batch, KV head); each wave streams one contiguous range of keys.
constexpr int kDecodeMaxSplits = 64;
constexpr int kDecodeWaves = 4;

inline int64_t decode_max_splits(int64_t L) {
    const int64_t n = (L + 255) / 256;
    return n < kDecodeMaxSplits ? n : kDecodeMaxSplits;
}

inline void decode_split_plan(int64_t L, int* n_split, int* wave_chunk) {
    const int64_t nmax = decode_max_splits(L);
    int64_t per_wave = (L + nmax * kDecodeWaves - 1) / (nmax * kDecodeWaves);
    per_wave = (per_wave + 31) / 32 * 32;
    const int64_t chunk = per_wave * kDecodeWaves;
    *n_split = (int)((L + chunk - 1) / chunk);
    *wave_chunk = (int)per_wave;
}

hipError_t launch_table_fill(void* table, int64_t n_cover, int head_dim, double rope_base,
                             hipStream_t stream);
void table_fill_host(void* table, int64_t n_cover, int head_dim, double rope_base);

hipError_t launch_prefill(const PrefillParams& p, int in_dtype, int out_dtype, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int out_dtype, hipStream_t stream);

}  // namespace jl
