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
    int64_t B, L, Hq, Hkv;   // L: keys (positions 0..L-1); G comes from L
    int64_t Lq;              // query rows, at positions q_off .. q_off + Lq - 1 = L - 1
    int64_t q_off;
    int64_t Lkv;             // rows per batch entry of k and v (>= L)
    int R;              // Hq / Hkv
    int BQ;             // query positions per workgroup (256 / R)
    int n_qtiles;
    int64_t w0;
    int64_t G;
    float sm_scale_log2;  // sm_scale * log2(e)
    double rope_base;
    int head_dim;
    // 0: compute every row.  1: recompute only the workgroups whose rows carry
    // the non-finite-row mark left by the bf16 kernel (NaN in element 0).
    int fixup;
    // bf16 kernel only: B*L*Hkv*D bf16 workspace that receives the keys in
    // their corrected view when G > 1 (laid out like k)
    void* krot;
    // which pairs and which view (Jet-Long §3.3 Eq. 6): kFused is the bifocal
    // rule in one softmax; the other three are the separate passes of the
    // inclusion-exclusion merge, each one plain masked attention in one view
    int mode;
    // bf16 kernel only: krot already holds this call's rotated keys
    int krot_ready;
    // paged caches (null block_table: k/v are [B, Lkv, Hkv, D]): key k of
    // sequence b is row k % page_size of page block_table[b * max_pages +
    // k / page_size] of k/v, which hold n_pages pages of page_size rows
    const int32_t* block_table;
    int64_t page_size, max_pages, n_pages;
    // the table the kernels expect: an offset table, or for the
    // frequency-interpolation view a position-indexed table for this call
    // (then G is set to max(2, L) when L > w_pretrained, so that the row of
    // position p, p - floor(p/G), is p itself)
    TableKey table_key;
};

enum PrefillMode {
    kFused = 0,        // q - k <= w0 in the stored view, the rest in the corrected view
    kLocalWindow = 1,  // A: stored view, keys q - w0 <= k <= q
    kRemoteAll = 2,    // B: corrected view, keys k <= q
    kRemoteWindow = 3, // C: corrected view, keys q - w0 <= k <= q
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
    // paged cache (block_table non-NULL): k/v are [n_pages, page_size, Hkv, D]
    // and key p of sequence b is row p % page_size of page
    // block_table[b * max_pages + p / page_size]; page_size is a multiple of 32
    const int32_t* block_table;
    int64_t page_size, max_pages, n_pages;
    int R;
    int n_split;        // workgroups per (batch, KV-head group)
    int wave_chunk;     // consecutive keys per wave (multiple of 32)
    int heads_per_wg;   // KV heads per workgroup (waves per head = 8 / heads_per_wg)
    int64_t w0;
    int64_t G;
    float sm_scale_log2;
    double rope_base;
    int head_dim;
    // contiguous caches only: [B, Lmax, Hkv, D] bf16 holding every remote
    // key (rows < L-1-w0) already in its corrected view under this G, or null
    const void* krot;
    // with krot: the row to write into krot, rotated under this G, for the
    // next step (the first local row, which the next step reads as remote
    // when G stays); -1 for none
    int64_t rot_row;
    TableKey table_key;
    // frequency-interpolation remote view: no table; the kernel forms the
    // rows it reads, (cos, sin)(n * fi_phi[i]) at positions n, from the
    // per-pair phi_i below (G = max(2, L) as for prefill); 0 otherwise
    int fi;
    double fi_phi[64];
};

// Rows [r0, r1) of a [B, Lmax, Hkv, D] bf16 key cache rotated into their
// corrected view under p.G (the rotated-key cache of jl_bifocal_decode_rkc),
// with p's table, which is checked against p's key (NaN rows if it does not
// match).
hipError_t launch_rotate_rows(const void* k, void* krot, const DecodeParams& p, int64_t r0, int64_t r1,
                              hipStream_t stream);

// Decode split plan.  A workgroup has 8 waves that cover up to 4 KV heads
// (wave w -> head w % WH, key sub-range w / WH) over one key range, so each
// key row is read in runs of WH heads (1 KB at D = 128); the grid holds about
// one workgroup per compute unit.  Four heads per workgroup (two waves per
// head, merged in LDS) measured faster than eight (whole rows) for the
// contiguous cache and clearly faster for the paged one; one or two heads
// (256-512 B runs) measured slower.
constexpr int kDecodeWaves = 8;
constexpr int kDecodeMaxHeadsPerWG = 4;
constexpr int kDecodeTargetWGs = 256;
constexpr int kDecodeMaxSplits = 256;

inline int64_t decode_max_splits(int64_t L) {
    const int64_t n = (L + 31) / 32;
    return n < kDecodeMaxSplits ? n : kDecodeMaxSplits;
}

inline int decode_heads_per_wg(int64_t Hkv) {
    return Hkv >= kDecodeMaxHeadsPerWG ? kDecodeMaxHeadsPerWG : (int)Hkv;
}

inline void decode_split_plan(int64_t B, int64_t Hkv, int64_t L, int* n_split, int* wave_chunk) {
    const int64_t WH = decode_heads_per_wg(Hkv);
    const int64_t NW = kDecodeWaves / WH;
    const int64_t groups = B * (Hkv / WH);
    const int64_t n_target = groups >= kDecodeTargetWGs ? 1 : kDecodeTargetWGs / groups;
    int64_t per_wave = (L + n_target * NW - 1) / (n_target * NW);
    per_wave = (per_wave + 31) / 32 * 32;
    const int64_t chunk = per_wave * NW;
    *n_split = (int)((L + chunk - 1) / chunk);
    *wave_chunk = (int)per_wave;
}

hipError_t launch_table_fill(void* table, int64_t n_cover, int head_dim, double rope_base,
                             hipStream_t stream);
void table_fill_host(void* table, int64_t n_cover, int head_dim, double rope_base);
// Channel reorder (interleaved RoPE pairs -> rotate-half pairs) of n_rows
// rows of D channels, elements of elem_bytes (2: bf16, 4: fp32).
hipError_t launch_interleaved_to_half(const void* x, void* out, int elem_bytes, int64_t n_rows, int D,
                                      hipStream_t stream);
hipError_t launch_table_fill_fi(void* table, int64_t L, int head_dim, double rope_base, int64_t w_pretrained,
                                double alpha, double beta, hipStream_t stream);
void table_fill_fi_host(void* table, int64_t L, int head_dim, double rope_base, int64_t w_pretrained, double alpha,
                        double beta);

// The three pass outputs of the unfused prefill and where their merge goes.
struct MergeParams {
    const float* o_a;     // [B, Lq, Hq, D] normalised pass outputs
    const float* o_b;
    const float* o_c;
    const float* lse_a;   // [B, Hq, Lq] natural-log sums of the passes
    const float* lse_b;
    const float* lse_c;
    void* out;            // [B, Lq, Hq, D], bf16 or fp32
    float* lse;           // [B, Hq, Lq] or null
    int64_t B, Lq, Hq, D;
};

hipError_t launch_prefill(const PrefillParams& p, int in_dtype, int out_dtype, hipStream_t stream);
hipError_t launch_ie_merge(const MergeParams& p, int out_dtype, hipStream_t stream);
hipError_t launch_prefill_bf16(const PrefillParams& p, int out_dtype, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int out_dtype, hipStream_t stream);

}  // namespace jl
