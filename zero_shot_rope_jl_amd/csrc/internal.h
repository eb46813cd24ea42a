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
    // bf16 kernel only: workspace that receives the keys in their corrected
    // view when G > 1, [B, krot_rows, Hkv, D] bf16 by position (krot_rows >=
    // L); rows [rot_lo, L) are rotated by the call, rows below rot_lo are
    // already there (a caller-kept state, chunked calls only)
    void* krot;
    int64_t krot_rows;
    int64_t rot_lo;
    // bf16 kernel only: the key tiles of each query tile are split over
    // n_ksplit workgroups (1: no split), which leave fp32 partials (acc[D],
    // max in log2 units, sum, 2 pad) [n_ksplit, B, Lq, Hq, D + 4] in `part`
    // for the combine kernel (rows 16-byte aligned)
    int n_ksplit;
    float* part;
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
    // bf16 kernel only, whole-sequence calls: non-null makes the grid one
    // workgroup per compute unit, each taking query tiles from kSchedQueues
    // counters (zeroed by a launch before the kernel) until all n_tiles are
    // done; null gives one workgroup per query tile
    uint32_t* sched;
    int64_t n_tiles;
};

// Tile queues of the bf16 prefill's dynamic grid: tile t (in the static
// grid's order, longest first) sits in queue t % kSchedQueues, which is the
// XCD that the static grid's round-robin dispatch gives it; each counter on
// its own 128-byte line.
constexpr int kSchedQueues = 8;
constexpr int kSchedStride = 32;
constexpr size_t kSchedBytes = (size_t)kSchedQueues * kSchedStride * sizeof(uint32_t);

enum PrefillMode {
    kFused = 0,        // q - k <= w0 in the stored view, the rest in the corrected view
    kLocalWindow = 1,  // A: stored view, keys q - w0 <= k <= q
    kRemoteAll = 2,    // B: corrected view, keys k <= q
    kRemoteWindow = 3, // C: corrected view, keys q - w0 <= k <= q
};

struct DecodeParams {
    // Lq query positions per sequence, L - Lq .. L - 1 (1 for a decode step):
    // q and out [B, Lq, Hq, D], lse [B, Hq, Lq]
    const void* q;
    const void* k;
    const void* v;
    void* out;
    float* lse;
    float* ws;          // split partials (acc[D], max, sum) [B, Lq, Hq, n_split, D + 2]
    const TableHeader* table;
    const float2* TF;   // (cos, sin)(n theta_i) rows, n < coverage
    int64_t B, L, Lmax, Hq, Hkv;
    // paged cache (block_table non-NULL): k/v are [n_pages, page_size, Hkv, D]
    // and key p of sequence b is row p % page_size of page
    // block_table[b * max_pages + p / page_size]; page_size is a multiple of 32
    const int32_t* block_table;
    int64_t page_size, max_pages, n_pages;
    int R;
    int Lq;             // query positions (R * Lq <= 16 * n_grp)
    int n_grp;          // 16-column groups of (position, query head) per KV head: 1, 2 or 4
    int n_split;        // workgroups per (batch, KV-head group)
    int wave_chunk;     // consecutive keys per wave (multiple of 32); with 2 or 4
                        // column groups, per workgroup (multiple of 64)
    int wave_extra;     // split kernel: waves 0 .. wave_extra-1 of a head take 32 keys more
    int wave_split_fastest;   // split kernel: a head's waves numbered split-fastest (1) or
                              // sub-range-fastest (0) along its keys
    int heads_per_wg;   // KV heads per workgroup of the split kernel (waves per head = 8 / heads_per_wg)
    int64_t w0;
    int64_t G;
    // keys k_lo .. L-1 are read; those >= kloc score in the stored view, the
    // rest in the corrected view.  The fused step reads every key with
    // kloc = L-1-w0 (0 when G = 1); the passes of the unfused step restrict
    // the keys to the window and put kloc at its start (pass A) or at L
    // (passes B and C: every key corrected).
    int64_t k_lo;
    int64_t kloc;
    float sm_scale_log2;
    double rope_base;
    int head_dim;
    // [B, krot_rows, Hkv, D] bf16 by position holding every remote key
    // (rows below the first query's window) already in its corrected view
    // under this G, or null
    const void* krot;
    int64_t krot_rows;
    // with krot (contiguous caches, Lq = 1): the row to write into krot,
    // rotated under this G, for the next step (the first local row, which the
    // next step reads as remote when G stays); -1 for none
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

inline size_t decode_align(size_t x) { return (x + 255u) & ~(size_t)255u; }

// Bytes of split partials for steps of up to L keys.
inline size_t decode_partial_bytes(int64_t B, int64_t Hq, int64_t D, int64_t L) {
    return (size_t)B * (size_t)Hq * (size_t)decode_max_splits(L) * (size_t)(D + 2) * sizeof(float);
}

inline int decode_heads_per_wg(int64_t Hkv) {
    return Hkv >= kDecodeMaxHeadsPerWG ? kDecodeMaxHeadsPerWG : (int)Hkv;
}

// Column groups for Lq query positions of R heads each: 16 columns per
// group, rounded up to 1, 2 or 4 groups; 0 when they need more than 4.
inline int decode_groups(int64_t Lq, int64_t R) {
    const int64_t cols = Lq * R;
    return cols <= 16 ? 1 : cols <= 32 ? 2 : cols <= 64 ? 4 : 0;
}

// Split plan of the kernel for 2 or 4 column groups: one KV head per
// workgroup, about 256 workgroups, key ranges in whole 64-key stages (its
// step).  The split count is at most ceil(256 / (B * Hkv)) and ceil(L / 64);
// the stages are dealt as in the split plan below: each workgroup takes
// floor(stages / n) of them and the first stages % n one more.
constexpr int kMultiStageKeys = 64;
inline void decode_multi_plan(int64_t B, int64_t Hkv, int64_t L, int* n_split, int* keys_per_wg, int* wg_extra) {
    const int64_t groups = B * Hkv;
    int64_t n = groups >= kDecodeTargetWGs ? 1 : (kDecodeTargetWGs + groups - 1) / groups;
    const int64_t steps = (L + kMultiStageKeys - 1) / kMultiStageKeys;
    if (n > steps) n = steps;
    *n_split = (int)n;
    *keys_per_wg = (int)(steps / n * kMultiStageKeys);
    *wg_extra = (int)(steps % n);
}

inline void decode_split_plan(int64_t B, int64_t Hkv, int64_t L, int* n_split, int* wave_chunk, int* wave_extra,
                              int* wave_split_fastest) {
    const int64_t WH = decode_heads_per_wg(Hkv);
    const int64_t NW = kDecodeWaves / WH;
    const int64_t groups = B * (Hkv / WH);
    const int64_t n_target = groups >= kDecodeTargetWGs ? 1 : kDecodeTargetWGs / groups;
    const int64_t steps = (L + 31) / 32;
    if (WH == 1) {
        // One KV head per workgroup (256-byte rows at D = 128): every plan
        // streams about the same rate, and the fastest measured rounds each
        // wave's share up to whole steps, a workgroup's waves taking
        // consecutive ranges.
        int64_t per_wave = (L + n_target * NW - 1) / (n_target * NW);
        per_wave = (per_wave + 31) / 32 * 32;
        *n_split = (int)((L + per_wave * NW - 1) / (per_wave * NW));
        *wave_chunk = (int)per_wave;
        *wave_extra = 0;
        *wave_split_fastest = 0;
        return;
    }
    // The ceil(L/32) steps of 32 keys of each KV head are dealt over its
    // waves: every wave takes floor(steps / waves) consecutive steps and the
    // first steps % waves waves one more, so that every workgroup of the
    // target grid gets keys (rounding each wave's share up to whole steps
    // instead would leave some of them idle).  The waves are numbered
    // split-fastest, so those extra steps fall on different workgroups.
    const int64_t waves = n_target * NW < steps ? n_target * NW : steps;
    *n_split = (int)((waves + NW - 1) / NW);
    const int64_t all = (int64_t)*n_split * NW;
    *wave_chunk = (int)(steps / all * 32);
    *wave_extra = (int)(steps % all);
    *wave_split_fastest = 1;
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

// Most key splits of one query tile in a chunked prefill.
constexpr int kMaxKSplit = 64;

hipError_t launch_prefill(const PrefillParams& p, int in_dtype, int out_dtype, hipStream_t stream);
hipError_t launch_ie_merge(const MergeParams& p, int out_dtype, hipStream_t stream);
hipError_t launch_prefill_bf16(const PrefillParams& p, int out_dtype, hipStream_t stream);
// bf16 caches with G > 1: rows [rot_lo, L) of p's keys into their corrected
// view in p.krot (nothing to do otherwise)
hipError_t launch_rotate_keys(const PrefillParams& p, hipStream_t stream);
hipError_t launch_decode(const DecodeParams& p, int out_dtype, hipStream_t stream);

// The fixed device scratch of jl_bifocal_decode_noalloc: its size, and its
// address on the current device (looked up once per device).
constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
hipError_t noalloc_scratch(void** ptr);

}  // namespace jl
