// Split-KV bifocal-attention decode for gfx950 (one new token per sequence).
//
// Method (Jet-Long §3.2): at each step the group size G is recomputed from
// the current length L and the cached keys, stored as RoPE(x_k, k), are read
// under that G by rotating them on the fly by f(k) - k (Eq. 5); the cache is
// never rewritten.  The query sits at position L-1; keys with
// (L-1) - k <= w0 use the stored vectors, the rest the corrected views (Eq. 1).
//
// Split kernel: workgroup = (key range, KV-head group, batch), 8 waves; wave w
// handles KV head w % WH over sub-range w / WH of the workgroup's keys, so the
// waves of a workgroup read whole key rows (all heads are contiguous in the
// cache) and the grid holds about one workgroup per compute unit.  A wave
// streams its keys 32 per step through two K register tiles and two LDS V
// slots: step i + 2's loads go out as step i's tile and slot are consumed
// (non-temporal loads).  K goes straight from HBM into MFMA A-operand
// registers (rows = keys); V is copied HBM -> the wave's LDS by buffer loads
// into LDS and read back transposed (ds_read_b64_tr_b16) as the A operand of
// O^T += V^T P^T.  The R query heads of the KV head are the MFMA
// N columns (16x16x32 bf16), so each K/V byte is read once per step for all R
// heads.
//
// Correction without per-key table traffic: for the 32 keys starting at
// kbase, n(k) = k - floor(k/G) = nb + dn with nb = n(kbase) and 0 <= dn < 32,
// and R(-n) = R(-nb) R(-dn).  Because R(a)x . y = x . R(-a)y, the remote score
//     R(-n_q) q . R(-n_k) k  =  [R(nb) R(-n_q) q] . [R(-dn) k],
// so the query absorbs the per-iteration base rotation (64 angles, one per
// lane, one table row) and each key is rotated only by dn, whose cos/sin rows
// 0..32 sit in LDS.
//
// Each workgroup leaves one fp32 partial (acc[D], m, l) per query head; the
// combine kernel merges a head's partials with the log-sum-exp rule (§3.3
// Eq. 6 with disjoint key sets).
//
// Several query positions (a short chunk of a chunked prefill, §3.2): the
// Lq positions L-Lq .. L-1 of the R heads give Lq * R <= 16 MFMA columns.
// A column keeps its own causal limit and window edge; the correction
// offsets are shared, since G comes from L for every position of the call.
// (More columns go to decode_multi_kernel below.)
//
// Pass modes (the unfused step): the same kernels read only the window's
// keys in the stored view (pass A), every key in the corrected view (B), or
// the window's keys in the corrected view (C); the merge kernel of the
// unfused prefill then applies Eq. 6 to the three results.
//
// Variants of the split kernel (template flags): PAGED reads the cache
// through a block table; RKC reads remote keys already rotated from a
// second cache (and writes ahead the row the next step needs); FI uses the
// frequency-interpolation remote view of the §4.7 ablation, whose table
// rows (cos, sin)(n * phi_i) the kernel forms itself.
#include <math.h>

#include <mutex>
#include <type_traits>

#include "internal.h"

namespace jl {

namespace {

constexpr int kDecThreads = kDecodeWaves * 64;
constexpr int kWaveKeys = 32;
constexpr int JROWS = kWaveKeys + 1;  // cos/sin(dn * theta) for dn = 0..32

// LDS ordering between lanes of one wave (write -> read, read -> write):
// wait for this wave's LDS operations and stop the compiler moving memory
// accesses across this point.
__device__ inline void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int D>
struct DecodeTile {
    static constexpr int NC = D / 32;    // 32-dim K chunks of the QK^T MFMA
    bf16x8 k[2][NC];                     // rows of the two 16-key blocks
};

// Cache reads are non-temporal: every byte is read once per step, and the
// streaming hint gave ~13% more read bandwidth for this access shape than
// ordinary loads.

// `rbase` is the cache row of key kbase; the 32 keys of a step occupy the
// consecutive rows from there (a page holds a multiple of 32 keys).
template <int D>
__device__ inline void load_k_blk(DecodeTile<D>& t, const __bf16* __restrict__ kc, int64_t cache_b, int64_t row,
                                  int kbase, int64_t rbase, int kend, int colh, int gq, int blk) {
    constexpr int NC = DecodeTile<D>::NC;
    // A-operand row colh of block blk holds key 8*(colh/4) + 4*blk + colh%4:
    // C rows then give P^T slots in natural key order
    const int dk = 8 * (colh >> 2) + 4 * blk + (colh & 3);
    const bool ok = kbase + dk < kend;
#pragma unroll
    for (int c = 0; c < NC; ++c)
        t.k[blk][c] = ok ? __builtin_nontemporal_load(
                               reinterpret_cast<const bf16x8*>(kc + cache_b + (rbase + dk) * row + 32 * c + 8 * gq))
                         : bf16x8{};
}

template <int D>
__device__ inline void load_k(DecodeTile<D>& t, const __bf16* __restrict__ kc, int64_t cache_b, int64_t row,
                              int kbase, int64_t rbase, int kend, int colh, int gq) {
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) load_k_blk<D>(t, kc, cache_b, row, kbase, rbase, kend, colh, gq, blk);
}

// (cos, sin)(n * phi) of the frequency-interpolation view, formed in the
// kernel: the angle is reduced to [-pi, pi] in float64 (n * phi reaches
// ~1e5 rad), then sin and cos are taken in fp32 (error ~2e-7 rad).
__device__ inline float2 fi_cs(double phi, int64_t n) {
    constexpr double kInvTwoPi = 0.15915494309189533577;
    constexpr double kTwoPi = 6.283185307179586476925;
    const double turns = (double)n * phi * kInvTwoPi;
    const float a = (float)((turns - rint(turns)) * kTwoPi);
    float sn, cs;
    sincosf(a, &sn, &cs);
    return make_float2(cs, sn);
}

// physical 16-byte chunk of logical chunk c in row `row` of a V slot
template <int D>
__device__ inline int dec_vswz(int row, int c) { return c ^ ((4 * (row & 3)) & (D / 8 - 1)); }
// cache policy of the V copies: non-temporal (streaming)
constexpr int kNtAux = 2;

template <int D, bool OUT_BF16, bool PAGED, bool RKC, bool FI, bool MQ = false>
__global__ __launch_bounds__(kDecThreads, 2) void decode_split_kernel(DecodeParams p) {
    constexpr int HALF = D / 2;
    constexpr int NC = D / 32;
    constexpr int NDB = D / 16;       // 16-dim blocks of O^T

    __shared__ __attribute__((aligned(16))) __bf16 sV0[kDecodeWaves][kWaveKeys * D];
    __shared__ __attribute__((aligned(16))) __bf16 sV1[kDecodeWaves][kWaveKeys * D];
    constexpr int JSTR = HALF + 2;    // padded row: rows start on different LDS banks
    __shared__ __attribute__((aligned(16))) float2 sJ[JROWS * JSTR];
    __shared__ __attribute__((aligned(16))) float2 sBase[kDecodeWaves][HALF];
    __shared__ float s_m[kDecodeWaves][16];
    __shared__ float s_l[kDecodeWaves][16];
    __shared__ int s_bad;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: key ranges and pages in SGPRs
    const int colh = lane & 15;   // MFMA column = query head within the group
    const int gq = lane >> 4;     // lane quad

    const int split = blockIdx.x;
    const int WH = p.heads_per_wg;
    const int NW = kDecodeWaves / WH;   // waves per head
    const int hw = wave % WH;
    const int sub = wave / WH;
    const int g = blockIdx.y * WH + hw;
    const int b = blockIdx.z;
    const int L = (int)p.L;
    const int Hq = (int)p.Hq;
    const int R = p.R;
    const int G = (int)p.G;
    const int Lq = MQ ? p.Lq : 1;   // MQ: several query positions (a short chunk)
    // this lane's column: query head rq at position L - Lq + jq (columns past
    // the last position compute on a zero query and are not written)
    const bool hvalid = colh < Lq * R;
    const int jq = MQ ? (hvalid ? colh / R : Lq - 1) : 0;
    const int rq = hvalid ? (MQ ? colh % R : colh) : 0;
    const int qpos = L - Lq + jq;
    // keys >= kloc score in the stored view: p.kloc is the last position's
    // edge (q - k <= w0 in the fused step, 0 when G == 1 makes every key
    // local), an earlier position's edge lies as many keys lower; kloc_lo
    // and kloc_hi bound the columns' edges
    const int kloc = p.kloc > 0 ? (int)p.kloc - (Lq - 1 - jq) : (int)p.kloc;
    const int kloc_lo = p.kloc > 0 ? (int)p.kloc - (Lq - 1) : (int)p.kloc;
    const int kloc_hi = (int)p.kloc;
    const float scale2 = p.sm_scale_log2;
    const __bf16* __restrict__ kc = static_cast<const __bf16*>(p.k);
    // rotated keys (RKC): remote keys are read in their corrected view,
    // [B, krot_rows, Hkv, D] by position, instead of being rotated here; a
    // step is read from there when its keys are remote for every column
    const __bf16* __restrict__ krc = static_cast<const __bf16*>(p.krot);
    auto rkc_step = [&](int kb) { return RKC && kb + kWaveKeys <= kloc_lo; };
    const __bf16* __restrict__ vc = static_cast<const __bf16*>(p.v);
    const float2* __restrict__ TF = p.TF;
    // row n, pair i of the correction table (formed here for the
    // frequency-interpolation view, which has no table)
    auto tf = [&](int64_t n, int i) -> float2 {
        if constexpr (FI) return fi_cs(p.fi_phi[i], n);
        else return table_cs(TF, HALF, n, i);
    };
    const int64_t row = p.Hkv * D;
    const int64_t cache_b = PAGED ? (int64_t)g * D : (int64_t)b * p.Lmax * row + (int64_t)g * D;
    const int64_t krot_b = (int64_t)b * p.krot_rows * row + (int64_t)g * D;

    // Cache row of key kb (a multiple of 32), in two parts so that the
    // block-table read can be issued well before its value is needed:
    // page_of reads the entry, row_in turns it into a row.  An entry outside
    // [0, n_pages) reads page 0 instead and marks the result, so no load
    // leaves the pages.  Contiguous caches: the row is kb.
    // The table is read through the constant address space (it is not
    // written during the kernel) so that its reads are scalar loads, whose
    // wait does not drain the cache loads in flight.
    bool bad_page = false;
    const int ps = PAGED ? (int)p.page_size : 1;
    const __attribute__((address_space(4))) int32_t* btab =
        (const __attribute__((address_space(4))) int32_t*)(p.block_table + (int64_t)b * p.max_pages);
    auto page_of = [&](int kb) -> int {
        if constexpr (!PAGED) return 0;
        else return btab[kb / ps];
    };
    auto row_in = [&](int pg, int kb) -> int64_t {
        if constexpr (!PAGED) {
            return kb;
        } else {
            if (pg < 0 || pg >= p.n_pages) {
                bad_page = true;
                pg = 0;
            }
            return (int64_t)pg * ps + kb % ps;
        }
    };
    auto row_of = [&](int kb) -> int64_t { return row_in(page_of(kb), kb); };

    // the first two steps' K and V go out before anything else (the set-up
    // below waits on the table and q); they stay within the cache whatever
    // the table check decides.  K goes HBM -> registers (two tiles, step i
    // computes from tile i & 1); V goes HBM -> this wave's LDS slot i & 1 by
    // buffer loads into LDS (no registers), 16-byte chunks XOR-swizzled by
    // row for the transposing reads of the PV product.
    // this wave's share of its head's steps, numbered split-fastest: the
    // waves that take one step more (the first wave_extra) are the first
    // waves of as many workgroups, so no compute unit holds more than one
    // such wave per head, and the heads of a workgroup read the same rows
    // (with one KV head per workgroup the plan numbers them sub-range-
    // fastest instead, with no extra steps)
    const int wj = p.wave_split_fastest ? sub * p.n_split + split : split * NW + sub;
    const int wstart = (int)p.k_lo + wj * p.wave_chunk + 32 * min(wj, p.wave_extra);
    const int wend0 = min(L, wstart + p.wave_chunk + (wj < p.wave_extra ? 32 : 0));
    constexpr int VCH = D / 8;                  // 16-byte chunks per V row
    constexpr int VRU = 64 / VCH;               // V rows per copy
    constexpr int VCOPIES = kWaveKeys / VRU;    // copies per step
    const uint32_t row_bytes = (uint32_t)(row * 2);
    const uint32_t v_voff =
        (uint32_t)(lane / VCH) * row_bytes + 16u * (uint32_t)dec_vswz<D>(lane / VCH, lane % VCH);
    auto stage_v = [&](int kb, int64_t rb, int kend, auto slot) __attribute__((always_inline)) {
        __bf16* dst = decltype(slot)::value ? sV1[wave] : sV0[wave];
        const int nrows = min(kend - kb, kWaveKeys);   // rows past the end read as zeros
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vc + cache_b + rb * row, (uint32_t)nrows * row_bytes);
#pragma unroll
        for (int u = 0; u < VCOPIES; ++u)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (__attribute__((address_space(3))) void*)(dst + u * 512), 16,
                                                     v_voff, (uint32_t)(u * VRU) * row_bytes, 0, kNtAux);
    };
    using Slot0 = std::integral_constant<int, 0>;
    using Slot1 = std::integral_constant<int, 1>;
    DecodeTile<D> t0, t1;
    int pg2 = 0;   // block-table entry of the step two ahead of the current one
    if (wstart < wend0) {
        const int64_t r0 = row_of(wstart);
        if (rkc_step(wstart)) load_k<D>(t0, krc, krot_b, row, wstart, wstart, wend0, colh, gq);
        else load_k<D>(t0, kc, cache_b, row, wstart, r0, wend0, colh, gq);
        stage_v(wstart, r0, wend0, Slot0{});
        const int k1 = wstart + kWaveKeys;
        if (k1 < wend0) {
            const int64_t r1 = row_of(k1);
            if (rkc_step(k1)) load_k<D>(t1, krc, krot_b, row, k1, k1, wend0, colh, gq);
            else load_k<D>(t1, kc, cache_b, row, k1, r1, wend0, colh, gq);
            stage_v(k1, r1, wend0, Slot1{});
        }
        if (PAGED && wstart + 2 * kWaveKeys < wend0) pg2 = page_of(wstart + 2 * kWaveKeys);
    }

    // rotated-key cache: one wave per (batch, KV head) reads the row that the
    // next step will need as remote (its wait falls in the first step's);
    // the rotated row is stored after the key loop
    const bool write_ahead = RKC && !PAGED && p.rot_row >= 0 && split == 0 && sub == 0 && lane < HALF;
    float wa_x = 0.f, wa_y = 0.f;
    float2 wa_cs = make_float2(1.f, 0.f);
    int64_t wa_o = 0;
    if (write_ahead) {
        wa_o = cache_b + p.rot_row * row + lane;
        wa_x = (float)kc[wa_o];
        wa_y = (float)kc[wa_o + HALF];
        wa_cs = tf(p.rot_row - p.rot_row / G, lane);
    }

    if (tid == 0) s_bad = FI ? 0 : !table_matches(p.table, p.table_key, D, p.rope_base, table_need(p.L, p.G));
    // rows 0..32 of the table are cos/sin(dn * theta_i); only rows < L are
    // guaranteed to exist and dn <= L-1, so copy no further
    if (!RKC)
        for (int i = tid; i < min(JROWS, L) * HALF; i += kDecThreads)
            sJ[(i / HALF) * JSTR + i % HALF] = tf(i / HALF, i % HALF);
    __syncthreads();
    const bool bad = s_bad;

    const int head = g * R + rq;

    // ---- query: stored fragments and the corrected view ---------------------
    // B operand of S^T = K Q^T: fragment c holds dims 32c + 8gq + [0, 8).  The
    // corrected view R(-n_q) q is kept in bf16 (the MFMA operand precision).
    bf16x8 qf[NC], qrem[NC];
    {
        const __bf16* qp = static_cast<const __bf16*>(p.q) + ((int64_t)(b * Lq + jq) * Hq + head) * D;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            qf[c] = hvalid ? *reinterpret_cast<const bf16x8*>(qp + 32 * c + 8 * gq) : bf16x8{};
            qrem[c] = qf[c];
        }
        if (G > 1 && !bad) {
            const int nq = qpos - qpos / G;
#pragma unroll
            for (int c = 0; c < NC / 2; ++c)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    float x = (float)qf[c][j], y = (float)qf[c + NC / 2][j];
                    rotate_back(x, y, tf(nq, 32 * c + 8 * gq + j));
                    qrem[c][j] = (__bf16)x;
                    qrem[c + NC / 2][j] = (__bf16)y;
                }
        }
    }

    f32x4 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x4{};
    float m_run = -INFINITY, l_run = 0.f;

    const int wend = bad ? wstart : wend0;
    float2* myBase = sBase[wave];

    // cos/sin(nb * theta_lane) of the current step's base offset nb = n(kbase):
    // read once, then advanced by the step's offset increment (<= 32) from the
    // LDS rows, so no step waits on a table load.
    float2 base = make_float2(1.f, 0.f);
    if (!RKC && lane < HALF && wstart < wend && G > 1) base = tf(wstart - wstart / G, lane);

    // the corrected query for the current step: R(nb) applied to R(-n_q) q
    bf16x8 qit[NC];
    int nb = 0;
    auto rotate_query = [&](int kb) {
        nb = kb - kb / G;
        wave_lds_sync();   // earlier reads of myBase are done
        if (lane < HALF) myBase[lane] = base;
        wave_lds_sync();
#pragma unroll
        for (int c = 0; c < NC / 2; ++c)
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const float2 cs = myBase[32 * c + 8 * gq + j];
                const float x = (float)qrem[c][j], y = (float)qrem[c + NC / 2][j];
                qit[c][j] = (__bf16)(x * cs.x - y * cs.y);
                qit[c + NC / 2][j] = (__bf16)(x * cs.y + y * cs.x);
            }
    };
    if (!RKC && G > 1 && wstart < wend && wstart < kloc_hi) rotate_query(wstart);

    // Step i computes from K tile i & 1 and V slot i & 1; as each part is
    // consumed it is refilled with step i + 2 (each 16-key half of K after
    // its scores, V after the PV product), so two steps of loads stay in
    // flight during the compute.
    const int tr_row = 8 * gq + (colh >> 2);   // transposing read: row and dims this lane addresses
    const int tr_dim = 4 * (colh & 3);
    auto step = [&](int kbase, DecodeTile<D>& cur, auto slot) __attribute__((always_inline)) {
        const int knext = kbase + kWaveKeys;
        const int k2 = kbase + 2 * kWaveKeys;
        // rows of step i + 2 (its table entry was read a step ago), then the
        // table entry of step i + 3
        const int64_t r2 = k2 < wend ? row_in(pg2, k2) : 0;
        if (PAGED && k2 + kWaveKeys < wend) pg2 = page_of(k2 + kWaveKeys);

        // some column scores a key of this step in the stored view / in the
        // corrected view
        const bool w_loc = (G == 1) || (kbase + kWaveKeys - 1 >= kloc_lo);
        const bool w_rem = (G > 1) && (kbase < kloc_hi);

        float s[2][4];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            f32x4 sl = f32x4{}, sr = f32x4{};
            if (w_loc) {
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    sl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.k[blk][c], qf[c], sl, 0, 0, 0);
            }
            if (RKC && w_rem) {
                // a step with local keys was read from the stored cache: read
                // this half's rows again, rotated, for its remote keys
                if (w_loc) load_k_blk<D>(cur, krc, krot_b, row, kbase, kbase, wend, colh, gq, blk);
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    sr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur.k[blk][c], qrem[c], sr, 0, 0, 0);
            } else if (w_rem) {
                const int key = kbase + 8 * (colh >> 2) + 4 * blk + (colh & 3);
                const int dn = (key < wend) ? (key - key / G) - nb : 0;
                bf16x8 kr[NC];
#pragma unroll
                for (int c = 0; c < NC / 2; ++c)
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        float x = (float)cur.k[blk][c][j], y = (float)cur.k[blk][c + NC / 2][j];
                        rotate_back(x, y, sJ[dn * JSTR + 32 * c + 8 * gq + j]);
                        kr[c][j] = (__bf16)x;
                        kr[c + NC / 2][j] = (__bf16)y;
                    }
#pragma unroll
                for (int c = 0; c < NC; ++c) sr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kr[c], qit[c], sr, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kk = kbase + 8 * gq + 4 * blk + i;   // key of C row gq*4+i
                float v;
                if (w_loc && w_rem) v = kk >= kloc ? sl[i] : sr[i];
                else v = w_loc ? sl[i] : sr[i];
                s[blk][i] = (kk < wend && (!MQ || kk <= qpos)) ? v * scale2 : -INFINITY;
            }
            // this half's K registers are free: start step i + 2's loads
            if (k2 < wend) {
                if (rkc_step(k2)) load_k_blk<D>(cur, krc, krot_b, row, k2, k2, wend, colh, gq, blk);
                else load_k_blk<D>(cur, kc, cache_b, row, k2, r2, wend, colh, gq, blk);
            }
        }

        // ---- online softmax per head column: 8 values here, 4 quads per head --
        // The reference m_run moves only when a score exceeds it by more than
        // kLazy (log2 units): probabilities stay below 2^kLazy (exact in fp32
        // and within bf16's range), and the accumulators are rescaled only on
        // the rare steps where some column's reference moves (a wave-uniform
        // branch).  A column's first step with a key in its causal range sets
        // it (m_run = -inf before); with several positions a column can meet
        // a step with none, whose probabilities must come out 0, not NaN.
        constexpr float kLazy = 8.f;
        float mx = -INFINITY;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[blk][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool move = mx > m_run + kLazy;
        if (__any(move)) {
            // a column that does not move keeps its scale (its m_run may still
            // be -inf, which a subtraction would turn into NaN)
            const float alpha = move ? fast_exp2(m_run - mx) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
            m_run = move ? mx : m_run;
        }
        float ls = 0.f;
        bf16x8 Bp;
        // (one position: every step holds a key of every column, so m_run is set)
        const float m_sub = (MQ && m_run == -INFINITY) ? 0.f : m_run;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pv = fast_exp2(s[blk][i] - m_sub);
                ls += pv;
                Bp[4 * blk + i] = (__bf16)pv;
            }
        l_run += ls;

        // ---- O^T += V^T P^T: V^T fragments by transposing reads of the slot ----
        const __bf16* V = decltype(slot)::value ? sV1[wave] : sV0[wave];
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int lc = (16 * db + tr_dim) >> 3, wi = tr_dim & 7;
            const bf16x4 lo = lds_read_tr16(V + tr_row * D + 8 * dec_vswz<D>(tr_row, lc) + wi);
            const bf16x4 hi = lds_read_tr16(V + (tr_row + 4) * D + 8 * dec_vswz<D>(tr_row + 4, lc) + wi);
            const bf16x8 A = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bp, acc[db], 0, 0, 0);
        }
        // the slot is consumed: start step i + 2's V copies into it
        if (k2 < wend) stage_v(k2, r2, wend, slot);
        if (!RKC && w_rem && knext < wend && lane < HALF) {
            const int stp = (knext - knext / G) - nb;   // 0 <= stp <= 32, stp < L
            const float2 j2 = sJ[stp * JSTR + lane];
            base = make_float2(base.x * j2.x - base.y * j2.y, base.y * j2.x + base.x * j2.y);
        }
        // the next step's corrected query, computed here so that it is off the
        // path from K's arrival to the next K loads
        if (!RKC && G > 1 && knext < wend && knext < kloc_hi) rotate_query(knext);
    };
    for (int kbase = wstart; kbase < wend; kbase += 2 * kWaveKeys) {
        step(kbase, t0, Slot0{});
        if (kbase + kWaveKeys < wend) step(kbase + kWaveKeys, t1, Slot1{});
    }
    // every copy into the V slots has landed before they are reused below
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (bad_page) l_run = NAN;   // poisons this head's output through the merge
    if (write_ahead) {
        // a table that does not match the call leaves NaN in the cache, so
        // later steps stay visibly wrong until the caller resets its state
        if (bad) wa_x = wa_y = NAN;
        else rotate_back(wa_x, wa_y, wa_cs);
        __bf16* kw = static_cast<__bf16*>(const_cast<void*>(p.krot));
        const int64_t wo = krot_b + p.rot_row * row + lane;
        kw[wo] = (__bf16)wa_x;
        kw[wo + HALF] = (__bf16)wa_y;
    }

    // ---- merge the NW waves of each head, write this split's partials ---------
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    __syncthreads();   // every wave is done with its V^T slice
    float* s_acc = reinterpret_cast<float*>(&sV0[0][0]);   // [wave][16 columns][D]
    static_assert(kDecodeWaves * 16 * D * 4 <= kDecodeWaves * kWaveKeys * D * 2, "merge scratch fits");
    if (gq == 0) {
        s_m[wave][colh] = m_run;
        s_l[wave][colh] = l_tot;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_acc[(wave * 16 + colh) * D + 16 * db + 4 * gq + i] = acc[db][i];
    __syncthreads();
    const int ncol = Lq * R;   // valid columns per KV head
    for (int idx = tid; idx < WH * ncol * D; idx += kDecThreads) {
        const int hx = idx / (ncol * D), c = (idx / D) % ncol, d = idx % D;
        float M = -INFINITY;
        for (int u = 0; u < NW; ++u) M = fmaxf(M, s_m[u * WH + hx][c]);
        float a = 0.f, l = 0.f;
        if (!bad) {
            for (int u = 0; u < NW; ++u) {
                const int w = u * WH + hx;
                const float m = s_m[w][c];
                const float fw = (m == -INFINITY) ? 0.f : fast_exp2(m - M);   // waves without keys
                a += fw * s_acc[(w * 16 + c) * D + d];
                l += fw * s_l[w][c];
            }
        } else {
            a = l = M = NAN;
        }
        const int hq = (blockIdx.y * WH + hx) * R + c % R;
        float* o = p.ws + ((((int64_t)b * Lq + c / R) * Hq + hq) * p.n_split + split) * (D + 2);
        o[d] = a;
        if (d == 0) {
            o[D] = M;
            o[D + 1] = l;
        }
    }
}

// Log-sum-exp merge of one head's split partials (up to 256 splits):
// workgroup = (head, batch, 16-dim block) of 512 threads.  Each thread loads
// one dimension of every 32nd split together with one split's (max, sum),
// all in one round trip; split weights go to LDS once.  Sixteen dimensions
// per workgroup (256 workgroups at 32 heads and D = 128) measured 0.3 µs
// faster per step than 32 (128 workgroups of 1024 threads), and faster than
// 8; each dimension's sum keeps the same order, so the result is the same.
constexpr int kCombDims = 16;                 // dimensions per workgroup
constexpr int kCombThreads = kCombDims * 32;  // 32 interleaved split groups
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(kCombThreads) void decode_combine_kernel(DecodeParams p) {
    __shared__ float sW[kDecodeMaxSplits];
    __shared__ float sRed[kCombThreads];
    __shared__ float sM, sL;
    const int head = blockIdx.x;
    const int bj = blockIdx.y;   // (batch, query position)
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ns = p.n_split;
    const float* base = p.ws + ((int64_t)bj * p.Hq + head) * ns * (D + 2);
    const int d = blockIdx.z * kCombDims + (tid % kCombDims);
    const int part = tid / kCombDims;   // 32 interleaved split groups
    // every load of the kernel goes out at once: this thread's partial sums
    // and, for thread t < ns, split t's max and row sum
    float pa[kDecodeMaxSplits / 32];
#pragma unroll
    for (int u = 0; u < kDecodeMaxSplits / 32; ++u) {
        const int s = part + 32 * u;
        pa[u] = s < ns ? base[s * (D + 2) + d] : 0.f;
    }
    const float m = tid < ns ? base[tid * (D + 2) + D] : -INFINITY;
    const float lsplit = tid < ns ? base[tid * (D + 2) + D + 1] : 0.f;
    float M = m;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
    if (lane == 0) sRed[wave] = M;
    __syncthreads();
    M = sRed[0];
#pragma unroll
    for (int w = 1; w < kCombThreads / 64; ++w) M = fmaxf(M, sRed[w]);
    const float wgt = tid < ns ? fast_exp2(m - M) : 0.f;
    if (tid < kDecodeMaxSplits) sW[tid] = wgt;
    float l = wgt * lsplit;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o);
    __syncthreads();
    if (lane == 0) sRed[wave] = l;
    __syncthreads();
    if (tid == 0) {
        float t = 0.f;
#pragma unroll
        for (int w = 0; w < kCombThreads / 64; ++w) t += sRed[w];
        sM = M;
        sL = t;
    }
    float a = 0.f;
#pragma unroll
    for (int u = 0; u < kDecodeMaxSplits / 32; ++u) {
        const int s = part + 32 * u;
        if (s < ns) a += sW[s] * pa[u];
    }
    __syncthreads();
    sRed[tid] = a;
    __syncthreads();
    if (tid < kCombDims) {
        float t = 0.f;
#pragma unroll
        for (int q = 0; q < 32; ++q) t += sRed[q * kCombDims + tid];
        const float lt = sL;
        const int64_t o = ((int64_t)bj * p.Hq + head) * D + d;
        if constexpr (OUT_BF16) static_cast<__bf16*>(p.out)[o] = (__bf16)(t / lt);
        else static_cast<float*>(p.out)[o] = t / lt;
        if (blockIdx.z == 0 && tid == 0 && p.lse)
            p.lse[((int64_t)(bj / p.Lq) * p.Hq + head) * p.Lq + bj % p.Lq] = (sM + log2f(lt)) * 0.69314718055994531f;
    }
}

// ---- several query positions: keys staged in LDS for every column group ----
//
// A short chunk of Lq positions (Jet-Long §3.2: the chunk's rows under G(L),
// remote keys in their corrected view) with 2 or 4 groups of 16 (position,
// query head) columns per KV head.  Workgroup = (key range, KV head, batch)
// with two waves per column group; every 64-key step is copied HBM -> LDS
// once (buffer loads into LDS, no registers), four steps deep, and each
// wave scores one 32-key half of the step for its 16 columns with the
// decode kernel's MFMA layout (K rows as A, queries as N columns; V^T
// through the transposing LDS read).  The copies of all groups' keys are
// then one HBM read, and the ring keeps up to 128 KB per compute unit in
// flight with no register cost.
//
// Remote keys are read rotated from p.krot (by position), stored keys from
// the cache.  A step that holds some column's window edge is visited twice:
// once in the corrected view (keys before each column's edge kept), once in
// the stored view (the rest).
constexpr int kMqKeys = 64;    // keys per stage
static_assert(kMqKeys == kMultiStageKeys, "the host plan deals whole stages");
constexpr int kMqStages = 4;   // LDS ring depth

// 16-byte buffer -> LDS copy per lane (lane l writes bytes [16l, 16l + 16)
// after the wave-uniform LDS base), issued so that the compiler does not
// track it: the compiler cannot tell this kernel's four stages apart and
// would make every LDS read wait for every copy in flight, which empties the
// ring.  The kernel orders the copies itself: each stage is waited for with
// s_waitcnt vmcnt (copies complete in issue order) and a barrier before any
// wave reads it, and a stage is refilled only after a barrier that follows
// every read of its previous contents.  The instruction writes no register;
// M0 (the LDS base) needs one wait state before the copy reads it.  The
// copies are non-temporal (streaming): every byte is read once per call, and
// the hint cut the 16-token chunk at 128K from 119.8 to 103.3 us.
__device__ inline void mq_copy16(__amdgpu_buffer_rsrc_t r, const void* lds_base, uint32_t voff, uint32_t soff) {
    const uint32_t m0v = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)lds_base;
    uint32_t saved;   // M0 is reserved to the compiler: restored before the asm ends
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\tbuffer_load_dwordx4 %2, %3, %4 offen nt lds\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved)
                 : "s"(m0v), "v"(voff), "s"(r), "s"(soff)
                 : "memory");
}

template <int D>
__device__ inline int mq_kswz(int row, int c) { return c ^ (row & (D / 8 - 1)); }
template <int D>
__device__ inline int mq_vswz(int row, int c) { return c ^ ((4 * (row & 3)) & (D / 8 - 1)); }

template <int D, bool OUT_BF16, bool PAGED, int NG>
__global__ __launch_bounds__(128 * NG) void decode_multi_kernel(DecodeParams p) {
    constexpr int NWV = 2 * NG;           // waves: column group x key half
    constexpr int NT = 64 * NWV;
    constexpr int NC = D / 32;            // 32-dim chunks of the score MFMA
    constexpr int NDB = D / 16;           // 16-dim blocks of O^T
    constexpr int CH = D / 8;             // 16-byte chunks per row
    constexpr int BK = kMqKeys;
    constexpr int PU = BK * CH / NT;      // 16-byte copies per thread per operand and stage
    constexpr int RU = NT / CH;           // rows per copy round
    static_assert(PU * NT == BK * CH && RU % CH == 0 && RU % 4 == 0, "copy rounds keep lane-constant swizzles");
    // four stages, K then V in each, as separate objects selected at compile
    // time (every LDS address of a step is then a constant offset)
    __shared__ __attribute__((aligned(16))) __bf16 sS0[2 * BK * D], sS1[2 * BK * D], sS2[2 * BK * D], sS3[2 * BK * D];
    __shared__ float s_m[NG][16], s_l[NG][16];
    __shared__ int s_bad;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int colh = lane & 15;
    const int gq = lane >> 4;
    const int grp = wave % NG;
    const int sub = wave / NG;            // key half of each step
    const int split = blockIdx.x;
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int L = (int)p.L;
    const int Hq = (int)p.Hq;
    const int R = p.R;
    const int G = (int)p.G;
    const int Lq = p.Lq;
    const int fcol = grp * 16 + colh;
    const bool hvalid = fcol < Lq * R;
    const int jq = hvalid ? fcol / R : Lq - 1;
    const int rq = hvalid ? fcol % R : 0;
    const int qpos = L - Lq + jq;
    const int kloc = p.kloc > 0 ? (int)p.kloc - (Lq - 1 - jq) : (int)p.kloc;
    const int kloc_lo = p.kloc > 0 ? (int)p.kloc - (Lq - 1) : (int)p.kloc;
    const int kloc_hi = (int)p.kloc;
    const float scale2 = p.sm_scale_log2;
    const int64_t kv_row = p.Hkv * D;
    const uint32_t row_bytes = (uint32_t)(kv_row * 2);

    // this workgroup's keys [kr0, kr1) in steps of BK; steps [t_rem, t_loc)
    // hold a window edge and are visited twice
    const int kr0 = split * p.wave_chunk + kMqKeys * min(split, p.wave_extra);
    const int kr1 = min(L, kr0 + p.wave_chunk + (split < p.wave_extra ? kMqKeys : 0));
    const int n_steps = kr1 > kr0 ? (kr1 - kr0 + BK - 1) / BK : 0;
    auto clampi = [](int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); };
    const int t_rem = G > 1 ? clampi(kloc_lo - kr0 < 0 ? -1 : (kloc_lo - kr0) / BK, 0, n_steps) : 0;
    const int t_loc = G > 1 ? clampi(kloc_hi - kr0 <= 0 ? 0 : (kloc_hi - kr0 + BK - 1) / BK, 0, n_steps) : 0;
    const int n_twice = t_loc > t_rem ? t_loc - t_rem : 0;
    const int NV = n_steps + n_twice;
    // visit v: its step's first key and its view
    auto visit_of = [&](int v, int& k0, bool& rem) __attribute__((always_inline)) {
        int t;
        if (v < t_rem) {
            t = v;
            rem = true;
        } else if (v < t_rem + 2 * n_twice) {
            t = t_rem + (v - t_rem) / 2;
            rem = ((v - t_rem) & 1) == 0;
        } else {
            t = v - n_twice;
            rem = false;
        }
        k0 = kr0 + t * BK;
    };

    // ---- staging -------------------------------------------------------------
    // One copy fills 64 consecutive 16-byte LDS slots (one per lane): slot
    // u * NT + tid holds row u * RU + tid / CH, physical chunk tid % CH, into
    // which this lane copies logical chunk swz(row, tid % CH).  Rows past L
    // (and every row of a visit past the last) read as zeros.
    const __bf16* kc = static_cast<const __bf16*>(p.k);
    const __bf16* vc = static_cast<const __bf16*>(p.v);
    const __bf16* krc = static_cast<const __bf16*>(p.krot);
    const int trow = tid / CH, tch = tid % CH;
    const uint32_t k_voff = (uint32_t)trow * row_bytes + 16u * (uint32_t)mq_kswz<D>(trow, tch);
    const uint32_t v_voff = (uint32_t)trow * row_bytes + 16u * (uint32_t)mq_vswz<D>(trow, tch);
    bool bad_page = false;
    auto cache_row = [&](int k0) __attribute__((always_inline)) -> int64_t {
        if constexpr (!PAGED) {
            return (int64_t)b * p.Lmax + k0;
        } else {
            typedef const __attribute__((address_space(4))) int32_t* ctab;
            const int ps = (int)p.page_size;
            int pg = ((ctab)(p.block_table + (int64_t)b * p.max_pages))[k0 / ps];
            if (pg < 0 || pg >= p.n_pages) {
                bad_page = true;
                pg = 0;
            }
            return (int64_t)pg * ps + k0 % ps;
        }
    };
    auto stage = [&](int v, __bf16* dK, __bf16* dV) __attribute__((always_inline)) {
        int k0 = 0;
        bool rem = false;
        uint32_t bytes = 0;
        const __bf16* ks = kc;
        const __bf16* vs = vc;
        if (v < NV) {
            visit_of(v, k0, rem);
            bytes = (uint32_t)min(L - k0, BK) * row_bytes;
            const int64_t crow = cache_row(k0);
            ks = rem ? krc + ((int64_t)b * p.krot_rows + k0) * kv_row + (int64_t)g * D
                     : kc + crow * kv_row + (int64_t)g * D;
            vs = vc + crow * kv_row + (int64_t)g * D;
        }
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(ks, bytes);
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vs, bytes);
#pragma unroll
        for (int u = 0; u < PU; ++u) {
            mq_copy16(rk, dK + (u * NWV + wave) * 512, k_voff, (uint32_t)(u * RU) * row_bytes);
            mq_copy16(rv, dV + (u * NWV + wave) * 512, v_voff, (uint32_t)(u * RU) * row_bytes);
        }
    };
    // outstanding copies allowed while waiting for the oldest stage: those
    // of the three stages issued after it (vmcnt field of s_waitcnt, expcnt
    // and lgkmcnt left at their maxima)
    constexpr int kAfter = 2 * PU * (kMqStages - 1);
    static_assert(kAfter < 64, "vmcnt holds 6 bits");
    constexpr int kWaitEnc = (kAfter & 15) | ((kAfter >> 4) << 14) | (7 << 4) | (15 << 8);

    stage(0, sS0, sS0 + BK * D);
    stage(1, sS1, sS1 + BK * D);
    stage(2, sS2, sS2 + BK * D);

    if (tid == 0) s_bad = !table_matches(p.table, p.table_key, D, p.rope_base, table_need(p.L, p.G));

    // ---- queries: stored and corrected views (bf16, the MFMA operand) ----
    const int head = g * R + rq;
    bf16x8 qf[NC], qrem[NC];
    {
        const __bf16* qp = static_cast<const __bf16*>(p.q) + ((int64_t)(b * Lq + jq) * Hq + head) * D;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            qf[c] = hvalid ? *reinterpret_cast<const bf16x8*>(qp + 32 * c + 8 * gq) : bf16x8{};
            qrem[c] = qf[c];
        }
        if (G > 1) {
            const int nq = qpos - qpos / G;
#pragma unroll
            for (int c = 0; c < NC / 2; ++c)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    float x = (float)qf[c][j], y = (float)qf[c + NC / 2][j];
                    rotate_back(x, y, table_cs(p.TF, D / 2, nq, 32 * c + 8 * gq + j));
                    qrem[c][j] = (__bf16)x;
                    qrem[c + NC / 2][j] = (__bf16)y;
                }
        }
    }

    f32x4 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x4{};
    float m_run = -INFINITY, l_run = 0.f;
    // A-operand row of this lane in each 16-key block (C rows then give P^T
    // in natural key order), and the transposing read's row and dims
    const int dk0 = 8 * (colh >> 2) + (colh & 3);
    const int tr_row = 8 * gq + (colh >> 2);
    const int tr_dim = 4 * (colh & 3);

    auto compute = [&](int v, const __bf16* K, const __bf16* V) __attribute__((always_inline)) {
        int k0;
        bool rem;
        visit_of(v, k0, rem);
        const int kb = k0 + 32 * sub;
        float s[2][4];
#pragma unroll
        for (int blk = 0; blk < 2; ++blk) {
            const int r = 32 * sub + dk0 + 4 * blk;
            f32x4 sc = f32x4{};
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const bf16x8 a = *reinterpret_cast<const bf16x8*>(K + r * D + 8 * mq_kswz<D>(r, 4 * c + gq));
                sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, rem ? qrem[c] : qf[c], sc, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int kk = kb + 8 * gq + 4 * blk + i;
                const bool keep = kk < L && kk <= qpos && (rem ? kk < kloc : kk >= kloc);
                s[blk][i] = keep ? sc[i] * scale2 : -INFINITY;
            }
        }
        // online softmax per column (lazy reference max, as in the split kernel)
        constexpr float kLazy = 8.f;
        float mx = -INFINITY;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[blk][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const bool move = mx > m_run + kLazy;
        if (__any(move)) {
            const float alpha = move ? fast_exp2(m_run - mx) : 1.f;
            l_run *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
            m_run = move ? mx : m_run;
        }
        const float m_sub = m_run == -INFINITY ? 0.f : m_run;
        float ls = 0.f;
        bf16x8 Bp;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pv = fast_exp2(s[blk][i] - m_sub);
                ls += pv;
                Bp[4 * blk + i] = (__bf16)pv;
            }
        l_run += ls;
        // O^T += V^T P^T: V^T rows (dims) through the transposing read
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const int r0 = 32 * sub + tr_row;
            const int lc = (16 * db + tr_dim) >> 3, wi = tr_dim & 7;
            const bf16x4 lo = lds_read_tr16(V + r0 * D + 8 * mq_vswz<D>(r0, lc) + wi);
            const bf16x4 hi = lds_read_tr16(V + (r0 + 4) * D + 8 * mq_vswz<D>(r0 + 4, lc) + wi);
            const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
            acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, Bp, acc[db], 0, 0, 0);
        }
    };

    // visit v computes from stage slot v % 4; first the slot that visit v - 1
    // used is refilled with visit v + 3 (a visit past the last copies zeros),
    // so that four stages are in flight while visit v's copies are awaited
    auto step = [&](int v, auto slot) __attribute__((always_inline)) {
        constexpr int S = decltype(slot)::value;
        __bf16* const Ss[4] = {sS0, sS1, sS2, sS3};
        __syncthreads();                         // visit v - 1 is done everywhere
        stage(v + 3, Ss[(S + 3) & 3], Ss[(S + 3) & 3] + BK * D);
        __builtin_amdgcn_s_waitcnt(kWaitEnc);   // this wave's copies of visit v have landed
        __syncthreads();                         // and everyone's
        compute(v, Ss[S], Ss[S] + BK * D);
    };
    for (int v = 0; v < NV; v += 4) {
        step(v, std::integral_constant<int, 0>{});
        if (v + 1 < NV) step(v + 1, std::integral_constant<int, 1>{});
        if (v + 2 < NV) step(v + 2, std::integral_constant<int, 2>{});
        if (v + 3 < NV) step(v + 3, std::integral_constant<int, 3>{});
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // the zero copies past the last visit
    __syncthreads();
    const bool bad = s_bad || __any(bad_page);   // a bad page poisons every column of this workgroup

    // ---- merge the two key halves of each column group, write the partials ----
    // The second-half waves leave their state in LDS (the first two K
    // stages, two groups each); the first-half waves merge it into theirs.
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    static_assert(2 * 16 * D * 4 <= BK * D * 2, "two groups' halves fit one K stage");
    float* half1 = reinterpret_cast<float*>(grp < 2 ? sS0 : sS1) + (grp & 1) * 16 * D;
    if (sub == 1) {
        if (gq == 0) {
            s_m[grp][colh] = m_run;
            s_l[grp][colh] = l_tot;
        }
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) half1[colh * D + 16 * db + 4 * gq + i] = acc[db][i];
    }
    __syncthreads();
    if (sub == 0 && hvalid) {
        const float m1 = s_m[grp][colh], l1 = s_l[grp][colh];
        const float M = fmaxf(m_run, m1);
        const float f0 = m_run == -INFINITY ? 0.f : fast_exp2(m_run - M);
        const float f1 = m1 == -INFINITY ? 0.f : fast_exp2(m1 - M);
        float* o = p.ws + ((((int64_t)b * Lq + jq) * Hq + head) * p.n_split + split) * (D + 2);
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int d = 16 * db + 4 * gq + i;
                o[d] = bad ? NAN : f0 * acc[db][i] + f1 * half1[colh * D + d];
            }
        if (gq == 0) {
            o[D] = bad ? NAN : M;
            o[D + 1] = bad ? NAN : f0 * l_tot + f1 * l1;
        }
    }
}

// Log-sum-exp merge of a (batch, position, head)'s split partials when the
// splits are few (the kernel above leaves ~256 / (B * Hkv) of them):
// workgroup of D threads, thread d sums dimension d over the splits in
// split order with the weights 2^(m_s - M) held in LDS.  A NaN max (bad
// table or page) makes its weight, and so the output, NaN.
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(D) void decode_combine_few_kernel(DecodeParams p) {
    __shared__ float sW[kDecodeMaxSplits];
    __shared__ float sRed[D / 64];
    const int head = blockIdx.x;
    const int bj = blockIdx.y;   // (batch, query position)
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int ns = p.n_split;
    const float* base = p.ws + ((int64_t)bj * p.Hq + head) * ns * (D + 2);
    float m = -INFINITY;
    for (int s = tid; s < ns; s += D) m = fmaxf(m, base[s * (D + 2) + D]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
    if (lane == 0) sRed[wave] = m;
    __syncthreads();
    float M = sRed[0];
#pragma unroll
    for (int w = 1; w < D / 64; ++w) M = fmaxf(M, sRed[w]);
    __syncthreads();
    float l = 0.f;
    for (int s = tid; s < ns; s += D) {
        const float ms = base[s * (D + 2) + D];
        const float wgt = ms == -INFINITY ? 0.f : fast_exp2(ms - M);   // splits without keys
        sW[s] = wgt;
        l += wgt * base[s * (D + 2) + D + 1];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o);
    if (lane == 0) sRed[wave] = l;
    __syncthreads();
    float lt = 0.f;
#pragma unroll
    for (int w = 0; w < D / 64; ++w) lt += sRed[w];
    float a = 0.f;
    for (int s = 0; s < ns; ++s) a += sW[s] * base[s * (D + 2) + tid];
    const int64_t o = ((int64_t)bj * p.Hq + head) * D + tid;
    if constexpr (OUT_BF16) static_cast<__bf16*>(p.out)[o] = (__bf16)(a / lt);
    else static_cast<float*>(p.out)[o] = a / lt;
    if (tid == 0 && p.lse)
        p.lse[((int64_t)(bj / p.Lq) * p.Hq + head) * p.Lq + bj % p.Lq] = (M + log2f(lt)) * 0.69314718055994531f;
}

template <int D, bool OUT_BF16, int NG>
void launch_multi(const DecodeParams& p, hipStream_t stream) {
    const dim3 grid(p.n_split, p.Hkv, p.B);
    if (p.block_table)
        hipLaunchKernelGGL((decode_multi_kernel<D, OUT_BF16, true, NG>), grid, dim3(128 * NG), 0, stream, p);
    else
        hipLaunchKernelGGL((decode_multi_kernel<D, OUT_BF16, false, NG>), grid, dim3(128 * NG), 0, stream, p);
    hipLaunchKernelGGL((decode_combine_few_kernel<D, OUT_BF16>), dim3(p.Hq, p.B * p.Lq), dim3(D), 0, stream, p);
}

template <int D, bool OUT_BF16>
hipError_t launch_dec(const DecodeParams& p, hipStream_t stream) {
    const dim3 grid(p.n_split, p.Hkv / p.heads_per_wg, p.B);
    if (p.n_grp > 1) {
        if (p.n_grp == 2) launch_multi<D, OUT_BF16, 2>(p, stream);
        else launch_multi<D, OUT_BF16, 4>(p, stream);
        return hipGetLastError();
    }
    if (p.Lq > 1 && p.block_table)   // a short chunk: rotated keys from the chunk workspace
        hipLaunchKernelGGL((decode_split_kernel<D, OUT_BF16, true, true, false, true>), grid, dim3(kDecThreads), 0,
                           stream, p);
    else if (p.Lq > 1)
        hipLaunchKernelGGL((decode_split_kernel<D, OUT_BF16, false, true, false, true>), grid, dim3(kDecThreads),
                           0, stream, p);
    else if (p.block_table && p.krot)
        hipLaunchKernelGGL((decode_split_kernel<D, OUT_BF16, true, true, false>), grid, dim3(kDecThreads), 0,
                           stream, p);
    else if (p.block_table)
        hipLaunchKernelGGL((decode_split_kernel<D, OUT_BF16, true, false, false>), grid, dim3(kDecThreads), 0,
                           stream, p);
    else if (p.krot)
        hipLaunchKernelGGL((decode_split_kernel<D, OUT_BF16, false, true, false>), grid, dim3(kDecThreads), 0,
                           stream, p);
    else if (p.fi)
        hipLaunchKernelGGL((decode_split_kernel<D, OUT_BF16, false, false, true>), grid, dim3(kDecThreads), 0,
                           stream, p);
    else
        hipLaunchKernelGGL((decode_split_kernel<D, OUT_BF16, false, false, false>), grid, dim3(kDecThreads), 0,
                           stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_combine_kernel<D, OUT_BF16>), dim3(p.Hq, p.B * p.Lq, D / kCombDims),
                       dim3(kCombThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

namespace {

// Rows [r0, r1) of every (batch, KV head) of a [B, Lmax, Hkv, D] bf16 key
// cache rotated by their correction offset, table row n(k) = k - floor(k/G),
// rounded to bf16, into the same place of krot (§3.2 Eq. 5 applied to the
// cached keys).  One thread per 8 rotation pairs of a row; HBM-bound.  A
// table whose header does not match the call writes NaN rows instead.
template <int D>
__global__ __launch_bounds__(256) void rotate_rows_kernel(const __bf16* __restrict__ k, __bf16* __restrict__ kr,
                                                          const float2* __restrict__ TF, int64_t n_items,
                                                          int64_t Lmax, int Hkv, int64_t r0, int64_t nrows,
                                                          int64_t G, const TableHeader* table, TableKey key,
                                                          double rope_base, int64_t L) {
    constexpr int HALF = D / 2;
    constexpr int CPR = HALF / 8;   // 8-pair items per row
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= n_items) return;
    const int c = (int)(t % CPR);
    const int64_t rh = t / CPR;     // (batch, row, head), head fastest
    const int h = (int)(rh % Hkv);
    const int64_t br = rh / Hkv;
    const int64_t pos = r0 + br % nrows;
    const int64_t b = br / nrows;
    const int64_t n = pos - pos / G;
    const int64_t o = ((b * Lmax + pos) * Hkv + h) * D + 8 * c;
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(k + o);
    const bf16x8 y = *reinterpret_cast<const bf16x8*>(k + o + HALF);
    bf16x8 xo, yo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float4 c4 = table_cs2(TF, HALF, n, 8 * c + 2 * e);
        float x0 = (float)x[2 * e], y0 = (float)y[2 * e];
        float x1 = (float)x[2 * e + 1], y1 = (float)y[2 * e + 1];
        rotate_back(x0, y0, make_float2(c4.x, c4.y));
        rotate_back(x1, y1, make_float2(c4.z, c4.w));
        xo[2 * e] = (__bf16)x0;
        yo[2 * e] = (__bf16)y0;
        xo[2 * e + 1] = (__bf16)x1;
        yo[2 * e + 1] = (__bf16)y1;
    }
    if (!table_matches(table, key, D, rope_base, table_need(L, G))) {
#pragma unroll
        for (int e = 0; e < 8; ++e) xo[e] = yo[e] = (__bf16)NAN;
    }
    *reinterpret_cast<bf16x8*>(kr + o) = xo;
    *reinterpret_cast<bf16x8*>(kr + o + HALF) = yo;
}

}  // namespace

hipError_t launch_rotate_rows(const void* k, void* krot, const DecodeParams& p, int64_t r0, int64_t r1,
                              hipStream_t stream) {
    if (r1 <= r0) return hipSuccess;
    const int64_t n_items = p.B * (r1 - r0) * p.Hkv * (p.head_dim / 16);
    const unsigned blocks = (unsigned)((n_items + 255) / 256);
    if (p.head_dim == 128)
        hipLaunchKernelGGL((rotate_rows_kernel<128>), dim3(blocks), dim3(256), 0, stream,
                           static_cast<const __bf16*>(k), static_cast<__bf16*>(krot), p.TF, n_items, p.Lmax,
                           (int)p.Hkv, r0, r1 - r0, p.G, p.table, p.table_key, p.rope_base, p.L);
    else
        hipLaunchKernelGGL((rotate_rows_kernel<64>), dim3(blocks), dim3(256), 0, stream,
                           static_cast<const __bf16*>(k), static_cast<__bf16*>(krot), p.TF, n_items, p.Lmax,
                           (int)p.Hkv, r0, r1 - r0, p.G, p.table, p.table_key, p.rope_base, p.L);
    return hipGetLastError();
}

// Scratch of jl_bifocal_decode_noalloc, for callers that cannot allocate
// (graph capture, serving loops): the split partials live in this fixed
// device array, one copy per device, held until the process ends.  Host code
// uses only the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void** ptr) {
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void* per_device[kMaxDevices] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!per_device[dev]) {
        void* a = nullptr;
        e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        per_device[dev] = a;
    }
    *ptr = per_device[dev];
    return hipSuccess;
}

hipError_t launch_decode(const DecodeParams& p, int out_dtype, hipStream_t stream) {
    const bool ob = out_dtype == 1;
    if (p.head_dim == 128) return ob ? launch_dec<128, true>(p, stream) : launch_dec<128, false>(p, stream);
    return ob ? launch_dec<64, true>(p, stream) : launch_dec<64, false>(p, stream);
}

}  // namespace jl
