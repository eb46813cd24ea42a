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
// streams its keys 32 per iteration with the next iteration's K and V in
// flight (non-temporal loads).  K goes straight from HBM into MFMA
// A-operand registers (rows = keys); V goes through wave-private LDS,
// transposed, to be the A operand of O^T += V^T P^T.  The R query heads of
// the KV head are the MFMA N columns (16x16x32 bf16), so each K/V byte is read
// once per step for all R heads.
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
// Variants of the split kernel (template flags): PAGED reads the cache
// through a block table; RKC reads remote keys already rotated from a
// second cache (and writes ahead the row the next step needs); FI uses the
// frequency-interpolation remote view of the §4.7 ablation, whose table
// rows (cos, sin)(n * phi_i) the kernel forms itself.
#include <math.h>

#include "internal.h"

namespace jl {

namespace {

constexpr int kDecThreads = kDecodeWaves * 64;
constexpr int kWaveKeys = 32;
constexpr int VSTR = kWaveKeys + 8;   // V^T row stride (keys) in LDS
constexpr int JROWS = kWaveKeys + 1;  // cos/sin(dn * theta) for dn = 0..32

// LDS ordering between lanes of one wave (write -> read, read -> write):
// wait for this wave's LDS operations and stop the compiler moving memory
// accesses across this point.
__device__ inline void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

template <int D>
struct DecodeTile {
    static constexpr int NC = D / 32;    // 32-dim K chunks of the QK^T MFMA
    static constexpr int KPL = D / 16;   // keys per lane in the V transpose
    bf16x8 k[2][NC];                     // rows of the two 16-key blocks
    bf16x8 v[KPL];                       // V rows for the transpose
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

template <int D>
__device__ inline void load_v(DecodeTile<D>& t, const __bf16* __restrict__ vc, int64_t cache_b, int64_t row,
                              int kbase, int64_t rbase, int kend, int lane) {
    constexpr int KPL = DecodeTile<D>::KPL;
    const int dg = lane % (D / 8);
    const int kg = lane / (D / 8);
#pragma unroll
    for (int e = 0; e < KPL; ++e) {
        const int dk = kg * KPL + e;
        t.v[e] = kbase + dk < kend
                     ? __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(vc + cache_b + (rbase + dk) * row + dg * 8))
                     : bf16x8{};
    }
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

template <int D, bool OUT_BF16, bool PAGED, bool RKC, bool FI>
__global__ __launch_bounds__(kDecThreads, 2) void decode_split_kernel(DecodeParams p) {
    constexpr int HALF = D / 2;
    constexpr int NC = D / 32;
    constexpr int NDB = D / 16;       // 16-dim blocks of O^T
    constexpr int KPL = D / 16;
    typedef __bf16 VW __attribute__((ext_vector_type(KPL)));

    __shared__ __attribute__((aligned(16))) __bf16 sVt[kDecodeWaves][D * VSTR];
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
    const int qpos = L - 1;
    // keys >= kloc are local (q - k <= w0); G == 1 makes every key local
    const int kloc = (G == 1) ? 0 : (int)max<int64_t>(0, (int64_t)qpos - p.w0);
    const float scale2 = p.sm_scale_log2;
    const __bf16* __restrict__ kc = static_cast<const __bf16*>(p.k);
    // rotated-key cache (RKC): remote keys are read in their corrected view
    // instead of being rotated here; a step is read from it when all of its
    // keys are remote
    const __bf16* __restrict__ krc = static_cast<const __bf16*>(p.krot);
    auto ksrc = [&](int kb) -> const __bf16* { return (RKC && kb + kWaveKeys <= kloc) ? krc : kc; };
    const __bf16* __restrict__ vc = static_cast<const __bf16*>(p.v);
    const float2* __restrict__ TF = p.TF;
    // row n, pair i of the correction table (formed here for the
    // frequency-interpolation view, which has no table)
    auto tf = [&](int64_t n, int i) -> float2 {
        if constexpr (FI) return fi_cs(p.fi_phi[i], n);
        else return TF[n * HALF + i];
    };
    const int64_t row = p.Hkv * D;
    const int64_t cache_b = PAGED ? (int64_t)g * D : (int64_t)b * p.Lmax * row + (int64_t)g * D;

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

    // the first step's K and V go out before anything else (the set-up below
    // waits on the table and q); they stay within the cache whatever the
    // table check decides
    const int wstart = (split * NW + sub) * p.wave_chunk;
    const int wend0 = min(L, wstart + p.wave_chunk);
    DecodeTile<D> cur;
    int64_t r_next = 0;   // cache row of the next step's first key
    int pg_ahead = 0;     // block-table entry of the step after next
    if (wstart < wend0) {
        const int64_t r0 = row_of(wstart);
        load_k<D>(cur, ksrc(wstart), cache_b, row, wstart, r0, wend0, colh, gq);
        load_v<D>(cur, vc, cache_b, row, wstart, r0, wend0, lane);
        if (wstart + kWaveKeys < wend0) r_next = row_of(wstart + kWaveKeys);
        if (wstart + 2 * kWaveKeys < wend0) pg_ahead = page_of(wstart + 2 * kWaveKeys);
    }

    // rotated-key cache: one wave per (batch, KV head) reads the row that the
    // next step will need as remote (its wait falls in the first step's);
    // the rotated row is stored after the key loop
    const bool write_ahead = RKC && p.rot_row >= 0 && split == 0 && sub == 0 && lane < HALF;
    float wa_x = 0.f, wa_y = 0.f;
    float2 wa_cs = make_float2(1.f, 0.f);
    int64_t wa_o = 0;
    if (write_ahead) {
        wa_o = cache_b + p.rot_row * row + lane;
        wa_x = (float)kc[wa_o];
        wa_y = (float)kc[wa_o + HALF];
        wa_cs = tf(p.rot_row - p.rot_row / G, lane);
    }

    if (tid == 0) s_bad = FI ? 0 : !table_matches(p.table, p.table_key, D, p.rope_base, p.L);
    // rows 0..32 of the table are cos/sin(dn * theta_i); only rows < L are
    // guaranteed to exist and dn <= L-1, so copy no further
    if (!RKC)
        for (int i = tid; i < min(JROWS, L) * HALF; i += kDecThreads)
            sJ[(i / HALF) * JSTR + i % HALF] = tf(i / HALF, i % HALF);
    __syncthreads();
    const bool bad = s_bad;

    const bool hvalid = colh < R;
    const int head = g * R + (hvalid ? colh : 0);

    // ---- query: stored fragments and the corrected view ---------------------
    // B operand of S^T = K Q^T: fragment c holds dims 32c + 8gq + [0, 8).  The
    // corrected view R(-n_q) q is kept in bf16 (the MFMA operand precision).
    bf16x8 qf[NC], qrem[NC];
    {
        const __bf16* qp = static_cast<const __bf16*>(p.q) + ((int64_t)b * Hq + head) * D;
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
    __bf16* myV = sVt[wave];
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
    if (!RKC && G > 1 && wstart < wend && wstart < kloc) rotate_query(wstart);

    // One register tile (loaded above): each part is reloaded for the next
    // step as soon as this step has consumed it (V after its transpose, each
    // 16-key half of K after its scores), so loads stay in flight during the
    // compute.
    for (int kbase = wstart; kbase < wend; kbase += kWaveKeys) {
        const int knext = kbase + kWaveKeys;
        // ---- V rows -> V^T in this wave's LDS slice --------------------------
        {
            const int dg = lane % (D / 8);
            const int kg = lane / (D / 8);
            wave_lds_sync();   // previous iteration's V^T reads are done
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                VW w;
#pragma unroll
                for (int e = 0; e < KPL; ++e) w[e] = cur.v[e][d];
                *reinterpret_cast<VW*>(&myV[(dg * 8 + d) * VSTR + kg * KPL]) = w;
            }
        }
        // V registers are free: start the next step's V loads
        if (knext < wend) load_v<D>(cur, vc, cache_b, row, knext, r_next, wend, lane);

        const bool w_loc = (G == 1) || (kbase + kWaveKeys - 1 >= kloc);
        const bool w_rem = (G > 1) && (kbase < kloc);

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
                if (w_loc) load_k_blk<D>(cur, krc, cache_b, row, kbase, kbase, wend, colh, gq, blk);
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
                s[blk][i] = kk < wend ? v * scale2 : -INFINITY;
            }
            // this half's K registers are free: start the next step's loads
            if (knext < wend) load_k_blk<D>(cur, ksrc(knext), cache_b, row, knext, r_next, wend, colh, gq, blk);
        }

        // ---- online softmax per head column: 8 values here, 4 quads per head --
        float mx = -INFINITY;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[blk][i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);   // finite: key kbase is valid
        const float alpha = fast_exp2(m_run - m_new);
        float ls = 0.f;
        bf16x8 Bp;
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pv = fast_exp2(s[blk][i] - m_new);
                ls += pv;
                Bp[4 * blk + i] = (__bf16)pv;
            }
        l_run = l_run * alpha + ls;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] *= alpha;

        // ---- O^T += V^T P^T ------------------------------------------------------
        wave_lds_sync();   // V^T written by the other lanes of this wave
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const bf16x8 A = *reinterpret_cast<const bf16x8*>(&myV[(16 * db + colh) * VSTR + 8 * gq]);
            acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bp, acc[db], 0, 0, 0);
        }
        if (!RKC && w_rem && knext < wend && lane < HALF) {
            const int step = (knext - knext / G) - nb;   // 0 <= step <= 32, step < L
            const float2 j2 = sJ[step * JSTR + lane];
            base = make_float2(base.x * j2.x - base.y * j2.y, base.y * j2.x + base.x * j2.y);
        }
        // the next step's corrected query, computed here so that it is off the
        // path from K's arrival to the next K loads
        if (!RKC && G > 1 && knext < wend && knext < kloc) rotate_query(knext);
        // rows of the step after next (its table entry was read a step ago);
        // then the table entry of the step after that
        r_next = knext + kWaveKeys < wend ? row_in(pg_ahead, knext + kWaveKeys) : 0;
        if (PAGED && knext + 2 * kWaveKeys < wend) pg_ahead = page_of(knext + 2 * kWaveKeys);
    }
    if (bad_page) l_run = NAN;   // poisons this head's output through the merge
    if (write_ahead) {
        // a table that does not match the call leaves NaN in the cache, so
        // later steps stay visibly wrong until the caller resets its state
        if (bad) wa_x = wa_y = NAN;
        else rotate_back(wa_x, wa_y, wa_cs);
        __bf16* kw = static_cast<__bf16*>(const_cast<void*>(p.krot));
        kw[wa_o] = (__bf16)wa_x;
        kw[wa_o + HALF] = (__bf16)wa_y;
    }

    // ---- merge the NW waves of each head, write this split's partials -------
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
    __syncthreads();   // every wave is done with its V^T slice
    float* s_acc = reinterpret_cast<float*>(&sVt[0][0]);   // [wave][16 heads][D]
    if (gq == 0) {
        s_m[wave][colh] = m_run;
        s_l[wave][colh] = l_tot;
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_acc[(wave * 16 + colh) * D + 16 * db + 4 * gq + i] = acc[db][i];
    __syncthreads();
    for (int idx = tid; idx < WH * R * D; idx += kDecThreads) {
        const int hx = idx / (R * D), r = (idx / D) % R, d = idx % D;
        float M = -INFINITY;
        for (int u = 0; u < NW; ++u) M = fmaxf(M, s_m[u * WH + hx][r]);
        float a = 0.f, l = 0.f;
        if (!bad) {
            for (int u = 0; u < NW; ++u) {
                const int w = u * WH + hx;
                const float m = s_m[w][r];
                const float f = (m == -INFINITY) ? 0.f : fast_exp2(m - M);   // waves without keys
                a += f * s_acc[(w * 16 + r) * D + d];
                l += f * s_l[w][r];
            }
        } else {
            a = l = M = NAN;
        }
        const int hq = (blockIdx.y * WH + hx) * R + r;
        float* o = p.ws + (((int64_t)b * Hq + hq) * p.n_split + split) * (D + 2);
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
    const int b = blockIdx.y;
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int ns = p.n_split;
    const float* base = p.ws + ((int64_t)b * p.Hq + head) * ns * (D + 2);
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
        const int64_t o = ((int64_t)b * p.Hq + head) * D + d;
        if constexpr (OUT_BF16) static_cast<__bf16*>(p.out)[o] = (__bf16)(t / lt);
        else static_cast<float*>(p.out)[o] = t / lt;
        if (blockIdx.z == 0 && tid == 0 && p.lse) p.lse[(int64_t)b * p.Hq + head] = (sM + log2f(lt)) * 0.69314718055994531f;
    }
}

template <int D, bool OUT_BF16>
hipError_t launch_dec(const DecodeParams& p, hipStream_t stream) {
    const dim3 grid(p.n_split, p.Hkv / p.heads_per_wg, p.B);
    if (p.block_table)
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
    hipLaunchKernelGGL((decode_combine_kernel<D, OUT_BF16>), dim3(p.Hq, p.B, D / kCombDims), dim3(kCombThreads), 0,
                       stream, p);
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
    const float4* cs = reinterpret_cast<const float4*>(TF + n * HALF + 8 * c);
    bf16x8 xo, yo;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const float4 c4 = cs[e];
        float x0 = (float)x[2 * e], y0 = (float)y[2 * e];
        float x1 = (float)x[2 * e + 1], y1 = (float)y[2 * e + 1];
        rotate_back(x0, y0, make_float2(c4.x, c4.y));
        rotate_back(x1, y1, make_float2(c4.z, c4.w));
        xo[2 * e] = (__bf16)x0;
        yo[2 * e] = (__bf16)y0;
        xo[2 * e + 1] = (__bf16)x1;
        yo[2 * e + 1] = (__bf16)y1;
    }
    if (!table_matches(table, key, D, rope_base, L)) {
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

hipError_t launch_decode(const DecodeParams& p, int out_dtype, hipStream_t stream) {
    const bool ob = out_dtype == 1;
    if (p.head_dim == 128) return ob ? launch_dec<128, true>(p, stream) : launch_dec<128, false>(p, stream);
    return ob ? launch_dec<64, true>(p, stream) : launch_dec<64, false>(p, stream);
}

}  // namespace jl
