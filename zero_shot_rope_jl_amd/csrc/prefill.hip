// Causal GQA bifocal-attention prefill for gfx950, generic kernel (serves
// fp32 inputs and the overflow fixup of bf16 calls; bf16 inputs go to the
// kernel of prefill_bf16.hip).  Like that kernel it also runs the three
// separate passes of the unfused form (PrefillParams::mode).
//
// Method (Jet-Long, §3 Eq. 1; §3.1 Eqs. 2-3; §3.2 Eq. 5; §3.3 Eq. 6): a
// query/key pair with q - k <= w0 scores with the stored RoPE vectors; a pair
// with q - k > w0 scores with both vectors rotated by their correction offset
// f(p) - p, f(p) = floor(p/G).  Both views feed one online softmax per query
// row, which realises the inclusion-exclusion merge exactly (the overlap term
// is removed by masking, not subtracted).
//
// Work decomposition
//   workgroup = 8 waves = 256 query rows = R query heads x (256/R) positions
//               of one KV head; wave = 32 positions of one query head.
//   The workgroup walks its key tiles (64 keys) in two phases: a remote
//   phase over every tile that holds a remote pair, with K rotated by its
//   correction on the global->LDS path and Q held in its corrected view, then
//   a local phase over every tile that holds a local pair, with stored K and
//   Q.  A tile that straddles the window edge is visited once per phase under
//   a mask, so only one Q view is ever live in registers and every other
//   tile runs without per-element masking.
//   Pipeline: LDS is double-buffered; the next tile's K, V and correction
//   rows are loaded into registers before the current tile's MFMAs and
//   written (K rotated where needed) to the other buffer after them, so one
//   barrier per tile suffices.  V stays row-major in LDS; the PV MFMA reads
//   its V^T operand with the transposing LDS load (ds_read_b64_tr_b16).
//   Each wave computes S^T = K Q^T with MFMA (keys on the M axis, queries on
//   N), so a query's 64 scores sit in one lane pair: the row max needs one
//   cross-half exchange and the row sum none until the end.  P^T is already
//   in the B-operand layout of O^T += V^T P^T.  The running max is only
//   raised (and the accumulator rescaled) when a tile's max exceeds it by
//   more than 2^8, which keeps every probability below 256.
#include <limits.h>
#include <math.h>

#include <type_traits>

#include "internal.h"

namespace jl {

namespace {

constexpr int kThreads = 512;
constexpr int BN = 64;                  // keys per tile
constexpr float kRescaleSlack = 8.0f;   // log2 units

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// ds_read_b64_tr_b16: within each 16-lane group, lane i receives element i%4
// of the 8-byte rows supplied by lanes i/4, i/4+4, i/4+8 and i/4+12.
__device__ inline bf16x4 lds_read_tr16(const __bf16* p) {
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

template <bool BF16> struct Elem;
template <> struct Elem<true> { using T = __bf16; };
template <> struct Elem<false> { using T = float; };

template <int D, bool BF16>
struct PrefillLayout {
    static constexpr int HALF = D / 2;
    static constexpr int KSTR = BF16 ? D + 8 : D + 4;      // K row stride (elements)
    // V rows [key][d]; bf16 rows are padded by 64 bytes so that the transposed
    // reads of 8 key rows spread over all LDS banks
    static constexpr int VSTR = BF16 ? D + 32 : D + 4;
    static constexpr int K_ELEMS = BN * KSTR;
    static constexpr int V_ELEMS = BN * VSTR;
    static constexpr int PPT = HALF * BN / kThreads;        // rotation pairs per thread
    static constexpr int NQ = BF16 ? D / 16 : D / 8;        // Q fragments per lane
    static constexpr int VPT = D / 8;                       // V elements per thread (8 threads per row)
};

// Registers holding one tile on its way from HBM to LDS.
template <int D, bool BF16>
struct Stage {
    using Lay = PrefillLayout<D, BF16>;
    using T = typename Elem<BF16>::T;
    typedef T KV __attribute__((ext_vector_type(Lay::PPT)));
    typedef T VV __attribute__((ext_vector_type(Lay::VPT)));
    KV x, y;                      // pair halves: dims f0.. and HALF + f0..
    float4 cs[Lay::PPT / 2];      // correction (cos, sin) of the pairs (remote view)
    VV v;                         // one row segment of V
};

// Query fragments (B operand of S^T = K Q^T).  bf16: fragment c holds dims
// 16c + 8hh + [0, 8); f32: fragment t holds dims 8t + 4hh + [0, 4).  Partner
// dims (+D/2) sit in fragment c + NQ/2.  The remote view rotates each pair by
// the query's correction offset.
template <int D, bool BF16, typename QF, typename T>
__device__ __forceinline__ void load_q_frags(QF* qv, const T* __restrict__ qrow, bool ok, bool remote_view,
                                             const float2* __restrict__ TF, int64_t nq, int hh) {
    using Lay = PrefillLayout<D, BF16>;
    constexpr int NQ = Lay::NQ;
    constexpr int W = BF16 ? 8 : 4;
#pragma unroll
    for (int c = 0; c < NQ; ++c) qv[c] = ok ? *reinterpret_cast<const QF*>(qrow + c * 2 * W + W * hh) : QF{};
    if (remote_view) {
#pragma unroll
        for (int c = 0; c < NQ / 2; ++c)
#pragma unroll
            for (int j = 0; j < W; ++j) {
                float x = (float)qv[c][j];
                float y = (float)qv[c + NQ / 2][j];
                rotate_back(x, y, table_cs(TF, Lay::HALF, nq, c * 2 * W + W * hh + j));
                qv[c][j] = (T)x;
                qv[c + NQ / 2][j] = (T)y;
            }
    }
}

// One 64-key tile for one wave: S^T = K Q^T for the two 32-key blocks, the
// optional window/causal mask (keys outside [rlo, rhi] relative to the lane's
// first key), the online-softmax update and O^T += V^T P^T.
template <int D, bool BF16, typename QF, typename T>
__device__ __forceinline__ void tile_step(const T* __restrict__ K, const T* __restrict__ V, const QF* qv,
                                          f32x16* acc, float& m_run, float& l_run, int col, int hh, int lane,
                                          bool masked, int rlo, int rhi, float scale2) {
    using Lay = PrefillLayout<D, BF16>;
    constexpr int NQ = Lay::NQ;
    constexpr int KSTR = Lay::KSTR;
    constexpr int VSTR = Lay::VSTR;
    constexpr int NDB = D / 32;

    f32x16 s0 = f32x16{}, s1 = f32x16{};
    if constexpr (BF16) {
        // A-operand row `col` holds key sigma(col) of each 32-key block; sigma
        // makes the C rows land so that P^T feeds the PV MFMA in natural order.
        const int a3 = col >> 3, hp = (col >> 2) & 1, e = col & 3;
        const int krow = 16 * (a3 >> 1) + 8 * hp + 4 * (a3 & 1) + e;
        const T* k0p = K + krow * KSTR + 8 * hh;
        const T* k1p = k0p + 32 * KSTR;
        // two-deep register pipeline for the K fragments: the reads for
        // chunk c+1 are in flight while chunk c's MFMAs issue
        bf16x8 A0 = *reinterpret_cast<const bf16x8*>(k0p);
        bf16x8 A1 = *reinterpret_cast<const bf16x8*>(k1p);
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            bf16x8 B0, B1;
            if (c + 1 < NQ) {
                B0 = *reinterpret_cast<const bf16x8*>(k0p + 16 * (c + 1));
                B1 = *reinterpret_cast<const bf16x8*>(k1p + 16 * (c + 1));
            }
            s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A0, qv[c], s0, 0, 0, 0);
            s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, qv[c], s1, 0, 0, 0);
            if (c + 1 < NQ) {
                A0 = B0;
                A1 = B1;
            }
        }
    } else {
        const T* k0p = K + col * KSTR + 4 * hh;
        const T* k1p = k0p + 32 * KSTR;
#pragma unroll
        for (int t = 0; t < NQ; ++t) {
            const f32x4 A0 = *reinterpret_cast<const f32x4*>(k0p + 8 * t);
            const f32x4 A1 = *reinterpret_cast<const f32x4*>(k1p + 8 * t);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                s0 = __builtin_amdgcn_mfma_f32_32x32x2f32(A0[e], qv[t][e], s0, 0, 0, 0);
                s1 = __builtin_amdgcn_mfma_f32_32x32x2f32(A1[e], qv[t][e], s1, 0, 0, 0);
            }
        }
    }
    if (masked) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int c0 = BF16 ? 16 * (i >> 3) + (i & 7) : (i >> 2) * 8 + (i & 3);
            s0[i] = ((c0 >= rlo) & (c0 <= rhi)) ? s0[i] : -INFINITY;
            s1[i] = ((c0 + 32 >= rlo) & (c0 + 32 <= rhi)) ? s1[i] : -INFINITY;
        }
    }

    // ---- online softmax (base 2, lazily rescaled) ---------------------------
    float mx = s0[0];
#pragma unroll
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s0[i]);
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s1[i]);
    mx = wave_max_xor32(mx) * scale2;
    const bool raise = mx > m_run + kRescaleSlack;
    if (__any(raise)) {
        const float m_new = raise ? mx : m_run;
        const float alpha = raise ? fast_exp2(m_run - m_new) : 1.f;   // 0 when m_run = -inf
        l_run *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
        m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.f : m_run;   // rows with no key yet
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        s0[i] = fast_exp2(fmaf(s0[i], scale2, -m_use));
        s1[i] = fast_exp2(fmaf(s1[i], scale2, -m_use));
    }

    // ---- O^T += V^T P^T ------------------------------------------------------
    if constexpr (BF16) {
        // A operand (V^T: rows = dims, k = keys) from row-major V through the
        // transposing LDS read: within each 16-lane group, lane c supplies 4
        // dims of one key row and lane i receives dim i of 4 key rows.
        const int Gq = lane >> 4, cq = lane & 15;
        const T* vbase = V + (8 * (Gq >> 1) + (cq >> 2)) * VSTR + 16 * (Gq & 1) + 4 * (cq & 3);
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        float lsum0 = 0.f, lsum1 = 0.f;
#pragma unroll
        for (int kc = 0; kc < 4; ++kc) {
            const f32x16& sp = (kc < 2) ? s0 : s1;
            const int o = 8 * (kc & 1);
            bf16x8 Bp;
#pragma unroll
            for (int j = 0; j < 8; ++j) Bp[j] = (__bf16)sp[o + j];
            // row sums of the probabilities as rounded for the MFMA
#pragma unroll
            for (int j = 0; j < 4; j += 2) {
                lsum0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{Bp[2 * j], Bp[2 * j + 1]}, ones, lsum0, false);
                lsum1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{Bp[2 * j + 2], Bp[2 * j + 3]}, ones, lsum1, false);
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const T* vp = vbase + 16 * kc * VSTR + 32 * db;
                const bf16x4 lo = lds_read_tr16(vp);
                const bf16x4 hi = lds_read_tr16(vp + 4 * VSTR);
                const bf16x8 A = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bp, acc[db], 0, 0, 0);
            }
        }
        l_run += lsum0 + lsum1;
    } else {
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const f32x16& sp = kb ? s1 : s0;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                ls += sp[i];
                const int key = 32 * kb + (i >> 2) * 8 + hh * 4 + (i & 3);
#pragma unroll
                for (int db = 0; db < NDB; ++db)
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(V[key * VSTR + db * 32 + col], sp[i], acc[db], 0,
                                                                   0, 0);
            }
        }
        l_run += ls;
    }
}

template <int D, bool BF16, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void prefill_kernel(PrefillParams p) {
    using Lay = PrefillLayout<D, BF16>;
    using T = typename Elem<BF16>::T;
    constexpr int HALF = Lay::HALF;
    constexpr int KSTR = Lay::KSTR;
    constexpr int VSTR = Lay::VSTR;
    constexpr int PPT = Lay::PPT;
    constexpr int NQ = Lay::NQ;
    constexpr int NDB = D / 32;   // 32-dim blocks of O^T
    using St = Stage<D, BF16>;
    using QF = typename std::conditional<BF16, bf16x8, f32x4>::type;

    __shared__ __attribute__((aligned(16))) T sK[2][Lay::K_ELEMS];
    __shared__ __attribute__((aligned(16))) T sV[2][Lay::V_ELEMS];
    __shared__ int s_bad;
    __shared__ int s_marked;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave index through readfirstlane: everything derived from it (rows,
    // tile classes, masks) is wave-uniform and branches on it are scalar
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hh = lane >> 5;      // lane half
    const int col = lane & 31;     // query column of the S^T / O^T tiles

    // Heads vary fastest over the grid so that the workgroups of one KV head
    // land on one XCD (dispatch is round-robin over the 8 XCDs) and share its
    // L2; query tiles are issued longest (last) first.
    int bid = blockIdx.x;
    const int g = (int)(bid % p.Hkv);
    bid /= (int)p.Hkv;
    const int b = (int)(bid % p.B);
    bid /= (int)p.B;
    const int qt = p.n_qtiles - 1 - bid;

    // positions: keys 0..L-1; queries q_off..L-1, stored as rows 0..Lq-1
    const int L = (int)p.L;
    const int Lq = (int)p.Lq;
    const int q_off = (int)p.q_off;
    const int64_t Lkv = p.Lkv;   // rows per batch entry of k and v
    const int Hq = (int)p.Hq;
    const int Hkv = (int)p.Hkv;
    const int G = (int)p.G;
    const int w0 = (int)p.w0;
    const int R = p.R;
    const int r = wave % R;
    const int pb = wave / R;
    const int head = g * R + r;
    const int q0 = q_off + qt * p.BQ;
    const int q_hi = min(q0 + p.BQ, L) - 1;
    const int p0 = q0 + pb * 32;
    const int p_hi = min(p0 + 31, L - 1);
    const int my_q = p0 + col;
    const bool wave_active = p0 < L;
    const float scale2 = p.sm_scale_log2;

    const T* __restrict__ qg = static_cast<const T*>(p.q);
    const T* __restrict__ kg = static_cast<const T*>(p.k);
    const T* __restrict__ vg = static_cast<const T*>(p.v);
    const float2* __restrict__ TF = p.TF;
    const int64_t kv_row = (int64_t)Hkv * D;
    const bool paged = p.block_table != nullptr;
    const int64_t kv_b = paged ? 0 : (int64_t)b * Lkv * kv_row;
    const T* __restrict__ kbase = kg + kv_b + (int64_t)g * D;
    const T* __restrict__ vbase = vg + kv_b + (int64_t)g * D;
    // Cache row of key k0 (a multiple of BN).  Paged caches: the page size is
    // a multiple of BN, so a tile lies in one page.  An entry outside
    // [0, n_pages) reads page 0 instead and this workgroup's rows are
    // written as NaN, so no load leaves the pages.
    bool bad_page = false;
    auto cache_row = [&](int k0) -> int64_t {
        if (!paged) return k0;
        const int ps = (int)p.page_size;
        int pg = p.block_table[(int64_t)b * p.max_pages + k0 / ps];
        if (pg < 0 || pg >= p.n_pages) {
            bad_page = true;
            pg = 0;
        }
        return (int64_t)pg * ps + k0 % ps;
    };

    if (p.fixup) {
        // Fixup pass: only a workgroup with a marked row (NaN in element 0)
        // recomputes; the row sets of both prefill kernels coincide.
        if (tid == 0) s_marked = 0;
        __syncthreads();
        if (tid < 256) {
            const int hq = g * R + tid / p.BQ;
            const int pos = q0 + tid % p.BQ;
            if (pos < L) {
                const int64_t o = (((int64_t)b * Lq + (pos - q_off)) * Hq + hq) * D;
                const float e0 = OUT_BF16 ? (float)static_cast<const __bf16*>(p.out)[o]
                                          : static_cast<const float*>(p.out)[o];
                if (e0 != e0) s_marked = 1;
            }
        }
        __syncthreads();
        if (!s_marked) return;
    }
    if (tid == 0) {
        const TableHeader* th = p.table;
        s_bad = !table_matches(th, p.table_key, D, p.rope_base, table_need(p.L, p.G));
    }
    __syncthreads();
    if (s_bad) {
        // The table does not belong to this (D, rope_base, L): poison the output.
        if (wave_active && my_q < L) {
            const int64_t o = (((int64_t)b * Lq + (my_q - q_off)) * Hq + head) * D;
            for (int d = hh; d < D; d += 2) {
                if constexpr (OUT_BF16) static_cast<__bf16*>(p.out)[o + d] = (__bf16)NAN;
                else static_cast<float*>(p.out)[o + d] = NAN;
            }
            if (hh == 0 && p.lse) p.lse[((int64_t)b * Hq + head) * Lq + (my_q - q_off)] = NAN;
        }
        return;
    }

    // ---- pass schedule (uniform over the workgroup) -------------------------
    // tile kt covers keys [64kt, 64kt + 63]; the last one is padded with zero
    // rows beyond L, which every mask below excludes.
    // The corrected-view phase walks tiles r0 .. r0 + nR - 1, then the
    // stored-view phase tiles nL0 .. nkt - 1.
    const int nkt = q_hi / BN + 1;
    const int mode = p.mode;
    int nR = 0;    // fused: tiles [0, nR) hold a pair with q - k > w0
    int nL0 = 0;   // fused: tiles [nL0, nkt) hold a pair with 0 <= q - k <= w0
    int r0 = 0;
    // first tile holding a key of some row's window [q - w0, q]
    const int win0 = q0 - w0 - (BN - 1) > 0 ? (q0 - w0) / BN : 0;
    if (mode == kFused) {
        if (G > 1) {
            nR = q_hi - w0 > 0 ? min(nkt, (q_hi - w0 + BN - 1) / BN) : 0;
            nL0 = win0;
        }
    } else if (mode == kLocalWindow) {
        nL0 = win0;
    } else if (mode == kRemoteAll) {
        nR = nkt;
        nL0 = nkt;
    } else {
        r0 = win0;
        nR = nkt - win0;
        nL0 = nkt;
    }
    const int NP = nR + (nkt - nL0);

    const bool q_ok = wave_active && my_q < L;
    const T* qrow = qg + (((int64_t)b * Lq + (q_ok ? my_q - q_off : 0)) * Hq + head) * D;
    QF qv[NQ];
    load_q_frags<D, BF16>(qv, qrow, q_ok, nR > 0, TF, q_ok ? (int64_t)(my_q - my_q / G) : 0, hh);

    // ---- staging of one tile: HBM -> registers -> LDS -----------------------
    St st;
    const int kr = tid >> 3;             // key row of this thread
    const int f0 = (tid & 7) * PPT;      // K: first frequency of this thread
    const int v0 = (tid & 7) * Lay::VPT; // V: first dim of this thread
    auto pass_k0 = [&](int pi) { return (pi < nR ? r0 + pi : nL0 + (pi - nR)) * BN; };
    auto stage_load = [&](int pi) {
        const int tk0 = pass_k0(pi);
        const int kpos = tk0 + kr;
        const bool ok = kpos < L;
        // the tile's first key is below L, so its row exists; rows past L
        // read that row and are zeroed below
        const int64_t trow = cache_row(tk0);
        const int64_t crow = ok ? trow + kr : trow;
        const T* krow = kbase + crow * kv_row;
        const T* vrow = vbase + crow * kv_row;
        st.x = ok ? *reinterpret_cast<const typename St::KV*>(krow + f0) : typename St::KV{};
        st.y = ok ? *reinterpret_cast<const typename St::KV*>(krow + HALF + f0) : typename St::KV{};
        st.v = ok ? *reinterpret_cast<const typename St::VV*>(vrow + v0) : typename St::VV{};
        if (pi < nR) {
            const int64_t n = ok ? kpos - kpos / G : 0;
#pragma unroll
            for (int j = 0; j < PPT / 2; ++j) st.cs[j] = table_cs2(TF, HALF, n, f0 + 2 * j);
        }
    };
    auto stage_store = [&](int pi, int buf) {
        T* Kd = sK[buf] + kr * KSTR + f0;
        if (pi < nR) {
            typename St::KV xr, yr;
#pragma unroll
            for (int j = 0; j < PPT; ++j) {
                const float4 c4 = st.cs[j >> 1];
                const float2 cs = (j & 1) ? make_float2(c4.z, c4.w) : make_float2(c4.x, c4.y);
                float x = (float)st.x[j], y = (float)st.y[j];
                rotate_back(x, y, cs);
                xr[j] = (T)x;
                yr[j] = (T)y;
            }
            *reinterpret_cast<typename St::KV*>(Kd) = xr;
            *reinterpret_cast<typename St::KV*>(Kd + HALF) = yr;
        } else {
            *reinterpret_cast<typename St::KV*>(Kd) = st.x;
            *reinterpret_cast<typename St::KV*>(Kd + HALF) = st.y;
        }
        *reinterpret_cast<typename St::VV*>(&sV[buf][kr * VSTR + v0]) = st.v;
    };

    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
    float m_run = -INFINITY;
    float l_run = 0.f;

    // ---- software pipeline over the passes --------------------------------------
    stage_load(0);
    stage_store(0, 0);
    __syncthreads();
    for (int pi = 0; pi < NP; ++pi) {
        const int buf = pi & 1;
        if (pi + 1 < NP) stage_load(pi + 1);
        if (pi == nR && nR > 0) load_q_frags<D, BF16>(qv, qrow, q_ok, false, TF, 0, hh);   // local view
        if (wave_active) {
            const bool rem = pi < nR;
            const int k0 = pass_k0(pi);
            const int k1 = k0 + BN - 1;
            bool act, masked;
            int klo, khi;
            if (mode == kFused) {
                if (rem) {
                    act = p_hi - k0 > w0;
                    masked = p0 - k1 <= w0;                          // some local pair here
                } else {
                    act = k0 <= p_hi && (G == 1 || p0 - k1 <= w0);
                    masked = k1 > p0 || (G > 1 && p_hi - k0 > w0);  // causal edge or remote pairs
                }
                // masked tiles keep keys in [klo, khi]: the remote view keeps
                // q - k > w0, the local view 0 <= q - k <= w0 (no lower bound
                // if G == 1)
                klo = (rem || G == 1) ? INT_MIN / 2 : my_q - w0;
                khi = rem ? my_q - w0 - 1 : my_q;
            } else {
                // one pass of the merge: keys [q - w0, q], or every k <= q
                const bool all = mode == kRemoteAll;
                act = k0 <= p_hi && (all || p0 - k1 <= w0);
                masked = k1 > p0 || (!all && p_hi - k0 > w0);
                klo = all ? INT_MIN / 2 : my_q - w0;
                khi = my_q;
            }
            if (act) {
                const int off = k0 + (BF16 ? 8 * hh : 4 * hh);
                tile_step<D, BF16>(sK[buf], sV[buf], qv, acc, m_run, l_run, col, hh, lane, masked, klo - off,
                                   khi - off, scale2);
            }
        }
        if (pi + 1 < NP) stage_store(pi + 1, buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue ---------------------------------------------------------------
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (q_ok) {
        const float inv = bad_page ? NAN : 1.f / l_tot;
        const int64_t o = (((int64_t)b * Lq + (my_q - q_off)) * Hq + head) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int d0 = db * 32 + a4 * 8 + hh * 4;
                if constexpr (OUT_BF16) {
                    bf16x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[db][4 * a4 + e] * inv);
                    *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(p.out) + o + d0) = w;
                } else {
                    f32x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = acc[db][4 * a4 + e] * inv;
                    *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + o + d0) = w;
                }
            }
        }
        if (hh == 0 && p.lse)
            p.lse[((int64_t)b * Hq + head) * Lq + (my_q - q_off)] =
                bad_page ? NAN : (m_run + log2f(l_tot)) * 0.69314718055994531f;
    }
}

template <int D, bool BF16, bool OUT_BF16>
hipError_t launch_one(const PrefillParams& p, hipStream_t stream) {
    const int64_t blocks = (int64_t)p.n_qtiles * p.Hkv * p.B;
    hipLaunchKernelGGL((prefill_kernel<D, BF16, OUT_BF16>), dim3((unsigned)blocks), dim3(kThreads), 0,
                       stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const PrefillParams& p, int in_dtype, int out_dtype, hipStream_t stream) {
    if (in_dtype == 1) {
        // bf16 inputs: the kernel of prefill_bf16.hip, then the fixup pass that
        // recomputes (with the online softmax here) any workgroup whose rows
        // it marked as non-finite; the pass exits at once when none is marked.
        const hipError_t e = launch_prefill_bf16(p, out_dtype, stream);
        if (e != hipSuccess) return e;
        PrefillParams pf = p;
        pf.fixup = 1;
        const bool ob = out_dtype == 1;
        if (p.head_dim == 128) return ob ? launch_one<128, true, true>(pf, stream) : launch_one<128, true, false>(pf, stream);
        return ob ? launch_one<64, true, true>(pf, stream) : launch_one<64, true, false>(pf, stream);
    }
    (void)out_dtype;
    if (p.head_dim == 128) return launch_one<128, false, false>(p, stream);
    return launch_one<64, false, false>(p, stream);
}

}  // namespace jl
