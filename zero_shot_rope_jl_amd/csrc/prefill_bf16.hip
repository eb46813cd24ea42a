// Causal GQA bifocal-attention prefill for gfx950, bf16 inputs.
//
// Method (Jet-Long, §3 Eq. 1; §3.1 Eqs. 2-3; §3.2 Eq. 5; §3.3 Eq. 6): a
// query/key pair with q - k <= w0 scores with the stored RoPE vectors; a pair
// with q - k > w0 scores with both vectors rotated by their correction offset
// f(p) - p, f(p) = floor(p/G).  Both views feed one online softmax per query
// row, which realises the inclusion-exclusion merge exactly (the overlap term
// is removed by masking, not subtracted).
//
// Work decomposition (one workgroup = 4 waves = 256 query rows of one KV head)
//   Rows are ordered head-major over the R = Hq/Hkv query heads of the KV
//   head and BQ = 256/R positions; wave w owns rows [64w, 64w + 64) as two
//   32-row query blocks.  Every K or V^T fragment read from LDS feeds the
//   MFMAs of both blocks, which halves LDS traffic per flop: with 32x32x16
//   bf16 MFMAs a single block would need the whole LDS read bandwidth of a
//   compute unit.  One wave per SIMD; the output accumulators live in AGPRs.
//
//   Key tiles of 64 are walked in two phases: a remote phase over every tile
//   that holds a remote pair (K rotated by its correction on the way into
//   LDS, Q in its corrected view), then a local phase over every tile that
//   holds a local pair (stored K and Q).  A tile that straddles the window
//   edge is visited once per phase under a mask.
//
//   Pipeline: LDS is double-buffered.  At the start of a tile the next tile's
//   V is streamed HBM -> LDS with global_load_lds (no registers; 16-byte
//   chunks XOR-swizzled by row so that the transposed reads below spread over
//   the LDS banks) and its K and correction rows are loaded into registers;
//   after the MFMAs K is rotated (remote view) and written to LDS.  One
//   barrier per tile.
//
//   Each wave computes S^T = K Q^T (keys on the MFMA M axis, queries on N):
//   a query's 64 scores sit in one lane pair, so the row max needs one
//   cross-half exchange and P^T is already the B operand of O^T += V^T P^T,
//   whose V^T operand comes from row-major V through ds_read_b64_tr_b16.
//   The running max is raised (and the accumulator rescaled) only when a
//   tile's max exceeds it by more than 2^8.
#include <limits.h>
#include <math.h>

#include "internal.h"

namespace jl {

namespace {

constexpr int kWaves = 4;
constexpr int kThreads = kWaves * 64;
constexpr int BN = 64;                  // keys per tile
constexpr float kRescaleSlack = 8.0f;   // log2 units

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ inline bf16x4 lds_read_tr16(const __bf16* p) {
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(p));
}

// 16-byte HBM -> LDS copy per lane; lane l writes bytes [16l, 16l + 16) after
// the wave-uniform LDS base.
__device__ inline void load_lds16(const void* src, void* lds_base) {
    __builtin_amdgcn_global_load_lds((__attribute__((address_space(1))) void*)(src),
                                     (__attribute__((address_space(3))) void*)(lds_base), 16, 0, 0);
}

__device__ inline void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// acc *= alpha in place in the accumulation registers.  Written out so that
// the compiler never keeps a VGPR copy of the accumulators for the (rare)
// rescale; the trailing nops cover an MFMA that reads the result next.
__device__ inline void scale_acc(f32x16& acc, float alpha) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float x = acc[i];
        float t;
        asm volatile(
            "v_accvgpr_read_b32 %1, %0\n\t"
            "v_mul_f32 %1, %1, %2\n\t"
            "v_accvgpr_write_b32 %0, %1"
            : "+a"(x), "=&v"(t)
            : "v"(alpha));
        acc[i] = x;
    }
    asm volatile("s_nop 2");
}

template <int D>
struct Lay5 {
    static constexpr int HALF = D / 2;
    static constexpr int NC = D / 16;           // 16-dim K chunks (MFMA k)
    static constexpr int NDB = D / 32;          // 32-dim O^T blocks
    static constexpr int KSTR = D + 8;          // K row stride (elements), padded
    static constexpr int CH = D / 8;            // 16-byte chunks per V row
    static constexpr int PPT = HALF * BN / kThreads;   // K pairs per thread
    static constexpr int TPR = kThreads / BN;          // threads per K row
};

// physical 16-byte chunk of logical chunk `c` in V row `row`
template <int D>
__device__ inline int vswz(int row, int c) {
    return c ^ ((4 * (row & 3)) & (Lay5<D>::CH - 1));
}

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(PrefillParams p) {
    using Lay = Lay5<D>;
    constexpr int HALF = Lay::HALF;
    constexpr int NC = Lay::NC;
    constexpr int NDB = Lay::NDB;
    constexpr int KSTR = Lay::KSTR;
    constexpr int CH = Lay::CH;
    constexpr int PPT = Lay::PPT;
    typedef __bf16 KV __attribute__((ext_vector_type(PPT)));

    __shared__ __attribute__((aligned(16))) __bf16 sK[2][BN * KSTR];
    __shared__ __attribute__((aligned(16))) __bf16 sV[2][BN * D];
    __shared__ int s_bad;

    // Naming an accumulation register keeps the compiler from assuming the
    // kernel needs none; it then gives the MFMAs their accumulation-register
    // form and the output accumulators stay out of the VGPR budget.
    asm volatile("" ::: "a255");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
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

    const int L = (int)p.L;
    const int Hq = (int)p.Hq;
    const int Hkv = (int)p.Hkv;
    const int G = (int)p.G;
    const int w0 = (int)p.w0;
    const int R = p.R;
    const int BQ = p.BQ;
    const int q0 = qt * BQ;
    const int q_hi = min(q0 + BQ, L) - 1;
    const float scale2 = p.sm_scale_log2;

    // the wave's two 32-row query blocks
    int head[2], pj0[2], pjhi[2], my_q[2];
    bool qok[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int rho = 64 * wave + 32 * j;
        head[j] = g * R + rho / BQ;
        pj0[j] = q0 + rho % BQ;
        pjhi[j] = min(pj0[j] + 31, L - 1);
        my_q[j] = pj0[j] + col;
        qok[j] = my_q[j] < L;
    }

    const __bf16* __restrict__ qg = static_cast<const __bf16*>(p.q);
    const float2* __restrict__ TF = p.TF;
    const int64_t kv_row = (int64_t)Hkv * D;
    const __bf16* __restrict__ kbase = static_cast<const __bf16*>(p.k) + (int64_t)b * L * kv_row + (int64_t)g * D;
    const __bf16* __restrict__ vbase = static_cast<const __bf16*>(p.v) + (int64_t)b * L * kv_row + (int64_t)g * D;

    if (tid == 0) {
        const TableHeader* th = p.table;
        s_bad = !(th->magic == kTableMagic && th->head_dim == D && th->rope_base == p.rope_base &&
                  th->n_cover >= p.L);
    }
    __syncthreads();
    if (s_bad) {
        // The table does not belong to this (D, rope_base, L): poison the output.
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            if (!qok[j]) continue;
            const int64_t o = (((int64_t)b * L + my_q[j]) * Hq + head[j]) * D;
            for (int d = hh; d < D; d += 2) {
                if constexpr (OUT_BF16) static_cast<__bf16*>(p.out)[o + d] = (__bf16)NAN;
                else static_cast<float*>(p.out)[o + d] = NAN;
            }
            if (hh == 0 && p.lse) p.lse[((int64_t)b * Hq + head[j]) * L + my_q[j]] = NAN;
        }
        return;
    }

    // ---- pass schedule (uniform over the workgroup) -------------------------
    const int nkt = q_hi / BN + 1;
    int nR = 0;    // remote phase: tiles [0, nR) hold a pair with q - k > w0
    int nL0 = 0;   // local phase: tiles [nL0, nkt) hold a pair with 0 <= q - k <= w0
    if (G > 1) {
        nR = q_hi - w0 > 0 ? min(nkt, (q_hi - w0 + BN - 1) / BN) : 0;
        nL0 = q0 - w0 - (BN - 1) > 0 ? (q0 - w0) / BN : 0;
    }
    const int NP = nR + (nkt - nL0);

    // ---- query fragments: B operand, fragment c = dims 16c + 8hh + [0, 8) ----
    // Rows past L read row L-1 (finite values, never stored).
    bf16x8 qv[2][NC];
    auto load_q = [&](bool remote_view) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int qpos = min(my_q[j], L - 1);
            const __bf16* qrow = qg + (((int64_t)b * L + qpos) * Hq + head[j]) * D;
#pragma unroll
            for (int c = 0; c < NC; ++c) qv[j][c] = *reinterpret_cast<const bf16x8*>(qrow + 16 * c + 8 * hh);
            if (remote_view) {
                const int64_t nq = qpos - qpos / G;
#pragma unroll
                for (int c = 0; c < NC / 2; ++c)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float x = (float)qv[j][c][e], y = (float)qv[j][c + NC / 2][e];
                        rotate_back(x, y, TF[nq * HALF + 16 * c + 8 * hh + e]);
                        qv[j][c][e] = (__bf16)x;
                        qv[j][c + NC / 2][e] = (__bf16)y;
                    }
            }
        }
    };

    // ---- staging of the next tile ------------------------------------------------
    // Every tile is rotated on its way into LDS: remote tiles by their
    // correction rows, local tiles by table row 0, which is exactly (1, 0).
    const int kr = tid / Lay::TPR;                 // K row of this thread
    const int f0 = (tid % Lay::TPR) * PPT;         // first frequency of this thread
    KV stx, sty;
    float4 stc[PPT / 2];
    auto tile_k0 = [&](int pi) { return (pi < nR ? pi : nL0 + (pi - nR)) * BN; };
    auto stage_load = [&](int pi, int buf) {
        const int k0 = tile_k0(pi);
        // V: 64 rows x CH chunks, BN*CH/256 wave-instructions of 64 chunks each
#pragma unroll
        for (int u = 0; u < BN * CH / kThreads; ++u) {
            const int P = (u * kWaves + wave) * 64 + lane;   // physical chunk in the tile
            const int row = P / CH;
            const int lc = vswz<D>(row, P % CH);           // logical chunk stored there
            const int key = min(k0 + row, L - 1);           // rows beyond L: finite, masked out
            load_lds16(vbase + (int64_t)key * kv_row + 8 * lc, &sV[buf][(u * kWaves + wave) * 64 * 8]);
        }
        const int kpos = min(k0 + kr, L - 1);
        const __bf16* krow = kbase + (int64_t)kpos * kv_row;
        stx = *reinterpret_cast<const KV*>(krow + f0);
        sty = *reinterpret_cast<const KV*>(krow + HALF + f0);
        const int64_t tn = pi < nR ? kpos - kpos / G : 0;
        const float4* t4 = reinterpret_cast<const float4*>(TF + tn * HALF + f0);
#pragma unroll
        for (int e = 0; e < PPT / 2; ++e) stc[e] = t4[e];
    };
    auto stage_store = [&](int buf) {
        __bf16* Kd = sK[buf] + kr * KSTR + f0;
        KV xr, yr;
#pragma unroll
        for (int e = 0; e < PPT; ++e) {
            const float4 c4 = stc[e >> 1];
            const float2 cs = (e & 1) ? make_float2(c4.z, c4.w) : make_float2(c4.x, c4.y);
            float x = (float)stx[e], y = (float)sty[e];
            rotate_back(x, y, cs);
            xr[e] = (__bf16)x;
            yr[e] = (__bf16)y;
        }
        *reinterpret_cast<KV*>(Kd) = xr;
        *reinterpret_cast<KV*>(Kd + HALF) = yr;
    };

    f32x16 acc[2][NDB];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[j][db] = f32x16{};
    float m_run[2] = {-INFINITY, -INFINITY};
    float l_run[2] = {0.f, 0.f};

    // K A-operand row of this lane in each 32-key block (sigma makes the C
    // rows land so that P^T feeds the PV MFMA in natural key order)
    const int a3 = col >> 3, hp = (col >> 2) & 1, ee = col & 3;
    const int krow_l = 16 * (a3 >> 1) + 8 * hp + 4 * (a3 & 1) + ee;
    // V^T operand through the transposing read: within each 16-lane group,
    // lane c supplies 4 dims of one key row, lane i receives dim i of 4 rows
    const int Gq = lane >> 4, cq = lane & 15;
    const int tr_row = 8 * (Gq >> 1) + (cq >> 2);
    const int tr_dim = 16 * (Gq & 1) + 4 * (cq & 3);

    // One tile: S, masks, online softmax and PV for both query blocks, with
    // the next tile's staging wrapped around it.  Tiles without a kept pair
    // for a block run fully masked rather than branch.
    auto tile = [&](int pi) {
        const int buf = pi & 1;
        stage_load(pi + 1 < NP ? pi + 1 : pi, buf ^ 1);   // the last tile refills the idle buffer
        const bool rem = pi < nR;
        const int k0 = tile_k0(pi);
        const int k1 = k0 + BN - 1;
        // per query block: masked?, kept key window [rlo, rhi] relative to
        // the lane's first key k0 + 8hh
        bool msk[2];
        int rlo[2], rhi[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            bool act;
            if (rem) {
                act = pjhi[j] - k0 > w0;
                msk[j] = pj0[j] - k1 <= w0;
            } else {
                act = k0 <= pjhi[j] && (G == 1 || pj0[j] - k1 <= w0);
                msk[j] = k1 > pj0[j] || (G > 1 && pjhi[j] - k0 > w0);
            }
            act = act && pj0[j] < L;
            const int klo = (rem || G == 1) ? INT_MIN / 2 : my_q[j] - w0;
            const int khi = rem ? my_q[j] - w0 - 1 : my_q[j];
            rlo[j] = act ? klo - k0 - 8 * hh : 1;
            rhi[j] = act ? khi - k0 - 8 * hh : 0;
            msk[j] = msk[j] || !act;
        }
        const __bf16* K = sK[buf];
        const __bf16* V = sV[buf];
        // two 32-key halves per tile keep the score and probability registers
        // of both query blocks small
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            // ---- S^T = K Q^T: each K fragment feeds both query blocks ---------
            f32x16 s[2] = {f32x16{}, f32x16{}};
            const __bf16* kp = K + (32 * kb + krow_l) * KSTR + 8 * hh;
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const bf16x8 A = *reinterpret_cast<const bf16x8*>(kp + 16 * c);
                s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, qv[0][c], s[0], 0, 0, 0);
                s[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, qv[1][c], s[1], 0, 0, 0);
            }
            // ---- masks and running max --------------------------------------------
            float mx[2];
            bool raise[2];
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                if (msk[j]) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) {
                        const int c0 = 32 * kb + 16 * (i >> 3) + (i & 7);
                        s[j][i] = ((c0 >= rlo[j]) & (c0 <= rhi[j])) ? s[j][i] : -INFINITY;
                    }
                }
                float m = s[j][0];
#pragma unroll
                for (int i = 1; i < 16; ++i) m = fmaxf(m, s[j][i]);
                mx[j] = wave_max_xor32(m) * scale2;
                raise[j] = mx[j] > m_run[j] + kRescaleSlack;
            }
            if (__any(raise[0] | raise[1])) {
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const float m_new = raise[j] ? mx[j] : m_run[j];
                    const float alpha = raise[j] ? fast_exp2(m_run[j] - m_new) : 1.f;   // 0 when m_run = -inf
                    l_run[j] *= alpha;
#pragma unroll
                    for (int db = 0; db < NDB; ++db) scale_acc(acc[j][db], alpha);
                    m_run[j] = m_new;
                }
            }
            // ---- probabilities (bf16, as the PV MFMA consumes them) ----------------
            bf16x8 P[2][2];
            const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const float m_use = m_run[j] == -INFINITY ? 0.f : m_run[j];   // rows with no key yet
                float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        P[j][h][e] = (__bf16)fast_exp2(fmaf(s[j][8 * h + e], scale2, -m_use));
                    ls0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{P[j][h][0], P[j][h][1]}, ones, ls0, false);
                    ls1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{P[j][h][2], P[j][h][3]}, ones, ls1, false);
                    ls0 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{P[j][h][4], P[j][h][5]}, ones, ls0, false);
                    ls1 = __builtin_amdgcn_fdot2_f32_bf16(bf16x2{P[j][h][6], P[j][h][7]}, ones, ls1, false);
                }
                l_run[j] += ls0 + ls1;
            }
            // ---- O^T += V^T P^T: each V^T fragment feeds both query blocks ---------
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int r0 = 32 * kb + 16 * h + tr_row;
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    // logical chunk of dims 32db + tr_dim and its swizzled place
                    const int lc = (32 * db + tr_dim) >> 3;
                    const int wi = tr_dim & 7;
                    const bf16x4 lo = lds_read_tr16(V + r0 * D + 8 * vswz<D>(r0, lc) + wi);
                    const bf16x4 hi = lds_read_tr16(V + (r0 + 4) * D + 8 * vswz<D>(r0 + 4, lc) + wi);
                    const bf16x8 A = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
                    acc[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, P[0][h], acc[0][db], 0, 0, 0);
                    acc[1][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, P[1][h], acc[1][db], 0, 0, 0);
                }
            }
        }
        stage_store(buf ^ 1);
        wait_vmem();   // the next tile's V has landed in LDS
        __syncthreads();
    };

    stage_load(0, 0);
    stage_store(0);
    wait_vmem();
    __syncthreads();
    if (nR > 0) {
        load_q(true);
        for (int pi = 0; pi < nR; ++pi) tile(pi);
    }
    load_q(false);
    for (int pi = nR; pi < NP; ++pi) tile(pi);

    // ---- epilogue ---------------------------------------------------------------
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const float l_tot = l_run[j] + __shfl_xor(l_run[j], 32);
        if (!qok[j]) continue;
        const float inv = 1.f / l_tot;
        const int64_t o = (((int64_t)b * L + my_q[j]) * Hq + head[j]) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int d0 = db * 32 + a4 * 8 + hh * 4;
                if constexpr (OUT_BF16) {
                    bf16x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[j][db][4 * a4 + e] * inv);
                    *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(p.out) + o + d0) = w;
                } else {
                    f32x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = acc[j][db][4 * a4 + e] * inv;
                    *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + o + d0) = w;
                }
            }
        }
        if (hh == 0 && p.lse)
            p.lse[((int64_t)b * Hq + head[j]) * L + my_q[j]] = (m_run[j] + log2f(l_tot)) * 0.69314718055994531f;
    }
}

template <int D, bool OUT_BF16>
hipError_t launch_one(const PrefillParams& p, hipStream_t stream) {
    const int64_t blocks = (int64_t)p.n_qtiles * p.Hkv * p.B;
    hipLaunchKernelGGL((prefill_bf16_kernel<D, OUT_BF16>), dim3((unsigned)blocks), dim3(kThreads), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const PrefillParams& p, int out_dtype, hipStream_t stream) {
    const bool ob = out_dtype == 1;
    if (p.head_dim == 128) return ob ? launch_one<128, true>(p, stream) : launch_one<128, false>(p, stream);
    return ob ? launch_one<64, true>(p, stream) : launch_one<64, false>(p, stream);
}

}  // namespace jl
