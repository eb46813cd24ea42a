// Causal GQA bifocal-attention prefill for gfx950.
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
//   key tiles of 64 are staged in LDS: K as stored (local view) and/or K
//   rotated by its correction (remote view) -- the rotation runs once per
//   workgroup per tile on the global->LDS path -- and V transposed.
//   Each wave computes S^T = K Q^T with MFMA (keys on the M axis, queries on
//   N), so a query's 64 scores sit in one lane pair: the row max needs one
//   cross-half exchange and the row sum none until the end.  P^T is already
//   in the B-operand layout of O^T += V^T P^T.
//   Tile classes per wave: local-only, remote-only or straddling (both
//   products, per-element select on q - k <= w0); tiles above the diagonal
//   are skipped.
#include <math.h>

#include <type_traits>

#include "internal.h"

namespace jl {

namespace {

constexpr int kThreads = 512;
constexpr int BN = 64;   // keys per tile

template <bool BF16> struct Elem;
template <> struct Elem<true> { using T = __bf16; };
template <> struct Elem<false> { using T = float; };

template <int D, bool BF16>
struct PrefillLayout {
    static constexpr int HALF = D / 2;
    static constexpr int KSTR = BF16 ? D + 8 : D + 4;      // K row stride (elements)
    // bf16: V^T[d][key] rows of BN keys; f32: V[key][d] rows of D values
    static constexpr int VSTR = BF16 ? BN + 8 : D + 4;
    static constexpr int K_ELEMS = BN * KSTR;
    static constexpr int V_ELEMS = BF16 ? D * VSTR : BN * VSTR;
    static constexpr int PPT = HALF * BN / kThreads;        // rotation pairs per thread
    static constexpr int NQ = BF16 ? D / 16 : D / 8;        // Q fragments per lane
};

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

    __shared__ __attribute__((aligned(16))) T sKloc[Lay::K_ELEMS];
    __shared__ __attribute__((aligned(16))) T sKrem[Lay::K_ELEMS];
    __shared__ __attribute__((aligned(16))) T sV[Lay::V_ELEMS];
    __shared__ int s_bad;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
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
    const int r = wave % R;
    const int pb = wave / R;
    const int head = g * R + r;
    const int q0 = qt * p.BQ;
    const int q_hi = min(q0 + p.BQ, L) - 1;
    const int p0 = q0 + pb * 32;
    const int p_hi = min(p0 + 31, L - 1);
    const int my_q = p0 + col;
    const bool wave_active = p0 < L;
    const float scale2 = p.sm_scale_log2;

    const T* __restrict__ qg = static_cast<const T*>(p.q);
    const T* __restrict__ kg = static_cast<const T*>(p.k);
    const T* __restrict__ vg = static_cast<const T*>(p.v);
    const float2* __restrict__ TL = p.TL;
    const float2* __restrict__ TH = p.TH;
    const int64_t kv_row = (int64_t)Hkv * D;

    if (tid == 0) {
        const TableHeader* th = p.table;
        s_bad = !(th->magic == kTableMagic && th->head_dim == D && th->rope_base == p.rope_base &&
                  th->n_cover >= p.L);
    }
    __syncthreads();
    if (s_bad) {
        // The table does not belong to this (D, rope_base, L): poison the output.
        if (wave_active && my_q < L) {
            const int64_t o = (((int64_t)b * L + my_q) * Hq + head) * D;
            for (int d = hh; d < D; d += 2) {
                if constexpr (OUT_BF16) static_cast<__bf16*>(p.out)[o + d] = (__bf16)NAN;
                else static_cast<float*>(p.out)[o + d] = NAN;
            }
            if (hh == 0 && p.lse) p.lse[((int64_t)b * Hq + head) * L + my_q] = NAN;
        }
        return;
    }

    // ---- Q fragments (B operand of S^T = K Q^T) -----------------------------
    // bf16: fragment c holds dims 16c + 8hh + [0, 8); f32: fragment t holds
    // dims 8t + 4hh + [0, 4).  Partner dims (+D/2) sit in fragment c + NQ/2.
    using QF = typename std::conditional<BF16, bf16x8, f32x4>::type;
    QF qf[NQ], qr[NQ];
    {
        const bool ok = wave_active && my_q < L;
        const int64_t qo = (((int64_t)b * L + (ok ? my_q : 0)) * Hq + head) * D;
        constexpr int W = BF16 ? 8 : 4;
#pragma unroll
        for (int c = 0; c < NQ; ++c) {
            const int d0 = c * 2 * W + W * hh;
            if (ok) qf[c] = *reinterpret_cast<const QF*>(qg + qo + d0);
            else qf[c] = QF{};
        }
        if (G > 1) {
            const int nq = ok ? my_q - my_q / G : 0;
#pragma unroll
            for (int c = 0; c < NQ / 2; ++c) {
#pragma unroll
                for (int j = 0; j < W; ++j) {
                    float x = (float)qf[c][j];
                    float y = (float)qf[c + NQ / 2][j];
                    rotate_back(x, y, corr_angle(TL, TH, HALF, nq, c * 2 * W + W * hh + j));
                    qr[c][j] = (T)x;
                    qr[c + NQ / 2][j] = (T)y;
                }
            }
        } else {
#pragma unroll
            for (int c = 0; c < NQ; ++c) qr[c] = qf[c];
        }
    }

    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};
    float m_run = -INFINITY;
    float l_run = 0.f;

    const int nkt = q_hi / BN + 1;
    for (int kt = 0; kt < nkt; ++kt) {
        const int k0 = kt * BN;
        const int k1 = min(k0 + BN, L) - 1;
        const bool wg_loc = (G == 1) || (q0 - k1 <= w0);
        const bool wg_rem = (G > 1) && (q_hi - k0 > w0);

        __syncthreads();   // previous tile's LDS reads are done
        // ---- K: stored view and/or corrected view --------------------------
        {
            typedef T KV __attribute__((ext_vector_type(PPT)));
            const int kr = tid >> 3;             // key row in tile
            const int f0 = (tid & 7) * PPT;      // first frequency index
            const int kpos = k0 + kr;
            const bool ok = kpos < L;
            const int64_t ko = ((int64_t)b * L + (ok ? kpos : 0)) * kv_row + (int64_t)g * D;
            KV xv = KV{}, yv = KV{};
            if (ok) {
                xv = *reinterpret_cast<const KV*>(kg + ko + f0);
                yv = *reinterpret_cast<const KV*>(kg + ko + HALF + f0);
            }
            if (wg_loc) {
                *reinterpret_cast<KV*>(&sKloc[kr * KSTR + f0]) = xv;
                *reinterpret_cast<KV*>(&sKloc[kr * KSTR + HALF + f0]) = yv;
            }
            if (wg_rem) {
                const int n = ok ? kpos - kpos / G : 0;
                KV xr, yr;
#pragma unroll
                for (int j = 0; j < PPT; ++j) {
                    float x = (float)xv[j], y = (float)yv[j];
                    rotate_back(x, y, corr_angle(TL, TH, HALF, n, f0 + j));
                    xr[j] = (T)x;
                    yr[j] = (T)y;
                }
                *reinterpret_cast<KV*>(&sKrem[kr * KSTR + f0]) = xr;
                *reinterpret_cast<KV*>(&sKrem[kr * KSTR + HALF + f0]) = yr;
            }
        }
        // ---- V ---------------------------------------------------------------
        if constexpr (BF16) {
            // transposed: sV[d][key], natural key order; each thread moves a
            // KPT-key x 4-dim block (8-byte row reads, KPT*2-byte column writes)
            constexpr int KPT = BN * D / (kThreads * 4);
            typedef __bf16 VW __attribute__((ext_vector_type(KPT)));
            const int dg = tid % (D / 4);
            const int kgp = tid / (D / 4);
            bf16x4 vv[KPT];
#pragma unroll
            for (int e = 0; e < KPT; ++e) {
                const int kpos = k0 + kgp * KPT + e;
                const int64_t vo = ((int64_t)b * L + kpos) * kv_row + (int64_t)g * D + dg * 4;
                vv[e] = kpos < L ? *reinterpret_cast<const bf16x4*>(vg + vo) : bf16x4{};
            }
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                VW w;
#pragma unroll
                for (int e = 0; e < KPT; ++e) w[e] = vv[e][d];
                *reinterpret_cast<VW*>(&sV[(dg * 4 + d) * VSTR + kgp * KPT]) = w;
            }
        } else {
            constexpr int FPT = D / 8;   // floats per thread, 8 threads per key row
            typedef float VW __attribute__((ext_vector_type(FPT)));
            const int kr = tid >> 3;
            const int c0 = (tid & 7) * FPT;
            const int kpos = k0 + kr;
            const int64_t vo = ((int64_t)b * L + kpos) * kv_row + (int64_t)g * D + c0;
            *reinterpret_cast<VW*>(&sV[kr * VSTR + c0]) =
                kpos < L ? *reinterpret_cast<const VW*>(vg + vo) : VW{};
        }
        __syncthreads();

        if (!wave_active || k0 > p_hi) continue;
        const bool w_loc = (G == 1) || (p0 - k1 <= w0);
        const bool w_rem = (G > 1) && (p_hi - k0 > w0);
        const int nkb = min(2, (p_hi - k0) / 32 + 1);   // 32-key blocks with a causal key

        // ---- S^T = K Q^T ---------------------------------------------------------
        f32x16 s[2];
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (kb >= nkb) break;
            f32x16 sl = f32x16{}, sr = f32x16{};
            if constexpr (BF16) {
                // A-operand row `col` holds key 32kb + sigma(col); sigma makes the
                // C rows land so that P^T feeds the PV MFMA in natural key order.
                const int a = col >> 3, hp = (col >> 2) & 1, e = col & 3;
                const int krow = 32 * kb + 16 * (a >> 1) + 8 * hp + 4 * (a & 1) + e;
                if (w_loc) {
#pragma unroll
                    for (int c = 0; c < NQ; ++c) {
                        const bf16x8 A = *reinterpret_cast<const bf16x8*>(&sKloc[krow * KSTR + 16 * c + 8 * hh]);
                        sl = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, qf[c], sl, 0, 0, 0);
                    }
                }
                if (w_rem) {
#pragma unroll
                    for (int c = 0; c < NQ; ++c) {
                        const bf16x8 A = *reinterpret_cast<const bf16x8*>(&sKrem[krow * KSTR + 16 * c + 8 * hh]);
                        sr = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, qr[c], sr, 0, 0, 0);
                    }
                }
            } else {
                const int krow = 32 * kb + col;
                if (w_loc) {
#pragma unroll
                    for (int t = 0; t < NQ; ++t) {
                        const f32x4 A = *reinterpret_cast<const f32x4*>(&sKloc[krow * KSTR + 8 * t + 4 * hh]);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            sl = __builtin_amdgcn_mfma_f32_32x32x2f32(A[e], qf[t][e], sl, 0, 0, 0);
                    }
                }
                if (w_rem) {
#pragma unroll
                    for (int t = 0; t < NQ; ++t) {
                        const f32x4 A = *reinterpret_cast<const f32x4*>(&sKrem[krow * KSTR + 8 * t + 4 * hh]);
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            sr = __builtin_amdgcn_mfma_f32_32x32x2f32(A[e], qr[t][e], sr, 0, 0, 0);
                    }
                }
            }
            // select the view per element, apply the causal mask, scale to log2
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                int koff;
                if constexpr (BF16) koff = 32 * kb + 16 * (i >> 3) + 8 * hh + (i & 7);
                else koff = 32 * kb + (i >> 2) * 8 + hh * 4 + (i & 3);
                const int key = k0 + koff;
                float vsc;
                if (w_loc && w_rem) vsc = (my_q - key <= w0) ? sl[i] : sr[i];
                else vsc = w_loc ? sl[i] : sr[i];
                s[kb][i] = (key > my_q) ? -INFINITY : vsc * scale2;
            }
        }

        // ---- online softmax (base 2) ---------------------------------------------
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (kb >= nkb) break;
#pragma unroll
            for (int i = 0; i < 16; ++i) mx = fmaxf(mx, s[kb][i]);
        }
        mx = wave_max_xor32(mx);
        const float m_new = fmaxf(m_run, mx);     // finite: key 0 is in the first tile
        const float alpha = fast_exp2(m_run - m_new);
        float ls = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            if (kb >= nkb) break;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const float pv = fast_exp2(s[kb][i] - m_new);
                s[kb][i] = pv;
                ls += pv;
            }
        }
        l_run = l_run * alpha + ls;
        m_run = m_new;
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[db] *= alpha;

        // ---- O^T += V^T P^T ----------------------------------------------------
        if constexpr (BF16) {
#pragma unroll
            for (int kc = 0; kc < 4; ++kc) {
                if (kc >= 2 * nkb) break;
                bf16x8 Bp;
#pragma unroll
                for (int j = 0; j < 8; ++j) Bp[j] = (__bf16)s[kc >> 1][8 * (kc & 1) + j];
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const bf16x8 A = *reinterpret_cast<const bf16x8*>(&sV[(db * 32 + col) * VSTR + 16 * kc + 8 * hh]);
                    acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, Bp, acc[db], 0, 0, 0);
                }
            }
        } else {
#pragma unroll
            for (int kb = 0; kb < 2; ++kb) {
                if (kb >= nkb) break;
#pragma unroll
                for (int i = 0; i < 16; ++i) {
                    const int key = 32 * kb + (i >> 2) * 8 + hh * 4 + (i & 3);
#pragma unroll
                    for (int db = 0; db < NDB; ++db)
                        acc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(sV[key * VSTR + db * 32 + col],
                                                                       s[kb][i], acc[db], 0, 0, 0);
                }
            }
        }
    }

    // ---- epilogue ---------------------------------------------------------------
    const float l_tot = l_run + __shfl_xor(l_run, 32);
    if (wave_active && my_q < L) {
        const float inv = 1.f / l_tot;
        const int64_t o = (((int64_t)b * L + my_q) * Hq + head) * D;
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
            p.lse[((int64_t)b * Hq + head) * L + my_q] = (m_run + log2f(l_tot)) * 0.69314718055994531f;
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
    const bool in_bf16 = in_dtype == 1;
    const bool out_bf16 = out_dtype == 1;
    if (p.head_dim == 128) {
        if (in_bf16) return out_bf16 ? launch_one<128, true, true>(p, stream) : launch_one<128, true, false>(p, stream);
        return launch_one<128, false, false>(p, stream);
    }
    if (in_bf16) return out_bf16 ? launch_one<64, true, true>(p, stream) : launch_one<64, true, false>(p, stream);
    return launch_one<64, false, false>(p, stream);
}

}  // namespace jl
