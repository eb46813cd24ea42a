// Split-KV bifocal-attention decode for gfx950 (one new token per sequence).
//
// Method (Jet-Long §3.2): at each step the group size G is recomputed from
// the current length L and the cached keys, stored as RoPE(x_k, k), are read
// under that G by rotating them on the fly by f(k) - k (Eq. 5); the cache is
// never rewritten.  The query sits at position L-1; keys with
// (L-1) - k <= w0 use the stored vectors, the rest the corrected views (Eq. 1).
//
// Split kernel: workgroup = (split of 512 keys, KV head, batch), 4 waves;
// each wave owns 32 consecutive keys per iteration.  K is read straight from
// HBM into MFMA A-operand registers (rows = keys) and rotated there; V goes
// through wave-private LDS, transposed, to be the A operand of
// O^T += V^T P^T.  The R query heads of the KV head are the MFMA N columns
// (16x16x32 bf16), so each K/V byte is read once per step for all R heads.
// Each workgroup leaves one fp32 partial (acc[D], m, l) per query head; the
// combine kernel merges the partials of a head with the log-sum-exp rule
// (§3.3 Eq. 6 with disjoint key sets).
#include <math.h>

#include "internal.h"

namespace jl {

namespace {

constexpr int kDecThreads = 256;
constexpr int kWaves = 4;
constexpr int kWaveKeys = 32;
constexpr int kIterKeys = kWaves * kWaveKeys;
constexpr int VSTR = kWaveKeys + 8;   // V^T row stride (keys) in LDS

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(kDecThreads) void decode_split_kernel(DecodeParams p) {
    constexpr int HALF = D / 2;
    constexpr int NC = D / 32;        // 32-dim K chunks of the QK^T MFMA
    constexpr int NDB = D / 16;       // 16-dim blocks of O^T
    constexpr int KPL = D / 16;       // keys per lane in the V transpose
    typedef __bf16 VW __attribute__((ext_vector_type(KPL)));

    __shared__ __attribute__((aligned(16))) __bf16 sVt[kWaves][D * VSTR];
    __shared__ float s_m[kWaves][16];
    __shared__ float s_l[kWaves][16];
    __shared__ int s_bad;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int colh = lane & 15;   // MFMA column = query head within the group
    const int gq = lane >> 4;     // lane quad

    const int split = blockIdx.x;
    const int g = blockIdx.y;
    const int b = blockIdx.z;
    const int L = (int)p.L;
    const int Hq = (int)p.Hq;
    const int Hkv = (int)p.Hkv;
    const int R = p.R;
    const int G = (int)p.G;
    const int qpos = L - 1;
    // keys >= kloc are local (q - k <= w0); G == 1 makes every key local
    const int kloc = (G == 1) ? 0 : (int)max<int64_t>(0, (int64_t)qpos - p.w0);
    const float scale2 = p.sm_scale_log2;
    const __bf16* __restrict__ kc = static_cast<const __bf16*>(p.k);
    const __bf16* __restrict__ vc = static_cast<const __bf16*>(p.v);
    const float2* __restrict__ TL = p.TL;
    const float2* __restrict__ TH = p.TH;
    const int64_t row = (int64_t)Hkv * D;
    const int64_t cache_b = (int64_t)b * p.Lmax * row + (int64_t)g * D;

    if (tid == 0) {
        const TableHeader* th = p.table;
        s_bad = !(th->magic == kTableMagic && th->head_dim == D && th->rope_base == p.rope_base &&
                  th->n_cover >= p.L);
    }
    __syncthreads();

    const bool hvalid = colh < R;
    const int head = g * R + (hvalid ? colh : 0);

    // ---- query fragments (B operand of S^T = K Q^T) -----------------------
    bf16x8 qf[NC], qr[NC];
    {
        const __bf16* qp = static_cast<const __bf16*>(p.q) + ((int64_t)b * Hq + head) * D;
#pragma unroll
        for (int c = 0; c < NC; ++c)
            qf[c] = hvalid ? *reinterpret_cast<const bf16x8*>(qp + 32 * c + 8 * gq) : bf16x8{};
        if (G > 1 && !s_bad) {
            const int nq = qpos - qpos / G;
#pragma unroll
            for (int c = 0; c < NC / 2; ++c)
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    float x = (float)qf[c][j], y = (float)qf[c + NC / 2][j];
                    rotate_back(x, y, corr_angle(TL, TH, HALF, nq, 32 * c + 8 * gq + j));
                    qr[c][j] = (__bf16)x;
                    qr[c + NC / 2][j] = (__bf16)y;
                }
        } else {
#pragma unroll
            for (int c = 0; c < NC; ++c) qr[c] = qf[c];
        }
    }

    f32x4 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x4{};
    float m_run = -INFINITY, l_run = 0.f;

    const int kstart = split * kDecodeChunk;
    const int kend = min(L, kstart + kDecodeChunk);
    __bf16* myV = sVt[wave];

    for (int it0 = kstart; it0 < kend && !s_bad; it0 += kIterKeys) {
        const int kbase = it0 + wave * kWaveKeys;
        const bool active = kbase < kend;
        // ---- V rows -> V^T (this wave's 32 keys) ---------------------------
        {
            const int dg = lane % (D / 8);
            const int kg = lane / (D / 8);
            bf16x8 vv[KPL];
#pragma unroll
            for (int e = 0; e < KPL; ++e) {
                const int key = kbase + kg * KPL + e;
                vv[e] = key < kend ? *reinterpret_cast<const bf16x8*>(vc + cache_b + (int64_t)key * row + dg * 8)
                                   : bf16x8{};
            }
#pragma unroll
            for (int d = 0; d < 8; ++d) {
                VW w;
#pragma unroll
                for (int e = 0; e < KPL; ++e) w[e] = vv[e][d];
                *reinterpret_cast<VW*>(&myV[(dg * 8 + d) * VSTR + kg * KPL]) = w;
            }
        }
        float s[2][4];
        if (active) {
            const bool w_loc = (G == 1) || (kbase + kWaveKeys - 1 >= kloc);
            const bool w_rem = (G > 1) && (kbase < kloc);
#pragma unroll
            for (int blk = 0; blk < 2; ++blk) {
                // A-operand row colh holds key 8*(colh/4) + 4*blk + colh%4, so
                // that C rows give P^T slots in natural key order
                const int key = kbase + 8 * (colh >> 2) + 4 * blk + (colh & 3);
                const bool ok = key < kend;
                bf16x8 kf[NC];
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    kf[c] = ok ? *reinterpret_cast<const bf16x8*>(kc + cache_b + (int64_t)key * row + 32 * c + 8 * gq)
                               : bf16x8{};
                f32x4 sl = f32x4{}, sr = f32x4{};
                if (w_loc) {
#pragma unroll
                    for (int c = 0; c < NC; ++c) sl = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[c], qf[c], sl, 0, 0, 0);
                }
                if (w_rem) {
                    const int n = ok ? key - key / G : 0;
#pragma unroll
                    for (int c = 0; c < NC / 2; ++c)
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            float x = (float)kf[c][j], y = (float)kf[c + NC / 2][j];
                            rotate_back(x, y, corr_angle(TL, TH, HALF, n, 32 * c + 8 * gq + j));
                            kf[c][j] = (__bf16)x;
                            kf[c + NC / 2][j] = (__bf16)y;
                        }
#pragma unroll
                    for (int c = 0; c < NC; ++c) sr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[c], qr[c], sr, 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int kk = kbase + 8 * gq + 4 * blk + i;   // key of C row gq*4+i
                    float v;
                    if (w_loc && w_rem) v = kk >= kloc ? sl[i] : sr[i];
                    else v = w_loc ? sl[i] : sr[i];
                    s[blk][i] = kk < kend ? v * scale2 : -INFINITY;
                }
            }
            // online softmax per head column: 8 values here, 4 quads per head
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
#pragma unroll
            for (int blk = 0; blk < 2; ++blk)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float pv = fast_exp2(s[blk][i] - m_new);
                    s[blk][i] = pv;
                    ls += pv;
                }
            l_run = l_run * alpha + ls;
            m_run = m_new;
#pragma unroll
            for (int db = 0; db < NDB; ++db) acc[db] *= alpha;
        }
        __syncthreads();   // V^T visible
        if (active) {
            bf16x8 Bp;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                Bp[j] = (__bf16)s[0][j];
                Bp[j + 4] = (__bf16)s[1][j];
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const bf16x8 A = *reinterpret_cast<const bf16x8*>(&myV[(16 * db + colh) * VSTR + 8 * gq]);
                acc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bp, acc[db], 0, 0, 0);
            }
        }
        __syncthreads();   // V^T reads done before the next overwrite
    }

    // ---- merge the 4 waves, write this split's partial --------------------
    float l_tot = l_run + __shfl_xor(l_run, 16);
    l_tot += __shfl_xor(l_tot, 32);
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
    float* ws = p.ws;
    for (int idx = tid; idx < R * D; idx += kDecThreads) {
        const int r = idx / D, d = idx % D;
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) M = fmaxf(M, s_m[w][r]);
        float a = 0.f, l = 0.f;
        if (!s_bad) {
#pragma unroll
            for (int w = 0; w < kWaves; ++w) {
                const float f = fast_exp2(s_m[w][r] - M);
                a += f * s_acc[(w * 16 + r) * D + d];
                l += f * s_l[w][r];
            }
        } else {
            a = NAN;
            l = NAN;
            M = NAN;
        }
        float* o = ws + (((int64_t)b * Hq + g * R + r) * p.n_split + split) * (D + 2);
        o[d] = a;
        if (d == 0) {
            o[D] = M;
            o[D + 1] = l;
        }
    }
}

template <int D, bool OUT_BF16>
__global__ __launch_bounds__(D) void decode_combine_kernel(DecodeParams p) {
    const int head = blockIdx.x;
    const int b = blockIdx.y;
    const int d = threadIdx.x;
    const int ns = p.n_split;
    const float* base = p.ws + ((int64_t)b * p.Hq + head) * ns * (D + 2);
    float M = -INFINITY;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, base[s * (D + 2) + D]);
    float a = 0.f, l = 0.f;
    for (int s = 0; s < ns; ++s) {
        const float f = fast_exp2(base[s * (D + 2) + D] - M);
        a += f * base[s * (D + 2) + d];
        l += f * base[s * (D + 2) + D + 1];
    }
    const int64_t o = ((int64_t)b * p.Hq + head) * D + d;
    if constexpr (OUT_BF16) static_cast<__bf16*>(p.out)[o] = (__bf16)(a / l);
    else static_cast<float*>(p.out)[o] = a / l;
    if (d == 0 && p.lse) p.lse[(int64_t)b * p.Hq + head] = (M + log2f(l)) * 0.69314718055994531f;
}

template <int D, bool OUT_BF16>
hipError_t launch_dec(const DecodeParams& p, hipStream_t stream) {
    hipLaunchKernelGGL((decode_split_kernel<D, OUT_BF16>), dim3(p.n_split, p.Hkv, p.B), dim3(kDecThreads), 0,
                       stream, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((decode_combine_kernel<D, OUT_BF16>), dim3(p.Hq, p.B), dim3(D), 0, stream, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_decode(const DecodeParams& p, int out_dtype, hipStream_t stream) {
    const bool ob = out_dtype == 1;
    if (p.head_dim == 128) return ob ? launch_dec<128, true>(p, stream) : launch_dec<128, false>(p, stream);
    return ob ? launch_dec<64, true>(p, stream) : launch_dec<64, false>(p, stream);
}

}  // namespace jl
