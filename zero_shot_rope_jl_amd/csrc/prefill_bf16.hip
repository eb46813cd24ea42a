// Causal GQA bifocal-attention prefill for gfx950, bf16 inputs.
//
// Method (Jet-Long, §3 Eq. 1; §3.1 Eqs. 2-3; §3.2 Eq. 5; §3.3 Eq. 6): a
// query/key pair with q - k <= w0 scores with the stored RoPE vectors; a pair
// with q - k > w0 scores with both vectors rotated by their correction offset
// f(p) - p, f(p) = floor(p/G).  Both views feed one softmax per query row,
// which realises the inclusion-exclusion merge exactly (the overlap term is
// removed by masking, not subtracted).
//
// Work decomposition (one workgroup = 8 waves = 256 query rows of one KV head)
//   Rows are ordered head-major over the R = Hq/Hkv query heads of the KV
//   head and BQ = 256/R positions; wave w owns the 32-row query block
//   [32w, 32w + 32).  Two waves per SIMD: while one issues MFMAs the other's
//   softmax VALU work runs beside them.  Every MFMA keeps its result and
//   accumulator in VGPRs (the library compiles this file in that form), so
//   scores feed the exponentials with no register-file copies.
//
//   Key tiles of BN = 128 are walked in two phases: a remote phase over every tile
//   that holds a remote pair (keys and Q in their corrected view), then a
//   local phase over every tile that holds a local pair (stored K and Q).  A
//   tile that straddles the window edge is visited once per phase under a
//   mask.  The remote view of the keys is formed once per call by
//   rotate_keys_kernel into the caller's workspace: every workgroup of a KV
//   head reads the same keys, so rotating them per visited tile would repeat
//   the same VALU work once per query tile.  The cache itself is never
//   written.
//
//   Staging: LDS is double-buffered.  During a tile the next tile's K and V
//   are copied HBM -> LDS with buffer loads into LDS (no registers, no VALU;
//   K rows padded to KSTR, V chunks XOR-swizzled by row so that the
//   transposed reads below spread over the banks).  One barrier per tile.
//
//   Scores: each wave computes S^T = K Q^T (keys on the MFMA M axis, queries
//   on N), so a query's scores sit in one lane pair and P^T is already the B
//   operand of O^T += V^T P^T, whose V^T operand comes from row-major V
//   through ds_read_b64_tr_b16.  Q is pre-multiplied by sm_scale * log2(e).
//   Each row's reference max m is fixed (rounded to bf16) at the first tile
//   that gives it a key and never moved; each score MFMA chain starts from
//   -m as its accumulator input, so P = exp2(S) needs no per-element
//   subtraction and the accumulators are touched by MFMAs only.  Probabilities above 1 are
//   harmless (fp32 and bf16 share the exponent range; the final division
//   restores the scale).
//
// The kernel's MODE template parameter also gives the three separate passes
// of the unfused form of §3.3 Eq. (6): the stored view over each row's window
// [q - w0, q], the corrected view over every key k <= q, and the corrected
// view over the window.  A mode changes only which tiles a workgroup visits
// and which keys each row keeps; kFused is the bifocal rule itself.
#include <limits.h>
#include <math.h>

#include <type_traits>

#include "internal.h"

namespace jl {

namespace {

// 32-row query blocks per wave.  1 gives 8 waves per workgroup, two per
// SIMD, whose MFMA and VALU work the hardware interleaves.  (2 would give 4
// waves, one per SIMD, each K or V^T fragment read from LDS feeding two
// MFMAs, but its accumulators and scores no longer fit the 256 VGPRs of the
// MFMAs' VGPR form.)
constexpr int NJ = 1;
constexpr int kWaves = 8 / NJ;
constexpr int kThreads = kWaves * 64;
// keys per tile: 128 halves the per-tile scalar set-up, copy issue and
// barrier per key against 64, and double-buffered K and V still fit in LDS
// (135 KB of 160 KB at D = 128)
constexpr int BN = 128;

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

__device__ inline void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int D>
struct Lay5 {
    static constexpr int HALF = D / 2;
    static constexpr int NC = D / 16;           // 16-dim K chunks (MFMA k)
    static constexpr int NDB = D / 32;          // 32-dim O^T blocks
    static constexpr int KSTR = D + 8;          // K row stride (elements), padded
    static constexpr int CH = D / 8;            // 16-byte chunks per K or V row
};

// physical 16-byte chunk of logical chunk `c` in V row `row`
template <int D>
__device__ inline int vswz(int row, int c) {
    return c ^ ((4 * (row & 3)) & (Lay5<D>::CH - 1));
}

// One query tile (one workgroup's share of the static grid, index `tile_id`
// in its order): the whole body of the kernel below.
template <int D, bool OUT_BF16, int MODE, bool PAGED>
__device__ __attribute__((always_inline)) inline void prefill_tile(const PrefillParams& p, const int tile_id) {
    using Lay = Lay5<D>;
    constexpr int HALF = Lay::HALF;
    constexpr int NC = Lay::NC;
    constexpr int NDB = Lay::NDB;
    constexpr int KSTR = Lay::KSTR;
    constexpr int CH = Lay::CH;

    // Two LDS buffers per operand, as separate objects and always selected at
    // compile time: the compiler can then tell that the HBM->LDS copy into
    // one buffer does not alias the reads of the other, and does not make
    // those reads wait for the copy.
    __shared__ __attribute__((aligned(16))) __bf16 sK0[BN * KSTR];
    __shared__ __attribute__((aligned(16))) __bf16 sK1[BN * KSTR];
    __shared__ __attribute__((aligned(16))) __bf16 sV0[BN * D];
    __shared__ __attribute__((aligned(16))) __bf16 sV1[BN * D];
    __shared__ int s_bad;

    // the thread index passes through an empty asm statement, so that the
    // lane-constant offsets derived from it are formed inside each tile's
    // body rather than hoisted out of the dynamic grid's loop and kept live
    // (in registers the body needs) across every tile
    int tid_opaque = (int)threadIdx.x;
    asm volatile("" : "+v"(tid_opaque));
    const int tid = tid_opaque;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hh = lane >> 5;      // lane half
    const int col = lane & 31;     // query column of the S^T / O^T tiles

    // Heads vary fastest over the tile order so that the tiles of one KV head
    // land on one XCD (the static grid's dispatch is round-robin over the 8
    // XCDs; the dynamic grid's queues follow it) and share its L2; query
    // tiles come longest (last) first.
    int bid = tile_id;
    const int g = (int)(bid % p.Hkv);
    bid /= (int)p.Hkv;
    const int b = (int)(bid % p.B);
    bid /= (int)p.B;
    const int ks = bid % p.n_ksplit;   // key split of this query tile (0 when unsplit)
    bid /= p.n_ksplit;
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
    const int BQ = p.BQ;
    const int q0 = q_off + qt * BQ;
    const int q_hi = min(q0 + BQ, L) - 1;
    const float scale2 = p.sm_scale_log2;

    // the wave's 32-row query blocks
    int head[NJ], pj0[NJ], pjhi[NJ], my_q[NJ];
    bool qok[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int rho = 32 * NJ * wave + 32 * j;
        head[j] = g * R + rho / BQ;
        pj0[j] = q0 + rho % BQ;
        pjhi[j] = min(pj0[j] + 31, L - 1);
        my_q[j] = pj0[j] + col;
        qok[j] = my_q[j] < L;
    }

    const __bf16* __restrict__ qg = static_cast<const __bf16*>(p.q);
    const float2* __restrict__ TF = p.TF;
    const int64_t kv_row = (int64_t)Hkv * D;
    const uint32_t row_bytes = (uint32_t)kv_row * 2u;
    const int64_t kv_b = PAGED ? 0 : (int64_t)b * Lkv * kv_row;
    const __bf16* __restrict__ kbase = static_cast<const __bf16*>(p.k) + kv_b + (int64_t)g * D;
    const __bf16* __restrict__ vbase = static_cast<const __bf16*>(p.v) + kv_b + (int64_t)g * D;
    // keys in their corrected view (only read by remote tiles, which exist only
    // when G > 1), laid out like k with L rows per batch entry
    const __bf16* __restrict__ krbase =
        G > 1 ? static_cast<const __bf16*>(p.krot) + (int64_t)b * p.krot_rows * kv_row + (int64_t)g * D : kbase;

    if (tid == 0) {
        const TableHeader* th = p.table;
        s_bad = !table_matches(th, p.table_key, D, p.rope_base, table_need(p.L, p.G));
    }
    __syncthreads();
    if (s_bad) {
        // The table does not belong to this (D, rope_base, L): poison the output
        // (a split marks its partials; the combine and fixup passes then poison
        // the rows).
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            if (!qok[j]) continue;
            if (p.n_ksplit > 1) {
                if (hh == 0)
                    p.part[((((int64_t)ks * p.B + b) * Lq + (my_q[j] - q_off)) * Hq + head[j]) * (D + 4) + D] = NAN;
                continue;
            }
            const int64_t o = (((int64_t)b * Lq + (my_q[j] - q_off)) * Hq + head[j]) * D;
            for (int d = hh; d < D; d += 2) {
                if constexpr (OUT_BF16) static_cast<__bf16*>(p.out)[o + d] = (__bf16)NAN;
                else static_cast<float*>(p.out)[o + d] = NAN;
            }
            if (hh == 0 && p.lse) p.lse[((int64_t)b * Hq + head[j]) * Lq + (my_q[j] - q_off)] = NAN;
        }
        return;
    }

    // ---- pass schedule (uniform over the workgroup) -------------------------
    // The corrected-view phase walks tiles r0 .. r0 + nR - 1, then the
    // stored-view phase tiles nL0 .. nkt - 1.
    const int nkt = q_hi / BN + 1;
    int nR = 0;    // fused: tiles [0, nR) hold a pair with q - k > w0
    int nL0 = 0;   // fused: tiles [nL0, nkt) hold a pair with 0 <= q - k <= w0
    int r0 = 0;
    if constexpr (MODE == kFused) {
        if (G > 1) {
            nR = q_hi - w0 > 0 ? min(nkt, (q_hi - w0 + BN - 1) / BN) : 0;
            nL0 = q0 - w0 - (BN - 1) > 0 ? (q0 - w0) / BN : 0;
        }
    } else {
        // first tile holding a key of some row's window [q - w0, q]
        const int win0 = q0 - w0 - (BN - 1) > 0 ? (q0 - w0) / BN : 0;
        if constexpr (MODE == kLocalWindow) {
            nL0 = win0;
        } else if constexpr (MODE == kRemoteAll) {
            nR = nkt;
            nL0 = nkt;
        } else {
            r0 = win0;
            nR = nkt - win0;
            nL0 = nkt;
        }
    }
    const int NP = nR + (nkt - nL0);
    // this workgroup's share of the tile list: a contiguous run, so a split
    // walks its tiles in the unsplit order
    const int pi_lo = (int)((int64_t)NP * ks / p.n_ksplit);
    const int pi_hi = (int)((int64_t)NP * (ks + 1) / p.n_ksplit);

    // ---- query fragments ---------------------------------------------------------
    // B operand, fragment c = dims 16c + 8hh + [0, 8), multiplied by
    // sm_scale * log2(e) before the bf16 rounding, so the MFMA yields scores in
    // log2 units.  Rows past L read row L-1 (finite values, never stored).
    bf16x8 qv[NJ][NC];
    auto load_q = [&](bool remote_view) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const int qpos = min(my_q[j], L - 1);
            const __bf16* qrow = qg + (((int64_t)b * Lq + (qpos - q_off)) * Hq + head[j]) * D;
            bf16x8 raw[NC];
#pragma unroll
            for (int c = 0; c < NC; ++c) raw[c] = *reinterpret_cast<const bf16x8*>(qrow + 16 * c + 8 * hh);
            if (remote_view) {
                const int64_t nq = qpos - qpos / G;
#pragma unroll
                for (int c = 0; c < NC / 2; ++c)
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        float x = (float)raw[c][e], y = (float)raw[c + NC / 2][e];
                        rotate_back(x, y, table_cs(TF, HALF, nq, 16 * c + 8 * hh + e));
                        qv[j][c][e] = (__bf16)(x * scale2);
                        qv[j][c + NC / 2][e] = (__bf16)(y * scale2);
                    }
            } else {
#pragma unroll
                for (int c = 0; c < NC; ++c)
#pragma unroll
                    for (int e = 0; e < 8; ++e) qv[j][c][e] = (__bf16)((float)raw[c][e] * scale2);
            }
        }
    };

    // ---- staging of the next tile ------------------------------------------------
    // K and V tiles are copied HBM -> LDS with buffer loads into LDS (no
    // registers, no VALU).  Remote tiles read the keys in their corrected view
    // (rotated once per call by rotate_keys_kernel), local tiles the stored
    // keys.  A copy instruction fills 64 consecutive 16-byte LDS slots, one per
    // lane, so each lane's HBM offset places its slot: V rows are dense with
    // their 16-byte chunks XOR-swizzled by row (for the transposed reads),
    // K rows keep a 16-byte pad (row stride KSTR) whose slot reads past the
    // tile and lands as zeros.  All offsets are lane constants over a tile
    // base held in a buffer resource; rows past L read as zeros (masked).
    constexpr int VU = BN * CH / kThreads;         // V copies per thread
    constexpr int VRU = kThreads / CH;             // V rows per copy step
    constexpr int KS = BN * (CH + 1);              // 16-byte slots of a K tile, pads included
    constexpr int KU = KS / kThreads;              // K copy rounds every wave takes
    constexpr int KREM = (KS - KU * kThreads) / 64;   // waves that take one more
    static_assert(VRU % 4 == 0, "V swizzle is lane-constant");
    static_assert((KS - KU * kThreads) % 64 == 0 && KREM < kWaves, "K slots fill whole copies");
    const uint32_t v_voff = (uint32_t)(tid / CH) * row_bytes + 16u * (uint32_t)vswz<D>(tid / CH, tid % CH);
    auto k_slot_voff = [&](int slot) __attribute__((always_inline)) {
        const int row = slot / (CH + 1), ch = slot % (CH + 1);
        return ch == CH ? 0x80000000u : (uint32_t)row * row_bytes + 16u * (uint32_t)ch;
    };
    uint32_t k_voff[KU + 1];
#pragma unroll
    for (int u = 0; u < KU; ++u) k_voff[u] = k_slot_voff((u * kWaves + wave) * 64 + lane);
    k_voff[KU] = wave < KREM ? k_slot_voff((KU * kWaves + wave) * 64 + lane) : 0u;
    auto tile_k0 = [&](int pi) __attribute__((always_inline)) { return (pi < nR ? r0 + pi : nL0 + (pi - nR)) * BN; };
    // Cache row of key k0 (a multiple of BN).  Paged caches: BN divides the
    // page size, so a tile lies in one page; its block-table entry is read
    // through the constant address space (a scalar load: the table is not
    // written during the kernel).  An entry outside [0, n_pages) reads page
    // 0 instead and marks this workgroup's rows, which the fixup pass then
    // writes as NaN, so no load leaves the pages.
    bool bad_page = false;
    auto cache_row = [&](int k0) __attribute__((always_inline)) -> int64_t {
        if constexpr (!PAGED) {
            return k0;
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
    // staging is issued in two parts spread over the tile, so that the
    // vector-memory queue never fills and stalls the wave: K at the start, V
    // with the first PV half
    auto stage_load_k = [&](int pi, auto buf) __attribute__((always_inline)) {
        char* sKd = reinterpret_cast<char*>(decltype(buf)::value ? sK1 : sK0);
        const int k0 = tile_k0(pi);
        const uint32_t tile_bytes = (uint32_t)min(L - k0, BN) * row_bytes;
        // corrected-view tiles read the rotated keys, laid out by position
        const __bf16* src = pi < nR ? krbase + (int64_t)k0 * kv_row : kbase + cache_row(k0) * kv_row;
        const __amdgpu_buffer_rsrc_t rk = make_rsrc(src, tile_bytes);
#pragma unroll
        for (int u = 0; u < KU; ++u) buffer_lds16(rk, sKd + (u * kWaves + wave) * 1024, k_voff[u], 0);
        if (KREM > 0 && wave < KREM) buffer_lds16(rk, sKd + (KU * kWaves + wave) * 1024, k_voff[KU], 0);
    };
    auto stage_load_v = [&](int pi, auto buf) __attribute__((always_inline)) {
        __bf16* sVd = decltype(buf)::value ? sV1 : sV0;
        const int k0 = tile_k0(pi);
        const uint32_t tile_bytes = (uint32_t)min(L - k0, BN) * row_bytes;
        // V: BN rows x CH chunks, VRU rows per copy step
        const __amdgpu_buffer_rsrc_t rv = make_rsrc(vbase + cache_row(k0) * kv_row, tile_bytes);
#pragma unroll
        for (int u = 0; u < VU; ++u)
            buffer_lds16(rv, &sVd[(u * kWaves + wave) * 64 * 8], v_voff, (uint32_t)(u * VRU) * row_bytes);
    };

    // ---- softmax state -------------------------------------------------------------
    // m_ref: the row's reference max (log2 units, a bf16 value), -inf until the
    // row meets its first key; negm: -m_ref (0 while unset) in every element,
    // the accumulator input of each score chain's first MFMA, which so
    // subtracts the reference at no cost; l_run: row sum of probabilities.
    f32x16 acc[NJ][NDB];
    float m_ref[NJ], l_run[NJ];
    f32x16 negm[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) acc[j][db] = f32x16{};
        m_ref[j] = -INFINITY;
        l_run[j] = 0.f;
        negm[j] = f32x16{};
    }

    // K A-operand row of this lane in each 32-key block (sigma makes the C
    // rows land so that P^T feeds the PV MFMA in natural key order)
    const int a3 = col >> 3, hp = (col >> 2) & 1, ee = col & 3;
    const int krow_l = 16 * (a3 >> 1) + 8 * hp + 4 * (a3 & 1) + ee;
    // V^T operand through the transposing read: within each 16-lane group,
    // lane c supplies 4 dims of one key row, lane i receives dim i of 4 rows
    const int Gq = lane >> 4, cq = lane & 15;
    const int tr_row = 8 * (Gq >> 1) + (cq >> 2);
    const int tr_dim = 16 * (Gq & 1) + 4 * (cq & 3);
    const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};

    // One MFMA operand fragment from LDS: K rows of 32-key block kb, chunk c
    // (the A operand of S^T = K Q^T), or V^T fragment t = 4h + db of block kb
    // (the A operand of O^T += V^T P^T: dims 32db.., keys 16h.. of the block)
    // through the transposing read.
    auto kfrag = [&](const __bf16* K, int kb, int c) __attribute__((always_inline)) -> bf16x8 {
        return *reinterpret_cast<const bf16x8*>(K + (32 * kb + krow_l) * KSTR + 8 * hh + 16 * c);
    };
    auto vfrag = [&](const __bf16* V, int kb, int t) __attribute__((always_inline)) -> bf16x8 {
        const int h = t / NDB, db = t % NDB;
        const int r0 = 32 * kb + 16 * h + tr_row;
        // logical chunk of dims 32db + tr_dim and its swizzled place
        const int lc = (32 * db + tr_dim) >> 3;
        const int wi = tr_dim & 7;
        const bf16x4 lo = lds_read_tr16(V + r0 * D + 8 * vswz<D>(r0, lc) + wi);
        const bf16x4 hi = lds_read_tr16(V + (r0 + 4) * D + 8 * vswz<D>(r0 + 4, lc) + wi);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };

    // Window-edge, causal-diagonal and ragged tiles mask scores per element;
    // a row meeting its first keys takes this half's max (rounded to bf16) as
    // its reference, which is subtracted here once and by the MFMA after.
    // Per query block of a tile: does it hold a kept pair (act), and is some
    // pair of the block outside the kept window (msk)?  Wave-uniform, and
    // written with selects so that it compiles without branches.
    auto block_state = [&](int j, bool rem, int k0, bool& act, bool& msk) __attribute__((always_inline)) {
        const int k1 = k0 + BN - 1;
        if constexpr (MODE == kFused) {
            const bool act_r = pjhi[j] - k0 > w0;
            const bool msk_r = pj0[j] - k1 <= w0;
            const bool act_l = (k0 <= pjhi[j]) & ((G == 1) | (pj0[j] - k1 <= w0));
            const bool msk_l = (k1 > pj0[j]) | ((G > 1) & (pjhi[j] - k0 > w0));
            act = (rem ? act_r : act_l) & (pj0[j] < L);
            msk = (rem ? msk_r : msk_l) | !act;
        } else {
            // kept keys [q - w0, q], or every k <= q for the all-keys pass
            constexpr bool all = MODE == kRemoteAll;
            act = (k0 <= pjhi[j]) & (all | (pj0[j] - k1 <= w0)) & (pj0[j] < L);
            msk = (k1 > pj0[j]) | (!all & (pjhi[j] - k0 > w0)) | !act;
        }
    };
    auto edge_fix = [&](f32x16 (&s)[NJ], int kb, bool rem, int k0) {
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            // kept key window [rlo, rhi] relative to the lane's first key k0 + 8hh
            bool act, msk;
            block_state(j, rem, k0, act, msk);
            int klo, khi;
            if constexpr (MODE == kFused) {
                klo = (rem || G == 1) ? INT_MIN / 2 : my_q[j] - w0;
                khi = rem ? my_q[j] - w0 - 1 : my_q[j];
            } else {
                klo = MODE == kRemoteAll ? INT_MIN / 2 : my_q[j] - w0;
                khi = my_q[j];
            }
            int rlo = act ? klo - k0 - 8 * hh : 1;
            int rhi = act ? khi - k0 - 8 * hh : 0;
            rlo = msk ? rlo : INT_MIN / 2;   // every pair kept
            rhi = msk ? rhi : INT_MAX / 2;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int c0 = 32 * kb + 16 * (i >> 3) + (i & 7);
                s[j][i] = ((c0 >= rlo) & (c0 <= rhi)) ? s[j][i] : -INFINITY;
            }
            float m = s[j][0];
#pragma unroll
            for (int i = 1; i < 16; ++i) m = fmaxf(m, s[j][i]);
            m = wave_max_xor32(m);
            const bool first = (m_ref[j] == -INFINITY) & (m != -INFINITY);
            const float mb = (float)(__bf16)m;
            const float d = first ? mb : 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) s[j][i] -= d;
            m_ref[j] = first ? mb : m_ref[j];
            const float nm = m_ref[j] != -INFINITY ? -m_ref[j] : 0.f;
#pragma unroll
            for (int i = 0; i < 16; ++i) negm[j][i] = nm;
        }
    };

    // One region: PV of block kbp (with its probabilities Pold), the scores
    // of block kbq into Snew, and the probabilities of the scores Scur into
    // Pnew with their row sums.  The three are independent, so the region is
    // written in the order it should issue, fenced by scheduling barriers:
    // PV and score MFMAs alternate, each operand fragment is read from LDS
    // PFD MFMAs ahead of its use, and each MFMA is followed by its share of
    // the exponentials, bf16 packs and row-sum dot products.  The row sum is
    // pinned in the region: left alone, the compiler sinks every row sum to
    // the tile's end, which keeps all four blocks' probabilities live and
    // leaves no registers for the fragments in flight.
    static_assert(NJ == 1, "the region schedule assumes one query block per wave");
    constexpr int PFD = 3;
    auto region = [&](auto has_pv, auto has_qk, auto has_probs, const __bf16* K, const __bf16* V, int kbp, int kbq,
                      const bf16x8 (&Pold)[NJ][2], f32x16 (&Snew)[NJ], const f32x16 (&Scur)[NJ],
                      bf16x8 (&Pnew)[NJ][2]) __attribute__((always_inline)) {
        constexpr bool HP = decltype(has_pv)::value, HQ = decltype(has_qk)::value;
        constexpr bool HPR = decltype(has_probs)::value;
        constexpr int M = (HP ? 2 * NDB : 0) + (HQ ? NC : 0);   // MFMAs in the region
        constexpr int PER = HPR ? 16 / M : 0;                    // exponentials per MFMA
        auto is_pv = [](int m) { return (HP && HQ) ? (m & 1) == 0 : HP; };
        auto idx = [](int m) { return (HP && HQ) ? (m >> 1) : m; };
        auto frag = [&](int m) __attribute__((always_inline)) {
            return is_pv(m) ? vfrag(V, kbp, idx(m)) : kfrag(K, kbq, idx(m));
        };
        bf16x8 F[M];
#pragma unroll
        for (int m = 0; m < PFD && m < M; ++m) F[m] = frag(m);
        float pe[16];
        float ls0 = 0.f, ls1 = 0.f;
#pragma unroll
        for (int m = 0; m < M; ++m) {
            if (m + PFD < M) F[m + PFD] = frag(m + PFD);
            if (is_pv(m)) {
                const int t = idx(m), h = t / NDB, db = t % NDB;
                acc[0][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F[m], Pold[0][h], acc[0][db], 0, 0, 0);
            } else {
                // the chain of block kbq starts from -m_ref
                const int c = idx(m);
                Snew[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F[m], qv[0][c], c == 0 ? negm[0] : Snew[0], 0, 0, 0);
            }
            if (HPR) {
                // P = exp2(S - m_ref) as rounded for the MFMA, and the row sums
                // of those rounded values
#pragma unroll
                for (int e = m * PER; e < (m + 1) * PER; ++e) {
                    pe[e] = fast_exp2(Scur[0][e]);
                    if (e & 1) {
                        const int h = e / 8, i = e % 8;
                        Pnew[0][h][i - 1] = (__bf16)pe[e - 1];
                        Pnew[0][h][i] = (__bf16)pe[e];
                        const bf16x2 pr = {Pnew[0][h][i - 1], Pnew[0][h][i]};
                        if (((i - 1) / 2) % 2 == 0) ls0 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ls0, false);
                        else ls1 = __builtin_amdgcn_fdot2_f32_bf16(pr, ones, ls1, false);
                    }
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        if (HPR) {
            l_run[0] += ls0 + ls1;
            asm volatile("" : "+v"(l_run[0]));
            // the probabilities stay in this region too, not beside their PV
            asm volatile("" ::"v"(Pnew[0][0]), "v"(Pnew[0][1]));
        }
    };

    // One tile: S(0) was issued by the caller right after the barrier (a
    // region of its own); then
    // the regions S(1)+softmax(0), PV(0)+S(2)+softmax(1), PV(1)+S(3)+softmax(2),
    // PV(2)+softmax(3) and PV(3).  The rare edge work (masks, reference max)
    // sits in uniform branches between regions and never touches the
    // accumulators.
    static_assert(BN == 128, "four 32-key score blocks per tile");
    auto tile_body = [&](auto buf, int pn, bool edge, bool rem, int k0, f32x16 (&S0)[NJ]) __attribute__((always_inline)) {
        using Other = std::integral_constant<int, 1 - decltype(buf)::value>;
        using T = std::true_type;
        using F = std::false_type;
        const __bf16* K = decltype(buf)::value ? sK1 : sK0;
        const __bf16* V = decltype(buf)::value ? sV1 : sV0;
        f32x16 S1[NJ], S2[NJ], S3[NJ];
        bf16x8 P0[NJ][2], P1[NJ][2], P2[NJ][2], P3[NJ][2];
        if (edge) edge_fix(S0, 0, rem, k0);
        region(F{}, T{}, T{}, K, V, 0, 1, P3, S1, S0, P0);   // P3 unused (no PV)
        if (edge) edge_fix(S1, 1, rem, k0);
        stage_load_v(pn, Other{});
        // the copies have no users in the kernel's data flow; left alone the
        // scheduler sinks them to the tile's end, where the closing wait would
        // then see their whole latency
        __builtin_amdgcn_sched_barrier(0);
        region(T{}, T{}, T{}, K, V, 0, 2, P0, S2, S1, P1);
        if (edge) edge_fix(S2, 2, rem, k0);
        region(T{}, T{}, T{}, K, V, 1, 3, P1, S3, S2, P2);
        if (edge) edge_fix(S3, 3, rem, k0);
        region(T{}, F{}, T{}, K, V, 2, 0, P2, S1, S3, P3);    // S1 unused (no scores)
        region(T{}, F{}, F{}, K, V, 3, 0, P3, S1, S3, P0);    // PV only
    };

    using Buf0 = std::integral_constant<int, 0>;
    using Buf1 = std::integral_constant<int, 1>;
    // tile pi computes from buffer pi & 1 (= buf) and stages tile pi + 1 into the other
    auto tile = [&](int pi, auto buf) __attribute__((always_inline)) {
        using Other = std::integral_constant<int, 1 - decltype(buf)::value>;
        if (pi == nR && pi > pi_lo) load_q(false);   // the local phase starts: stored Q
        // the first score MFMAs go out right after the barrier, ahead of the
        // tile's scalar set-up: a region with S(0) only
        f32x16 s0[NJ];
        {
            bf16x8 noP[NJ][2];   // not read: the region has no PV and no softmax
            f32x16 noS[NJ];
            region(std::false_type{}, std::true_type{}, std::false_type{}, decltype(buf)::value ? sK1 : sK0,
                   decltype(buf)::value ? sV1 : sV0, 0, 0, noP, s0, noS, noP);
        }
        const int pn = pi + 1 < pi_hi ? pi + 1 : pi;   // the last tile refills the idle buffer
        stage_load_k(pn, Other{});
        const bool rem = pi < nR;
        const int k0 = tile_k0(pi);
        bool any_msk = false, any_unset = false;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            // a block whose rows all lie past L (the last query tile of a call
            // whose length is not a multiple of its rows) is never stored: it
            // takes the unmasked path, whose values for it may come out
            // non-finite and are never read.  Left to the masked path it never
            // sets a reference max and so slowed every tile of its workgroup.
            if (pj0[j] >= L) continue;
            bool act, msk;
            block_state(j, rem, k0, act, msk);
            any_msk = any_msk | msk;
            any_unset = any_unset | (m_ref[j] == -INFINITY);
        }
        const bool edge = any_msk || __any(any_unset);
        tile_body(buf, pn, edge, rem, k0, s0);
        wait_vmem();   // the next tile's V has landed in LDS
        __syncthreads();
    };

    if (pi_lo < pi_hi) {
        stage_load_k(pi_lo, Buf0{});
        stage_load_v(pi_lo, Buf0{});
    }
    wait_vmem();
    __syncthreads();
    load_q(pi_lo < nR);
    int pi = pi_lo;
    for (; pi + 1 < pi_hi; pi += 2) {
        tile(pi, Buf0{});
        tile(pi + 1, Buf1{});
    }
    if (pi < pi_hi) tile(pi, Buf0{});

    // ---- epilogue ---------------------------------------------------------------
    // A row whose probabilities overflowed (a later score above its fixed
    // reference by more than the fp32 exponent range) comes out non-finite;
    // it is marked with NaN in element 0 for the fixup pass, which recomputes
    // its workgroup with a running max.
    if (p.n_ksplit > 1) {
        // a split leaves its unnormalised partial (acc, max, sum) per row; a
        // row whose values overflowed (or that read a bad page) carries NaN
        // as its max, which the combine kernel turns into the fixup mark
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const float l_tot = l_run[j] + __shfl_xor(l_run[j], 32);
            bool finite = l_tot < INFINITY;
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int i = 0; i < 16; ++i) finite = finite && fabsf(acc[j][db][i]) < INFINITY;
            const bool row_ok = finite && __shfl_xor((int)finite, 32) && !bad_page;
            if (!qok[j]) continue;
            float* o = p.part + ((((int64_t)ks * p.B + b) * Lq + (my_q[j] - q_off)) * Hq + head[j]) * (D + 4);
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4) {
                    const int d0 = db * 32 + a4 * 8 + hh * 4;
                    *reinterpret_cast<f32x4*>(o + d0) = f32x4{acc[j][db][4 * a4], acc[j][db][4 * a4 + 1],
                                                              acc[j][db][4 * a4 + 2], acc[j][db][4 * a4 + 3]};
                }
            if (hh == 0) {
                o[D] = row_ok ? m_ref[j] : NAN;
                o[D + 1] = l_tot;
            }
        }
        return;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const float l_tot = l_run[j] + __shfl_xor(l_run[j], 32);
        const float inv = 1.f / l_tot;
        bool finite = l_tot > 0.f && l_tot < INFINITY;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
            for (int i = 0; i < 16; ++i) finite = finite && fabsf(acc[j][db][i] * inv) < INFINITY;
        const bool row_ok = finite && __shfl_xor((int)finite, 32) && !bad_page;
        if (!qok[j]) continue;
        const int64_t o = (((int64_t)b * Lq + (my_q[j] - q_off)) * Hq + head[j]) * D;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) {
                const int d0 = db * 32 + a4 * 8 + hh * 4;
                if constexpr (OUT_BF16) {
                    bf16x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = (__bf16)(acc[j][db][4 * a4 + e] * inv);
                    if (d0 == 0 && !row_ok) w[0] = (__bf16)NAN;
                    *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(p.out) + o + d0) = w;
                } else {
                    f32x4 w;
#pragma unroll
                    for (int e = 0; e < 4; ++e) w[e] = acc[j][db][4 * a4 + e] * inv;
                    if (d0 == 0 && !row_ok) w[0] = NAN;
                    *reinterpret_cast<f32x4*>(static_cast<float*>(p.out) + o + d0) = w;
                }
            }
        }
        if (hh == 0 && p.lse)
            p.lse[((int64_t)b * Hq + head[j]) * Lq + (my_q[j] - q_off)] = (m_ref[j] + log2f(l_tot)) * 0.69314718055994531f;
    }
}

// The keys in their corrected view (§3.2 Eq. 5 applied to K): rows
// rot_lo .. rot_lo + nrows - 1 of every (batch, KV head) rotated by their
// correction offset, table row n(k) = k - floor(k/G), rounded to bf16, into
// [B, krot_rows, Hkv, D] by position.  One thread per 8 rotation pairs of a
// row; HBM-bound (one read and one write of K, table rows shared by the KV
// heads of a position through L2).
// The XCD (accelerator complex die, 0..7) the calling wave runs on.
__device__ inline int xcd_index() {
    uint32_t x;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(x));
    return (int)(x & 7u);
}

// Dynamic grid: the next tile for the workgroup of the calling thread, from
// the queue of its own XCD while that lasts (the tiles the static grid would
// have sent there, longest first), then from the other queues in turn; -1
// once every queue is empty.  The counters only grow, so an empty queue stays
// empty.
__device__ inline int next_tile(const PrefillParams& p, int& queue, int& left) {
    while (left > 0) {
        const uint32_t i = atomicAdd(p.sched + queue * kSchedStride, 1u);
        const int64_t t = queue + (int64_t)kSchedQueues * i;
        if (t < p.n_tiles) return (int)t;
        queue = (queue + 1) % kSchedQueues;
        --left;
    }
    return -1;
}

// Static grid (p.sched null): one workgroup per query tile.  Dynamic grid:
// one workgroup per compute unit, each taking tiles until none is left, so
// that an XCD that runs faster than another (their clocks differ under the
// same load) takes over the other's last tiles instead of idling while it
// finishes them.  Every tile is computed as in the static grid, so the
// results are the same.
template <int D, bool OUT_BF16, int MODE, bool PAGED>
__global__ __launch_bounds__(kThreads) void prefill_bf16_kernel(PrefillParams p) {
    __shared__ int s_tile;
    const bool dyn = p.sched != nullptr;
    int queue = 0, left = kSchedQueues;
    if (dyn && threadIdx.x == 0) queue = xcd_index();
    int tile = (int)blockIdx.x;
    for (;;) {
        if (dyn) {
            if (threadIdx.x == 0) s_tile = next_tile(p, queue, left);
            __syncthreads();
            tile = __builtin_amdgcn_readfirstlane(s_tile);
            __syncthreads();   // read by every wave before thread 0 writes the next one
            if (tile < 0) break;
        }
        prefill_tile<D, OUT_BF16, MODE, PAGED>(p, tile);
        if (!dyn) break;
    }
}

__global__ __launch_bounds__(64) void sched_reset_kernel(uint32_t* s) {
    if (threadIdx.x < kSchedQueues) s[threadIdx.x * kSchedStride] = 0u;
}

template <int D, bool PAGED>
__global__ __launch_bounds__(256) void rotate_keys_kernel(const __bf16* __restrict__ k, __bf16* __restrict__ kr,
                                                          const float2* __restrict__ TF, int64_t n_items,
                                                          int64_t nrows, int64_t Lkv, int Hkv, int64_t G,
                                                          PrefillParams pp) {
    constexpr int HALF = D / 2;
    constexpr int CPR = HALF / 8;   // 8-pair items per row
    const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (t >= n_items) return;
    const int64_t item = t / CPR;   // (b, position - rot_lo, head), head fastest
    const int c = (int)(t % CPR);
    const int64_t bp = item / Hkv;
    const int64_t pos = pp.rot_lo + bp % nrows;
    const int64_t n = pos - pos / G;
    const int64_t bb = bp / nrows;
    // the output: row pos of batch entry bb, [B, krot_rows, Hkv, D]
    const int64_t row = (bb * pp.krot_rows + pos) * Hkv + item % Hkv;
    // k holds Lkv rows per batch entry (or pages), the output L
    int64_t crow;
    if constexpr (PAGED) {
        // an entry outside [0, n_pages) reads page 0; the attention kernel
        // marks the rows that use it
        int64_t pg = pp.block_table[bb * pp.max_pages + pos / pp.page_size];
        pg = (pg < 0 || pg >= pp.n_pages) ? 0 : pg;
        crow = pg * pp.page_size + pos % pp.page_size;
    } else {
        crow = bb * Lkv + pos;
    }
    const __bf16* src = k + (crow * Hkv + item % Hkv) * D + 8 * c;
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(src);
    const bf16x8 y = *reinterpret_cast<const bf16x8*>(src + HALF);
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
    __bf16* dst = kr + row * D + 8 * c;
    *reinterpret_cast<bf16x8*>(dst) = xo;
    *reinterpret_cast<bf16x8*>(dst + HALF) = yo;
}

// Log-sum-exp merge of the key splits of each row (§3.3 Eq. 6 with disjoint
// key sets).  One workgroup of 256 threads per (batch, row, head): thread t
// takes 4 output dimensions (t % (D/4)) of every split s = t / (D/4) + g *
// (256 / (D/4)), so all of a row's partials are read in one round trip, and
// the splits' maxima, sums and weighted rows are reduced through LDS.  The
// maxima are in log2 units; splits without keys for the row (max -inf) weigh
// nothing.  A NaN max (overflow, bad page or table) or a non-finite result
// writes NaN in element 0, the mark the fixup pass recomputes.  The splits
// are summed in split order.
constexpr int kCombThreads = 256;
template <int D, bool OUT_BF16>
__global__ __launch_bounds__(kCombThreads) void split_combine_kernel(PrefillParams p) {
    constexpr int D4 = D / 4;
    constexpr int SG = kCombThreads / D4;             // split groups
    constexpr int PER = kMaxKSplit / SG;              // splits per thread at most
    static_assert(SG * PER == kMaxKSplit, "every split has a thread");
    __shared__ float sM[kMaxKSplit], sL[kMaxKSplit];
    __shared__ float4 sA[SG][D4];
    __shared__ float sRow[2];
    const int64_t r = blockIdx.x;                     // (b, row, head), head fastest
    const int64_t rows = p.B * p.Lq * p.Hq;
    const int64_t stride = rows * (D + 4);            // one split's partials
    const float* base = p.part + r * (D + 4);
    const int t = threadIdx.x, d4 = t % D4, sg = t / D4;
    const int n = p.n_ksplit;
    float4 v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int sp = sg + u * SG;
        v[u] = sp < n ? *reinterpret_cast<const float4*>(base + sp * stride + 4 * d4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (t < n) {
        sM[t] = base[t * stride + D];
        sL[t] = base[t * stride + D + 1];
    }
    __syncthreads();
    if (t == 0) {
        float M = -INFINITY;
        bool bad = false;
        for (int sp = 0; sp < n; ++sp) {
            bad = bad || (sM[sp] != sM[sp]);
            M = fmaxf(M, sM[sp]);
        }
        float l = 0.f;
        for (int sp = 0; sp < n; ++sp) {
            const float w = (sM[sp] == -INFINITY) ? 0.f : fast_exp2(sM[sp] - M);
            sM[sp] = w;   // the split's weight from here on
            l += w * sL[sp];
        }
        sRow[0] = bad ? NAN : M;
        sRow[1] = l;
    }
    __syncthreads();
    float4 a = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int sp = sg + u * SG;
        if (sp < n) {
            const float w = sM[sp];
            a.x += w * v[u].x;
            a.y += w * v[u].y;
            a.z += w * v[u].z;
            a.w += w * v[u].w;
        }
    }
    sA[sg][d4] = a;
    __syncthreads();
    if (t >= D4) return;
    a = sA[0][t];
#pragma unroll
    for (int g = 1; g < SG; ++g) {
        const float4 b = sA[g][t];
        a.x += b.x;
        a.y += b.y;
        a.z += b.z;
        a.w += b.w;
    }
    const float M = sRow[0], l = sRow[1];
    const float inv = 1.f / l;
    const float4 o = make_float4(a.x * inv, a.y * inv, a.z * inv, a.w * inv);
    const bool ok = M == M && l > 0.f && l < INFINITY && fabsf(o.x) < INFINITY && fabsf(o.y) < INFINITY &&
                    fabsf(o.z) < INFINITY && fabsf(o.w) < INFINITY;
    // the D/4 threads left are lanes of one wave: any of them that finds its
    // dims non-finite marks the row through element 0
    const bool row_bad = __any(!ok);
    const int64_t off = r * D + 4 * t;
    if constexpr (OUT_BF16) {
        bf16x4 w = {(__bf16)o.x, (__bf16)o.y, (__bf16)o.z, (__bf16)o.w};
        if (t == 0 && row_bad) w[0] = (__bf16)NAN;
        *reinterpret_cast<bf16x4*>(static_cast<__bf16*>(p.out) + off) = w;
    } else {
        float4 w = o;
        if (t == 0 && row_bad) w.x = NAN;
        *reinterpret_cast<float4*>(static_cast<float*>(p.out) + off) = w;
    }
    if (t == 0 && p.lse) {
        const int64_t h = r % p.Hq, row = (r / p.Hq) % p.Lq, b = r / (p.Hq * p.Lq);
        p.lse[(b * p.Hq + h) * p.Lq + row] = (M + log2f(l)) * 0.69314718055994531f;
    }
}

template <int D, bool PAGED>
void rotate_keys(const PrefillParams& p, hipStream_t stream) {
    if (p.G <= 1 || p.rot_lo >= p.L) return;
    const int64_t n_items = p.B * (p.L - p.rot_lo) * p.Hkv * (D / 16);
    hipLaunchKernelGGL((rotate_keys_kernel<D, PAGED>), dim3((unsigned)((n_items + 255) / 256)), dim3(256), 0, stream,
                       static_cast<const __bf16*>(p.k), static_cast<__bf16*>(p.krot), p.TF, n_items, p.L - p.rot_lo,
                       p.Lkv, (int)p.Hkv, p.G, p);
}

template <int D, bool OUT_BF16, int MODE, bool PAGED = false>
hipError_t launch_one(const PrefillParams& p, hipStream_t stream) {
    if (MODE != kLocalWindow && !p.krot_ready) rotate_keys<D, PAGED>(p, stream);
    const int64_t blocks = (int64_t)p.n_qtiles * p.Hkv * p.B * p.n_ksplit;
    // the dynamic grid (one workgroup per compute unit, a workgroup's LDS
    // fills one) pays when the static grid takes more than two rounds
    int dev = 0, n_cu = 0;
    const bool dyn = p.sched && !PAGED && p.n_ksplit == 1 && hipGetDevice(&dev) == hipSuccess &&
                     hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
                     n_cu > 0 && blocks > 2 * (int64_t)n_cu;
    PrefillParams pk = p;
    pk.sched = dyn ? p.sched : nullptr;
    pk.n_tiles = blocks;
    if (dyn) hipLaunchKernelGGL(sched_reset_kernel, dim3(1), dim3(64), 0, stream, p.sched);
    hipLaunchKernelGGL((prefill_bf16_kernel<D, OUT_BF16, MODE, PAGED>), dim3((unsigned)(dyn ? n_cu : blocks)),
                       dim3(kThreads), 0, stream, pk);
    if (p.n_ksplit > 1)
        hipLaunchKernelGGL((split_combine_kernel<D, OUT_BF16>), dim3((unsigned)(p.B * p.Lq * p.Hq)),
                           dim3(kCombThreads), 0, stream, p);
    return hipGetLastError();
}

template <int D, bool OUT_BF16>
hipError_t launch_mode(const PrefillParams& p, hipStream_t stream) {
    if (p.block_table) return launch_one<D, OUT_BF16, kFused, true>(p, stream);   // paged caches: fused only
    switch (p.mode) {
        case kLocalWindow: return launch_one<D, OUT_BF16, kLocalWindow>(p, stream);
        case kRemoteAll: return launch_one<D, OUT_BF16, kRemoteAll>(p, stream);
        case kRemoteWindow: return launch_one<D, OUT_BF16, kRemoteWindow>(p, stream);
        default: return launch_one<D, OUT_BF16, kFused>(p, stream);
    }
}

}  // namespace

hipError_t launch_rotate_keys(const PrefillParams& p, hipStream_t stream) {
    if (p.head_dim == 128) {
        if (p.block_table) rotate_keys<128, true>(p, stream);
        else rotate_keys<128, false>(p, stream);
    } else {
        if (p.block_table) rotate_keys<64, true>(p, stream);
        else rotate_keys<64, false>(p, stream);
    }
    return hipGetLastError();
}

hipError_t launch_prefill_bf16(const PrefillParams& p, int out_dtype, hipStream_t stream) {
    const bool ob = out_dtype == 1;
    if (p.head_dim == 128) return ob ? launch_mode<128, true>(p, stream) : launch_mode<128, false>(p, stream);
    return ob ? launch_mode<64, true>(p, stream) : launch_mode<64, false>(p, stream);
}

}  // namespace jl
