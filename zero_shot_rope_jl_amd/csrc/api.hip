// C ABI of libjetlong.so: argument validation (host only, before any HIP
// call), the schedule of Jet-Long §3.1 Eq. (2), and kernel dispatch.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "internal.h"
#include "jetlong.h"

namespace {

thread_local std::string g_err;

constexpr int64_t kMaxLen = int64_t(1) << 30;   // positions are int32 in the kernels

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int64_t group_size(int64_t L, int64_t w_pretrained) {
    const int64_t g = (L + w_pretrained - 1) / w_pretrained;   // ceil, L >= 1
    return g < 1 ? 1 : g;
}

int check_rope(int64_t head_dim, double rope_base) {
    if (head_dim != 64 && head_dim != 128)
        return fail(JL_EUNSUPPORTED, "head_dim %lld not supported (64 or 128)", (long long)head_dim);
    if (!std::isfinite(rope_base) || !(rope_base > 1.0))
        return fail(JL_EINVAL, "rope_base must be finite and > 1 (got %g)", rope_base);
    return JL_OK;
}

// Ramp bounds of the frequency-interpolation view (turns per pretrained
// window): finite, alpha < beta.
int check_fi_ramp(double alpha, double beta) {
    if (!std::isfinite(alpha) || !std::isfinite(beta) || !(alpha < beta))
        return fail(JL_EINVAL, "fi_alpha and fi_beta must be finite with fi_alpha < fi_beta (got %g, %g)", alpha,
                    beta);
    return JL_OK;
}

// The frequency-interpolation view of one call, or none.
struct FiArgs {
    double alpha, beta;
};

// G handed to the kernels for the frequency-interpolation view: 1 when
// s = 1 (every view is the stored one), else max(2, L), so that the row of
// position p < L, p - floor(p/G), is p.
int64_t fi_group(int64_t L, int64_t w_pretrained) { return L > w_pretrained ? (L > 2 ? L : 2) : 1; }

int check_attention_common(int64_t B, int64_t L, int64_t Hq, int64_t Hkv, int64_t D, int64_t w0,
                           int64_t w_pretrained, double rope_base, float sm_scale, int in_dtype,
                           int out_dtype) {
    if (B < 1 || L < 1 || Hq < 1 || Hkv < 1)
        return fail(JL_EINVAL, "B, L, Hq, Hkv must be >= 1 (got %lld, %lld, %lld, %lld)", (long long)B,
                    (long long)L, (long long)Hq, (long long)Hkv);
    if (L > kMaxLen) return fail(JL_EINVAL, "L %lld exceeds 2^30", (long long)L);
    if (B > 65535) return fail(JL_EINVAL, "B %lld exceeds 65535", (long long)B);
    if (Hq % Hkv != 0) return fail(JL_EINVAL, "Hq %% Hkv != 0 (%lld, %lld)", (long long)Hq, (long long)Hkv);
    if (w0 < 0) return fail(JL_EINVAL, "w0 must be >= 0 (got %lld)", (long long)w0);
    if (w_pretrained < 1) return fail(JL_EINVAL, "w_pretrained must be >= 1 (got %lld)", (long long)w_pretrained);
    if (!std::isfinite(sm_scale) || !(sm_scale > 0.f))
        return fail(JL_EINVAL, "sm_scale must be finite and > 0 (got %g)", (double)sm_scale);
    if ((in_dtype != JL_F32 && in_dtype != JL_BF16) || (out_dtype != JL_F32 && out_dtype != JL_BF16))
        return fail(JL_EINVAL, "unknown dtype code (in %d, out %d)", in_dtype, out_dtype);
    if (int rc = check_rope(D, rope_base)) return rc;
    if (in_dtype == JL_F32 && out_dtype != JL_F32)
        return fail(JL_EUNSUPPORTED, "f32 input requires f32 output");
    return JL_OK;
}

}  // namespace

extern "C" {

JL_API const char* jl_last_error(void) { return g_err.c_str(); }

JL_API int jl_device_info(int device, int* n_cu, int* max_clock_khz) {
    g_err.clear();
    if (!n_cu || !max_clock_khz) return fail(JL_EINVAL, "n_cu and max_clock_khz must be non-NULL");
    hipError_t e = hipDeviceGetAttribute(n_cu, hipDeviceAttributeMultiprocessorCount, device);
    if (e == hipSuccess) e = hipDeviceGetAttribute(max_clock_khz, hipDeviceAttributeClockRate, device);
    if (e != hipSuccess) return fail(JL_EHIP, "device %d attributes: %s", device, hipGetErrorString(e));
    return JL_OK;
}

JL_API int jl_version(void) { return 13; }

JL_API int jl_schedule(int64_t L, int64_t w_pretrained, int64_t head_dim, double rope_base, int64_t* G_out,
                       void* table, size_t table_bytes, size_t* table_bytes_needed, void* hip_stream) {
    g_err.clear();
    if (!G_out) return fail(JL_EINVAL, "G_out is NULL");
    if (L < 1 || L > kMaxLen) return fail(JL_EINVAL, "L must be in [1, 2^30] (got %lld)", (long long)L);
    if (w_pretrained < 1) return fail(JL_EINVAL, "w_pretrained must be >= 1 (got %lld)", (long long)w_pretrained);
    if (int rc = check_rope(head_dim, rope_base)) return rc;
    // the offsets of every call with L' <= L and this w_pretrained are below
    // n(L-1) + 1 (they grow with L' and with G)
    const int64_t n_cover = jl::table_need(L, group_size(L, w_pretrained));
    const size_t need = jl::table_bytes_for(n_cover, (int)head_dim);
    if (table_bytes_needed) *table_bytes_needed = need;
    if (table) {
        if (!aligned16(table)) return fail(JL_EINVAL, "table must be 16-byte aligned");
        if (table_bytes < need)
            return fail(JL_ESPACE, "table holds %zu bytes, %zu needed for L=%lld", table_bytes, need, (long long)L);
    }
    *G_out = group_size(L, w_pretrained);
    if (!table) return JL_OK;
    (void)hipGetLastError();
    hipError_t e = jl::launch_table_fill(table, n_cover, (int)head_dim, rope_base,
                                         static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(JL_EHIP, "table fill launch failed: %s", hipGetErrorString(e));
    return JL_OK;
}

JL_API int jl_table_fill_host(int64_t L, int64_t head_dim, double rope_base, void* table, size_t table_bytes) {
    g_err.clear();
    if (!table) return fail(JL_EINVAL, "table is NULL");
    if (L < 1 || L > kMaxLen) return fail(JL_EINVAL, "L must be in [1, 2^30] (got %lld)", (long long)L);
    if (int rc = check_rope(head_dim, rope_base)) return rc;
    const size_t need = jl::table_bytes_for(L, (int)head_dim);
    if (table_bytes < need) return fail(JL_ESPACE, "table holds %zu bytes, %zu needed", table_bytes, need);
    jl::table_fill_host(table, L, (int)head_dim, rope_base);
    return JL_OK;
}

JL_API int jl_fi_table(int64_t L, int64_t w_pretrained, int64_t head_dim, double rope_base, double fi_alpha,
                       double fi_beta, void* table, size_t table_bytes, size_t* table_bytes_needed,
                       void* hip_stream) {
    g_err.clear();
    if (L < 1 || L > kMaxLen) return fail(JL_EINVAL, "L must be in [1, 2^30] (got %lld)", (long long)L);
    if (w_pretrained < 1) return fail(JL_EINVAL, "w_pretrained must be >= 1 (got %lld)", (long long)w_pretrained);
    if (int rc = check_rope(head_dim, rope_base)) return rc;
    if (int rc = check_fi_ramp(fi_alpha, fi_beta)) return rc;
    const size_t need = jl::table_bytes_for(L, (int)head_dim);
    if (table_bytes_needed) *table_bytes_needed = need;
    if (!table) return JL_OK;
    if (!aligned16(table)) return fail(JL_EINVAL, "table must be 16-byte aligned");
    if (table_bytes < need)
        return fail(JL_ESPACE, "table holds %zu bytes, %zu needed for L=%lld", table_bytes, need, (long long)L);
    (void)hipGetLastError();
    hipError_t e = jl::launch_table_fill_fi(table, L, (int)head_dim, rope_base, w_pretrained, fi_alpha, fi_beta,
                                            static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(JL_EHIP, "table fill launch failed: %s", hipGetErrorString(e));
    return JL_OK;
}

JL_API int jl_fi_table_fill_host(int64_t L, int64_t w_pretrained, int64_t head_dim, double rope_base,
                                 double fi_alpha, double fi_beta, void* table, size_t table_bytes) {
    g_err.clear();
    if (!table) return fail(JL_EINVAL, "table is NULL");
    if (L < 1 || L > kMaxLen) return fail(JL_EINVAL, "L must be in [1, 2^30] (got %lld)", (long long)L);
    if (w_pretrained < 1) return fail(JL_EINVAL, "w_pretrained must be >= 1 (got %lld)", (long long)w_pretrained);
    if (int rc = check_rope(head_dim, rope_base)) return rc;
    if (int rc = check_fi_ramp(fi_alpha, fi_beta)) return rc;
    const size_t need = jl::table_bytes_for(L, (int)head_dim);
    if (table_bytes < need) return fail(JL_ESPACE, "table holds %zu bytes, %zu needed", table_bytes, need);
    jl::table_fill_fi_host(table, L, (int)head_dim, rope_base, w_pretrained, fi_alpha, fi_beta);
    return JL_OK;
}

JL_API int jl_rope_interleaved_to_half(const void* x, void* out, int dtype, int64_t n_rows, int64_t D,
                                       void* hip_stream) {
    g_err.clear();
    if (!x || !out) return fail(JL_EINVAL, "x and out must be non-NULL");
    if (dtype != JL_F32 && dtype != JL_BF16) return fail(JL_EINVAL, "unknown dtype code %d", dtype);
    if (D != 64 && D != 128) return fail(JL_EUNSUPPORTED, "head_dim %lld not supported (64 or 128)", (long long)D);
    if (n_rows < 0 || n_rows > (int64_t(1) << 40)) return fail(JL_EINVAL, "n_rows out of range (%lld)", (long long)n_rows);
    if (!aligned16(x) || !aligned16(out)) return fail(JL_EINVAL, "x and out must be 16-byte aligned");
    const int eb = dtype == JL_BF16 ? 2 : 4;
    const uintptr_t xa = reinterpret_cast<uintptr_t>(x), oa = reinterpret_cast<uintptr_t>(out);
    const uintptr_t bytes = (uintptr_t)n_rows * (uintptr_t)D * (uintptr_t)eb;
    if (n_rows > 0 && xa < oa + bytes && oa < xa + bytes) return fail(JL_EINVAL, "x and out overlap");
    (void)hipGetLastError();
    hipError_t e = jl::launch_interleaved_to_half(x, out, eb, n_rows, (int)D, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(JL_EHIP, "channel reorder launch failed: %s", hipGetErrorString(e));
    return JL_OK;
}

}  // extern "C"

namespace {
// Layout of the whole-sequence prefill's workspace (bf16 inputs): the keys
// in their corrected view [B, L, Hkv, D] bf16 when G > 1, then (from a
// 256-byte boundary) the tile counters of the bf16 kernel's dynamic grid.
size_t prefill_ws_sched_offset(int in_dtype, int64_t B, int64_t L, int64_t Hkv, int64_t D, int64_t w_pretrained) {
    const bool rotated_keys = in_dtype == JL_BF16 && group_size(L, w_pretrained) > 1;
    return rotated_keys ? jl::decode_align((size_t)B * (size_t)L * (size_t)Hkv * (size_t)D * 2u) : 0u;
}
}  // namespace

extern "C" {

JL_API int jl_bifocal_prefill_workspace(int in_dtype, int64_t B, int64_t L, int64_t Hkv, int64_t D,
                                        int64_t w_pretrained, size_t* bytes) {
    g_err.clear();
    if (!bytes) return fail(JL_EINVAL, "bytes is NULL");
    if (B < 1 || Hkv < 1 || L < 1 || L > kMaxLen)
        return fail(JL_EINVAL, "B, Hkv, L must be >= 1 and L <= 2^30");
    if (w_pretrained < 1) return fail(JL_EINVAL, "w_pretrained must be >= 1 (got %lld)", (long long)w_pretrained);
    if (D != 64 && D != 128) return fail(JL_EUNSUPPORTED, "head_dim %lld not supported", (long long)D);
    if (in_dtype != JL_F32 && in_dtype != JL_BF16) return fail(JL_EUNSUPPORTED, "unknown in_dtype %d", in_dtype);
    *bytes = prefill_ws_sched_offset(in_dtype, B, L, Hkv, D, w_pretrained) +
             (in_dtype == JL_BF16 ? jl::kSchedBytes : 0u);
    return JL_OK;
}

}  // extern "C"

namespace {

// Argument checks shared by every prefill entry point (all but the
// workspace size): Lq queries at positions L - Lq .. L - 1 over keys 0..L-1
// held in k/v with Lkv rows per batch entry.
int check_prefill(const char* who, const void* q, const void* k, const void* v, const void* out, const float* lse,
                  int in_dtype, int out_dtype, int64_t B, int64_t Lq, int64_t L, int64_t Lkv, int64_t Hq,
                  int64_t Hkv, int64_t D, int64_t w0, int64_t w_pretrained, double rope_base, float sm_scale,
                  const void* table, size_t table_bytes, const void* workspace, bool fi = false) {
    if (!q || !k || !v || !out || !table) return fail(JL_EINVAL, "%s: q, k, v, out and table must be non-NULL", who);
    if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned16(table) ||
        !aligned16(lse) || !aligned16(workspace))
        return fail(JL_EINVAL, "%s: device pointers must be 16-byte aligned", who);
    if (int rc = check_attention_common(B, L, Hq, Hkv, D, w0, w_pretrained, rope_base, sm_scale, in_dtype,
                                        out_dtype))
        return rc;
    if (Lq < 1 || Lq > L || Lkv < L || Lkv > kMaxLen)
        return fail(JL_EINVAL, "%s: need 1 <= Lq <= L <= Lmax <= 2^30 (Lq=%lld, L=%lld, Lmax=%lld)", who,
                    (long long)Lq, (long long)L, (long long)Lkv);
    const int64_t R = Hq / Hkv;
    if (R != 1 && R != 2 && R != 4 && R != 8)
        return fail(JL_EUNSUPPORTED, "GQA ratio Hq/Hkv = %lld not supported (1, 2, 4, 8)", (long long)R);
    // the table rows the call reads (the interpolation view indexes by position)
    const size_t need = jl::table_bytes_for(fi ? L : jl::table_need(L, group_size(L, w_pretrained)), (int)D);
    if (table_bytes < need)
        return fail(JL_ESPACE, "table holds %zu bytes, %zu needed for L=%lld", table_bytes, need, (long long)L);
    const int64_t n_qtiles = (Lq + 256 / R - 1) / (256 / R);
    if (n_qtiles * Hkv * B > 0x7fffffffLL) return fail(JL_EINVAL, "grid too large");
    return JL_OK;
}

jl::PrefillParams make_prefill_params(const void* q, const void* k, const void* v, void* out, float* lse, int64_t B,
                                      int64_t Lq, int64_t L, int64_t Lkv, int64_t Hq, int64_t Hkv, int64_t D,
                                      int64_t w0, int64_t w_pretrained, double rope_base, float sm_scale,
                                      const void* table, void* krot) {
    const int64_t R = Hq / Hkv;
    const int BQ = 256 / (int)R;
    jl::PrefillParams p{};
    p.q = q;
    p.k = k;
    p.v = v;
    p.out = out;
    p.lse = lse;
    p.table = static_cast<const jl::TableHeader*>(table);
    p.TF = reinterpret_cast<const float2*>(static_cast<const char*>(table) + jl::kTableHeaderBytes);
    p.B = B;
    p.L = L;
    p.Lq = Lq;
    p.q_off = L - Lq;
    p.Lkv = Lkv;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.R = (int)R;
    p.BQ = BQ;
    p.n_qtiles = (int)((Lq + BQ - 1) / BQ);
    p.w0 = w0 < L ? w0 : L;   // any w0 >= L-1 makes every pair local
    p.G = group_size(L, w_pretrained);
    p.sm_scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
    p.rope_base = rope_base;
    p.head_dim = (int)D;
    p.krot = krot;
    p.krot_rows = L;
    p.rot_lo = 0;
    p.n_ksplit = 1;
    p.part = nullptr;
    p.mode = jl::kFused;
    p.table_key = jl::TableKey{jl::kTableMagic, 0, 0, 0.0, 0.0};
    return p;
}

// Key splits of a chunk's query tiles: when the query tiles of a chunk give
// fewer than 128 workgroups, each one's key tiles are split over several
// workgroups, whose partials a combine kernel merges: as many splits as keep
// the grid within one workgroup per compute unit (256 on MI355X; a
// workgroup's LDS fills its CU), at least 4 key tiles each and at most 64
// splits.  One full round measured 10-32% faster than about 512 workgroups
// (two rounds) for 32-960-token chunks over a 128K cache.  bf16 inputs only.
// The split count grows with L, so a plan for a larger L bounds it.
constexpr int64_t kPlanCUs = 256;
int64_t chunk_ksplit(int in_dtype, int64_t B, int64_t Lq, int64_t L, int64_t Hq, int64_t Hkv) {
    if (in_dtype != JL_BF16) return 1;
    const int64_t R = Hq / Hkv, BQ = 256 / R;
    const int64_t wgs = (Lq + BQ - 1) / BQ * Hkv * B;
    const int64_t tiles = (L + 127) / 128;
    if (wgs >= 128 || tiles < 8) return 1;
    int64_t s = kPlanCUs / wgs;
    if (s > tiles / 4) s = tiles / 4;
    if (s > jl::kMaxKSplit) s = jl::kMaxKSplit;
    return s < 1 ? 1 : s;
}

// Short chunks run on the decode kernels: when the chunk's Lq positions of
// the R query heads of a KV head make at most 64 MFMA columns (bf16 caches),
// a chunk is a decode step with several query positions, which reads the
// cache once for all of them (and its remote keys from the chunk's rotated
// keys) instead of walking 256-row query tiles.  Returns the column groups
// of 16: 1 (the split kernel), 2 or 4 (the kernel that stages keys in LDS
// for every group), or 0 for the prefill kernels.
int chunk_decode_groups(int in_dtype, int64_t B, int64_t Lq, int64_t Hq, int64_t Hkv) {
    if (in_dtype != JL_BF16) return 0;
    if (Hkv % 8 != 0 && 8 % Hkv != 0) return 0;
    if (B * Lq > 65535) return 0;   // the combine's grid holds (batch, position) in y
    return jl::decode_groups(Lq, Hq / Hkv);
}

// Bytes of the decode kernels' split partials for chunks of up to Lq tokens
// over up to Lcap keys, [B, lq, Hq, n_split, D + 2] fp32: for each column
// group count, its longest chunk and the most splits its plan can give.
size_t chunk_decode_part_bytes(int in_dtype, int64_t B, int64_t Lq, int64_t Lcap, int64_t Hq, int64_t Hkv,
                               int64_t D) {
    size_t best = 0;
    const int64_t R = Hq / Hkv;
    for (int ng = 1; ng <= 4; ng *= 2) {
        int64_t lq = 16 * ng / R < Lq ? 16 * ng / R : Lq;
        if (lq < 1 || chunk_decode_groups(in_dtype, B, lq, Hq, Hkv) != ng) continue;
        int64_t n_split;
        if (ng == 1) {
            // the split kernel: up to 4 KV heads per workgroup
            const int64_t groups = B * (Hkv / jl::decode_heads_per_wg(Hkv));
            const int64_t n_target = groups >= jl::kDecodeTargetWGs ? 1 : jl::kDecodeTargetWGs / groups;
            n_split = n_target < jl::decode_max_splits(Lcap) ? n_target : jl::decode_max_splits(Lcap);
        } else {
            // the staged kernel: one KV head per workgroup, 64-key stages
            const int64_t groups = B * Hkv;
            const int64_t n_target =
                groups >= jl::kDecodeTargetWGs ? 1 : (jl::kDecodeTargetWGs + groups - 1) / groups;
            const int64_t steps = (Lcap + jl::kMultiStageKeys - 1) / jl::kMultiStageKeys;
            n_split = n_target < steps ? n_target : steps;
        }
        const size_t b = (size_t)B * (size_t)lq * (size_t)Hq * (size_t)n_split * (size_t)(D + 2) * sizeof(float);
        if (b > best) best = b;
    }
    return best;
}

// Workspace of chunk calls of up to Lq tokens over a cache of Lcap rows per
// sequence: the keys' remote view [B, Lcap, Hkv, D] bf16 by position (bf16
// inputs, when a G > 1 is possible), then room for the split partials of any
// such call (of the prefill kernels' key splits or of the decode kernels).
struct ChunkLayout {
    size_t krot, part, total;
};

// The partial rows (split x query row) of the largest need among chunks of
// up to Lq tokens over up to Lcap keys.  The split count falls as the query
// tiles grow, so the need peaks at the end of a run of Lq with the same tile
// count; past 128 workgroups nothing is split.
int64_t chunk_part_rows(int in_dtype, int64_t B, int64_t Lq, int64_t Lcap, int64_t Hq, int64_t Hkv) {
    const int64_t BQ = 256 / (Hq / Hkv);
    int64_t best = 0;
    for (int64_t t = 1; (t - 1) * BQ < Lq; ++t) {
        const int64_t lq = t * BQ < Lq ? t * BQ : Lq;
        if (t * Hkv * B >= 128) break;
        const int64_t s = chunk_ksplit(in_dtype, B, lq, Lcap, Hq, Hkv);
        if (s > 1 && s * lq > best) best = s * lq;
    }
    return best;
}

ChunkLayout chunk_layout(int in_dtype, int64_t B, int64_t Lq, int64_t Lcap, int64_t Hq, int64_t Hkv, int64_t D,
                         int64_t w_pretrained) {
    ChunkLayout c{};
    const bool rotated = in_dtype == JL_BF16 && group_size(Lcap, w_pretrained) > 1;
    c.krot = 0;
    c.part = jl::decode_align(rotated ? (size_t)B * (size_t)Lcap * (size_t)Hkv * (size_t)D * 2u : 0u);
    const int64_t rows = chunk_part_rows(in_dtype, B, Lq, Lcap, Hq, Hkv);
    const size_t split_bytes = (size_t)rows * (size_t)B * (size_t)Hq * (size_t)(D + 4) * sizeof(float);
    const size_t dec_bytes = chunk_decode_part_bytes(in_dtype, B, Lq, Lcap, Hq, Hkv, D);
    c.total = c.part + (split_bytes > dec_bytes ? split_bytes : dec_bytes);
    return c;
}

// Chunk set-up shared by the contiguous and paged forms: workspace checks,
// the rotated keys (only the rows the state does not cover are rotated) and
// the key splits.  Updates *state when given.
int setup_chunk(const char* who, jl::PrefillParams& p, int in_dtype, int64_t Lcap, int64_t D, int64_t w_pretrained,
                void* workspace, size_t workspace_bytes, jl_rotated_keys* state) {
    const ChunkLayout c = chunk_layout(in_dtype, p.B, p.Lq, Lcap, p.Hq, p.Hkv, D, w_pretrained);
    if (c.total > 0 && (!workspace || workspace_bytes < c.total))
        return fail(JL_ESPACE, "%s: workspace holds %zu bytes, %zu needed", who,
                    workspace ? workspace_bytes : (size_t)0, c.total);
    if (state && (state->rows < 0 || state->rows > Lcap))
        return fail(JL_EINVAL, "%s: state.rows must be in [0, %lld] (got %lld)", who, (long long)Lcap,
                    (long long)state->rows);
    char* w = static_cast<char*>(workspace);
    p.krot = c.part > 0 ? w + c.krot : nullptr;
    p.krot_rows = Lcap;
    p.n_ksplit = (int)chunk_ksplit(in_dtype, p.B, p.Lq, p.L, p.Hq, p.Hkv);
    const bool dec = chunk_decode_groups(in_dtype, p.B, p.Lq, p.Hq, p.Hkv) > 0;
    p.part = (p.n_ksplit > 1 || dec) ? reinterpret_cast<float*>(w + c.part) : nullptr;
    p.rot_lo = 0;
    if (state && p.G > 1) {
        // rows below state->rows already hold their remote view under this G
        const bool kept = state->G == p.G && state->rows <= p.L;
        // a chunk on the decode kernels reads rotated rows only below its last
        // position's window edge, L-1-w0: when the state covers them, nothing
        // is rotated now (a later chunk that needs more rotates every row it
        // lacks, up to its own L, in one pass)
        const int64_t need = p.L - 1 - p.w0 > 0 ? p.L - 1 - p.w0 : 0;
        if (dec && kept && state->rows >= need) {
            p.rot_lo = p.L;
        } else {
            if (kept) p.rot_lo = state->rows;
            state->G = p.G;
            state->rows = p.L;
        }
    } else if (state) {
        state->G = p.G;
        state->rows = 0;   // G = 1: nothing rotated
    }
    return JL_OK;
}

void set_decode_range(jl::DecodeParams& p, int64_t L, int mode);

// A short chunk (chunk_decode_groups > 0) on the decode kernels: the keys the
// state lacks are rotated as for the prefill kernels, then one split launch
// scores every position's keys (remote ones read rotated from p.krot) and the
// combine writes out [B, Lq, Hq, D] and lse [B, Hq, Lq].
int chunk_on_decode(const char* who, const jl::PrefillParams& p, int out_dtype, hipStream_t stream) {
    (void)hipGetLastError();
    hipError_t e = jl::launch_rotate_keys(p, stream);
    if (e != hipSuccess) return fail(JL_EHIP, "%s key rotation launch failed: %s", who, hipGetErrorString(e));
    jl::DecodeParams d{};
    d.q = p.q;
    d.k = p.k;
    d.v = p.v;
    d.out = p.out;
    d.lse = p.lse;
    d.ws = p.part;
    d.table = p.table;
    d.TF = p.TF;
    d.table_key = p.table_key;
    d.B = p.B;
    d.L = p.L;
    d.Lmax = p.block_table ? 0 : p.Lkv;
    d.block_table = p.block_table;
    d.page_size = p.page_size;
    d.max_pages = p.max_pages;
    d.n_pages = p.n_pages;
    d.Hq = p.Hq;
    d.Hkv = p.Hkv;
    d.R = p.R;
    d.Lq = (int)p.Lq;
    d.n_grp = chunk_decode_groups(JL_BF16, p.B, p.Lq, p.Hq, p.Hkv);
    d.heads_per_wg = d.n_grp == 1 ? jl::decode_heads_per_wg(p.Hkv) : 1;
    d.w0 = p.w0 < p.L ? p.w0 : p.L;
    d.G = p.G;
    d.sm_scale_log2 = p.sm_scale_log2;
    d.rope_base = p.rope_base;
    d.head_dim = p.head_dim;
    d.krot = p.G > 1 ? p.krot : nullptr;
    d.krot_rows = p.krot_rows;
    d.rot_row = -1;
    set_decode_range(d, p.L, jl::kFused);
    e = jl::launch_decode(d, out_dtype, stream);
    if (e != hipSuccess) return fail(JL_EHIP, "%s launch failed: %s", who, hipGetErrorString(e));
    return JL_OK;
}

// Both fused prefill entry points.
int prefill_impl(const char* who, const void* q, const void* k, const void* v, void* out, float* lse, int in_dtype,
                 int out_dtype, int64_t B, int64_t Lq, int64_t L, int64_t Lkv, int64_t Hq, int64_t Hkv, int64_t D,
                 int64_t w0, int64_t w_pretrained, double rope_base, float sm_scale, const void* table,
                 size_t table_bytes, void* workspace, size_t workspace_bytes, void* hip_stream,
                 const FiArgs* fi = nullptr, bool chunk = false, jl_rotated_keys* state = nullptr) {
    g_err.clear();
    if (int rc = check_prefill(who, q, k, v, out, lse, in_dtype, out_dtype, B, Lq, L, Lkv, Hq, Hkv, D, w0,
                               w_pretrained, rope_base, sm_scale, table, table_bytes, workspace, fi != nullptr))
        return rc;
    if (fi)
        if (int rc = check_fi_ramp(fi->alpha, fi->beta)) return rc;
    if (!chunk) {
        size_t ws_need = 0;
        jl_bifocal_prefill_workspace(in_dtype, B, L, Hkv, D, w_pretrained, &ws_need);
        if (ws_need > 0 && (!workspace || workspace_bytes < ws_need))
            return fail(JL_ESPACE, "workspace holds %zu bytes, %zu needed", workspace ? workspace_bytes : (size_t)0,
                        ws_need);
    }
    jl::PrefillParams p = make_prefill_params(q, k, v, out, lse, B, Lq, L, Lkv, Hq, Hkv, D, w0, w_pretrained,
                                              rope_base, sm_scale, table, workspace);
    if (!chunk && in_dtype == JL_BF16)
        p.sched = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) +
                                              prefill_ws_sched_offset(in_dtype, B, L, Hkv, D, w_pretrained));
    if (chunk)
        if (int rc = setup_chunk(who, p, in_dtype, Lkv, D, w_pretrained, workspace, workspace_bytes, state)) return rc;
    if (fi) {
        p.G = fi_group(L, w_pretrained);
        p.table_key = jl::TableKey{jl::kTableMagicFI, L, w_pretrained, fi->alpha, fi->beta};
    }
    if (chunk && chunk_decode_groups(in_dtype, B, Lq, Hq, Hkv) > 0)
        return chunk_on_decode(who, p, out_dtype, static_cast<hipStream_t>(hip_stream));
    (void)hipGetLastError();
    hipError_t e = jl::launch_prefill(p, in_dtype, out_dtype, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(JL_EHIP, "%s launch failed: %s", who, hipGetErrorString(e));
    return JL_OK;
}

// Workspace of the unfused prefill: the rotated keys (bf16 inputs, G > 1),
// then the three passes' fp32 outputs and log-sum-exps, each at a 256-byte
// boundary.
struct UnfusedLayout {
    size_t krot, o[3], l[3], sched, total;
};

UnfusedLayout unfused_layout(int in_dtype, int64_t B, int64_t L, int64_t Hq, int64_t Hkv, int64_t D,
                             int64_t w_pretrained) {
    auto up = [](size_t x) { return (x + 255u) & ~(size_t)255u; };
    UnfusedLayout u{};
    size_t off = 0;
    const bool rotated_keys = in_dtype == JL_BF16 && group_size(L, w_pretrained) > 1;
    u.krot = off;
    off = up(off + (rotated_keys ? (size_t)B * (size_t)L * (size_t)Hkv * (size_t)D * 2u : 0u));
    for (int i = 0; i < 3; ++i) {
        u.o[i] = off;
        off = up(off + (size_t)B * (size_t)L * (size_t)Hq * (size_t)D * 4u);
    }
    for (int i = 0; i < 3; ++i) {
        u.l[i] = off;
        off = up(off + (size_t)B * (size_t)Hq * (size_t)L * 4u);
    }
    // bf16 inputs: the tile counters of the bf16 kernel's dynamic grid (each
    // pass clears them before it runs)
    u.sched = off;
    u.total = off + (in_dtype == JL_BF16 ? jl::kSchedBytes : 0u);
    return u;
}

}  // namespace

extern "C" {

JL_API int jl_bifocal_prefill(const void* q, const void* k, const void* v, void* out, float* lse, int in_dtype,
                              int out_dtype, int64_t B, int64_t L, int64_t Hq, int64_t Hkv, int64_t D, int64_t w0,
                              int64_t w_pretrained, double rope_base, float sm_scale, const void* table,
                              size_t table_bytes, void* workspace, size_t workspace_bytes, void* hip_stream) {
    return prefill_impl("prefill", q, k, v, out, lse, in_dtype, out_dtype, B, L, L, L, Hq, Hkv, D, w0,
                        w_pretrained, rope_base, sm_scale, table, table_bytes, workspace, workspace_bytes, hip_stream);
}

JL_API int jl_bifocal_prefill_fi(const void* q, const void* k, const void* v, void* out, float* lse, int in_dtype,
                                 int out_dtype, int64_t B, int64_t L, int64_t Hq, int64_t Hkv, int64_t D, int64_t w0,
                                 int64_t w_pretrained, double rope_base, double fi_alpha, double fi_beta,
                                 float sm_scale, const void* table, size_t table_bytes, void* workspace,
                                 size_t workspace_bytes, void* hip_stream) {
    const FiArgs fi{fi_alpha, fi_beta};
    return prefill_impl("prefill_fi", q, k, v, out, lse, in_dtype, out_dtype, B, L, L, L, Hq, Hkv, D, w0,
                        w_pretrained, rope_base, sm_scale, table, table_bytes, workspace, workspace_bytes, hip_stream,
                        &fi);
}

JL_API int jl_bifocal_prefill_chunk_workspace(int in_dtype, int64_t B, int64_t Lq, int64_t Lcap, int64_t Hq,
                                              int64_t Hkv, int64_t D, int64_t w_pretrained, size_t* bytes) {
    g_err.clear();
    if (!bytes) return fail(JL_EINVAL, "bytes is NULL");
    if (B < 1 || Hq < 1 || Hkv < 1 || Lq < 1 || Lq > Lcap || Lcap > kMaxLen)
        return fail(JL_EINVAL, "need B, Hq, Hkv >= 1 and 1 <= Lq <= Lcap <= 2^30");
    if (Hq % Hkv != 0) return fail(JL_EINVAL, "Hq %% Hkv != 0 (%lld, %lld)", (long long)Hq, (long long)Hkv);
    if (w_pretrained < 1) return fail(JL_EINVAL, "w_pretrained must be >= 1 (got %lld)", (long long)w_pretrained);
    if (D != 64 && D != 128) return fail(JL_EUNSUPPORTED, "head_dim %lld not supported", (long long)D);
    if (in_dtype != JL_F32 && in_dtype != JL_BF16) return fail(JL_EUNSUPPORTED, "unknown in_dtype %d", in_dtype);
    *bytes = chunk_layout(in_dtype, B, Lq, Lcap, Hq, Hkv, D, w_pretrained).total;
    return JL_OK;
}

JL_API int jl_bifocal_prefill_chunk(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                                    int in_dtype, int out_dtype, int64_t B, int64_t Lq, int64_t L, int64_t Lmax,
                                    int64_t Hq, int64_t Hkv, int64_t D, int64_t w0, int64_t w_pretrained,
                                    double rope_base, float sm_scale, const void* table, size_t table_bytes,
                                    void* workspace, size_t workspace_bytes, jl_rotated_keys* state,
                                    void* hip_stream) {
    return prefill_impl("prefill_chunk", q, k_cache, v_cache, out, lse, in_dtype, out_dtype, B, Lq, L, Lmax, Hq,
                        Hkv, D, w0, w_pretrained, rope_base, sm_scale, table, table_bytes, workspace,
                        workspace_bytes, hip_stream, nullptr, true, state);
}

JL_API int jl_bifocal_prefill_unfused_workspace(int in_dtype, int64_t B, int64_t L, int64_t Hq, int64_t Hkv,
                                                int64_t D, int64_t w_pretrained, size_t* bytes) {
    g_err.clear();
    if (!bytes) return fail(JL_EINVAL, "bytes is NULL");
    if (B < 1 || Hq < 1 || Hkv < 1 || L < 1 || L > kMaxLen)
        return fail(JL_EINVAL, "B, Hq, Hkv, L must be >= 1 and L <= 2^30");
    if (w_pretrained < 1) return fail(JL_EINVAL, "w_pretrained must be >= 1 (got %lld)", (long long)w_pretrained);
    if (D != 64 && D != 128) return fail(JL_EUNSUPPORTED, "head_dim %lld not supported", (long long)D);
    if (in_dtype != JL_F32 && in_dtype != JL_BF16) return fail(JL_EUNSUPPORTED, "unknown in_dtype %d", in_dtype);
    *bytes = unfused_layout(in_dtype, B, L, Hq, Hkv, D, w_pretrained).total;
    return JL_OK;
}

JL_API int jl_bifocal_prefill_unfused(const void* q, const void* k, const void* v, void* out, float* lse,
                                      int in_dtype, int out_dtype, int64_t B, int64_t L, int64_t Hq, int64_t Hkv,
                                      int64_t D, int64_t w0, int64_t w_pretrained, double rope_base, float sm_scale,
                                      const void* table, size_t table_bytes, void* workspace,
                                      size_t workspace_bytes, void* hip_stream) {
    const char* who = "prefill_unfused";
    g_err.clear();
    if (int rc = check_prefill(who, q, k, v, out, lse, in_dtype, out_dtype, B, L, L, L, Hq, Hkv, D, w0,
                               w_pretrained, rope_base, sm_scale, table, table_bytes, workspace))
        return rc;
    if (!workspace) return fail(JL_EINVAL, "%s: workspace must be non-NULL", who);
    const UnfusedLayout u = unfused_layout(in_dtype, B, L, Hq, Hkv, D, w_pretrained);
    if (workspace_bytes < u.total)
        return fail(JL_ESPACE, "workspace holds %zu bytes, %zu needed", workspace_bytes, u.total);
    char* ws = static_cast<char*>(workspace);
    const hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    (void)hipGetLastError();
    // passes A, B, C (B rotates the keys into the workspace, C reuses them)
    const int modes[3] = {jl::kLocalWindow, jl::kRemoteAll, jl::kRemoteWindow};
    for (int i = 0; i < 3; ++i) {
        jl::PrefillParams p = make_prefill_params(q, k, v, ws + u.o[i], reinterpret_cast<float*>(ws + u.l[i]), B, L,
                                                  L, L, Hq, Hkv, D, w0, w_pretrained, rope_base, sm_scale, table,
                                                  ws + u.krot);
        p.mode = modes[i];
        p.krot_ready = i == 2;
        if (in_dtype == JL_BF16) p.sched = reinterpret_cast<uint32_t*>(ws + u.sched);
        const hipError_t e = jl::launch_prefill(p, in_dtype, JL_F32, stream);
        if (e != hipSuccess) return fail(JL_EHIP, "%s pass %d launch failed: %s", who, i, hipGetErrorString(e));
    }
    jl::MergeParams m{};
    m.o_a = reinterpret_cast<const float*>(ws + u.o[0]);
    m.o_b = reinterpret_cast<const float*>(ws + u.o[1]);
    m.o_c = reinterpret_cast<const float*>(ws + u.o[2]);
    m.lse_a = reinterpret_cast<const float*>(ws + u.l[0]);
    m.lse_b = reinterpret_cast<const float*>(ws + u.l[1]);
    m.lse_c = reinterpret_cast<const float*>(ws + u.l[2]);
    m.out = out;
    m.lse = lse;
    m.B = B;
    m.Lq = L;
    m.Hq = Hq;
    m.D = D;
    const hipError_t e = jl::launch_ie_merge(m, out_dtype, stream);
    if (e != hipSuccess) return fail(JL_EHIP, "%s merge launch failed: %s", who, hipGetErrorString(e));
    return JL_OK;
}

JL_API int jl_bifocal_prefill_chunk_paged(const void* q, const void* k_pages, const void* v_pages,
                                          const int32_t* block_table, void* out, float* lse, int in_dtype,
                                          int out_dtype, int64_t B, int64_t Lq, int64_t L, int64_t n_pages,
                                          int64_t page_size, int64_t max_pages, int64_t Hq, int64_t Hkv, int64_t D,
                                          int64_t w0, int64_t w_pretrained, double rope_base, float sm_scale,
                                          const void* table, size_t table_bytes, void* workspace,
                                          size_t workspace_bytes, jl_rotated_keys* state, void* hip_stream) {
    const char* who = "prefill_chunk_paged";
    g_err.clear();
    if (!block_table) return fail(JL_EINVAL, "%s: block_table must be non-NULL", who);
    if (reinterpret_cast<uintptr_t>(block_table) & 3u)
        return fail(JL_EINVAL, "%s: block_table must be 4-byte aligned", who);
    if (int rc = check_prefill(who, q, k_pages, v_pages, out, lse, in_dtype, out_dtype, B, Lq, L, L, Hq, Hkv, D, w0,
                               w_pretrained, rope_base, sm_scale, table, table_bytes, workspace))
        return rc;
    if (page_size < 128 || page_size % 128 != 0 || page_size > kMaxLen)
        return fail(JL_EINVAL, "%s: page_size must be a positive multiple of 128 (got %lld)", who,
                    (long long)page_size);
    if (n_pages < 1 || max_pages < 1 || max_pages > kMaxLen || max_pages * page_size < L ||
        max_pages * page_size > kMaxLen)
        return fail(JL_EINVAL, "%s: need n_pages >= 1 and L <= max_pages * page_size <= 2^30 (%lld, %lld, L=%lld)", who,
                    (long long)n_pages, (long long)max_pages, (long long)L);
    if (in_dtype != JL_BF16) return fail(JL_EUNSUPPORTED, "%s reads a bf16 cache only", who);
    jl::PrefillParams p = make_prefill_params(q, k_pages, v_pages, out, lse, B, Lq, L, L, Hq, Hkv, D, w0,
                                              w_pretrained, rope_base, sm_scale, table, workspace);
    // the rotated keys are kept by position for max_pages * page_size rows
    if (int rc = setup_chunk(who, p, in_dtype, max_pages * page_size, D, w_pretrained, workspace, workspace_bytes,
                             state))
        return rc;
    p.block_table = block_table;
    p.page_size = page_size;
    p.max_pages = max_pages;
    p.n_pages = n_pages;
    if (chunk_decode_groups(in_dtype, B, Lq, Hq, Hkv) > 0)
        return chunk_on_decode(who, p, out_dtype, static_cast<hipStream_t>(hip_stream));
    (void)hipGetLastError();
    hipError_t e = jl::launch_prefill(p, in_dtype, out_dtype, static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(JL_EHIP, "%s launch failed: %s", who, hipGetErrorString(e));
    return JL_OK;
}

JL_API int jl_bifocal_decode_workspace(int64_t B, int64_t Hq, int64_t D, int64_t L, size_t* bytes) {
    g_err.clear();
    if (!bytes) return fail(JL_EINVAL, "bytes is NULL");
    if (B < 1 || Hq < 1 || L < 1 || L > kMaxLen) return fail(JL_EINVAL, "B, Hq, L must be >= 1 and L <= 2^30");
    if (D != 64 && D != 128) return fail(JL_EUNSUPPORTED, "head_dim %lld not supported", (long long)D);
    *bytes = jl::decode_partial_bytes(B, Hq, D, L);
    return JL_OK;
}

}  // extern "C"

namespace {

// Workspace of the unfused decode step: the split partials of the fused
// step (the passes run one after another and share them), then the three
// passes' fp32 outputs [B, Hq, D] and log-sum-exps [B, Hq].
struct UnfusedDecodeLayout {
    size_t o[3], l[3], total;
};

UnfusedDecodeLayout unfused_decode_layout(int64_t B, int64_t Hq, int64_t D, int64_t L) {
    UnfusedDecodeLayout u{};
    size_t off = jl::decode_align(jl::decode_partial_bytes(B, Hq, D, L));
    for (int i = 0; i < 3; ++i) {
        u.o[i] = off;
        off = jl::decode_align(off + (size_t)B * (size_t)Hq * (size_t)D * sizeof(float));
    }
    for (int i = 0; i < 3; ++i) {
        u.l[i] = off;
        off = jl::decode_align(off + (size_t)B * (size_t)Hq * sizeof(float));
    }
    u.total = off;
    return u;
}

// The keys a decode launch reads and how it scores them (p.G and p.w0 set):
// the fused step reads every key, the passes of the unfused step (§3.3
// Eq. 6) read the window's keys in the stored view (A), every key in the
// corrected view (B) or the window's keys in the corrected view (C).  With
// G = 1 the corrected view is the stored one.  The split plan covers the
// keys read.
void set_decode_range(jl::DecodeParams& p, int64_t L, int mode) {
    const int64_t kwin = L - 1 - p.w0 > 0 ? L - 1 - p.w0 : 0;   // first key of the window
    const int64_t all_stored = 0, none_stored = p.G == 1 ? 0 : L;
    switch (mode) {
    case jl::kLocalWindow: p.k_lo = kwin; p.kloc = all_stored; break;
    case jl::kRemoteAll: p.k_lo = 0; p.kloc = none_stored; break;
    case jl::kRemoteWindow: p.k_lo = kwin; p.kloc = none_stored; break;
    default: p.k_lo = 0; p.kloc = p.G == 1 ? 0 : kwin; break;
    }
    p.wave_extra = 0;
    if (p.n_grp > 1) jl::decode_multi_plan(p.B, p.Hkv, L - p.k_lo, &p.n_split, &p.wave_chunk, &p.wave_extra);
    else jl::decode_split_plan(p.B, p.Hkv, L - p.k_lo, &p.n_split, &p.wave_chunk, &p.wave_extra,
                               &p.wave_split_fastest);
}

// Both decode entry points.  Contiguous cache: block_table == NULL, k/v
// [B, Lmax, Hkv, D].  Paged cache: k/v [n_pages, page_size, Hkv, D] and
// block_table [B, max_pages].
int decode_impl(const char* who, const void* q, const void* k_cache, const void* v_cache, const int32_t* block_table,
                int64_t page_size, int64_t max_pages, int64_t n_pages, void* out, float* lse, int in_dtype,
                int out_dtype, int64_t B, int64_t L, int64_t Lmax, int64_t Hq, int64_t Hkv, int64_t D, int64_t w0,
                int64_t w_pretrained, double rope_base, float sm_scale, const void* table, size_t table_bytes,
                void* workspace, size_t workspace_bytes, void* hip_stream, void* krot = nullptr,
                jl_rotated_keys* rk_state = nullptr, const FiArgs* fi = nullptr, bool unfused = false,
                bool noalloc = false) {
    g_err.clear();
    if (!q || !k_cache || !v_cache || !out || (!table && !fi) || (!workspace && !noalloc))
        return fail(JL_EINVAL, "%s: q, the caches, out, table and workspace must be non-NULL", who);
    if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out) || !aligned16(table) ||
        !aligned16(workspace) || !aligned16(lse))
        return fail(JL_EINVAL, "%s: device pointers must be 16-byte aligned", who);
    if (int rc = check_attention_common(B, L, Hq, Hkv, D, w0, w_pretrained, rope_base, sm_scale, in_dtype,
                                        out_dtype))
        return rc;
    if (block_table) {
        if (reinterpret_cast<uintptr_t>(block_table) & 3u)
            return fail(JL_EINVAL, "%s: block_table must be 4-byte aligned", who);
        if (page_size < 32 || page_size % 32 != 0 || page_size > kMaxLen)
            return fail(JL_EINVAL, "%s: page_size must be a positive multiple of 32 (got %lld)", who,
                        (long long)page_size);
        if (n_pages < 1 || max_pages < 1 || max_pages * page_size < L)
            return fail(JL_EINVAL, "%s: need n_pages >= 1 and max_pages * page_size >= L (%lld, %lld, L=%lld)",
                        who, (long long)n_pages, (long long)max_pages, (long long)L);
    } else if (Lmax < L || Lmax > kMaxLen) {
        return fail(JL_EINVAL, "need L <= Lmax <= 2^30 (L=%lld, Lmax=%lld)", (long long)L, (long long)Lmax);
    }
    if (in_dtype != JL_BF16) return fail(JL_EUNSUPPORTED, "decode reads a bf16 cache only");
    const int64_t R = Hq / Hkv;
    if (R != 1 && R != 2 && R != 4 && R != 8 && R != 16)
        return fail(JL_EUNSUPPORTED, "GQA ratio Hq/Hkv = %lld not supported (1..16, power of 2)", (long long)R);
    if (fi) {
        if (int rc = check_fi_ramp(fi->alpha, fi->beta)) return rc;
    } else {
        const size_t need = jl::table_bytes_for(jl::table_need(L, group_size(L, w_pretrained)), (int)D);
        if (table_bytes < need)
            return fail(JL_ESPACE, "table holds %zu bytes, %zu needed for L=%lld", table_bytes, need, (long long)L);
    }
    const UnfusedDecodeLayout ul = unfused_decode_layout(B, Hq, D, L);
    const size_t ws_need = unfused ? ul.total : jl::decode_partial_bytes(B, Hq, D, L);
    if (!noalloc && workspace_bytes < ws_need)
        return fail(JL_ESPACE, "workspace holds %zu bytes, %zu needed", workspace_bytes, ws_need);
    if (Hkv > 65535) return fail(JL_EINVAL, "Hkv exceeds 65535");
    if (Hkv % 8 != 0 && 8 % Hkv != 0)
        return fail(JL_EUNSUPPORTED, "decode needs Hkv dividing 8 or a multiple of 8 (got %lld)", (long long)Hkv);
    if (krot) {
        if (!aligned16(krot)) return fail(JL_EINVAL, "%s: the rotated-key cache must be 16-byte aligned", who);
        if (!rk_state) return fail(JL_EINVAL, "%s: state is NULL", who);
        if (rk_state->rows < 0 || rk_state->rows > Lmax)
            return fail(JL_EINVAL, "%s: state.rows must be in [0, Lmax] (got %lld)", who, (long long)rk_state->rows);
    }

    jl::DecodeParams p{};
    p.q = q;
    p.k = k_cache;
    p.v = v_cache;
    p.out = out;
    p.lse = lse;
    p.table = static_cast<const jl::TableHeader*>(table);
    p.TF = table ? reinterpret_cast<const float2*>(static_cast<const char*>(table) + jl::kTableHeaderBytes) : nullptr;
    p.table_key = jl::TableKey{jl::kTableMagic, 0, 0, 0.0, 0.0};
    p.B = B;
    p.L = L;
    p.Lmax = block_table ? 0 : Lmax;
    p.block_table = block_table;
    p.page_size = page_size;
    p.max_pages = max_pages;
    p.n_pages = n_pages;
    p.Hq = Hq;
    p.Hkv = Hkv;
    p.R = (int)R;
    p.Lq = 1;
    p.n_grp = 1;
    p.heads_per_wg = jl::decode_heads_per_wg(Hkv);
    p.w0 = w0 < L ? w0 : L;
    p.G = group_size(L, w_pretrained);
    p.sm_scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
    p.rope_base = rope_base;
    p.head_dim = (int)D;
    p.krot = krot;
    p.krot_rows = Lmax;
    p.rot_row = -1;
    if (fi) {
        p.G = fi_group(L, w_pretrained);
        p.fi = 1;
        for (int i = 0; i < (int)D / 2; ++i)
            p.fi_phi[i] = jl::fi_phi(rope_base, (int)D, L, w_pretrained, fi->alpha, fi->beta, i);
    }
    set_decode_range(p, L, jl::kFused);
    if (noalloc) {
        // the partials of this step's split plan must fit the fixed scratch
        const size_t need = (size_t)B * (size_t)Hq * (size_t)p.n_split * (size_t)(D + 2) * sizeof(float);
        if (need > jl::kNoAllocScratchBytes)
            return fail(JL_ESPACE, "%s: the step needs %zu bytes of scratch, the library's fixed scratch holds %zu",
                        who, need, jl::kNoAllocScratchBytes);
        (void)hipGetLastError();
        const hipError_t es = jl::noalloc_scratch(&workspace);
        if (es != hipSuccess) return fail(JL_EHIP, "%s: scratch lookup failed: %s", who, hipGetErrorString(es));
    }
    p.ws = static_cast<float*>(workspace);
    (void)hipGetLastError();
    if (krot) {
        // bring the rotated-key cache up to date for this step: every key with
        // (L-1) - k > w0 must be there, rotated under this step's G.  The
        // decode kernel itself then writes row kloc (local now, the first
        // remote row of the next step if G stays), so a step that follows
        // its predecessor under the same G needs no separate rotation.
        const int64_t kloc = p.G == 1 ? 0 : (L - 1 - p.w0 > 0 ? L - 1 - p.w0 : 0);
        int64_t r0 = rk_state->G == p.G ? rk_state->rows : 0;
        if (r0 > kloc) r0 = kloc;
        hipError_t er = jl::launch_rotate_rows(k_cache, krot, p, r0, kloc, static_cast<hipStream_t>(hip_stream));
        if (er != hipSuccess) return fail(JL_EHIP, "%s key rotation launch failed: %s", who, hipGetErrorString(er));
        if (kloc > 0) {
            p.rot_row = kloc;
            if (rk_state->G != p.G) rk_state->rows = 0;
            rk_state->G = p.G;
            if (rk_state->rows < kloc + 1) rk_state->rows = kloc + 1;
        }
    }
    const hipStream_t stream = static_cast<hipStream_t>(hip_stream);
    if (!unfused) {
        hipError_t e = jl::launch_decode(p, out_dtype, stream);
        if (e != hipSuccess) return fail(JL_EHIP, "%s launch failed: %s", who, hipGetErrorString(e));
        return JL_OK;
    }
    // the unfused step: passes A, B and C one after the other (they share the
    // split partials), each writing fp32 output and log-sum-exp, then
    // the inclusion-exclusion merge (§3.3 Eq. 6)
    char* w = static_cast<char*>(workspace);
    const int modes[3] = {jl::kLocalWindow, jl::kRemoteAll, jl::kRemoteWindow};
    for (int i = 0; i < 3; ++i) {
        jl::DecodeParams pi = p;
        set_decode_range(pi, L, modes[i]);
        pi.out = w + ul.o[i];
        pi.lse = reinterpret_cast<float*>(w + ul.l[i]);
        hipError_t e = jl::launch_decode(pi, JL_F32, stream);
        if (e != hipSuccess) return fail(JL_EHIP, "%s pass %d launch failed: %s", who, i, hipGetErrorString(e));
    }
    jl::MergeParams m{};
    m.o_a = reinterpret_cast<const float*>(w + ul.o[0]);
    m.o_b = reinterpret_cast<const float*>(w + ul.o[1]);
    m.o_c = reinterpret_cast<const float*>(w + ul.o[2]);
    m.lse_a = reinterpret_cast<const float*>(w + ul.l[0]);
    m.lse_b = reinterpret_cast<const float*>(w + ul.l[1]);
    m.lse_c = reinterpret_cast<const float*>(w + ul.l[2]);
    m.out = out;
    m.lse = lse;
    m.B = B;
    m.Lq = 1;
    m.Hq = Hq;
    m.D = D;
    hipError_t e = jl::launch_ie_merge(m, out_dtype, stream);
    if (e != hipSuccess) return fail(JL_EHIP, "%s merge launch failed: %s", who, hipGetErrorString(e));
    return JL_OK;
}

}  // namespace

extern "C" {

JL_API int jl_bifocal_decode(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                             int in_dtype, int out_dtype, int64_t B, int64_t L, int64_t Lmax, int64_t Hq,
                             int64_t Hkv, int64_t D, int64_t w0, int64_t w_pretrained, double rope_base,
                             float sm_scale, const void* table, size_t table_bytes, void* workspace,
                             size_t workspace_bytes, void* hip_stream) {
    return decode_impl("decode", q, k_cache, v_cache, nullptr, 0, 0, 0, out, lse, in_dtype, out_dtype, B, L, Lmax,
                       Hq, Hkv, D, w0, w_pretrained, rope_base, sm_scale, table, table_bytes, workspace,
                       workspace_bytes, hip_stream);
}

JL_API int jl_bifocal_decode_unfused_workspace(int64_t B, int64_t Hq, int64_t D, int64_t L, size_t* bytes) {
    g_err.clear();
    if (!bytes) return fail(JL_EINVAL, "bytes is NULL");
    if (B < 1 || Hq < 1 || L < 1 || L > kMaxLen) return fail(JL_EINVAL, "B, Hq, L must be >= 1 and L <= 2^30");
    if (D != 64 && D != 128) return fail(JL_EUNSUPPORTED, "head_dim %lld not supported", (long long)D);
    *bytes = unfused_decode_layout(B, Hq, D, L).total;
    return JL_OK;
}

JL_API int jl_bifocal_decode_unfused(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                                     int in_dtype, int out_dtype, int64_t B, int64_t L, int64_t Lmax, int64_t Hq,
                                     int64_t Hkv, int64_t D, int64_t w0, int64_t w_pretrained, double rope_base,
                                     float sm_scale, const void* table, size_t table_bytes, void* workspace,
                                     size_t workspace_bytes, void* hip_stream) {
    return decode_impl("decode_unfused", q, k_cache, v_cache, nullptr, 0, 0, 0, out, lse, in_dtype, out_dtype, B, L,
                       Lmax, Hq, Hkv, D, w0, w_pretrained, rope_base, sm_scale, table, table_bytes, workspace,
                       workspace_bytes, hip_stream, nullptr, nullptr, nullptr, true);
}

JL_API int jl_bifocal_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                                     int in_dtype, int out_dtype, int64_t B, int64_t L, int64_t Lmax, int64_t Hq,
                                     int64_t Hkv, int64_t D, int64_t w0, int64_t w_pretrained, double rope_base,
                                     float sm_scale, const void* table, size_t table_bytes, void* hip_stream) {
    return decode_impl("decode_noalloc", q, k_cache, v_cache, nullptr, 0, 0, 0, out, lse, in_dtype, out_dtype, B, L,
                       Lmax, Hq, Hkv, D, w0, w_pretrained, rope_base, sm_scale, table, table_bytes, nullptr, 0,
                       hip_stream, nullptr, nullptr, nullptr, false, true);
}

JL_API int jl_bifocal_decode_rkc(const void* q, const void* k_cache, const void* v_cache, void* krot_cache,
                                 jl_rotated_keys* state, void* out, float* lse, int in_dtype, int out_dtype, int64_t B,
                                 int64_t L, int64_t Lmax, int64_t Hq, int64_t Hkv, int64_t D, int64_t w0,
                                 int64_t w_pretrained, double rope_base, float sm_scale, const void* table,
                                 size_t table_bytes, void* workspace, size_t workspace_bytes, void* hip_stream) {
    if (!krot_cache) {
        g_err.clear();
        return fail(JL_EINVAL, "decode_rkc: krot_cache must be non-NULL");
    }
    return decode_impl("decode_rkc", q, k_cache, v_cache, nullptr, 0, 0, 0, out, lse, in_dtype, out_dtype, B, L, Lmax,
                       Hq, Hkv, D, w0, w_pretrained, rope_base, sm_scale, table, table_bytes, workspace,
                       workspace_bytes, hip_stream, krot_cache, state);
}

JL_API int jl_bifocal_decode_fi(const void* q, const void* k_cache, const void* v_cache, void* out, float* lse,
                                int in_dtype, int out_dtype, int64_t B, int64_t L, int64_t Lmax, int64_t Hq,
                                int64_t Hkv, int64_t D, int64_t w0, int64_t w_pretrained, double rope_base,
                                double fi_alpha, double fi_beta, float sm_scale, void* workspace,
                                size_t workspace_bytes, void* hip_stream) {
    const FiArgs fi{fi_alpha, fi_beta};
    return decode_impl("decode_fi", q, k_cache, v_cache, nullptr, 0, 0, 0, out, lse, in_dtype, out_dtype, B, L, Lmax,
                       Hq, Hkv, D, w0, w_pretrained, rope_base, sm_scale, nullptr, 0, workspace, workspace_bytes,
                       hip_stream, nullptr, nullptr, &fi);
}

JL_API int jl_bifocal_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                                   const int32_t* block_table, void* out, float* lse, int in_dtype, int out_dtype,
                                   int64_t B, int64_t L, int64_t n_pages, int64_t page_size, int64_t max_pages,
                                   int64_t Hq, int64_t Hkv, int64_t D, int64_t w0, int64_t w_pretrained,
                                   double rope_base, float sm_scale, const void* table, size_t table_bytes,
                                   void* workspace, size_t workspace_bytes, void* hip_stream) {
    if (!block_table) {
        g_err.clear();
        return fail(JL_EINVAL, "decode_paged: block_table must be non-NULL");
    }
    return decode_impl("decode_paged", q, k_pages, v_pages, block_table, page_size, max_pages, n_pages, out, lse,
                       in_dtype, out_dtype, B, L, 0, Hq, Hkv, D, w0, w_pretrained, rope_base, sm_scale, table,
                       table_bytes, workspace, workspace_bytes, hip_stream);
}

}  // extern "C"
