/*
 * jetlong.h -- C ABI of the MI355X (gfx950) Jet-Long bifocal RoPE attention
 * library (libjetlong.so).
 *
 * Method: "Jet-Long: Efficient Long-Context Extension with Dynamic Bifocal
 * RoPE", §3.  For a call that holds L tokens, a query at position q and a key
 * at position k (0-based, k <= q) score
 *     local  (q - k <= w0):  RoPE(x_q, q)    . RoPE(x_k, k)        (§3, Eq. 1)
 *     remote (q - k >  w0):  RoPE(x_q, f(q)) . RoPE(x_k, f(k))
 * with f(x) = floor(x / G) (§3.1, Eq. 3) and G = max(1, ceil(L / w_pretrained))
 * (§3.1, Eq. 2).  The cache holds RoPE(x_k, k) and is never rewritten (§3.2,
 * Eq. 4); the remote view is formed inside each call by rotating stored
 * vectors by f(p) - p (§3.2, Eq. 5): queries and decode keys as they are
 * read, prefill keys once per call into a caller-provided workspace.  The two views are merged exactly inside one online
 * softmax, which is the inclusion-exclusion merge of §3.3 (Eq. 6) with the
 * overlap term cancelled by masking instead of subtraction.
 *
 * Conventions (readings where the pages are silent):
 *   - RoPE pairs channel i with channel i + D/2, theta_i = base^(-2i/D).
 *   - Query head h reads KV head h / (Hq / Hkv).
 *   - sm_scale multiplies the raw dot product; softmax and LSE are fp32,
 *     LSE is a natural logarithm.
 *
 * Memory: every pointer argument named q, k, v, out, lse, k_cache, v_cache,
 * table and workspace is a DEVICE pointer, owned by the caller, and must be
 * 16-byte aligned.  Tensors are dense row-major in the layout given at each
 * call.  The library never allocates device memory, keeps no per-call state
 * and never synchronises: work is enqueued on `hip_stream` (a hipStream_t;
 * NULL = the default stream) and the call returns.
 *
 * Errors: every argument is validated on the host before any HIP call.  A
 * non-zero return leaves every output untouched; jl_last_error() then
 * describes the failure (thread-local, valid until the next call on that
 * thread).  JL_EHIP is returned if a kernel launch fails.
 */
#ifndef JETLONG_H
#define JETLONG_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define JL_API __attribute__((visibility("default")))
#else
#define JL_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

enum {
    JL_OK = 0,
    JL_EINVAL = 1,        /* bad shape, value or pointer                        */
    JL_EUNSUPPORTED = 2,  /* valid but not implemented (head_dim, dtype, GQA)   */
    JL_EHIP = 3,          /* HIP runtime / launch failure                       */
    JL_ESPACE = 4         /* table or workspace smaller than required           */
};

enum { JL_F32 = 0, JL_BF16 = 1 };

/* Message for the last non-OK return on this thread ("" if none). */
JL_API const char* jl_last_error(void);

/* Library ABI version (increments on any signature or layout change). */
JL_API int jl_version(void);

/*
 * jl_device_info -- compute units and peak shader clock (kHz) of HIP device
 * `device`, as the runtime reports them (for rooflines: the dense bf16
 * MFMA peak of a CDNA4 device is n_cu * 4096 FLOP per clock).  Makes HIP
 * calls.  Errors: NULL outputs -> JL_EINVAL, a runtime error -> JL_EHIP.
 */
JL_API int jl_device_info(int device, int* n_cu, int* max_clock_khz);

/*
 * jl_rotated_keys -- host-side state of keys kept in their remote view (a
 * rotated-key cache, or a chunk workspace): rows 0 .. rows-1 hold their keys in the remote view under group
 * size G.  Start from {0, 0}; the library updates it on each call.
 */
typedef struct jl_rotated_keys {
    int64_t G;
    int64_t rows;
} jl_rotated_keys;

/*
 * jl_schedule -- §3.1 Eq. (2) and the correction-angle table for §3.2 Eq. (5).
 *
 *   *G_out = max(1, ceil(L / w_pretrained)).
 *   *table_bytes_needed = bytes of a table covering the correction offsets
 *       n = p - f(p) of every position p < L under this G, i.e. n < n_cover
 *       with n_cover = n(L-1) + 1, for this head_dim.
 *
 * If `table` is non-NULL, the call also enqueues on `hip_stream` a float64
 * kernel that fills the table for (head_dim, rope_base) covering n < n_cover.
 * The entries do not depend on G, and the offsets of a call grow with its L
 * and its G, so one table built for the largest length serves every later
 * call with L no larger, w_pretrained no smaller and the same head_dim and
 * rope_base (decode steps that cross a G change included).  w_pretrained = 1
 * sizes it for any window (n_cover = L).  A call whose offsets the table does
 * not cover, or whose head_dim or rope_base differ, writes NaN outputs.
 *
 * Table layout (opaque to callers; documented for completeness): a 64-byte
 * header {magic, head_dim, n_cover, rope_base}, then two levels of fp32
 * (cos, sin) pairs, each angle formed in float64 and rounded once to fp32:
 * 1024 rows TL[l][i] = (cos, sin)(l * theta_i), then ceil(n_cover / 1024)
 * rows TH[h][i] = (cos, sin)(1024 h * theta_i), i < D/2.  The entry of offset
 * n is the complex product TL[n mod 1024] * TH[n / 1024] (within a few fp32
 * ulp).  Size: (1024 + ceil(n_cover / 1024)) * D * 4 bytes + 64: 0.57 MB for
 * L = 128K at any window, 0.92 MB for L = 2^20 with w_pretrained = 2^18,
 * D = 128.
 *
 * With table == NULL no HIP call is made.  Errors: L < 1, w_pretrained < 1,
 * head_dim not in {64, 128} (JL_EUNSUPPORTED), rope_base <= 1 or not finite,
 * G_out == NULL -> JL_EINVAL; table_bytes < needed -> JL_ESPACE.
 */
JL_API int jl_schedule(int64_t L, int64_t w_pretrained, int64_t head_dim, double rope_base,
                int64_t* G_out, void* table, size_t table_bytes,
                size_t* table_bytes_needed, void* hip_stream);

/*
 * jl_bifocal_prefill_workspace -- device bytes of scratch jl_bifocal_prefill
 * (and jl_bifocal_prefill_fi) needs.  bf16 inputs: when G = max(1,
 * ceil(L / w_pretrained)) > 1 the keys in their remote view (§3.2 Eq. 5),
 * B * L * Hkv * D bf16 laid out like k; then, from the next 256-byte
 * boundary (at offset 0 when G = 1), 1 KiB of counters through which the
 * workgroups of the attention kernel share out its query tiles.  fp32
 * inputs: 0.  Pure host call.
 *
 * Errors: bytes == NULL, B, L, Hkv < 1 or L > 2^30, w_pretrained < 1 ->
 * JL_EINVAL; D not in {64, 128} or in_dtype not JL_F32 / JL_BF16 ->
 * JL_EUNSUPPORTED.
 */
JL_API int jl_bifocal_prefill_workspace(int in_dtype, int64_t B, int64_t L, int64_t Hkv, int64_t D,
                                        int64_t w_pretrained, size_t* bytes);

/*
 * jl_bifocal_prefill -- causal bifocal attention over a whole sequence
 * (§3 Eq. 1 with §3.1 Eqs. 2-3, §3.2 Eq. 5, §3.3 Eq. 6).
 *
 *   q   [B, L, Hq,  D]  in_dtype   stored RoPE(x, p) for positions p = 0..L-1
 *   k   [B, L, Hkv, D]  in_dtype   stored RoPE(x, p)
 *   v   [B, L, Hkv, D]  in_dtype
 *   out [B, L, Hq,  D]  out_dtype
 *   lse [B, Hq, L]      fp32 natural-log softmax denominators, or NULL
 *
 * G is computed from this call's L.  dtypes: in = JL_F32 -> out = JL_F32;
 * in = JL_BF16 -> out in {JL_BF16, JL_F32}.  D in {64, 128}; Hq / Hkv in
 * {1, 2, 4, 8}.  `table` must have been filled by jl_schedule for this D and
 * rope_base with coverage >= L; if its header does not match (D, rope_base,
 * coverage) the kernels write NaN to `out` (the host cannot read it).
 * `workspace` holds workspace_bytes >= jl_bifocal_prefill_workspace(...)
 * bytes of device scratch, owned by the caller; it may be NULL when that
 * size is 0 (fp32 inputs).  Its contents on entry do not matter and are
 * overwritten (the counters are cleared by a launch of the call itself), so
 * two calls in flight at once need two workspaces.
 *
 * Errors: JL_EINVAL for B, L, Hq, Hkv < 1, Hq % Hkv != 0, w0 < 0,
 * w_pretrained < 1, sm_scale not finite or <= 0, NULL or misaligned pointers;
 * JL_EUNSUPPORTED for other D, dtype pairs or GQA ratios; JL_ESPACE if
 * table_bytes is below jl_schedule's requirement for L or workspace_bytes
 * below jl_bifocal_prefill_workspace's.
 */
JL_API int jl_bifocal_prefill(const void* q, const void* k, const void* v, void* out, float* lse,
                       int in_dtype, int out_dtype, int64_t B, int64_t L, int64_t Hq,
                       int64_t Hkv, int64_t D, int64_t w0, int64_t w_pretrained,
                       double rope_base, float sm_scale, const void* table,
                       size_t table_bytes, void* workspace, size_t workspace_bytes,
                       void* hip_stream);

/*
 * jl_bifocal_prefill_unfused_workspace -- device bytes of scratch
 * jl_bifocal_prefill_unfused needs: the keys in their remote view (bf16
 * inputs with G > 1, as for jl_bifocal_prefill), then three fp32 pass
 * outputs [B, L, Hq, D] and three fp32 log-sum-exps [B, Hq, L], each part at
 * a 256-byte boundary, then (bf16 inputs) 1 KiB of tile counters as in
 * jl_bifocal_prefill's workspace.  Pure host call.  Errors as for
 * jl_bifocal_prefill_workspace (Hq < 1 -> JL_EINVAL as well).
 */
JL_API int jl_bifocal_prefill_unfused_workspace(int in_dtype, int64_t B, int64_t L, int64_t Hq,
                                                int64_t Hkv, int64_t D, int64_t w_pretrained,
                                                size_t* bytes);

/*
 * jl_bifocal_prefill_unfused -- the same result as jl_bifocal_prefill,
 * computed the way §3.3 Eq. (6) writes it: three separate causal attention
 * passes, then their inclusion-exclusion merge.
 *
 *   A: stored vectors, keys q - w0 <= k <= q        (the local window)
 *   B: remote view (§3.2 Eq. 5), every key k <= q
 *   C: remote view, keys q - w0 <= k <= q
 *   out = (W_A O_A + W_B O_B - W_C O_C) / (W_A + W_B - W_C),
 *   lse = log(W_A + W_B - W_C)
 *
 * with O_X a pass's normalised output and W_X its softmax denominator (the
 * passes keep fp32 outputs and log-sum-exps in the workspace).  It is the
 * unfused baseline that the fused kernel is measured against; the fused call
 * is the one to use.  Arguments, layouts, dtypes and errors as for
 * jl_bifocal_prefill, except that `workspace` (never NULL) must hold
 * jl_bifocal_prefill_unfused_workspace(...) bytes (JL_ESPACE otherwise).
 * Four or five kernel launches on `hip_stream` (key rotation, A, B, C,
 * merge, plus each pass's overflow check).
 */
JL_API int jl_bifocal_prefill_unfused(const void* q, const void* k, const void* v, void* out,
                                      float* lse, int in_dtype, int out_dtype, int64_t B, int64_t L,
                                      int64_t Hq, int64_t Hkv, int64_t D, int64_t w0,
                                      int64_t w_pretrained, double rope_base, float sm_scale,
                                      const void* table, size_t table_bytes, void* workspace,
                                      size_t workspace_bytes, void* hip_stream);

/*
 * jl_bifocal_prefill_chunk -- a chunk of Lq new tokens appended to a cache
 * (chunked prefill, or several decode tokens at once): the rows at positions
 * L-Lq .. L-1 of jl_bifocal_prefill over L tokens (§3 Eq. 1, §3.2 Eqs. 4-5,
 * §3.3 Eq. 6).  G = max(1, ceil(L / w_pretrained)) comes from L, the count
 * of every key the chunk sees, so a chunk that crosses a multiple of
 * w_pretrained is computed under the new G (the cache is not rewritten).
 *
 *   q       [B, Lq,   Hq,  D]  in_dtype   stored RoPE(x, p), p = L-Lq .. L-1
 *   k_cache [B, Lmax, Hkv, D]  in_dtype   rows 0..L-1 valid (the chunk's own
 *   v_cache [B, Lmax, Hkv, D]  in_dtype   rows already written by the caller)
 *   out     [B, Lq,   Hq,  D]  out_dtype
 *   lse     [B, Hq,   Lq]      fp32, or NULL
 *
 * Cache rows L..Lmax-1 are never read into the result (they may hold
 * anything, NaN included).
 * dtypes, D, GQA ratios and table as for jl_bifocal_prefill.  `workspace`
 * must hold jl_bifocal_prefill_chunk_workspace(in_dtype, B, Lq, Lmax, Hq, Hkv,
 * D, w_pretrained) bytes (NULL when that is 0).  It holds the keys in their
 * remote view, [B, Lmax, Hkv, D] bf16 by position, and the partials of the
 * key splits: when the chunk's query tiles are few (short chunks), each
 * tile's keys are split over several workgroups and merged with the
 * log-sum-exp rule (§3.3 Eq. 6 with disjoint key sets).  A bf16 chunk whose
 * Lq positions give at most 64 (position, query head) pairs per KV head
 * (Lq * Hq / Hkv <= 64, with B * Lq <= 65535 and Hkv dividing 8 or a multiple
 * of 8) runs on the decode kernels instead: one pass over the cache serves
 * every position, remote keys read from the workspace's rotated rows, and
 * the splits' partials [B, Lq, Hq, splits, D + 2] fp32 go to the workspace.
 *
 * `state` (host, may be NULL) describes the workspace's rotated keys: with
 * state->G equal to this call's G, rows below state->rows are not rotated
 * again, only rows state->rows .. L-1; the call then sets state to {G, L}.
 * A chunk on the decode kernels reads rotated rows only below L-1-w0: when
 * the state (same G) already covers those, it rotates nothing and leaves
 * the state as it is.
 * Pass the same workspace and state to the chunks of one sequence (start
 * from {0, 0}, and reset to {0, 0} after rewriting cached keys below
 * state->rows); a chunk then rotates only its own new keys, except when G
 * changes.  With state NULL every key row 0..L-1 is rotated on each call.
 * The cache itself is never written.
 *
 * Errors: as for jl_bifocal_prefill, plus JL_EINVAL unless
 * 1 <= Lq <= L <= Lmax <= 2^30 or if state->rows is outside [0, Lmax].
 */
JL_API int jl_bifocal_prefill_chunk(const void* q, const void* k_cache, const void* v_cache, void* out,
                             float* lse, int in_dtype, int out_dtype, int64_t B, int64_t Lq,
                             int64_t L, int64_t Lmax, int64_t Hq, int64_t Hkv, int64_t D,
                             int64_t w0, int64_t w_pretrained, double rope_base, float sm_scale,
                             const void* table, size_t table_bytes, void* workspace,
                             size_t workspace_bytes, jl_rotated_keys* state, void* hip_stream);

/*
 * jl_bifocal_prefill_chunk_workspace -- bytes of scratch for a chunk of Lq
 * tokens over a cache of Lcap rows per sequence (Lmax for
 * jl_bifocal_prefill_chunk, max_pages * page_size for the paged form): the
 * keys' remote view when G can exceed 1 (bf16 inputs, Lcap > w_pretrained),
 * B * Lcap * Hkv * D * 2 bytes rounded up to 256, then room for the split
 * partials of any chunk of up to Lq tokens: the larger of max(splits * Lq')
 * * B * Hq * (D + 4) fp32 over the chunks Lq' <= Lq that the prefill kernels
 * split, and B * Lq' * Hq * splits * (D + 2) fp32 over those that run on the
 * decode kernels (none when neither applies).  The same size serves every
 * Lq' <= Lq and L <= Lcap.  Pure host call.
 */
JL_API int jl_bifocal_prefill_chunk_workspace(int in_dtype, int64_t B, int64_t Lq, int64_t Lcap, int64_t Hq,
                                              int64_t Hkv, int64_t D, int64_t w_pretrained, size_t* bytes);

/*
 * jl_bifocal_prefill_chunk_paged -- jl_bifocal_prefill_chunk over a paged
 * cache: the chunk's rows at positions L-Lq .. L-1 attend to keys 0..L-1
 * held in pages (§3 Eq. 1, §3.2 Eqs. 4-5, §3.3 Eq. 6), under G(L).
 *
 *   q                [B, Lq, Hq, D]                 bf16
 *   k_pages, v_pages [n_pages, page_size, Hkv, D]   bf16
 *   block_table      [B, max_pages] int32 (device): key position p of
 *                    sequence b is row p % page_size of page
 *                    block_table[b * max_pages + p / page_size]
 *   out, lse         as for jl_bifocal_prefill_chunk
 *
 * page_size must be a positive multiple of 128 (a 128-key tile never
 * crosses a page) and L <= max_pages * page_size <= 2^30.  The workspace
 * holds jl_bifocal_prefill_chunk_workspace(JL_BF16, B, Lq, max_pages *
 * page_size, Hq, Hkv, D, w_pretrained) bytes; the keys in their remote view
 * go there laid out by position, not by page, and `state` works as for
 * jl_bifocal_prefill_chunk.  Results are bit-identical to
 * jl_bifocal_prefill_chunk over the same keys held contiguously.  A block
 * table entry outside [0, n_pages) is never followed: every output row whose
 * workgroup needs that page (at least every row at or after the page's first
 * position; on the decode kernels, every row of the chunk's heads that read
 * it) is written as NaN.
 *
 * Errors: as for jl_bifocal_prefill_chunk, plus JL_EINVAL for a NULL or
 * misaligned block_table, a page_size that is not a positive multiple of 128,
 * n_pages < 1 or max_pages * page_size outside [L, 2^30]; in_dtype other
 * than JL_BF16 -> JL_EUNSUPPORTED.
 */
JL_API int jl_bifocal_prefill_chunk_paged(const void* q, const void* k_pages, const void* v_pages,
                                          const int32_t* block_table, void* out, float* lse,
                                          int in_dtype, int out_dtype, int64_t B, int64_t Lq,
                                          int64_t L, int64_t n_pages, int64_t page_size,
                                          int64_t max_pages, int64_t Hq, int64_t Hkv, int64_t D,
                                          int64_t w0, int64_t w_pretrained, double rope_base,
                                          float sm_scale, const void* table, size_t table_bytes,
                                          void* workspace, size_t workspace_bytes, jl_rotated_keys* state,
                                          void* hip_stream);

/*
 * jl_bifocal_decode_workspace -- bytes of fp32 scratch that jl_bifocal_decode
 * (and its paged, rotated-key and interpolation forms) needs for steps that
 * attend up to L keys: the split-KV partials (acc[D], max, sum) of every
 * query head, B * Hq * min(ceil(L/32), 256) * (D + 2) floats.  Pure host call.
 * Calls that share a workspace must not overlap in time (keep them on one
 * stream).
 */
JL_API int jl_bifocal_decode_workspace(int64_t B, int64_t Hq, int64_t D, int64_t L, size_t* bytes);

/*
 * jl_bifocal_decode -- one generation step (§3.2: cached keys are read under
 * the G of the current length; the cache is not rewritten).
 *
 *   q        [B, 1, Hq, D]      bf16, the new token's query at position L-1
 *   k_cache  [B, Lmax, Hkv, D]  bf16, rows 0..L-1 valid (the caller has
 *   v_cache  [B, Lmax, Hkv, D]  bf16   already written the new row L-1)
 *   out      [B, 1, Hq, D]      out_dtype (JL_BF16 or JL_F32)
 *   lse      [B, Hq]            fp32 natural log, or NULL
 *
 * L counts every key including the new one; G = max(1, ceil(L/w_pretrained)).
 * Keys with (L-1) - k <= w0 are local, the rest remote.  Cache rows L..Lmax-1
 * are never read into the result (they may hold anything, NaN included).
 * `workspace` must
 * hold jl_bifocal_decode_workspace(B, Hq, D, L) bytes.  in_dtype must be
 * JL_BF16.  Errors as for prefill, plus L > Lmax -> JL_EINVAL and a short
 * workspace -> JL_ESPACE.
 */
JL_API int jl_bifocal_decode(const void* q, const void* k_cache, const void* v_cache, void* out,
                      float* lse, int in_dtype, int out_dtype, int64_t B, int64_t L,
                      int64_t Lmax, int64_t Hq, int64_t Hkv, int64_t D, int64_t w0,
                      int64_t w_pretrained, double rope_base, float sm_scale,
                      const void* table, size_t table_bytes, void* workspace,
                      size_t workspace_bytes, void* hip_stream);

/*
 * jl_bifocal_decode_noalloc -- jl_bifocal_decode with no workspace argument
 * and no allocation, for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Same arguments (minus workspace) and the same result, bit for
 * bit, as jl_bifocal_decode on a contiguous cache.
 *
 * The split partials go to a fixed 16 MiB device array inside the library
 * (one per device, held until the process ends; its address is looked up
 * on the first call on each device).  A step needs
 * B * Hq * n_split * (D + 2) * 4 bytes, n_split <= min(ceil(L/32), 256) from
 * the split plan (2 MiB for B = 1, Hq = 32, D = 128 at L = 128K); a step
 * that needs more than 16 MiB returns JL_ESPACE.  Every call on a device
 * shares that device's array: calls that overlap in time on one device
 * (other streams, other threads) race and must not be issued.  Nothing in
 * the array needs clearing between calls.  Errors otherwise as for
 * jl_bifocal_decode.
 */
JL_API int jl_bifocal_decode_noalloc(const void* q, const void* k_cache, const void* v_cache, void* out,
                                     float* lse, int in_dtype, int out_dtype, int64_t B, int64_t L,
                                     int64_t Lmax, int64_t Hq, int64_t Hkv, int64_t D, int64_t w0,
                                     int64_t w_pretrained, double rope_base, float sm_scale,
                                     const void* table, size_t table_bytes, void* hip_stream);

/*
 * jl_bifocal_decode_unfused_workspace -- bytes of scratch for
 * jl_bifocal_decode_unfused: the decode partials above (rounded up to 256
 * bytes), then three fp32 pass outputs [B, Hq, D] and three log-sum-exps
 * [B, Hq], each rounded up to 256 bytes.  Pure host call.
 */
JL_API int jl_bifocal_decode_unfused_workspace(int64_t B, int64_t Hq, int64_t D, int64_t L, size_t* bytes);

/*
 * jl_bifocal_decode_unfused -- the same step as jl_bifocal_decode (same
 * arguments and result up to rounding), computed as §3.3 Eq. (6) writes it:
 * three separate attention passes over the cache, each a full decode launch,
 *   A: stored view, keys with (L-1) - k <= w0,
 *   B: remote view, every key k <= L-1,
 *   C: remote view, keys with (L-1) - k <= w0,
 * then O = (W_A O_A + W_B O_B - W_C O_C) / (W_A + W_B - W_C) with W_X the
 * passes' softmax denominators.  It is the unfused baseline that the fused
 * step is measured against (§4.8, Tab. 7).  `workspace` must hold
 * jl_bifocal_decode_unfused_workspace(B, Hq, D, L) bytes.  Errors as for
 * jl_bifocal_decode.
 */
JL_API int jl_bifocal_decode_unfused(const void* q, const void* k_cache, const void* v_cache, void* out,
                                     float* lse, int in_dtype, int out_dtype, int64_t B, int64_t L,
                                     int64_t Lmax, int64_t Hq, int64_t Hkv, int64_t D, int64_t w0,
                                     int64_t w_pretrained, double rope_base, float sm_scale,
                                     const void* table, size_t table_bytes, void* workspace,
                                     size_t workspace_bytes, void* hip_stream);

/*
 * jl_bifocal_decode_paged -- jl_bifocal_decode over a paged cache (a block
 * table maps each sequence's positions to fixed-size pages, as serving
 * engines keep their caches).
 *
 *   k_pages, v_pages [n_pages, page_size, Hkv, D]  bf16
 *   block_table      [B, max_pages] int32 (device): key position p of
 *                    sequence b is row p % page_size of page
 *                    block_table[b * max_pages + p / page_size]
 *
 * page_size must be a positive multiple of 32 and max_pages * page_size >=
 * L; the pages that cover positions 0..L-1 must be written, the new token's
 * row included.  Everything else as for jl_bifocal_decode (one L for every
 * sequence of the batch).  A page index outside [0, n_pages) is not followed:
 * the kernel reads page 0 in its place and writes NaN for that sequence's
 * heads.
 *
 * Errors: as for jl_bifocal_decode, plus JL_EINVAL for a NULL or misaligned
 * block_table, a page_size that is not a positive multiple of 32, n_pages < 1
 * or max_pages * page_size < L.
 */
JL_API int jl_bifocal_decode_paged(const void* q, const void* k_pages, const void* v_pages,
                            const int32_t* block_table, void* out, float* lse, int in_dtype,
                            int out_dtype, int64_t B, int64_t L, int64_t n_pages, int64_t page_size,
                            int64_t max_pages, int64_t Hq, int64_t Hkv, int64_t D, int64_t w0,
                            int64_t w_pretrained, double rope_base, float sm_scale, const void* table,
                            size_t table_bytes, void* workspace, size_t workspace_bytes,
                            void* hip_stream);

/*
 * jl_bifocal_decode_rkc -- jl_bifocal_decode with a rotated-key cache: the
 * same step (§3.2 Eqs. 4-5), with every remote key read already in its
 * remote view R(f(k) - k)·k from `krot_cache` instead of being rotated as it
 * is read.  k_cache itself is never written.
 *
 *   krot_cache [B, Lmax, Hkv, D] bf16, caller-owned, laid out like k_cache
 *   state      host jl_rotated_keys describing krot_cache; {0, 0} for a new
 *              cache (or after the caller rewrites rows of k_cache it covers)
 *
 * Before the step the call enqueues, on `hip_stream`, the rotation of the
 * rows that the step needs and `state` does not cover: every row
 * k < L-1-w0 under this step's G.  The step itself also writes row L-1-w0
 * (still local) rotated under G, the row the next step reads as remote, so
 * consecutive steps under one G enqueue no rotation; when G changes (every
 * w_pretrained tokens) the rotation covers every remote row (one pass over
 * the keys).  After a step with remote keys, state = {G, L-w0}.  `state` is
 * updated at enqueue time, so calls that share a cache must be ordered on
 * one stream, and a call captured into a HIP graph does not stand for later
 * steps (its rotation range was decided when it was enqueued).  The result equals jl_bifocal_decode's up to bf16 rounding
 * (the remote view of each key is rounded once, in the cache).  Everything
 * else as for jl_bifocal_decode.
 *
 * A call given a table that does not match it (its output is NaN, as for
 * jl_bifocal_decode) also writes NaN into the rows it rotates, so later
 * steps stay NaN until `state` is reset to {0, 0}.
 *
 * Errors: as for jl_bifocal_decode, plus JL_EINVAL for a NULL or
 * misaligned krot_cache, a NULL state, or state->rows outside [0, Lmax].
 */
JL_API int jl_bifocal_decode_rkc(const void* q, const void* k_cache, const void* v_cache,
                                 void* krot_cache, jl_rotated_keys* state, void* out, float* lse,
                                 int in_dtype, int out_dtype, int64_t B, int64_t L, int64_t Lmax,
                                 int64_t Hq, int64_t Hkv, int64_t D, int64_t w0,
                                 int64_t w_pretrained, double rope_base, float sm_scale,
                                 const void* table, size_t table_bytes, void* workspace,
                                 size_t workspace_bytes, void* hip_stream);

/*
 * jl_table_fill_host -- fill a HOST buffer with the table jl_schedule writes
 * on the device for w_pretrained = 1 (covering every offset n < L; same
 * layout, same float64 formulas compiled for the host).  Lets the table
 * builder be checked without a GPU.  Errors as for jl_schedule.
 */
JL_API int jl_table_fill_host(int64_t L, int64_t head_dim, double rope_base, void* table,
                       size_t table_bytes);

/*
 * jl_rope_interleaved_to_half -- for models whose RoPE rotates adjacent
 * channel pairs (2i, 2i+1) instead of (i, i + D/2): reorder the channels of
 * n_rows rows of D channels so that pair i lands on (i, i + D/2),
 *     out[r][i] = x[r][2i],  out[r][i + D/2] = x[r][2i + 1].
 * Applied to q and k alike (never to v), it makes every call of this
 * library compute that model's scores exactly: a dot product is unchanged
 * by a common permutation of its operands' channels, and each pair's
 * rotation moves with the pair.  The output (a function of v) is not
 * permuted.  (A model can instead permute its q and k projection weights
 * once.)
 *
 *   x, out   device [n_rows, D] of `dtype` (JL_BF16 or JL_F32), 16-byte
 *            aligned, not overlapping; q [B, L, Hq, D] is n_rows = B*L*Hq
 *
 * Enqueued on hip_stream.  Errors: JL_EINVAL (NULL, misaligned or
 * overlapping buffers, unknown dtype, n_rows < 0), JL_EUNSUPPORTED (D not
 * 64 or 128), JL_EHIP.
 */
JL_API int jl_rope_interleaved_to_half(const void* x, void* out, int dtype, int64_t n_rows, int64_t D,
                                       void* hip_stream);

/*
 * ---- Frequency-interpolation remote view (the ablation of §4.7) ----------
 *
 * The same bifocal rule with the remote pairs (q - k > w0) scored after
 * YaRN-style frequency interpolation instead of position aliasing: the
 * local window keeps RoPE(x, p); a remote query or key moves to the phase
 * p * theta'_i, with
 *     theta'_i = (1 - gamma_i) theta_i / s + gamma_i theta_i,
 *     s = max(1, L / w_pretrained)        (the continuous ratio of §3.1),
 *     gamma_i = clamp((r_i - fi_alpha) / (fi_beta - fi_alpha), 0, 1),
 *     r_i = w_pretrained theta_i / (2 pi) (turns of pair i per window).
 * The pages name the variant but give no ramp; this is YaRN's form, with
 * its bounds as arguments (YaRN uses 1 and 32) and no attention
 * temperature.  A stored vector reaches its remote view by the rotation
 * R(-p phi_i), phi_i = theta_i - theta'_i, so the machinery of Eq. 5 applies
 * with position-indexed rows.  Unlike G, s changes with every L.
 */

/*
 * jl_fi_table -- the table of the frequency-interpolation view for one call:
 * (cos, sin)(p * phi_i) for positions p < L in jl_schedule's two-level
 * layout (1024 rows of l * phi_i, then ceil(L / 1024) rows of 1024 h * phi_i;
 * angles formed in float64 and stored fp32), after a header recording (L,
 * w_pretrained, fi_alpha, fi_beta, head_dim, rope_base).  Same size as
 * jl_schedule's table for L with w_pretrained = 1 (*table_bytes_needed);
 * table may be NULL to query the size only.  The
 * fill is enqueued on hip_stream.  jl_bifocal_prefill_fi checks the header
 * and writes NaN outputs when it was built for anything else.
 *
 * Errors: JL_EINVAL (L outside [1, 2^30], w_pretrained < 1, rope_base not
 * finite and > 1, fi_alpha / fi_beta not finite with fi_alpha < fi_beta, a
 * misaligned table), JL_EUNSUPPORTED (head_dim not 64 or 128), JL_ESPACE
 * (table_bytes too small), JL_EHIP.
 */
JL_API int jl_fi_table(int64_t L, int64_t w_pretrained, int64_t head_dim, double rope_base,
                       double fi_alpha, double fi_beta, void* table, size_t table_bytes,
                       size_t* table_bytes_needed, void* hip_stream);

/*
 * jl_fi_table_fill_host -- the same table written into a HOST buffer (the
 * same float64 formulas compiled for the host).  Errors as jl_fi_table,
 * plus JL_EINVAL for a NULL table.
 */
JL_API int jl_fi_table_fill_host(int64_t L, int64_t w_pretrained, int64_t head_dim, double rope_base,
                                 double fi_alpha, double fi_beta, void* table, size_t table_bytes);

/*
 * jl_bifocal_prefill_fi -- jl_bifocal_prefill with the remote pairs in the
 * frequency-interpolation view.  Arguments, layouts, workspace
 * (jl_bifocal_prefill_workspace with the same w_pretrained) and errors as
 * jl_bifocal_prefill, except that `table` comes from jl_fi_table for this
 * (L, w_pretrained, fi_alpha, fi_beta), and fi_alpha / fi_beta are checked
 * as there.  When L <= w_pretrained (s = 1) the result is plain causal
 * attention.
 */
JL_API int jl_bifocal_prefill_fi(const void* q, const void* k, const void* v, void* out, float* lse,
                                 int in_dtype, int out_dtype, int64_t B, int64_t L, int64_t Hq,
                                 int64_t Hkv, int64_t D, int64_t w0, int64_t w_pretrained,
                                 double rope_base, double fi_alpha, double fi_beta, float sm_scale,
                                 const void* table, size_t table_bytes, void* workspace,
                                 size_t workspace_bytes, void* hip_stream);

/*
 * jl_bifocal_decode_fi -- jl_bifocal_decode with the remote keys in the
 * frequency-interpolation view for this step's L.  It takes no table: s
 * changes every step, so the kernel forms the few rows it reads from
 * per-pair phi_i computed on the host in float64.  Arguments, layouts,
 * workspace and errors as jl_bifocal_decode (no table arguments), plus the
 * fi_alpha / fi_beta check.
 */
JL_API int jl_bifocal_decode_fi(const void* q, const void* k_cache, const void* v_cache, void* out,
                                float* lse, int in_dtype, int out_dtype, int64_t B, int64_t L,
                                int64_t Lmax, int64_t Hq, int64_t Hkv, int64_t D, int64_t w0,
                                int64_t w_pretrained, double rope_base, double fi_alpha,
                                double fi_beta, float sm_scale, void* workspace,
                                size_t workspace_bytes, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* JETLONG_H */
