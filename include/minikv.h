/*
 * minikv.h -- C ABI of libminikv.so, MiniKV-style compressed-KV attention on
 * AMD Instinct MI355X (gfx950).
 *
 * The method (arXiv 2411.18077, as described by the "Pith review of MiniKV:
 * Pushing the Limits of LLM Inference via 2-Bit Layer-Discriminative KV Cache"
 * and its verdict record):
 *   1. prefill attention that also returns, for every key, the attention it
 *      received summed over all query rows (two passes, memory linear in n);
 *   2. a one-time selection of heavy hitters (top-k by that score) plus a
 *      recent window, with per-layer (pyramid) budgets;
 *   3. KIVI-style asymmetric INT2 packing of the selected tokens: keys per
 *      channel over groups of tokens, values per token over groups of
 *      channels, sixteen 2-bit codes per 32-bit word, fp16 scale and zero;
 *   4. decode attention that reads the packed cache and dequantises it in
 *      registers, plus an fp16 residual buffer for newly generated tokens.
 *
 * Conventions for every call
 *  - Return value: MINIKV_OK (0) or a negative status.  On error nothing is
 *    launched and no host-side counter changes; minikv_last_error() gives a
 *    thread-local message.  No C++ exception crosses this boundary.
 *  - Arguments are validated on the host before any HIP call; the first HIP
 *    call of a compute entry point checks (once per device) that the current
 *    device is gfx950.
 *  - Device pointers are caller-owned (the library never allocates device
 *    memory), must be 16-byte aligned and point to contiguous arrays in the
 *    layouts stated below.  fp16 data is passed as raw 16-bit storage.
 *  - `stream` is a hipStream_t (NULL = the default stream); work is enqueued
 *    asynchronously on it.  Host-side counters in minikv_layer_cache are
 *    updated when the call returns, i.e. in stream order.
 *  - Concurrent calls on different caches are allowed; calls on the same
 *    cache or overlapping outputs must be ordered by the caller.
 *
 * Index conventions: a "unit" is one (batch b, kv head h) pair, unit index
 * b * n_kv_heads + h.  Query head hq belongs to kv head hq / (Hq / Hkv).
 */
#ifndef MINIKV_H
#define MINIKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Exported symbols; everything else in the library is hidden. */
#define MINIKV_API __attribute__((visibility("default")))

#define MINIKV_OK 0
#define MINIKV_EINVAL (-1)        /* bad argument: dims, pointer, size      */
#define MINIKV_EUNSUPPORTED (-2)  /* valid but unsupported: device, D, g    */
#define MINIKV_ECAPACITY (-3)     /* packed region or residual would overflow */
#define MINIKV_EHIP (-4)          /* a HIP runtime call or launch failed    */

/* Shapes shared by all calls of one layer.
 *   batch        B >= 1
 *   n_q_heads    Hq >= 1, a multiple of n_kv_heads
 *   n_kv_heads   Hkv >= 1; g = Hq / Hkv must be 1, 2, 4 or 8
 *   head_dim     D, 64 or 128
 *   group_k      Gk: tokens per key quantisation group; 16, 32, 64 or 128
 *   group_v      Gv: channels per value quantisation group; 16, 32, 64 or
 *                128 and dividing D
 *   residual_cap nr: fp16 residual slots per unit (KIVI's streaming buffer,
 *                128 on the MiniKV pages); a multiple of Gk, at most 256.  */
typedef struct minikv_dims {
    int32_t batch;
    int32_t n_q_heads;
    int32_t n_kv_heads;
    int32_t head_dim;
    int32_t group_k;
    int32_t group_v;
    int32_t residual_cap;
} minikv_dims;

/* One layer's compressed cache.  Device arrays (sizes from
 * minikv_cache_layout), cap = capacity:
 *   kq      int32  [B][Hkv][cap][D/16]   word (t, j) holds the 2-bit codes of
 *                                        channels 16j..16j+15 of packed token
 *                                        t; channel 16j+e at bits 2e..2e+1
 *   k_scale fp16   [B][Hkv][cap/Gk][D]   per key group and channel
 *   k_zero  fp16   [B][Hkv][cap/Gk][D]
 *   vq      int32  [B][Hkv][cap/16][D]   word (w, c) holds the codes of
 *                                        packed tokens 16w..16w+15 of channel
 *                                        c; token 16w+e at bits 2e..2e+1
 *           (each word runs along the dimension attention sums over:
 *           channels for q.k, tokens for p.v)
 *   v_scale fp16   [B][Hkv][cap][D/Gv]   per token and channel group
 *   v_zero  fp16   [B][Hkv][cap][D/Gv]
 *   k_res   fp16   [B][Hkv][nr][D]       residual keys, slots 0..n_res-1
 *   v_res   fp16   [B][Hkv][nr][D]
 * Host fields: capacity (packed tokens per unit, multiple of Gk), n_packed
 * (multiple of Gk, <= capacity) and n_res (< nr), maintained by the library.
 * Dequantised value of a code: code * scale + zero, computed in fp32.      */
typedef struct minikv_layer_cache {
    int32_t *kq;
    uint16_t *k_scale;
    uint16_t *k_zero;
    int32_t *vq;
    uint16_t *v_scale;
    uint16_t *v_zero;
    uint16_t *k_res;
    uint16_t *v_res;
    int32_t capacity;
    int32_t n_packed;
    int32_t n_res;
} minikv_layer_cache;

/* ------------------------------------------------------------------ info */

/* Library version as major*10000 + minor*100 + patch. */
MINIKV_API int32_t minikv_version(void);
/* Name of a status code ("MINIKV_OK", ...). */
MINIKV_API const char *minikv_status_str(int32_t status);
/* Message of the last failing call on this thread ("" if none). */
MINIKV_API const char *minikv_last_error(void);

/* ---------------------------------------------------------- host helpers */

/* Per-layer budgets.  Pith review of MiniKV, "Assumptions & free
 * parameters": 25% of the prompt as heavy hitters plus 25% as recent window
 * per layer, and a pyramid (depth d = 7) that interpolates the heavy-hitter
 * budget linearly across layers, larger in lower layers.
 *   r = floor(n * rw_num / rw_den), k = floor(n * hh_num / hh_den);
 *   pyramid != 0 and n_layers > 1: k_min = floor(k / depth),
 *   k_max = 2k - k_min, k_out[l] = k_min + floor((k_max - k_min) *
 *   (n_layers-1-l) / (n_layers-1)); otherwise k_out[l] = k;
 *   every k_out[l] is clamped to n - r.
 * k_out: host array [n_layers]; r_out: host scalar.  EINVAL on bad input. */
MINIKV_API int32_t minikv_pyramid_budgets(int32_t n, int32_t n_layers, int32_t hh_num,
                               int32_t hh_den, int32_t rw_num, int32_t rw_den,
                               int32_t depth, int32_t pyramid, int32_t *k_out,
                               int32_t *r_out);

/* Closed-form cache size of the verdict record's referee report (Appendix I
 * of the paper): K and V over budget*lprompt + lgen tokens at `bits` per
 * element plus fp16 scale and zero per `group` elements, against fp16 K and
 * V over lprompt + lgen tokens.  budget = budget_num / budget_den.  Bytes. */
MINIKV_API int32_t minikv_cache_bytes_closed_form(int32_t n_layers, int32_t n_heads,
                                       int32_t head_dim, int32_t lprompt,
                                       int32_t lgen, int32_t budget_num,
                                       int32_t budget_den, int32_t bits,
                                       int32_t group, uint64_t *minikv_bytes,
                                       uint64_t *full_bytes);

/* Byte sizes of the eight device arrays of a cache with `capacity` packed
 * tokens per unit, in the order kq, k_scale, k_zero, vq, v_scale, v_zero,
 * k_res, v_res.  EINVAL if capacity is not a non-negative multiple of Gk. */
MINIKV_API int32_t minikv_cache_layout(const minikv_dims *dims, int32_t capacity,
                            size_t out_bytes[8]);

/* Workspace bytes of minikv_prefill_select for prompt length n (0 when the
 * caller supplies `lse`; the LSE buffer otherwise).  O(n): the n x n score
 * matrix is never stored. */
MINIKV_API int32_t minikv_prefill_ws_bytes(const minikv_dims *dims, int32_t n,
                                int32_t lse_given, size_t *out);

/* Workspace bytes of minikv_decode_attn for a cache of `capacity` packed
 * tokens (split-KV partial results). */
MINIKV_API int32_t minikv_decode_ws_bytes(const minikv_dims *dims, int32_t capacity,
                               size_t *out);

/* Workspace bytes of minikv_decode_attn_mass for a cache of `capacity`
 * packed tokens: the decode partials plus every token's logit and each
 * head's softmax normaliser. */
MINIKV_API int32_t minikv_decode_mass_ws_bytes(const minikv_dims *dims,
                                               int32_t capacity, size_t *out);

/* ---------------------------------------------------------- compute calls */

/* Prefill attention, both passes (Pith review of MiniKV, "What carries the
 * argument": the prefill kernel returns the attention output and the
 * per-key cumulative attention; Fig. 4: two-pass kernel parallelism).
 *   q    fp16 [B][Hq][n][D];  k, v fp16 [B][Hkv][n][D]
 *   o    fp16 [B][Hq][n][D]   softmax(q k^T / sqrt(D), causal) v
 *   lse  fp32 [B][Hq][n]      natural-log normaliser of each row
 *   col  fp32 [B][Hkv][n]     col[u][j] = sum over the unit's g query heads
 *                             and all rows i >= j of P[h][i][j]
 * n = 0 is a no-op.  EINVAL for null/misaligned pointers or n < 0. */
MINIKV_API int32_t minikv_prefill_attn(const minikv_dims *dims, int32_t n, const void *q,
                            const void *k, const void *v, void *o, float *lse,
                            float *col, void *stream);

/* Persistent heavy-hitter + recent-window selection (Pith review of MiniKV,
 * "What carries the argument": heavy hitters chosen once, at the end of
 * prefill, from the cumulative scores; "Assumptions": plus a recent window).
 *   col  fp32 [B][Hkv][n] (finite values)
 *   sel  int32 [B][Hkv][n_hh + n_recent]: per unit the n_hh candidates of
 *        [0, n - n_recent) with the largest score -- ties to the lower
 *        index -- in ascending order, followed by n-n_recent .. n-1.
 * Requires 0 <= n_recent <= n and 0 <= n_hh <= n - n_recent. */
MINIKV_API int32_t minikv_select(const minikv_dims *dims, int32_t n, const float *col,
                      int32_t n_hh, int32_t n_recent, int32_t *sel,
                      void *stream);

/* minikv_prefill_attn followed by minikv_select.  lse may be NULL, in which
 * case the workspace (minikv_prefill_ws_bytes) holds it; ws may be NULL when
 * lse is given. */
MINIKV_API int32_t minikv_prefill_select(const minikv_dims *dims, int32_t n,
                              const void *q, const void *k, const void *v,
                              void *o, float *col, float *lse, int32_t n_hh,
                              int32_t n_recent, int32_t *sel, void *ws,
                              size_t ws_bytes, void *stream);

/* Quantise and pack the selected tokens of every unit into `cache` (Pith
 * review of MiniKV, "Assumptions": group size 16 for per-channel keys and
 * per-token values; verdict record key_machinery: 16 codes per int32, fp16
 * scale and zero).
 *   k, v fp16 [B][Hkv][n][D]; sel int32 [B][Hkv][n_sel], ascending, in
 *   [0, n).  The kernels clamp every index into [0, n) before reading a row
 *   (a negative index reads row n - 1), so a bad index never reads outside
 *   the unit's rows of k and v; the result for such an index is not
 *   meaningful and is not diagnosed (the indices live in device memory).
 * The first floor(n_sel/Gk)*Gk selected tokens are packed (in the order of
 * sel); the remaining n_sel mod Gk are copied to the fp16 residual.  Sets
 * n_packed and n_res.  Codec per group x_1..x_G (fp32 arithmetic, RNE):
 * scale = fp16((max - min) / 3), zero = min (-0 -> +0), code = the integer
 * nearest to (x - zero) / scale with ties to even, clamped to [0, 3]
 * (0 when scale == 0).  ECAPACITY if floor(n_sel/Gk)*Gk > capacity. */
MINIKV_API int32_t minikv_pack(const minikv_dims *dims, int32_t n, const void *k,
                    const void *v, const int32_t *sel, int32_t n_sel,
                    minikv_layer_cache *cache, void *stream);

/* Append one new token per unit to the fp16 residual (KIVI's streaming
 * buffer, cited by the verdict record; MiniKV keeps nr = 128).  When the
 * residual then holds residual_cap tokens they are packed as above onto the
 * end of the packed region and the residual is emptied.
 *   k_new, v_new fp16 [B][Hkv][D].
 * ECAPACITY, with no side effect, if that flush would exceed capacity.
 * EHIP if a launch fails: the host counters are then unchanged, and what
 * the launches before it enqueued wrote only residual slot n_res and packed
 * tokens past n_packed, i.e. outside the cache's valid contents. */
MINIKV_API int32_t minikv_append(const minikv_dims *dims, minikv_layer_cache *cache,
                      const void *k_new, const void *v_new, void *stream);

/* Decode attention over the cache (verdict record, forward implications:
 * the fixed layout allows fused dequantisation during decoding).
 *   q fp16 [B][Hq][D];  o fp16 [B][Hq][D]
 *   o[b][hq] = softmax_t(q . k_t / sqrt(D)) v_t over the n_packed packed
 *   tokens (dequantised) and the n_res residual tokens of unit
 *   (b, hq / g).
 * ws: at least minikv_decode_ws_bytes(dims, capacity) bytes of scratch for
 *   the split partial results; calls that share a workspace must not overlap
 *   in time.
 * EINVAL if the cache holds no token or the workspace is too small (both
 * checked on the host, before any launch); EUNSUPPORTED if capacity exceeds
 * 511 * 1024 packed tokens. */
MINIKV_API int32_t minikv_decode_attn(const minikv_dims *dims,
                           const minikv_layer_cache *cache, const void *q,
                           void *o, void *ws, size_t ws_bytes, void *stream);

/* minikv_decode_attn for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  Same arguments minus the workspace, same results bit for bit:
 * the split partials go to a 16 MiB array that the library keeps in device
 * memory on every GPU it runs on, until the process ends.  Every call on one
 * GPU shares that array, so calls that overlap in time on one GPU (any
 * streams) race and must be ordered by the caller.  No allocation, no
 * memset.  ECAPACITY if the call's split partials would exceed 16 MiB
 * (units * splits * g * (D + 2) * 4 bytes; e.g. 640 kv heads with 4096
 * packed tokens need 1.7 MB); otherwise the errors of minikv_decode_attn. */
MINIKV_API int32_t minikv_decode_attn_noalloc(const minikv_dims *dims,
                                              const minikv_layer_cache *cache,
                                              const void *q, void *o,
                                              void *stream);

/* minikv_append followed by minikv_decode_attn (the new token attends to
 * itself), with the same results bit for bit.  On a step that does not flush
 * the residual, the append happens inside the decode launch: the kernel reads
 * the new token from k_new/v_new and stores it in its residual slot.  On a
 * flushing step it runs the two calls in order.  Arguments and errors as for
 * the two calls; nothing changes if either would fail. */
MINIKV_API int32_t minikv_append_decode(const minikv_dims *dims,
                                        minikv_layer_cache *cache,
                                        const void *k_new, const void *v_new,
                                        const void *q, void *o, void *ws,
                                        size_t ws_bytes, void *stream);

/* Persistence audit (verdict record for MiniKV, referee_report
 * major_comments[0] and the falsifier field: the heavy hitters chosen at the
 * end of prefill are assumed to stay the tokens decoding attends to, and the
 * test of that is the attention decoding actually pays to each kept token).
 * minikv_decode_attn, and in addition
 *   mass[(b * Hkv + kvh) * mass_stride + t] += sum over the g query heads
 *     of kv head kvh of softmax weight of cache token t
 * for t < n_packed + n_res, in cache order (packed tokens, then residual
 * slots; a flush keeps every token's index).  mass is fp32, caller-owned
 * and caller-zeroed; calls accumulate into it, so after s steps it holds
 * each token's decode-time cumulative attention.  o is bit-identical to
 * minikv_decode_attn's.
 * ws: at least minikv_decode_mass_ws_bytes(dims, capacity) bytes.
 * EINVAL if mass is NULL or mass_stride < n_packed + n_res; otherwise the
 * errors of minikv_decode_attn. */
MINIKV_API int32_t minikv_decode_attn_mass(const minikv_dims *dims,
                                           const minikv_layer_cache *cache,
                                           const void *q, void *o, float *mass,
                                           int32_t mass_stride, void *ws,
                                           size_t ws_bytes, void *stream);

/* ================================================== fused prefill tail
 *
 * The prefill phase's own cost (the Pith review's referee report names a
 * prefill-phase slowdown) ends with a selection and a pack after the two
 * attention passes.  minikv_prefill_select_pack runs the whole tail in one
 * call.  With fuse_select = 1 the heavy-hitter + recent-window selection of
 * a unit runs inside the second pass, in the last workgroup to finish that
 * unit's key columns (no separate selection launch; a unit's selection can
 * overlap the other units' second pass); with 0 the selection kernel runs
 * after the second pass.  The pack of every unit follows.  Either way the
 * results are those of minikv_prefill_select followed by minikv_pack with
 * the same sel, bit for bit.  On MI355X the units of a layer finish their
 * second pass together, so the fused selection (one 256-thread workgroup
 * per unit) lands on the critical path: measured 6% slower at 4096 tokens
 * and equal at 32768 and 131072; 0 is the faster choice there. */

/* Workspace bytes of minikv_prefill_select_pack: the LSE when lse is NULL
 * (lse_given = 0), then one 32-bit completion counter per unit. */
MINIKV_API int32_t minikv_prefill_tail_ws_bytes(const minikv_dims *dims, int32_t n,
                                                int32_t lse_given, size_t *out);

/* Prefill attention, selection and pack of one layer (see above).
 * Arguments as for minikv_prefill_select and minikv_pack (sel: n_hh +
 * n_recent indices per unit, written, then packed into `cache`); ws is
 * required (the counters).  fuse_select: 1 fused, 0 separate (EINVAL
 * otherwise).  Sets cache->n_packed and n_res.  ECAPACITY, with no side
 * effect, if the selection does not fit the cache. */
MINIKV_API int32_t minikv_prefill_select_pack(const minikv_dims *dims, int32_t n,
                                              const void *q, const void *k,
                                              const void *v, void *o, float *col,
                                              float *lse, int32_t n_hh,
                                              int32_t n_recent, int32_t *sel,
                                              minikv_layer_cache *cache,
                                              int32_t fuse_select, void *ws,
                                              size_t ws_bytes, void *stream);

/* ============================================== mixed-precision caches
 *
 * Two neighbours of MiniKV on the same pages keep more than one precision
 * in one layer's cache:
 *  - MiKV ("Don't Discard, but Keep It Small: Context-Preserving KV Cache
 *    Compression with Importance-Aware Adaptive Precision", the authors'
 *    responses [W1] and, on the implementation, [W2]): the tokens an
 *    eviction policy would drop are kept at low precision and the important
 *    ones at high precision; the pairs are regrouped by precision (attention
 *    does not depend on the order of the cached pairs), each group stored
 *    contiguously and attended with its own INTn x FP16 product.
 *  - DiffKV (pith.science verdict record for arXiv 2412.03131,
 *    key_machinery and core_discovery): keys get more bits than values;
 *    tokens whose significance (the average attention they receive from
 *    later tokens, max over a GQA group's query heads) exceeds alpha_h / N
 *    are kept at K8V4, those above alpha_l / N at K4V2, the rest pruned,
 *    decided per kv head.
 *
 * A mixed cache holds up to MINIKV_MAX_SEGMENTS packed segments plus one
 * fp16 residual.  Segment codes of b bits are stored as b/2 planes of 2-bit
 * codes; plane p holds bits 2p..2p+1 of every code, each plane in exactly
 * the kq / vq word layout of minikv_layer_cache, plane-major within a unit:
 *   kq      int32 [B][Hkv][key_bits/2][cap][D/16]
 *   k_scale, k_zero fp16 [B][Hkv][cap/Gk][D]
 *   vq      int32 [B][Hkv][value_bits/2][cap/16][D]
 *   v_scale, v_zero fp16 [B][Hkv][cap][D/Gv]
 * Codec of a b-bit group: scale = fp16((max - min) / (2^b - 1)), zero =
 * min, code = the integer nearest to (x - zero) / scale, ties to even,
 * clamped to [0, 2^b - 1].  (key_bits, value_bits) is one of (2, 2),
 * (4, 4), (4, 2), (8, 4).  Mixed-cache calls need group_v == 16.
 *
 * n_packed is the host-side count of packed tokens per unit; when n_unit
 * (device int32 [B*Hkv]) is set, each unit holds its own count n_unit[u]
 * (a multiple of Gk) and n_packed is an upper bound of them (the decode
 * grid covers n_packed; a caller that reads the counts back may lower it to
 * their maximum).  Decode attends over every segment's packed tokens and
 * the n_res residual tokens in one softmax.  flush_seg names the segment
 * that receives residual flushes; it must not use n_unit. */
#define MINIKV_MAX_SEGMENTS 3

typedef struct minikv_segment {
    int32_t *kq;
    uint16_t *k_scale;
    uint16_t *k_zero;
    int32_t *vq;
    uint16_t *v_scale;
    uint16_t *v_zero;
    int32_t key_bits;
    int32_t value_bits;
    int32_t capacity;
    int32_t n_packed;
    int32_t *n_unit;
} minikv_segment;

typedef struct minikv_mixed_cache {
    minikv_segment seg[MINIKV_MAX_SEGMENTS];
    int32_t n_seg;
    int32_t flush_seg;
    uint16_t *k_res;
    uint16_t *v_res;
    int32_t n_res;
} minikv_mixed_cache;

/* Byte sizes of a segment's six device arrays (kq, k_scale, k_zero, vq,
 * v_scale, v_zero) for `capacity` packed tokens per unit.  EINVAL if the
 * bit widths are not a supported pair or capacity is not a non-negative
 * multiple of Gk. */
MINIKV_API int32_t minikv_segment_layout(const minikv_dims *dims, int32_t key_bits,
                                         int32_t value_bits, int32_t capacity,
                                         size_t out_bytes[6]);

/* Workspace bytes of minikv_pack_mikv: the unselected tokens' indices. */
MINIKV_API int32_t minikv_mikv_ws_bytes(const minikv_dims *dims, int32_t n,
                                        int32_t n_sel, size_t *out);

/* MiKV pack (see above): the n_sel selected tokens of every unit (sel as for
 * minikv_pack: ascending, in [0, n); e.g. the heavy hitters and recent
 * window of minikv_prefill_select, H2O's policy, which MiKV's experiments
 * use) go to seg[0], the other n - n_sel tokens, ascending, to seg[1], each
 * at its own bit widths (MiKV's average of 3 bits: seg[0] INT4 keys and
 * values, seg[1] INT2).  Each segment takes whole key groups; the
 * remaining n_sel mod Gk selected tokens and then the (n - n_sel) mod Gk
 * unselected ones stay fp16 as residual slots 0 .. n_res - 1.  Needs
 * n_seg == 2, flush_seg == 0 (generated tokens join the high-precision
 * segment), no n_unit.  Sets both segments' n_packed and n_res.
 * ws: minikv_mikv_ws_bytes bytes.  ECAPACITY, with no side effect, if a
 * segment or the residual would overflow. */
MINIKV_API int32_t minikv_pack_mikv(const minikv_dims *dims, int32_t n, const void *k,
                                    const void *v, const int32_t *sel, int32_t n_sel,
                                    minikv_mixed_cache *cache, void *ws,
                                    size_t ws_bytes, void *stream);

/* minikv_append for a mixed cache: the flush packs the residual onto the
 * end of seg[flush_seg] at that segment's bit widths. */
MINIKV_API int32_t minikv_append_mixed(const minikv_dims *dims,
                                       minikv_mixed_cache *cache,
                                       const void *k_new, const void *v_new,
                                       void *stream);

/* Workspace bytes of minikv_decode_mixed for this cache's segments (from
 * their capacities). */
MINIKV_API int32_t minikv_decode_mixed_ws_bytes(const minikv_dims *dims,
                                                const minikv_mixed_cache *cache,
                                                size_t *out);

/* Decode attention over a mixed cache: o[b][hq] = softmax over every packed
 * token of every segment and the residual tokens of unit (b, hq / g), the
 * codes of each segment dequantised in registers at its own bit widths.
 * q, o fp16 [B][Hq][D].  EINVAL if the cache holds no token. */
MINIKV_API int32_t minikv_decode_mixed(const minikv_dims *dims,
                                       const minikv_mixed_cache *cache,
                                       const void *q, void *o, void *ws,
                                       size_t ws_bytes, void *stream);

/* Workspace bytes of minikv_prefill_diffkv (the LSE, 0 when given). */
MINIKV_API int32_t minikv_diffkv_ws_bytes(const minikv_dims *dims, int32_t n,
                                          int32_t lse_given, size_t *out);

/* DiffKV prefill: the attention output and LSE of minikv_prefill_attn, and
 * every prompt token's significance
 *   score[b][kvh][j] = max over the g query heads h of kv head kvh of
 *                      (sum over rows i >= j of P[h][i][j]) / (n - j),
 * fp32 [B][Hkv][n] (the per-head column sum, then one fp32 division).
 * lse may be NULL when ws holds minikv_diffkv_ws_bytes bytes. */
MINIKV_API int32_t minikv_prefill_diffkv(const minikv_dims *dims, int32_t n,
                                         const void *q, const void *k, const void *v,
                                         void *o, float *score, float *lse, void *ws,
                                         size_t ws_bytes, void *stream);

/* DiffKV tiers of every unit from its significance scores, thresholds
 * thr = alpha / n in fp32 (one division): c_hi = the count of scores above
 * alpha_hi / n and c_kept = the count above alpha_lo / n, each rounded up
 * to a multiple of Gk (at most floor(n / Gk) * Gk; c_kept >= c_hi).  The
 * high tier is the first c_hi tokens by (score descending, index
 * ascending), the low tier the next c_kept - c_hi; the others are pruned.
 *   idx_hi, idx_lo int32 [B][Hkv][n]: each tier ascending in its first
 *                  n_hi[u] / n_lo[u] entries
 *   n_hi, n_lo     int32 [B*Hkv] (device)
 * alpha_lo <= alpha_hi. */
MINIKV_API int32_t minikv_tier_diffkv(const minikv_dims *dims, int32_t n,
                                      const float *score, float alpha_hi,
                                      float alpha_lo, int32_t *idx_hi,
                                      int32_t *idx_lo, int32_t *n_hi,
                                      int32_t *n_lo, void *stream);

/* DiffKV pack: the high tier into seg[0] (key_bits 8, value_bits 4) and the
 * low tier into seg[1] (4, 2), with per-unit counts: sets seg[0].n_unit =
 * n_hi, seg[1].n_unit = n_lo and both n_packed to floor(n / Gk) * Gk (the
 * bound).  seg[2] (8, 4, no n_unit) receives the generated tokens
 * (flush_seg == 2); its n_packed and n_res are set to 0.  Needs n_seg == 3
 * and each tier segment's capacity >= floor(n / Gk) * Gk. */
MINIKV_API int32_t minikv_pack_diffkv(const minikv_dims *dims, int32_t n, const void *k,
                                      const void *v, const int32_t *idx_hi,
                                      const int32_t *idx_lo, int32_t *n_hi,
                                      int32_t *n_lo, minikv_mixed_cache *cache,
                                      void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MINIKV_H */
