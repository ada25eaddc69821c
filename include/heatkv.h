/*
 * heatkv.h - C ABI of the MI355X (gfx950) head-scale KV-pruning hot path.
 *
 * What the library computes (sources are the pages the method is described on):
 *   - Next-scale generation: a visual autoregressive model emits token maps of
 *     growing size, one scale at a time, every token of a scale conditioned on
 *     all earlier scales; the KV cache grows with every scale (HeatKV project
 *     page, Abstract; Pith page of arXiv 2605.14877, Figure 2 caption).  Tokens
 *     inside a scale are in raster order (same page, Figure 3 caption).
 *   - Head-scale pruning: whole (layer, head, source-scale) segments are
 *     removed from the cache by a static schedule built offline from S-CAS,
 *     the attention mass each head puts on each earlier scale; early sink
 *     scales are always kept (HeatKV project page, Method steps 2-5; Pith
 *     page, Figure 4 caption).
 *
 * Vocabulary and shapes used below:
 *   L layers, H heads, D head_dim, B batch, K scales with n_s tokens each.
 *   keep[l][h][s] (uint8) = 1 when segment s of head (l, h) is cached once
 *   scale s completes.  The final scale K-1 is never cached; keep[.][.][K-1]
 *   is ignored.
 *   Per-scale tensors q, k_cur, v_cur, out are [B][n_t][H][D], contiguous,
 *   row-major, of the context's dtype.
 *
 * Cache layout (the caller allocates two buffers, one for K and one for V,
 * of hk_layout()'s size; the library only writes and reads them):
 *   cap[l][h]  = sum of n_s over s <= K-2 with keep[l][h][s] = 1;
 *   heads are laid out one after another in row-major (l, h) order and head
 *   (l, h) owns B * cap[l][h] * D elements, as [B][cap[l][h]][D];
 *   after scale k has been appended, rows [0, len_before(l,h,k+1)) of (l,h,b)
 *   hold the kept segments s <= k in scale order, where
 *   len_before(l,h,t) = sum of n_s over kept s < t.
 *
 * Conventions:
 *   - Every function returns HK_OK (0) or a negative HK_E* status and never
 *     aborts; hk_last_error() returns this thread's text of the last failure.
 *   - Device pointers are HIP device memory on the context's device, 16-byte
 *     aligned.  hip_stream is a hipStream_t (NULL = the null stream).  Device
 *     work is enqueued asynchronously on that stream; faults during execution
 *     surface at the caller's next synchronisation.
 *   - The library allocates device memory only in hk_create* (small tables,
 *     S-CAS partial sums, the key-range split workspace and, with 4-bit
 *     storage, a one-layer bf16 scratch) and frees it in hk_destroy; nothing
 *     allocates on the per-scale calls.
 *   - A context is not thread-safe: calls on one context must be serialised
 *     by the caller.  Its per-scale calls share that device workspace, so
 *     calls on one context issued to different streams must not overlap on
 *     the device (order the streams, or use one stream per context).
 */
#ifndef HEATKV_H
#define HEATKV_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define HK_OK 0
#define HK_EINVAL (-1)        /* bad argument: shape, range, null, alignment */
#define HK_EBUDGET (-2)       /* budget below the cost of the sink scales */
#define HK_EORDER (-3)        /* per-layer scale order violated */
#define HK_EHIP (-4)          /* HIP runtime or launch error */
#define HK_EUNSUPPORTED (-5)  /* dtype / head_dim combination not compiled */

/* element types */
#define HK_DTYPE_F32 0
#define HK_DTYPE_BF16 1

/* compile-time limits */
#define HK_MAX_SCALES 16

typedef struct hk_ctx hk_ctx; /* opaque; owned by the library */

/* Text of this thread's last non-OK return ("" if none). Owned by the library,
 * valid until the next call on this thread. */
const char* hk_last_error(void);

/* Build the static keep-mask from an S-CAS table and a memory budget.
 *
 * Follows the HeatKV project page, Method steps 3-5 (rank head-scale pairs by
 * their contribution to future predictions; remove low-ranked pairs to meet
 * the budget; keep the early sink scales; one static, prompt-independent
 * schedule) and the Figure 4 caption of the Pith page of arXiv 2605.14877
 * (per-source-scale orderings O_i of the heads from least to most dependent,
 * pruning set = union of a prefix of each O_i).  Readings taken:
 *   importance(l,h,s) = sum over t = s+1..K-1 of scas[l][h][t][s], summed in
 *     double in ascending t;
 *   prunable scales are n_sink..K-2, each with ordering O_s of the flat head
 *     index f = l*H+h ascending by (importance, f);
 *   F = L*H*sum_{s<=K-2} n_s, budget = floor(budget_frac * F) token slots;
 *   heads kept per prunable scale = min(L*H, floor((budget - sink cost) /
 *     sum of n_s over prunable s)); N = L*H - that; the first N heads of each
 *     O_s are dropped (greedy early pruning with one prefix length).
 *
 *   scale_tokens  host int32 [K], n_s >= 1
 *   scas          host float [L][H][K][K], row t over sources s <= t
 *   budget_frac   in (0, 1]
 *   n_sink        in [0, K-1]
 *   keep_out      host uint8 [L][H][K] (written; keep_out[.][.][K-1] = 0)
 *   retained_out  host int64 [K] or NULL: token slots per sequence held after
 *                 each scale k (sum over kept s <= min(k, K-2) of n_s)
 *   n_pruned_out  host int32 or NULL: N
 * Errors: HK_EINVAL (bad sizes, ranges, NULL), HK_EBUDGET (budget below the
 * sink cost).  K <= HK_MAX_SCALES is not required here. */
int hk_build_schedule(int L, int H, int K, const int32_t* scale_tokens, const float* scas,
                      double budget_frac, int n_sink, uint8_t* keep_out,
                      int64_t* retained_out, int32_t* n_pruned_out);

/* Size of one cache buffer (K or V; both have the same size) for a keep-mask,
 * in elements, and optionally the per-head capacities and element offsets of
 * the layout described at the top of this file.
 *   cache_elems_out  host int64 (required)
 *   cap_out          host int64 [L][H] or NULL
 *   base_out         host int64 [L][H] or NULL
 * Errors: HK_EINVAL. */
int hk_layout(int L, int H, int K, const int32_t* scale_tokens, const uint8_t* keep,
              int B, int D, int64_t* cache_elems_out, int64_t* cap_out, int64_t* base_out);

/* Progressive (lazy) schedule: the pruning set grows from scale to scale and
 * segments of earlier scales are dropped from the middle of a head's cache
 * when it does.
 *
 * Follows the Figure 4 caption of the Pith page of arXiv 2605.14877: after
 * scale k the pruning set G_k is the union over scales i <= k of the prefix
 * of length N_k of the ordering O_i, which is to be gone from the cache once
 * scale k is done; and the signature of its Algorithm 2, CacheSizeAfterLayer(k, l, G_k,
 * G_{k-1}, ...), which tracks the cache size layer by layer inside a scale.
 * Readings taken:
 *   orderings, prunable scales, sinks and the budget floor(budget_frac * F)
 *     are those of hk_build_schedule;
 *   N_k = the smallest N >= N_{k-1} for which the cache fits the budget
 *     (greedy and lazy: nothing is pruned before the budget needs it);
 *   with per_layer != 0 the budget must hold after every layer of scale k,
 *     where layers 0..l hold their segments s <= k outside G_k and layers
 *     l+1.. their segments s <= k-1 outside G_{k-1}; with per_layer == 0
 *     only at the end of each scale.
 *
 *   expire_out   host uint8 [L][H][K]: expire[l][h][s] = the first k >= s
 *                with (l, h, s) in G_k, else K-1 (kept to the end).  The
 *                queries of scales t with s < t <= expire read segment s from
 *                the cache; expire == s means it is never stored.
 *   prefix_out   host int32 [K] or NULL: N_k (N_{K-1} = N_{K-2})
 *   live_out     host int64 [K][L] or NULL: cache size in token slots per
 *                sequence after layer l of scale k (row K-1 repeats the end
 *                of scale K-2)
 * Errors: as hk_build_schedule (HK_EBUDGET when the sink scales alone do not
 * fit). */
int hk_build_progressive_schedule(int L, int H, int K, const int32_t* scale_tokens,
                                  const float* scas, double budget_frac, int n_sink,
                                  int per_layer, uint8_t* expire_out, int32_t* prefix_out,
                                  int64_t* live_out);

/* Cache size, in token slots per sequence, once layer `layer` has finished
 * scale `step` (the accounting of Algorithm 2 on the Pith page of arXiv
 * 2605.14877, read as: layers 0..layer hold, per head, the segments s <=
 * min(step, K-2) with expire > that bound; the later layers what they held at
 * the end of step-1, nothing before step 0).
 *   expire  host uint8 [L][H][K], each entry in [s, K-1]
 * Errors: HK_EINVAL. */
int hk_cache_size_after_layer(int L, int H, int K, const int32_t* scale_tokens,
                              const uint8_t* expire, int step, int layer, int64_t* out);

/* A second schedule generator: condensed plus local scales, as expiry steps
 * for hk_create_expiry (the AMS-KV paper's abstract: tokens of local scales
 * matter most, a little memory for the coarsest, condensed, scales
 * stabilises generation, and layers with weak inter-scale key/value
 * similarity are cache-demanding and get more).  Readings taken:
 *   scales 0..n_condensed-1 stay cached to the end (expire = K-1);
 *   any other segment s is read by the next w scales and leaves at step
 *     min(s + w, K-1), with w = window_demanding in the n_demanding layers
 *     of lowest similarity[l] (ties: lower layer first), else w = window;
 *   every head of a layer gets the same schedule.
 *   similarity  host float [L], or NULL when n_demanding = 0
 *   expire_out  host uint8 [L][H][K]
 * Errors: HK_EINVAL. */
int hk_build_scale_window_schedule(int L, int H, int K, const int32_t* scale_tokens,
                                   int n_condensed, int window, int window_demanding,
                                   const float* similarity, int n_demanding,
                                   uint8_t* expire_out);

/* hk_layout for a schedule given as expiry steps (hk_layout(keep) equals
 * this with expire = keep ? K-1 : s).  Head (l, h) gets the most rows it
 * holds at the end of any scale:
 *   cap[l][h] = max over k <= K-2 of the sum of n_s over s <= k with
 *   expire[l][h][s] > k;
 * at scale t rows [0, len) of (l, h, b) hold the segments s < t with
 * expire >= t, in scale order.
 * Errors: HK_EINVAL (also for an expire entry outside [s, K-1]). */
int hk_layout_expiry(int L, int H, int K, const int32_t* scale_tokens, const uint8_t* expire,
                     int B, int D, int64_t* cache_elems_out, int64_t* cap_out,
                     int64_t* base_out);

/* Create a context on the current HIP device.  Copies scale_tokens and keep,
 * and uploads the small per-head tables.  k_cache / v_cache are caller-owned
 * device buffers of hk_layout() elements each; they must outlive the context.
 * Supported: dtype HK_DTYPE_BF16 with D = 128 (matrix-core path), and
 * HK_DTYPE_F32 with D in {16, 32, 64, 128}; K <= HK_MAX_SCALES.
 * Errors: HK_EINVAL, HK_EUNSUPPORTED, HK_EHIP (allocation or copy failed). */
int hk_create(hk_ctx** out, int L, int H, int D, int B, int K, const int32_t* scale_tokens,
              const uint8_t* keep, int dtype, void* k_cache, void* v_cache);

/* hk_create for a schedule given as expiry steps (hk_build_progressive_schedule's
 * output, or any table with entries in [s, K-1]); the cache buffers hold
 * hk_layout_expiry() elements.  Scale t attends, per head, the held segments
 * s < t with expire >= t.  hk_append_scale of scale t first moves the
 * surviving segments down over those that expire at t (an in-place gather,
 * one workgroup per (layer, head, batch entry), in ascending row order) and
 * then stores segment t behind them.  Because the move and the store
 * overwrite rows that scale t's attention reads, a layer where any head
 * drops a segment at step t needs hk_attend (or hk_attend_with_scas) of
 * (layer, t) before hk_append_scale of (layer, t), and no attend of (layer, t)
 * after it, else HK_EORDER; hk_attend_append runs the two in that order
 * (as separate launches at such steps).
 * Errors: as hk_create. */
int hk_create_expiry(hk_ctx** out, int L, int H, int D, int B, int K,
                     const int32_t* scale_tokens, const uint8_t* expire, int dtype,
                     void* k_cache, void* v_cache);

/* Pooled layout for an expiry-step schedule (hk_build_progressive_schedule's
 * output, or any table with entries in [s, K-1]): instead of a region per
 * head sized to that head's own peak, every head's rows live in one pool of
 * rows per batch entry, and a segment that leaves the cache (Pith page of
 * arXiv 2605.14877, Figure 4 caption: G_k is gone once scale k is done)
 * gives its rows to segments stored later, so no stored row ever moves and
 * the pool holds exactly the most token slots the cache holds at once.
 * Rows are handed out in generation order -- for each scale k and each layer
 * l: the segments of layer l that expire at k give back their rows, then the
 * segments (l, h, k) that are stored take rows, lowest free rows first (the
 * per-layer accounting of Algorithm 2, Appendix A of the same page) -- so
 * pool_rows equals the largest per-layer cache size of
 * hk_build_progressive_schedule's live_out.
 *   pool_elems_out  host int64 (required): B * pool_rows * D, the elements of
 *                   each buffer (K or V), laid out [B][pool_rows][D]
 *   pool_rows_out   host int64 or NULL
 *   seg_rows_out    host int32 [L][H][sum of n_s over s <= K-2] or NULL: for
 *                   each head, segment after segment in scale order, the pool
 *                   row of each of the segment's n_s rows, -1 for a segment
 *                   that is never stored
 * Errors: HK_EINVAL. */
int hk_layout_pooled(int L, int H, int K, const int32_t* scale_tokens, const uint8_t* expire,
                     int B, int D, int64_t* pool_elems_out, int64_t* pool_rows_out,
                     int32_t* seg_rows_out);

/* Create a context over a pooled cache (hk_layout_pooled) in the caller's
 * k_pool / v_pool (bf16, head_dim 128, B * pool_rows * 128 elements each).
 * Attention reads every held row through a per-(step, layer, head) map of
 * pool rows; appends write the stored segments to their pool rows; dropped
 * segments cost nothing (no gather).  Order rules, beyond hk_create's: a
 * step is attended only before its own append (attend(l, t) needs the last
 * appended step of layer l to be t-1), and append(l, t) needs every layer to
 * have appended t-1 and the layers before l to have appended t, because the
 * rows it takes may have been freed by those layers' segments (HK_EORDER
 * otherwise).  hk_attend_append runs the attention and the append as two
 * launches.
 * Errors: as hk_create; HK_EUNSUPPORTED unless bf16 with D = 128. */
int hk_create_pooled(hk_ctx** out, int L, int H, int D, int B, int K, const int32_t* scale_tokens,
                     const uint8_t* expire, void* k_pool, void* v_pool);

/* 4-bit storage of the retained cache (VAR-Q summary page, Key
 * contributions and Method: quantization groups indexed by (block, channel),
 * a block being one scale's segment, optionally cut into sub-blocks along
 * the token axis; low-bit values packed into bytes when written and unpacked
 * for attention).  Readings taken:
 *   sub-block j of a stored n-token segment is rows [j*n/m, (j+1)*n/m)
 *     (rounded down), m = sub_blocks (the page's ratio r = 1/m);
 *   per (sub-block, channel) group, in float32: lo = min, step = (max - lo)
 *     / 15, code = round-half-even((x - lo) / step) clamped to [0, 15], 0 when
 *     step = 0; an empty sub-block stores (0, 0); the value read back is
 *     lo + code * step, rounded to bf16;
 *   two codes per byte, even channel in the low nibble.
 * Only the segments the static keep-mask keeps are stored (pruning and
 * quantization compose).  Buffer layout (one buffer for K, one for V, bytes):
 *   codes of head (l, h) from code_base(l, h) = sum over earlier heads of
 *     B * cap * 64, as [B][cap][64];
 *   from param_offset (256-byte aligned) the groups of head (l, h), as
 *     [B][m * stored segments][128] float2 (step, lo), segments in scale
 *     order.
 * Supported: bf16 inputs with D = 128.
 *   store_bytes_out   host int64 (required): bytes of each buffer
 *   param_offset_out  host int64 or NULL
 * Errors: HK_EINVAL, HK_EUNSUPPORTED. */
int hk_layout_int4(int L, int H, int K, const int32_t* scale_tokens, const uint8_t* keep, int B,
                   int D, int sub_blocks, int64_t* store_bytes_out, int64_t* param_offset_out);

/* Create a context whose cache is stored in 4 bits (hk_layout_int4) in the
 * caller's k_store / v_store.  Queries, current keys and values and outputs
 * stay bf16 [B][n_t][H][128].  hk_append_scale (and the append half of
 * hk_attend_append) quantizes the scale's stored segments into the buffers;
 * hk_attend / hk_attend_with_scas first unpack the layer's held rows into a
 * bf16 scratch the context owns (the largest layer's bf16 cache, allocated
 * here) and then run the bf16 attention on it, so the matrix-core kernel
 * does no per-query-tile unpacking.  Order rules as hk_create.
 * Errors: as hk_create (HK_EUNSUPPORTED unless D = 128). */
int hk_create_int4(hk_ctx** out, int L, int H, int D, int B, int K, const int32_t* scale_tokens,
                   const uint8_t* keep, int sub_blocks, void* k_store, void* v_store);

/* Free the context's device tables (synchronises the device first). NULL is OK. */
int hk_destroy(hk_ctx* ctx);

/* Start a new generation: every layer's cache is considered empty again. */
int hk_reset(hk_ctx* ctx);

/* Block-causal attention of scale `step` in `layer` (HeatKV project page,
 * Abstract and Method step 5: each scale attends to the key-value segments of
 * earlier scales that survive pruning; Pith page of arXiv 2605.14877,
 * Figure 2 caption: next-scale prediction conditions each scale on all
 * earlier ones, and Figure 3 caption: tokens of a scale in raster order).
 *
 * For every (b, h) and query i of scale step:
 *   out[b][i][h][:] = softmax_j(softmax_scale * q[b][i][h][:] . key_j) value_j
 * over the keys j of the kept segments s < step of head (layer, h), read from
 * the cache in scale order, followed by the n_step keys of k_cur[b][:][h][:]
 * (the scale being generated).  Scores and the softmax are fp32; with bf16
 * the products run on the matrix cores, probabilities are rounded to bf16 for
 * the value product, and out is rounded to bf16 (nearest even).
 * Order: requires that hk_append_scale has covered (layer, step-1) since the
 * last hk_reset (not needed for step 0).  Under a schedule whose segments
 * leave the cache after they were stored (hk_create_expiry), the append of a
 * step that drops segments moves the survivors, so attending (layer, step)
 * after the append of any step u >= step that drops segments of that layer
 * returns HK_EORDER.
 * Errors: HK_EINVAL, HK_EORDER, HK_EHIP. */
int hk_attend(hk_ctx* ctx, int layer, int step, const void* q, const void* k_cur,
              const void* v_cur, void* out, float softmax_scale, void* hip_stream);

/* hk_attend, plus this step's S-CAS row (HeatKV project page, Abstract and
 * Method step 2: attention probabilities aggregated per layer, head, source
 * scale and future scale).  Reading taken: for each query of scale step, the
 * probability mass on the keys of source s, averaged over the n_step queries
 * and then over the batch:
 *   scas_table[layer][h][step][s], s = 0..step, overwritten for every h;
 * dropped sources get exactly 0; entries s > step are not written.
 *   scas_table  device float [L][H][K][K]
 * The cross-workgroup sum runs in a fixed order (deterministic).
 * Errors: as hk_attend. */
int hk_attend_with_scas(hk_ctx* ctx, int layer, int step, const void* q, const void* k_cur,
                        const void* v_cur, void* out, float softmax_scale,
                        float* scas_table, void* hip_stream);

/* Streaming calibration: hk_attend_with_scas over one batch of calibration
 * images, adding instead of overwriting.  For every head h and source s <=
 * step, the per-image S-CAS (mass on source s averaged over the step's
 * queries) summed over the batch's B images is added to
 *   scas_sum[layer][h][step][s]   (device double [L][H][K][K]).
 * Calling it for every (layer, step) of N batches and dividing by the N*B
 * images (hk_scas_mean) gives the S-CAS table of the whole calibration set:
 * a small offline calibration set is aggregated into one table (HeatKV
 * project page, Method steps 1-2; Results: rankings stay stable with a small
 * calibration set).  Each call's contribution is summed in a fixed order.
 * Errors: as hk_attend_with_scas. */
int hk_attend_with_scas_sum(hk_ctx* ctx, int layer, int step, const void* q, const void* k_cur,
                            const void* v_cur, void* out, float softmax_scale, double* scas_sum,
                            void* hip_stream);

/* scas_out = scas_sum / images, element by element (host arrays of L*H*K*K).
 * Errors: HK_EINVAL (null, images <= 0). */
int hk_scas_mean(int L, int H, int K, const double* scas_sum, double images, float* scas_out);

/* Stability of the schedule's rankings between two S-CAS tables, e.g. from
 * two disjoint calibration subsets (HeatKV project page, Results; Pith page
 * of arXiv 2605.14877, Figure 6 caption: ranking stability across
 * calibration runs).  The pages do not define the measure; two are given:
 *   rho_out[s] (host double [K]): for each prunable source scale
 *     s = n_sink..K-2, the Spearman rank correlation between the positions
 *     of the L*H heads in the two orderings O_s (hk_build_schedule's
 *     orderings, ties by flat index); NaN for the other scales and when
 *     L*H < 2;
 *   jaccard_out (host double): |G_a & G_b| / |G_a | G_b| of the pruned
 *     (layer, head, scale) sets of the two keep-masks hk_build_schedule
 *     builds at budget_frac (1 when both are empty).
 * Errors: as hk_build_schedule. */
int hk_ranking_stability(int L, int H, int K, const int32_t* scale_tokens, const float* scas_a,
                         const float* scas_b, double budget_frac, int n_sink, double* rho_out,
                         double* jaccard_out);

/* hk_attend (or, with scas_table != NULL, hk_attend_with_scas) of scale
 * `step` in `layer`, followed by hk_append_scale of the same scale and layer,
 * for callers that run the two back to back.  With bf16 both happen in one
 * launch: every workgroup stages every key and value tile of its key range
 * anyway, and the one with query tile (key tile mod query tiles) also writes
 * that tile's kept current-scale rows into the cache (rows the launch itself
 * never reads), so the scale is read from HBM once instead of twice.  The
 * final scale (step = K-1) is only attended.
 * Order: as hk_attend, and the layer's last appended scale must be step-1.
 * Errors: as hk_attend. */
int hk_attend_append(hk_ctx* ctx, int layer, int step, const void* q, const void* k_cur,
                     const void* v_cur, void* out, float softmax_scale, float* scas_table,
                     void* hip_stream);

/* Compact scale `step` into the cache for layers [layer_begin, layer_end):
 * for every kept (l, h) (keep[l][h][step] = 1) and every b, copies the rows
 * k_cur_l[b][:][h][:] (and likewise V) to rows
 * [len_before(l,h,step), +n_step) of (l, h, b), bit for bit (HeatKV project
 * page, Method step 5: pruning during inference as scales are generated; a
 * dropped segment is simply never written).
 *   k_cur, v_cur        device, layer l's tensor at k_cur + (l - layer_begin)
 *                       * layer_stride_elems, each [B][n_step][H][D]
 *   layer_stride_elems  element stride between consecutive layers' tensors
 *                       (ignored when one layer is given)
 * Order: each layer's scales must be appended in order 0, 1, ..., K-2 since
 * the last hk_reset; step = K-1 is rejected (the final scale is never cached).
 * Errors: HK_EINVAL, HK_EORDER, HK_EHIP. */
int hk_append_scale(hk_ctx* ctx, int layer_begin, int layer_end, int step, const void* k_cur,
                    const void* v_cur, int64_t layer_stride_elems, void* hip_stream);

/* The launch plan hk_attend / hk_attend_with_scas use for scale `step`:
 * query rows per workgroup (bf16: 128 or 256, fp32: 64) and key-range splits
 * (1 = none; an S-CAS launch never splits).  A split launch is followed by a
 * merge kernel.  For tools and benchmarks that attribute kernel time.
 *   with_scas           0 for hk_attend, 1 for hk_attend_with_scas
 *   rows_per_workgroup  host int32 (written)
 *   splits              host int32 (written)
 * Errors: HK_EINVAL. */
int hk_attend_plan(const hk_ctx* ctx, int step, int with_scas, int32_t* rows_per_workgroup,
                   int32_t* splits);

/* The plan hk_create picks for a bf16 launch, on the host and without a
 * context: B batch entries, H heads, n queries per head (the scale's tokens)
 * and at most max_keys keys per head (held rows plus n).  A cost model of
 * launch rounds, key tiles per workgroup and the merge of split launches
 * (constants measured on the MI355X) picks the query rows per workgroup
 * (128 or 256) and the key-range splits (1 to 16, 256-row tiles only, at
 * most one per 64-key tile; allow_split = 0, as for S-CAS launches, forces
 * 1).
 *   rows_per_workgroup, splits  host int32 (written)
 * Errors: HK_EINVAL (a size < 1 or a null pointer). */
int hk_plan_attend_bf16(int B, int H, int n, int max_keys, int allow_split,
                        int32_t* rows_per_workgroup, int32_t* splits);

/* Token slots per sequence held by the whole cache (all layers and heads)
 * once scale `step` has been appended: the sum of n_s over the segments s <=
 * min(step, K-2) held at the end of that step (HeatKV project page, Method
 * steps 4-5: the cache must stay within the memory budget as scales are
 * generated; Results, Table 1 excerpt, where the full cache factors over
 * scales 0..K-2 only).  With a static keep-mask: the kept segments.
 *   out   host int64 (written)
 * Errors: HK_EINVAL (null, step outside [0, K)). */
int hk_retained_tokens(const hk_ctx* ctx, int step, int64_t* out);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): attention
 * of one layer at scale `step`, as hk_attend_with_scas (scas_table != NULL)
 * or hk_attend (scas_table == NULL), with no context and no allocation.
 * The per-head tables and the S-CAS partial sums live in a device array of
 * HK_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 * process ends; every call on a GPU shares it, so calls that overlap on one
 * GPU (other streams or threads) race.  The launch is never split over key
 * ranges (the S-CAS launch plan), so outputs equal hk_attend_with_scas's bit
 * for bit.
 *   H <= HK_NOALLOC_MAX_HEADS heads, bf16, head_dim 128, B batch entries
 *   scale_tokens   host int32 [K]
 *   keep           host uint8 [H][K]: this layer's static keep-mask
 *   k_cache, v_cache  device bf16: this layer's cache as hk_layout lays out
 *                  one layer (head h at the sum over h' < h of B*cap[h']*128
 *                  elements, [B][cap[h]][128]), holding every kept segment
 *                  s < step (e.g. a context's cache + base[layer][0])
 *   q, k_cur, v_cur, out  device bf16 [B][n_step][H][128]
 *   scas_table     device float [H][K][K] or NULL; row `step` of every head
 *                  is overwritten (entries s <= step)
 * The current device must be the one holding the buffers.
 * Errors: HK_EINVAL (sizes, nulls, alignment; H above the limit; B * H *
 * query tiles whose S-CAS partial sums would not fit the array),
 * HK_EUNSUPPORTED (K > HK_MAX_SCALES), HK_EHIP. */
#define HK_NOALLOC_MAX_HEADS 32
#define HK_NOALLOC_SCRATCH_BYTES (4 << 20)
int hk_attend_noalloc(int H, int B, int K, const int32_t* scale_tokens, const uint8_t* keep,
                      int step, const void* k_cache, const void* v_cache, const void* q,
                      const void* k_cur, const void* v_cur, void* out, float softmax_scale,
                      float* scas_table, void* hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* HEATKV_H */
