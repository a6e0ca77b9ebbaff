/*
 * sekv.h - C ABI of the SeKV decode path on AMD Instinct MI355X (gfx950).
 *
 * SeKV keeps a long prompt as a resolution-adaptive cache (SeKV paper,
 * Sec. 3): surprisal-guided spans, each with a small routing summary and a
 * coarse mean key/value on the GPU and low-rank SVD factors of its keys and
 * values in a second tier; anchor tokens and a local window stay at full
 * resolution.  Each decode step routes the query against the summaries and
 * runs one softmax over anchors, window, zoomed spans rebuilt from their
 * factors, and the coarse entries of every other span.
 *
 * Conventions for every call:
 *   - Pointers marked "device" are HIP device pointers the caller owns; they
 *     must stay valid until the work queued on the given stream(s) completes.
 *     Host pointers are read or written before the call returns.
 *   - The library owns an sekv_cache and everything reachable from it
 *     (device buffers, the factor pool, staging); sekv_cache_destroy frees it.
 *   - Errors: argument errors are found on the host before any HIP call and
 *     return SEKV_ERR_INVALID; failed allocations or a full host pool return
 *     SEKV_ERR_NOMEM; a failing HIP call returns SEKV_ERR_HIP.  Faults inside
 *     queued kernels surface at the caller's next synchronisation.  Every
 *     failing call leaves a message for sekv_last_error() on the calling
 *     thread, and a failing build leaves *out == NULL.
 *   - A cache may be used by one host thread and one stream order at a time
 *     (its decode calls share per-cache scratch: the chunk zoom masks the
 *     layer launch writes and its tail launch reads); distinct caches are
 *     independent.
 *   - Layouts are row-major C arrays; [a][b] means b varies fastest.
 *     L = n_layers, Hq = n_q_heads, Hkv = n_kv_heads, G = Hq / Hkv (query
 *     heads per KV head; query head h reads KV head h / G), d = head_dim,
 *     dr = route_dim, N = tokens, S_c = compressed spans of the cache.
 */
#ifndef SEKV_H
#define SEKV_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SEKV_OK = 0,
  SEKV_ERR_INVALID = 1,
  SEKV_ERR_NOMEM = 2,
  SEKV_ERR_HIP = 3,
  SEKV_ERR_UNSUPPORTED = 4
} sekv_status;

/* storage type of keys, values, coarse means and summaries */
typedef enum { SEKV_F32 = 0, SEKV_BF16 = 1 } sekv_dtype;

/* how the per-span truncated SVD is computed: exactly (Gram matrix and
 * one-sided Jacobi in float64), or by a randomized range finder with power
 * iterations (SeKV paper Sec. 3.2 names a randomized SVD) for spans of
 * 41..640 tokens, the others exactly; the randomized mode needs max_rank <= 32 */
typedef enum { SEKV_SVD_EXACT = 0, SEKV_SVD_RANDOMIZED = 1 } sekv_svd_mode;

/* where the span factors live: device HBM, or pinned host memory fetched per
 * step for the zoomed spans only (SeKV paper Sec. 3.2: bases on the CPU,
 * fetched asynchronously for selected spans) */
typedef enum { SEKV_TIER_DEVICE = 0, SEKV_TIER_HOST_PINNED = 1 } sekv_tier;

/* how a host-tier decode call moves the zoomed spans' factor blocks to HBM
 * staging (see sekv_set_fetch_mode) */
typedef enum { SEKV_FETCH_GATHER = 0, SEKV_FETCH_MEMCPY = 1 } sekv_fetch_mode;

typedef struct {
  int32_t n_layers;
  int32_t n_q_heads;
  int32_t n_kv_heads;     /* must divide n_q_heads; at most 8 query heads per KV head */
  int32_t head_dim;       /* d; must be 128 */
  int32_t route_dim;      /* dr; 1..64 (the paper uses 32) */
  int32_t window;         /* most recent tokens kept at full resolution (paper: 512) */
  int32_t max_rank;       /* rank cap R, 1..head_dim (paper: 32) */
  int32_t min_span_len;   /* spans shorter than this stay at full resolution (>= 1) */
  double alpha;           /* boundary sensitivity: anchor iff s_t > mean + alpha * std (paper: 1.0) */
  double gamma;           /* size-prior coefficient of the gate, p = sigmoid(q~.s + gamma ln n) */
  int32_t kv_dtype;       /* sekv_dtype */
  int32_t factor_tier;    /* sekv_tier */
  uint64_t host_pool_cap_bytes;  /* host tier: refuse a pool larger than this (0 = no cap) */
  int32_t svd_mode;       /* sekv_svd_mode */
  int32_t append_capacity; /* tokens sekv_append_tokens may add over the cache's life
                              (device-tier factors only); 0 = the cache never grows */
} sekv_config;

typedef struct {
  int32_t n_tokens;
  int32_t n_anchors;
  int32_t n_spans;        /* all spans, compressed and short */
  int32_t n_compressed;   /* S_c */
  int32_t n_dense;        /* window + anchors + short-span tokens */
  int32_t factor_tier;
  double mu, sigma, threshold;   /* surprisal statistics of the build */
  uint64_t resident_bytes;       /* dense rows, means, summaries, tables on the device */
  uint64_t factor_bytes;         /* sum over (layer, KV head, span) of 4 (rK + rV) (n + d + 1) */
  uint64_t factor_pool_bytes;    /* bytes allocated for the pool, padding included */
  int32_t open_start, open_len;  /* retired tokens not yet closed into a span (appends) */
  int32_t n_appended;            /* tokens added by sekv_append_tokens so far */
  int32_t append_capacity;       /* as configured */
} sekv_cache_info;

/* Output of sekv_route for one layer; every buffer is device memory the
 * caller allocates with the sizes below (S_c from sekv_cache_info). */
typedef struct {
  uint8_t* mask;         /* [Hq][S_c]  1 iff head h zooms span j */
  int32_t* list;         /* [Hq][S_c]  zoomed span ids of head h, ascending; first count[h] valid */
  int32_t* count;        /* [Hq] */
  int32_t* union_list;   /* [Hkv][S_c] ids zoomed by any head of the group, ascending */
  int32_t* union_count;  /* [Hkv] */
  double* prob;          /* [Hq][S_c] gate values p, or NULL to skip */
} sekv_route_out;

typedef struct sekv_cache sekv_cache;

/* Segmentation alone (SeKV paper Sec. 3.1): mean and population standard
 * deviation of the surprisal over all n_tokens positions (float64), anchors
 * are positions before the last `window` ones whose surprisal exceeds
 * mean + alpha * std, spans are the maximal runs of other positions before
 * the window, and spans of at least min_span_len tokens are compressed.
 * surprisal_dev: device float32 [n_tokens].  Writes the counts (host
 * pointers, any may be NULL); synchronises `stream`. */
sekv_status sekv_segment(const sekv_config* cfg, int32_t n_tokens, const float* surprisal_dev,
                         int32_t* n_anchors, int32_t* n_spans, int32_t* n_compressed,
                         hipStream_t stream);

/* Build the cache from a prefilled prompt (SeKV paper Sec. 3.1-3.2):
 * segmentation as in sekv_segment; for every (layer, KV head) and compressed
 * span j: normalised surprisal weights w_t = s_t / sum_j s (1/n if the sum is
 * 0), coarse mean key and value sum_t w_t k_t and sum_t w_t v_t, and for every
 * query head h of the group the routing summary W_h kbar_j, all accumulated in
 * float64 and rounded once, to nearest even, to kv_dtype; the truncated SVD of
 * the span's key matrix and of its value matrix, keeping
 * r_j = min(max(rank, 1), n_j, d, max_rank) components (hard gates on Eq. 8),
 * stored as float32 factors in the configured tier.  Anchors, the window and
 * short-span tokens are copied to a contiguous full-resolution set.
 *   k_dev, v_dev:  device [L][Hkv][N][d] in kv_dtype
 *   w_route_dev:   device float32 [L][Hq][dr][d]  (summary projections W_h)
 *   rank_by_pos_dev: device int32 [L][Hkv][N]: requested rank of the span that
 *                  starts at each position; NULL requests max_rank everywhere.
 * Inputs are only read during the call (it synchronises `stream`); the cache
 * holds no pointer to them afterwards. */
sekv_status sekv_build_spans(const sekv_config* cfg, int32_t n_tokens, const float* surprisal_dev,
                             const void* k_dev, const void* v_dev, const float* w_route_dev,
                             const int32_t* rank_by_pos_dev, hipStream_t stream, sekv_cache** out);

sekv_status sekv_cache_info_get(const sekv_cache* cache, sekv_cache_info* out);

/* Copy the span table to host arrays sized from sekv_cache_info (any may be
 * NULL): anchors [n_anchors], span_start/span_len/kind [n_spans] (kind 0 =
 * compressed, 1 = short), cspan [n_compressed] (index into the span arrays of
 * each compressed span), dense_pos [n_dense] (ascending). */
sekv_status sekv_cache_copy_spans(const sekv_cache* cache, int32_t* anchors, int32_t* span_start,
                                  int32_t* span_len, uint8_t* kind, int32_t* cspan,
                                  int32_t* dense_pos);

/* Copy one (layer, KV head) of the cache's stored representation to host
 * memory (any pointer may be NULL), for inspection and tests:
 *   kbar, vbar [S_c][d] and summary [G][S_c][dr], in kv_dtype;
 *   rank_k, rank_v [S_c] int32: retained ranks of each span's key factors and
 *   of its value factors (equal after the build, see sekv_apply_gates);
 * sekv_cache_copy_factors copies the factors of compressed span j, kv = 0
 * keys, 1 values: u [n_j][r], sigma [r], vt [r][d], all float32, with r that
 * matrix's rank. */
sekv_status sekv_cache_copy_group(const sekv_cache* cache, int32_t layer, int32_t kv_head,
                                  void* kbar, void* vbar, void* summary, int32_t* rank_k,
                                  int32_t* rank_v);
sekv_status sekv_cache_copy_factors(const sekv_cache* cache, int32_t layer, int32_t kv_head,
                                    int32_t span, int32_t kv, float* u, float* sigma, float* vt);

/* Append decode tokens to the cache's local window and retire the tokens that
 * leave it (SeKV paper Sec. 3.3: every decode step attends over the
 * mixed-resolution memory; the summary page, sec. 2: the most recent `window`
 * tokens stay at full resolution; how tokens leave the window is not stated).
 * Reading: each appended token enters the window at full resolution; a token
 * that leaves the window is compared with the build's threshold (the prompt's
 * mean + alpha std, computed once): above it, it becomes an anchor;
 * otherwise it joins the open run of retired tokens since the last retired
 * anchor, which stays at full resolution until the next retired anchor closes
 * it into a span.  A closed span of at least min_span_len tokens is
 * compressed exactly as the build compresses spans (surprisal weights, coarse
 * mean key and value, routing summaries, truncated SVD of its keys and of its
 * values at the rank requested at its first token, exact SVD); a shorter one
 * stays at full resolution.  Nothing the build or earlier appends made
 * changes.
 *   n_new >= 1 tokens, in order, following the cache's last token:
 *   surprisal_dev: device float32 [n_new]
 *   k_dev, v_dev:  device [L][Hkv][n_new][d] in kv_dtype
 *   w_route_dev:   device float32 [L][Hq][dr][d], the summary projections of
 *                  the build
 *   rank_dev:      device int32 [L][Hkv][n_new], the rank requested for a span
 *                  that starts at each new token, or NULL for max_rank.
 * The span table, full-resolution set, compressed spans and decode geometry
 * grow; S_c (and with it the route buffer sizes) and the decode workspace
 * size may change: read them again (sekv_cache_info_get,
 * sekv_decode_workspace_bytes) before the next decode call.  Synchronises
 * `stream`; no decode call of this cache may be in flight.  Errors:
 * SEKV_ERR_INVALID for NULL arguments, n_new < 1 or a non-finite surprisal
 * (nothing changed); SEKV_ERR_UNSUPPORTED for a cache built without
 * append_capacity (or with host-tier factors, where it must be 0);
 * SEKV_ERR_NOMEM when n_appended + n_new exceeds append_capacity (nothing
 * changed); after SEKV_ERR_HIP the cache must be destroyed. */
sekv_status sekv_append_tokens(sekv_cache* cache, int32_t n_new, const float* surprisal_dev,
                               const void* k_dev, const void* v_dev, const float* w_route_dev,
                               const int32_t* rank_dev, hipStream_t stream);

/* Route one layer (SeKV paper Sec. 3.2 gate and Sec. 3.3 Eq. 9), float64
 * throughout: q~_h = P_h q_h; x_j = q~_h . s_{h,j} + gamma ln n_j;
 * p_j = 1 / (1 + e^-x_j); span j is zoomed by head h iff p_j > tau_h.
 * Fills `out`: per-head mask and ascending list, per-group ascending union.
 *   q_dev:    device float32 [Hq][d]
 *   proj_dev: device float32 [Hq][dr][d]  (query projections P_h of this layer)
 *   tau_dev:  device float32 [Hq]
 * Asynchronous on `stream`. */
sekv_status sekv_route(const sekv_cache* cache, int32_t layer, const float* q_dev,
                       const float* proj_dev, const float* tau_dev, const sekv_route_out* out,
                       hipStream_t stream);

/* Bytes of device workspace sekv_decode_attn and sekv_route_attn need
 * (256-byte aligned): one partial softmax state per head and work item. */
size_t sekv_decode_workspace_bytes(const sekv_cache* cache);

/* Attention of one layer over the mixed-resolution memory (SeKV paper
 * Sec. 3.3): one softmax, scale 1/sqrt(d), over every full-resolution row of
 * the group, one coarse entry (kbar_j, vbar_j) with ln n_j added to its scaled
 * score for every compressed span the head did not zoom, and the n_j rows
 * U_j diag(sigma_j) V_j^T of every span it zoomed (keys from the span's key
 * factors, values from its value factors, each at its own rank).
 * Accumulates in float32.
 *   q_dev: device float32 [Hq][d]; route: the output of sekv_route for this
 *   layer and query (its mask and union lists are read); o_dev: device float32
 *   [Hq][d]; ws_dev: device workspace of at least
 *   sekv_decode_workspace_bytes(cache) bytes.
 * Runs on `stream`.  With host-tier factors, the zoomed spans' factors are
 * copied into device staging on `fetch_stream` (NULL = `stream`) while the
 * full-resolution and coarse entries are processed on `stream`. */
sekv_status sekv_decode_attn(const sekv_cache* cache, int32_t layer, const float* q_dev,
                             const sekv_route_out* route, float* o_dev, void* ws_dev,
                             size_t ws_bytes, hipStream_t stream, hipStream_t fetch_stream);

/* Route and attend one layer in one call (SeKV paper Sec. 3.2 gate, Sec. 3.3
 * Eq. 9 and the mixed-resolution softmax): the result is the same as
 * sekv_route followed by sekv_decode_attn with the same arguments, and `route`
 * receives the same mask, lists and counts (and prob, if non-NULL).  With
 * device-tier factors the layer is three kernel launches on `stream`: the
 * route; then the zoomed spans (shared among workgroups in proportion to each
 * KV head's union) side by side with the full-resolution rows and coarse
 * entries; then the merge and lists.  With host-tier factors it
 * runs as sekv_route then sekv_decode_attn (fetch on `fetch_stream`).
 * Arguments as for those two calls. */
sekv_status sekv_route_attn(const sekv_cache* cache, int32_t layer, const float* q_dev,
                            const float* proj_dev, const float* tau_dev,
                            const sekv_route_out* route, float* o_dev, void* ws_dev,
                            size_t ws_bytes, hipStream_t stream, hipStream_t fetch_stream);

/* Route and attend one layer like sekv_route_attn, with no workspace
 * argument and no allocation: for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, hosts that forbid
 * hipMalloc).  The partial softmax states go to a scratch array of
 * SEKV_NOALLOC_SCRATCH_BYTES that the library holds on each device until the
 * process ends (it calls neither hipMalloc nor hipFree, nor any allocating
 * routine).  Every call on a device shares that device's scratch: calls that
 * may overlap on one device (other streams, other threads) race and must be
 * serialised by the caller; each call writes every part of the scratch it
 * reads, so nothing needs clearing between calls.  Arguments, results and
 * errors as for sekv_route_attn; SEKV_ERR_UNSUPPORTED if the cache needs more
 * than SEKV_NOALLOC_SCRATCH_BYTES of partial states
 * (sekv_decode_workspace_bytes), which holds the 128K-context Llama-3-8B and
 * Qwen2.5-14B shapes with room to spare. */
#define SEKV_NOALLOC_SCRATCH_BYTES (8 * 1024 * 1024)
sekv_status sekv_route_attn_noalloc(const sekv_cache* cache, int32_t layer, const float* q_dev,
                                    const float* proj_dev, const float* tau_dev,
                                    const sekv_route_out* route, float* o_dev, hipStream_t stream,
                                    hipStream_t fetch_stream);

/* Matched-budget cap of one layer's zoom decisions (SeKV paper Sec. 3.3,
 * zoom-in decoding: past the GPU KV budget, spans are kept in decreasing order
 * of their gate value until the budget is filled).  Per KV head g, the
 * candidates are the spans of route->union_list[g]; a candidate's key is the
 * largest gate value p among the heads of g that zoomed it, ties going to the
 * lower span id; the kept candidates are the longest prefix of that order
 * whose total length sum n_j is at most budget_tokens (the budget counts the
 * tokens one KV head reconstructs in this layer).  A kept span stays zoomed
 * for the heads that selected it; a dropped one leaves the mask of every head
 * of g and reverts to its coarse entry.
 *   route: the output of sekv_route or sekv_route_attn for this cache, made
 *          with prob != NULL; its mask, list, count, union_list and
 *          union_count are rewritten in place (lists stay ascending), prob is
 *          only read.  Pass the result to sekv_decode_attn.
 *   budget_tokens >= 0; 0 zooms nothing, a budget at least the union's total
 *          length changes nothing.
 * Asynchronous on `stream`; the route buffers must not be in use by other
 * work until it completes.  Errors: SEKV_ERR_INVALID for a NULL cache, route
 * buffer or prob, or a negative budget; SEKV_ERR_UNSUPPORTED for caches of
 * more than 2^19 compressed spans. */
sekv_status sekv_cap_budget(const sekv_cache* cache, const sekv_route_out* route,
                            int64_t budget_tokens, hipStream_t stream);

/* The same cap with one budget for the whole layer (SeKV paper Sec. 3.3
 * defines the budget as the peak GPU-resident KV of a decoding step,
 * reconstructed spans included; a step reaches that peak inside one layer,
 * since a layer's reconstructed spans are needed only while it attends).  The
 * candidates are the (KV head g, span j) pairs of every union of the layer,
 * keyed as above, in one order: key descending, ties to the lower KV head,
 * then the lower span id; the kept candidates are the longest prefix whose
 * total length sum n_j (counted once per KV head that reconstructs j) is at
 * most budget_tokens.  A kept (g, j) stays zoomed for the heads of g that
 * selected it; a dropped one leaves their masks.  Two launches on `stream`
 * (the decisions, then their application in place); arguments and errors as
 * for sekv_cap_budget.  Uses the cache's per-layer decision scratch, so calls
 * on one cache must not overlap. */
sekv_status sekv_cap_budget_layer(const sekv_cache* cache, const sekv_route_out* route,
                                  int64_t budget_tokens, hipStream_t stream);

/* Soft-gated reconstruction (SeKV paper Sec. 3.2 low-rank paragraph, Eq. 8:
 * K^_j = U_j diag(g_j * sigma_j) V_j^T with per-component gates in [0, 1],
 * components with negligible gates not stored), applied to a built cache.
 * The value matrix of a span has gates of its own (same paragraph), so keys
 * and values are gated separately and may end with different ranks.  For
 * every (layer, KV head, compressed span) and each of its two matrices, gate
 * i belongs to the i-th largest singular value of that matrix's stored
 * factors (i < its rank); the components with gate >= eps stay, in order,
 * with sigma scaled by the gate; a matrix keeps at least one component, the
 * one with the largest gate (lowest index on ties).  The factor pool is
 * repacked to the new ranks, so zoomed spans then move
 * 4 (rK' + rV') (n + d + 1) bytes.  Calling it again gates the gated factors.
 *   key_gates_dev, value_gates_dev: device float32 [L][Hkv][S_c][max_rank]
 *              each (S_c from sekv_cache_info; entries past a matrix's rank
 *              are ignored), each used gate in [0, 1]; read during the call.
 * Synchronises `stream`.  Errors: SEKV_ERR_INVALID for NULL arguments, a
 * non-finite eps or a gate outside [0, 1] (nothing changed);
 * SEKV_ERR_UNSUPPORTED for host-tier caches; SEKV_ERR_NOMEM if the new pool
 * does not fit (nothing changed); after SEKV_ERR_HIP the cache must be
 * destroyed. */
sekv_status sekv_apply_gates(sekv_cache* cache, const float* key_gates_dev,
                             const float* value_gates_dev, float eps, hipStream_t stream);

/* HBM residency cache for host-tier factors (SeKV paper Sec. 3.2 keeps the
 * span bases on the CPU and fetches them for the selected spans; its
 * limitations name that transfer as the cost of the CPU tier).  Once enabled,
 * each host-tier sekv_decode_attn / sekv_route_attn keeps the zoomed spans'
 * factor blocks in HBM, so a span zoomed again in a later call (same layer and
 * KV head) is read from HBM instead of crossing the host link.  Block
 * (layer, KV head, span) may occupy either of two sets given by fixed hashes of
 * that key, one slot of slot_bytes (rounded up to 256) per set,
 * capacity_bytes / slot_bytes sets.  Within one call, a set goes to the block
 * it already holds if that block is zoomed, else to the lowest key that wants
 * it; spans that get neither of their sets, and blocks larger than a slot, are
 * copied to per-layer staging as without the cache.
 * Outputs do not depend on the cache (a block is the same bytes wherever it is
 * read from).
 *   capacity_bytes: 0 disables the cache and frees it.
 * The call synchronises the device (it frees and allocates device memory and
 * clears the tables), so no work of this cache may be in flight on another
 * thread.  Errors: SEKV_ERR_INVALID for a NULL or device-tier cache, a zero
 * slot size, or a capacity below one slot; SEKV_ERR_UNSUPPORTED for more
 * than 2^30 sets or more than 2^39 (layer, KV head, span) blocks;
 * SEKV_ERR_NOMEM if the tables do not fit; on failure the cache is left
 * disabled. */
sekv_status sekv_set_residency(sekv_cache* cache, uint64_t capacity_bytes, uint64_t slot_bytes);

/* Counters of the residency cache since it was enabled or last reset
 * (synchronises the device): out[0] blocks read from the cache, out[1] blocks
 * copied over the host link, out[2] and out[3] their bytes counted as
 * 4 (rK + rV) (n + d + 1) per block, out[4] sets, out[5] slot bytes.  reset != 0 zeroes
 * the counters afterwards.  SEKV_ERR_INVALID if the cache is not enabled. */
sekv_status sekv_residency_stats(const sekv_cache* cache, uint64_t out[6], int32_t reset);

/* Batched decode: the same layer of `batch` independent sequences
 * (1 <= batch <= SEKV_MAX_BATCH), one cache each, in one layer launch and one
 * tail launch (the per-sequence computation of sekv_route_attn /
 * sekv_decode_attn; batch-4
 * serving).  The caches must share n_layers, n_q_heads, n_kv_heads,
 * head_dim, route_dim and kv_dtype, and must be distinct (each holds its own
 * chunk zoom masks); their context lengths may differ.  For sequence i the
 * arguments are those of the single-sequence call: q_devs[i], routes[i],
 * o_devs[i], and ws_devs[i] with ws_bytes[i] bytes (at least
 * sekv_decode_workspace_bytes(caches[i])).  proj_dev and tau_dev are one
 * model layer's, shared by the batch.  Outputs equal those of the
 * single-sequence calls bit for bit.  Sequences whose factors are host-tier,
 * or that have no compressed span, run through the single-sequence path on
 * `stream` (fetch included).  The pointer arrays are host memory, read during
 * the call.  Errors: SEKV_ERR_INVALID for a NULL array or pointer, a batch size
 * outside the range, mixed model shapes, a repeated cache or a short
 * workspace, checked before anything is launched. */
#define SEKV_MAX_BATCH 8
sekv_status sekv_route_attn_batch(const sekv_cache* const* caches, int32_t batch, int32_t layer,
                                  const float* const* q_devs, const float* proj_dev,
                                  const float* tau_dev, const sekv_route_out* routes,
                                  float* const* o_devs, void* const* ws_devs,
                                  const size_t* ws_bytes, hipStream_t stream);
sekv_status sekv_decode_attn_batch(const sekv_cache* const* caches, int32_t batch, int32_t layer,
                                   const float* const* q_devs, const sekv_route_out* routes,
                                   float* const* o_devs, void* const* ws_devs,
                                   const size_t* ws_bytes, hipStream_t stream);

/* Fetch of a host-tier cache's factor blocks (SeKV paper Sec. 3.2: bases on
 * the CPU, fetched for the selected spans; the summary page asks that the
 * fetch be asynchronous).  SEKV_FETCH_GATHER (default): one kernel on the
 * fetch stream reads the union spans' blocks from mapped pinned memory, driven
 * by the route's union lists on the device, so the host never waits.
 * SEKV_FETCH_MEMCPY: the union lists are copied to the host (the call waits
 * for the route), then one hipMemcpyAsync per run of consecutive union spans
 * moves their blocks on the fetch stream.  Outputs are the same bit for bit.
 * Applies to later calls; a residency cache (sekv_set_residency) takes
 * precedence.  Errors: SEKV_ERR_INVALID for a NULL or device-tier cache or an
 * unknown mode. */
sekv_status sekv_set_fetch_mode(sekv_cache* cache, int32_t mode);

/* Test hook for the failure path of the host-tier factor fetch (the link the
 * SeKV paper Sec. 3.2 fetches factors over): the next n host-tier fetches
 * (sekv_decode_attn, or the attention half of sekv_route_attn) fail with
 * SEKV_ERR_HIP before anything of theirs is queued, and the cache stays
 * usable.  n = 0 cancels.  Process-wide; SEKV_ERR_INVALID for n < 0. */
sekv_status sekv_test_fail_fetch(int32_t n);

void sekv_cache_destroy(sekv_cache* cache);

/* Message of the last failing call on this thread ("" if none). */
const char* sekv_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SEKV_H */
