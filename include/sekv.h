/*
 * sekv.h -- C ABI of the SeKV mixed-resolution decode-attention library for
 * AMD Instinct MI355X (gfx950).
 *
 * The method (SeKV, "Resolution-Adaptive KV Cache with Hierarchical Semantic
 * Memory"):
 *   prefill  -- cut each sequence into spans where token surprisal exceeds
 *               mu + alpha*sigma, keep the boundary tokens (and a local window)
 *               as full-resolution anchors, summarise every span by the
 *               surprisal-weighted mean of its keys and values, and store a
 *               truncated SVD of each span's key and value matrices.
 *               [long-form summary page "SeKV：面向长上下文推理的分辨率自适应
 *               KV Cache 与层级语义记忆", sections 2.1-2.2, eqs. (1), (2), (6)]
 *   decode   -- score the query against every span summary, zoom into spans
 *               whose sigmoid score exceeds a per-(layer, head) threshold,
 *               rebuild their tokens from the SVD bases, and run one softmax
 *               over anchors, zoomed tokens and the log|S|-corrected summaries
 *               of the other spans.
 *               [same page, section 2.3, eqs. (5), (9), Figure 2; review page
 *               "SeKV：支持分层语义记忆的分辨率自适应KV缓存…", workflow paragraph]
 *
 * Readings fixed by this library where the pages are silent:
 *   mu/sigma are the population mean/std in fp64; both rules use a strict '>';
 *   members of a span = its positions minus anchors; empty spans are dropped;
 *   |S| = member count, natural log; the learned routing projection is the
 *   identity, so the routing score is q.kbar/(|kbar| sqrt(d)) + ln|S|; the
 *   trained rank gate is a hard rank r_S = choices[splitmix64(seed ^ layer<<40
 *   ^ g<<32 ^ k) mod n_choices], r_eff = min(r_S, |S|, d); a zoomed span adds
 *   only its rebuilt tokens, a non-zoomed span one entry with logit
 *   q.kbar/sqrt(d) + ln|S|; query head h reads kv head h / (Hq/Hkv).
 *
 * Conventions
 *   * Every call returns sekv_status (0 = OK); no C++ exception crosses the ABI.
 *     On error the text of the failure is kept in sekv_last_error(ctx).
 *   * "dev" pointers are HIP device memory on the context's device, "host"
 *     pointers ordinary host memory.  The caller owns every pointer it passes.
 *   * All device work is stream-ordered on the stream passed in (NULL = the
 *     legacy default stream).  Calls on one context are not thread-safe and
 *     must not overlap on different streams: they share internal buffers.
 *   * KV tensors are row-major [B][H_kv][n][d] in the context's KV dtype
 *     (float32 or bfloat16 bit patterns); q and outputs are float32.
 */
#ifndef SEKV_H
#define SEKV_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sekv_status {
  SEKV_OK = 0,
  SEKV_ERR_INVALID = 1, /* bad argument: shape, NaN/negative surprisal, NaN tau, ... */
  SEKV_ERR_OOM = 2,     /* device or pinned-host allocation failed */
  SEKV_ERR_HIP = 3,     /* a HIP runtime call failed; see sekv_last_error */
  SEKV_ERR_STATE = 4    /* call out of order (layer not built, ...) */
} sekv_status;

typedef enum sekv_dtype { SEKV_F32 = 0, SEKV_BF16 = 1 } sekv_dtype;

/* Where the per-span SVD bases live between decode steps.
 * HOST        -- pinned host memory (the pages' CPU tier), read in place by the
 *                decode kernel: only the zoomed spans' bytes cross the host
 *                link, and the step stays asynchronous (two kernels) and
 *                capturable into a HIP graph.
 * DEVICE      -- device memory (the whole store fits in HBM on MI355X at 128K
 *                context): the decode step is fully device-side and
 *                asynchronous, two kernels (attention with in-place zoom, then
 *                the combine), and capturable into a HIP graph.
 * HOST_STAGED -- pinned host memory; every decode step learns the zoom list
 *                (one host sync), copies the zoomed spans' bases into a device
 *                staging buffer on a side stream (sekv_zoom_fetch), then runs
 *                the zoomed segment from staging. */
typedef enum sekv_basis_home {
  SEKV_BASES_HOST = 0,
  SEKV_BASES_DEVICE = 1,
  SEKV_BASES_HOST_STAGED = 2
} sekv_basis_home;

typedef struct sekv_config {
  int32_t n_layers;     /* L >= 1 */
  int32_t batch;        /* B >= 1 independent sequences */
  int32_t n_ctx;        /* 1 <= n < 2^24 tokens per sequence */
  int32_t n_q_heads;    /* H_q <= 64, a multiple of n_kv_heads, H_q/H_kv in {1, 2, 4, 8} */
  int32_t n_kv_heads;   /* H_kv >= 1, batch * H_kv <= 512 */
  int32_t d_head;       /* 64 or 128 */
  int32_t kv_dtype;     /* sekv_dtype */
  int32_t local_window; /* w >= 0: the last w positions are anchors */
  int32_t basis_home;   /* sekv_basis_home */
  int32_t device;       /* HIP device ordinal */
} sekv_config;

typedef struct sekv_ctx sekv_ctx;

/* Create a context.  Allocates the span tables and per-layer bookkeeping;
 * per-layer artefacts are allocated by sekv_build / sekv_import_head.
 * Errors: INVALID (shape rules above), OOM, HIP. */
sekv_status sekv_create(const sekv_config* cfg, sekv_ctx** out);

/* Free everything the context owns.  NULL is accepted. */
void sekv_destroy(sekv_ctx* ctx);

/* Text of the last failure on this context ("" if none).  Valid until the
 * next call on the context.  NULL ctx returns the text of the last failed
 * sekv_create in this process. */
const char* sekv_last_error(const sekv_ctx* ctx);

/* ------------------------------------------------------------------ build */

/* Prefill builder for one layer [summary page 2.1-2.2, eqs. (1), (2), (6)].
 *   H      dev float32 [B][n]       per-token surprisal, finite and >= 0
 *   K, V   dev KV dtype [B][H_kv][n][d]
 *   alpha  boundary sensitivity (finite)
 *   rank_choices host int32 [n_choices] (each >= 1), rank_seed: the hard
 *          per-span rank r_S described above.
 * Steps: segmentation (on the first build of the context; later layers must
 * present the same H and alpha, which is checked), weighted-mean summaries,
 * anchor gather, batched one-sided-Jacobi truncated SVD of each span's key
 * and value member rows, basis packing (and, for SEKV_BASES_HOST, a copy into
 * the pinned host store).  The call synchronises `stream` once (after the
 * segmentation) and again before returning; H, K, V may be freed on return.
 * Errors: INVALID (NaN/Inf/negative H, alpha not finite, bad rank choice,
 * layer out of range), STATE (H or alpha differ from the first build), OOM, HIP. */
sekv_status sekv_build(sekv_ctx* ctx, int32_t layer, const float* H, const void* K, const void* V,
                       double alpha, const int32_t* rank_choices, int32_t n_choices,
                       uint64_t rank_seed, hipStream_t stream);

/* Span table of sequence b (shared by every layer and head).
 *   m, n_anchors, m_max (max over sequences) are written when non-NULL.
 *   mstart/mcount host int32 [m]: first member position and member count of
 *   each kept span, in position order (spans added by re-segmentation follow
 *   the prefill's).  anchors host int32 [n_anchors], ascending: the positions
 *   of the window rows as of the last build or re-segmentation (tokens
 *   appended since then are not listed).  Pass NULL arrays to query sizes only.
 * Errors: STATE before the first build/import, INVALID (b out of range). */
sekv_status sekv_get_spans(const sekv_ctx* ctx, int32_t b, int32_t* m, int32_t* n_anchors,
                           int32_t* m_max, int32_t* mstart, int32_t* mcount, int32_t* anchors);

/* Packed basis layout of one (layer, b, kv head g).  For span k with c = mcount[k],
 * c8 = c rounded up to a multiple of 8, and r = rank[k], the store holds from
 * element offset basis_off[k] four row-major blocks
 *     A_K^T [r][c8] | B_K^T [r][d] | A_V^T [r][c8] | B_V^T [r][d]
 * where A = U_r Sigma_r (c x r) and B^T = V_r^T (r x d) are the truncated SVD
 * factors of the span's member rows (X ~ A B^T); A is stored transposed
 * (rank-major, one row per singular component) with columns c..c8-1 zero, so
 * every block starts on a 16-byte boundary.  A span takes 2*r*(c8 + d)
 * elements; spans follow each other in span order.
 *   rank host int32 [m], basis_off host int64 [m] (elements), basis_elems
 *   total elements; any may be NULL.
 * Errors: STATE (layer not built), INVALID. */
sekv_status sekv_get_bases_layout(const sekv_ctx* ctx, int32_t layer, int32_t b, int32_t g,
                                  int32_t* rank, int64_t* basis_off, int64_t* basis_elems);

/* ----------------------------------------------------------------- decode */

/* One decode step of one layer for every sequence and query head.
 *   q         dev float32 [B][H_q][d]
 *   tau       host float32 [H_q]: zoom thresholds of this layer, on the
 *             probability scale of eq. (9); tau <= 0 zooms every span,
 *             tau >= 1 none.  NaN -> INVALID.
 *   out       dev float32 [B][H_q][d]: attention output
 *   zoom_mask dev uint8 [B][H_q][m_max] or NULL: 1 where the head zoomed the
 *             span; entries at or beyond the sequence's m are left untouched.
 * DEVICE and HOST bases: fully asynchronous on `stream` (two kernels);
 * capturable into a HIP graph once the layer has been decoded eagerly (the
 * first calls size the work schedule from the zoom counts they measure).
 * HOST_STAGED bases: route kernel, then the zoomed spans' bases are copied
 * from the pinned store to device staging on the context's side stream (see
 * sekv_zoom_fetch), then the zoomed-segment and anchor kernel and the
 * combine; synchronises `stream` once, after routing.
 * Errors: STATE (layer not built, or a graph capture before the first eager
 * call), INVALID, HIP. */
sekv_status sekv_decode_attn(sekv_ctx* ctx, int32_t layer, const float* q, const float* tau,
                             float* out, uint8_t* zoom_mask, hipStream_t stream);

/* sekv_decode_attn with a zoom budget per query head [summary page, section
 * 2.3, the budget rule after eq. (9)]: when more than budget[h] spans of a
 * sequence pass head h's threshold, only the budget[h] with the highest
 * routing score are zoomed (the sigmoid gate is monotone in the score), equal
 * scores going to the lower span index; the others contribute their summary
 * entry as non-zoomed spans do.
 *   budget host int32 [H_q]: most zoomed spans per (sequence, query head);
 *          a negative entry leaves that head uncapped.  NULL -> INVALID.
 * Adds two kernels before the route kernel (the routing scores, then one
 * radix-select workgroup per (sequence, query head) writing the capped
 * decisions to the zoom mask, or to an internal mask when zoom_mask is NULL).
 * Other arguments, asynchrony, capture and errors as sekv_decode_attn. */
sekv_status sekv_decode_attn_budget(sekv_ctx* ctx, int32_t layer, const float* q, const float* tau,
                                    const int32_t* budget, float* out, uint8_t* zoom_mask,
                                    hipStream_t stream);

/* sekv_decode_attn for callers that cannot allocate memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same kernels, with the split-K partials, the projected queries and (when
 * zoom_mask is NULL) the zoom mask in a device array of
 * SEKV_NOALLOC_SCRATCH_BYTES that the library holds on each GPU until the
 * process ends.  Calls no hipMalloc, hipFree or other allocating routine, and
 * no host synchronisation.  Arguments and result as sekv_decode_attn.
 * It runs the layer's work schedule as the last sekv_decode_attn on that
 * layer left it (it does not refine the schedule): decode the layer once with
 * sekv_decode_attn first, and again after appending tokens or re-segmenting.
 * Every call on one GPU shares that GPU's scratch array: calls that overlap
 * in time on one GPU (other streams, other contexts, other threads) race and
 * corrupt each other's results; serialise them on one stream.
 * DEVICE and HOST bases only (staged bases and the basis cache allocate).
 * Errors: STATE (layer not built, no current schedule, HOST_STAGED bases or a
 * basis cache), INVALID (bad arguments, or a decode that needs more scratch
 * than SEKV_NOALLOC_SCRATCH_BYTES: B*H_q*slots*(4+d)*4 bytes of partials,
 * slots <= 512, plus B*H_q*d_r*4 and B*H_q*m_max, each rounded up to 256),
 * HIP. */
#define SEKV_NOALLOC_SCRATCH_BYTES (16u << 20)
sekv_status sekv_decode_attn_noalloc(sekv_ctx* ctx, int32_t layer, const float* q, const float* tau,
                                     float* out, uint8_t* zoom_mask, hipStream_t stream);

/* Stage-1 routing scores only [eq. (5) with the identity projection]:
 *   scores dev float32 [B][H_q][m_max] = q.kbar/(|kbar| sqrt(d)) + ln|S|
 * (ln|S| alone when kbar = 0).  Entries beyond a sequence's m are untouched.
 * A diagnostic / calibration entry point; asynchronous on `stream`. */
sekv_status sekv_route_scores(sekv_ctx* ctx, int32_t layer, const float* q, float* scores,
                              hipStream_t stream);

/* Copy the bases of selected spans from the pinned host store into the
 * context's device staging buffer (HOST bases only) [the asynchronous CPU
 * fetch of zoomed spans, summary page Figure 2].
 *   entries host int32 [B*H_kv][m_max]: for each (b, g) the first counts[b*H_kv+g]
 *           entries are span ids k (0 <= k < m_b) in the low 24 bits and a bit
 *           mask of the group's zooming query heads in bits 24..31 (bit i =
 *           query head g*G+i).  Each span id at most once per (b, g).
 *   counts  host int32 [B*H_kv]
 * The copy is one kernel on `side` that reads the mapped pinned store (runs of
 * adjacent spans coalesced, cut into pieces of at most 32768 elements, one
 * workgroup each), followed by the upload of the staging table, and `done`
 * (may be NULL) is recorded on `side` after it.  The staging table describes
 * exactly these spans until the next fetch; the decode entry point calls this
 * itself.  The host arrays may be reused after `done`.
 * Errors: STATE (DEVICE bases, layer not built), INVALID (bad id, duplicate),
 * OOM (staging too small), HIP. */
sekv_status sekv_zoom_fetch(sekv_ctx* ctx, int32_t layer, const int32_t* entries,
                            const int32_t* counts, hipStream_t side, hipEvent_t done);

/* ------------------------------------------------------ artefact exchange */

/* Install a span table for sequence b instead of building one (test hook:
 * lets a decode run on artefacts built elsewhere).  All sequences must be
 * imported before any sekv_import_head.  Host int32 arrays as in
 * sekv_get_spans; spans must be disjoint, ascending, inside [0, n), and the
 * anchors ascending and disjoint from the members.
 * Errors: INVALID, STATE (a build already fixed the table), OOM, HIP. */
sekv_status sekv_import_spans(sekv_ctx* ctx, int32_t b, int32_t m, const int32_t* mstart,
                              const int32_t* mcount, int32_t n_anchors, const int32_t* anchors);

/* Fix the packed-basis layout of a layer that is not built here (test hook):
 *   rank host int32 [B][H_kv][m_max], m_max as returned by sekv_get_spans (it
 *   includes the spare rows of sekv_reserve_spans): r_eff of every (b, g,
 *   span); entries at or beyond a sequence's m are ignored;
 *   1 <= rank <= min(mcount, d).
 * Allocates the layer's summaries, anchors and basis store (zero-filled);
 * sekv_import_head then fills them head by head.  A layer produced by
 * sekv_build already has its layout and needs no call.
 * Errors: INVALID, STATE (span table not set), OOM, HIP. */
sekv_status sekv_import_layout(sekv_ctx* ctx, int32_t layer, const int32_t* rank);

/* Install the artefacts of one (layer, b, kv head g) from host memory:
 *   kbar, vbar host KV dtype [m][d]; KA, VA host KV dtype [n_anchors][d];
 *   rank host int32 [m] (1 <= rank[k] <= min(mcount[k], d));
 *   bases host KV dtype, packed as described at sekv_get_bases_layout,
 *   basis_elems elements.
 * The layer needs a layout (sekv_build or sekv_import_layout) and the ranks
 * must equal that layout's; imports are synchronous, and drop the layer's
 * device basis cache (after a device synchronisation).  The layer is
 * decodable once every (b, g) has artefacts (all of them, after a build).
 * Errors: INVALID, STATE (no layout), OOM, HIP. */
sekv_status sekv_import_head(sekv_ctx* ctx, int32_t layer, int32_t b, int32_t g, const void* kbar,
                             const void* vbar, const void* KA, const void* VA, const int32_t* rank,
                             const void* bases, int64_t basis_elems);

/* Copy the artefacts of one (layer, b, g) to host memory (same layouts as
 * sekv_import_head; any pointer may be NULL).  KA / VA hold the layer's
 * window rows: sekv_get_window of them (the anchors plus the tokens appended
 * since the last build or re-segmentation).  Synchronous.
 * Errors: STATE (layer not built), INVALID, HIP. */
sekv_status sekv_export_head(const sekv_ctx* ctx, int32_t layer, int32_t b, int32_t g, void* kbar,
                             void* vbar, void* KA, void* VA, int32_t* rank, void* bases);

/* ------------------------------------------------------------ basis cache */

/* Device cache of host-resident bases with predictive prefetch, for
 * SEKV_BASES_HOST contexts [summary page, Figure 2: the zoomed spans' bases are
 * fetched asynchronously from the CPU; the pages point to prefetching the
 * spans likely needed next].  `bytes` of device memory are split evenly over
 * the layers, each share a ring whose oldest entries are evicted first.  After
 * each decode of layer l the zoom mask comes back to pinned memory; while a
 * layer decodes, the spans that the next layer zoomed at its previous step
 * (any head of the group) and that are not cached are copied into that
 * layer's ring on the context's side stream, and the next layer's decode
 * waits for that copy.  The decode kernel reads a zoomed span from the cache
 * when it is there and in place from the pinned store otherwise, so results do
 * not depend on the prediction.  bytes = 0 frees the cache.  Synchronises the
 * device.  With a cache, sekv_decode_attn is not capturable (it plans on the
 * host).  Statistics: sekv_stats.cache_*.
 * Errors: INVALID (other homes, bytes < 0), OOM, HIP. */
sekv_status sekv_set_basis_cache(sekv_ctx* ctx, int64_t bytes);

/* ---------------------------------------------------------- decode-time append */

/* Append n_new decoded tokens per sequence to layer `layer`'s local window
 * [summary page, Figure 2 and eq. (17): the recent tokens stay at full
 * resolution on the GPU].  They become full-resolution entries of the shared
 * softmax (like the anchors) for every later decode step of this layer.
 *   K_new, V_new dev KV dtype [B][H_kv][n_new][d]; n_new >= 0.
 * The tokens that pass beyond the last w positions stay at full resolution
 * until sekv_resegment_window turns them into spans.  Asynchronous on
 * `stream`, except when the window storage must grow
 * (geometrically): then the call copies the rows and synchronises `stream`.
 * Not capturable; a decode graph captured before an append does not see the
 * new tokens (capture again after appending).  Each layer appends on its own
 * (in a model, layer l appends its token before it decodes).
 * Errors: STATE (layer not built, capture), INVALID, OOM, HIP. */
sekv_status sekv_append_tokens(sekv_ctx* ctx, int32_t layer, const void* K_new, const void* V_new, int32_t n_new,
                               hipStream_t stream);

/* Full-resolution entries (anchors + appended tokens) of sequence b in layer
 * `layer`.  Errors: STATE (no layout), INVALID. */
sekv_status sekv_get_window(const sekv_ctx* ctx, int32_t layer, int32_t b, int32_t* n_anchors);

/* ------------------------------------------------- window re-segmentation */

/* Spare span rows per sequence for spans that re-segmentation adds later.
 * Call before the first sekv_build (the per-span arrays take their row stride,
 * the maximum span count plus `extra`, from the first build).  extra in
 * [0, 2^22].  Errors: STATE (the span table exists), INVALID. */
sekv_status sekv_reserve_spans(sekv_ctx* ctx, int32_t extra);

/* Surprisal of n_new decoded tokens per sequence, in the order they were (or
 * will be) appended with sekv_append_tokens.  H_new host fp32 [B][n_new],
 * finite and >= 0; copied.  Only for contexts whose span table came from
 * sekv_build (which records the prefill surprisal and threshold).
 * Errors: STATE (no surprisal record), INVALID. */
sekv_status sekv_append_surprisal(sekv_ctx* ctx, const float* H_new, int32_t n_new);

/* Streaming re-segmentation of the full-resolution window [summary page,
 * section 2.1 and Figure 2, applied to decoded tokens], all layers at once.
 * The window holds the last w positions; an older row (an appended token, or a
 * prefill anchor once appended tokens push it out) leaves it unless its
 * surprisal lies strictly above the prefill threshold mu + alpha sigma (such a
 * row is a boundary and stays a full-resolution anchor).  Every maximal run of
 * consecutive leaving positions becomes one new span, numbered after the
 * existing ones, with the weighted-mean summaries, routing summary, hard rank
 * (the rank choices and seed of the layer's build) and truncated SVD bases of
 * the prefill builder; the remaining rows stay in position order.  Earlier
 * spans and cuts never move.  Requires every layer built by sekv_build, the
 * same number of window rows in every layer (append to every layer first) and
 * the surprisal of every appended token.  Synchronous on `stream`; changes the
 * span table (sekv_get_spans), the bases layout and every layer's window, so
 * decode graphs must be captured again; clears the basis caches.  After it,
 * sekv_build is refused.  Not capturable.
 * Errors: STATE (not built by sekv_build, layers differ, surprisal missing,
 * capture), OOM (no span rows left: sekv_reserve_spans), INVALID, HIP.  These
 * refusals come before anything changes; an OOM or HIP error while the layers
 * are rebuilt leaves the context unusable (destroy it). */
sekv_status sekv_resegment_window(sekv_ctx* ctx, hipStream_t stream);

/* ------------------------------------------- routing projection, rank gates */

/* Routing projection of one layer [summary page, section 2.2, eq. (3); section
 * 2.3, eq. (5)].  W^(l,g) maps keys of kv head g into a d_route-dimensional
 * routing space; the builder then stores, per span, the routing summary
 *     Kbar_S = sum_t w_t W K_t / |sum_t w_t W K_t|      (zero if the sum is zero)
 * (computed as W kbar_S / |W kbar_S| from the unrounded weighted mean, which is
 * the same vector since sum_t w_t = 1), and decode scores query head h of kv
 * head g with (W^(l,g) q_h).Kbar_S / sqrt(d_route) + ln|S|.  The summary-entry
 * logit of a non-zoomed span keeps q.kbar_S/sqrt(d) + ln|S| in key space.
 *   W       host float32 [H_kv][d_route][d], finite; copied.
 *   d_route 0 (back to the identity projection and the cosine score) or a
 *           multiple of 8 in [8, d].
 * Must precede the layer's sekv_build / sekv_import_layout (STATE otherwise).
 * A routed layer decodes with one more small kernel per step (the query
 * projection).  Errors: INVALID, STATE, OOM, HIP. */
sekv_status sekv_set_routing(sekv_ctx* ctx, int32_t layer, int32_t d_route, const float* W);

/* Install (test hook) or read the routing summaries of one (layer, b, kv head g)
 * of a routed layer: host KV dtype [m][d_route].  An imported routed layer is
 * decodable once every head has both sekv_import_head and this.  Synchronous.
 * Errors: STATE (no layout, no routing projection, export of a head without
 * summaries), INVALID, HIP. */
sekv_status sekv_import_route_summary(sekv_ctx* ctx, int32_t layer, int32_t b, int32_t g, const void* Kr);
sekv_status sekv_export_route_summary(const sekv_ctx* ctx, int32_t layer, int32_t b, int32_t g, void* Kr);

/* Soft rank gates of eq. (6) [summary page, section 2.2]: multiply component i
 * of span k's stored key factor A_K = U_r Sigma_r by gate_k[k][i] (and of the
 * value factor by gate_v[k][i]), so that the rebuilt matrix becomes
 * sum_i m_i sigma_i u_i v_i^T.  Each exact product of a stored value and a gate
 * is rounded once to the KV dtype (nearest, ties to even).  The factors are
 * changed in place: applying gates twice multiplies them.
 *   gate_k, gate_v host float32 [m][d] (entries i >= rank[k] ignored), each in
 *   [0, 1]; either may be NULL (that factor is left alone).
 * Works on device and host basis stores; synchronises `stream` before it
 * returns.  A device basis cache of the layer (sekv_set_basis_cache) is
 * dropped first, after a device synchronisation, so that no cached copy of an
 * ungated factor is read afterwards.  Errors: STATE (head has no artefacts),
 * INVALID (gate outside [0, 1] or NaN), OOM, HIP. */
sekv_status sekv_apply_rank_gates(sekv_ctx* ctx, int32_t layer, int32_t b, int32_t g, const float* gate_k,
                                  const float* gate_v, hipStream_t stream);

/* ------------------------------------------------------------- diagnostics */

typedef struct sekv_stats {
  uint64_t decode_calls;          /* sekv_decode_attn calls */
  uint64_t fetch_calls;           /* sekv_zoom_fetch calls */
  uint64_t spans_fetched;         /* (b, g, span) bases copied to staging */
  uint64_t bytes_fetched;         /* bytes copied host -> staging */
  uint64_t memcpy_calls;          /* copy launches issued by fetches (one kernel per staged fetch or cache prefetch) */
  int64_t device_resident_bytes;  /* anchors + summaries (+ routing summaries) + tables (+ bases if DEVICE) */
  int64_t host_basis_bytes;       /* pinned store (HOST) */
  int64_t full_kv_bytes;          /* 2 * L * B * H_kv * n * d * elem: the full cache */
  uint64_t tokens_appended;       /* (b, layer) rows added by sekv_append_tokens */
  uint64_t cache_zoomed;          /* (layer-step, b, g, span) zoomed, counted by the cache's predictor */
  uint64_t cache_hits;            /* ... of which the bases were in the device cache */
  uint64_t cache_spans_fetched;   /* spans copied into the device cache by prefetch */
  uint64_t cache_bytes_fetched;   /* their bytes */
} sekv_stats;

sekv_status sekv_get_stats(const sekv_ctx* ctx, sekv_stats* out);

/* Per-(layer, query head) zoom counters [summary page, section 3.4 and Figures
 * 5-6, which read router health from the zoom rate of every (layer, head)].
 *   counts host uint64 [B][H_q] (or NULL): spans zoomed by each (sequence, query
 *          head) of `layer`, summed over the layer's decode calls since its
 *          layout was made (sekv_build, sekv_import_layout) or since the last
 *          reset; a span zoomed by several query heads of a group counts for
 *          each of them.
 *   calls  host uint64 (or NULL): the number of those decode calls.
 *   reset  nonzero: zero both counters after reading.
 * The counters live on the device and are advanced by the combine kernel of
 * every decode call (graph replays included, no host synchronisation); the
 * zoom rate of a head is counts / (calls * m) with m the sequence's span count.
 * This call synchronises the device.  Errors: INVALID (layer out of range),
 * STATE (layer has no layout), HIP. */
sekv_status sekv_get_zoom_counts(sekv_ctx* ctx, int32_t layer, uint64_t* counts, uint64_t* calls,
                                 int32_t reset);

#ifdef __cplusplus
}
#endif

#endif /* SEKV_H */
