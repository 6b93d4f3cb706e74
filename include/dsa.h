/*
 * dsa.h -- C ABI of the MI355X (gfx950) DeepSeek Sparse Attention step.
 *
 * The step, per query token t of request r (SemiAnalysis, "Sparse Savings,
 * Persistent Demand: inside GLM-5.3", section "DeepSeek Sparse Attention"):
 *   1. lightning indexer ("Lightning Indexer"): for every visible token s,
 *        I[t,s] = sigma_s * sum_h w[t,h] * ReLU(q_idx[t,h,:] . k[s,:])
 *   2. top-K: keep the K highest-scoring visible tokens (all of them when a
 *      query sees K or fewer); equal scores go to the lower token index;
 *   3. sparse MLA in MQA mode ("Sparse MLA", "MLA Modifications"):
 *        z_j = scale * q_mla[t,h,:] . kv[s_j, 0:d+r]
 *        out[t,h,:] = softmax(z) . kv[s_j, 0:d]   (V = first d columns)
 * Query j (0-based) of request r sits at position p = L_r - q_len_r + j and
 * sees tokens [0, p] (n = p + 1 tokens).  L_r counts the new query tokens.
 *
 * Conventions shared by every entry point
 *   - All array arguments are DEVICE pointers unless marked "host".  The
 *     caller owns every buffer; the library never allocates or frees, does
 *     not synchronise (outside the debug check below), keeps no state
 *     between calls, and is reentrant.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *     default stream).  Only host-visible arguments are validated; a bad
 *     device value (page id, index) is undefined behaviour and surfaces at
 *     the caller's next synchronisation.
 *   - Debug mode: with DSA_DEBUG set in the environment (to anything but ""
 *     or "0"; read on every call), each entry point first runs the check of
 *     dsa_check_batch on the device values it will read (page ids against
 *     the caches' num_blocks when given, selections against their rows'
 *     visible counts) and returns DSA_ERR_BAD_DEVICE_ARG, with nothing else
 *     launched, when one is out of range; after launching it waits for
 *     `stream` and returns DSA_ERR_LAUNCH if the work failed.  So in debug
 *     mode every call synchronises, and calls under stream capture return
 *     DSA_ERR_UNSUPPORTED.
 *   - Return value: DSA_OK (0) or a negative dsa_status; nothing is printed
 *     and no exception crosses the ABI.  On error nothing was launched.
 *   - Paged caches: logical token s of request r lives in physical block
 *     page_table[r * max_blocks + s / block_size], slot s % block_size; a
 *     cache of row width W is laid out [num_blocks][block_size][W].
 *   - Token indices are LOGICAL positions within the request (so a second
 *     layer with its own latent pool can reuse them: "IndexShare").
 *   - Device tensors start 16-byte aligned (as device allocators return
 *     them); the kernels use 16-byte vector loads and stores.
 *   - Workspaces: pass at least dsa_workspace_size(op, ...) bytes, 256-byte
 *     aligned.  Contents on entry are ignored; on return they are garbage.
 *     Calls that share a workspace must be ordered on one stream.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef void *dsa_stream_t; /* a hipStream_t */

enum dsa_status {
    DSA_OK = 0,
    DSA_ERR_INVALID_ARG = -1,   /* null pointer, negative size, inconsistent shape */
    DSA_ERR_UNSUPPORTED = -2,   /* dtype or shape combination not implemented */
    DSA_ERR_WORKSPACE = -3,     /* workspace smaller than dsa_workspace_size() */
    DSA_ERR_DEVICE = -4,        /* current device is not gfx950 */
    DSA_ERR_LAUNCH = -5,        /* a HIP launch returned an error */
    DSA_ERR_TOO_LARGE = -6,     /* batch beyond dsa_decode_step_noalloc's built-in scratch */
    DSA_ERR_BAD_DEVICE_ARG = -7 /* a device value out of range (dsa_check_batch, DSA_DEBUG) */
};

/* Storage formats.  DSA_E4M3 is the OCP e4m3fn fp8 format (max 448). */
enum dsa_dtype { DSA_F32 = 0, DSA_BF16 = 1, DSA_E4M3 = 2, DSA_MXFP4 = 3 };

/* Operations for dsa_workspace_size(). */
enum dsa_op {
    DSA_OP_TOPK = 1,
    DSA_OP_MLA_DECODE = 2,
    DSA_OP_MLA_PREFILL = 3,
    DSA_OP_DECODE_STEP = 4
};

/* Batch geometry.  The struct itself lives in host memory. */
typedef struct {
    int32_t num_requests;          /* host: B >= 1 */
    int32_t total_q;               /* host: T = sum of q_len_r >= 1 */
    int32_t max_q_len;             /* host: upper bound of q_len_r */
    int32_t max_context_len;       /* host: upper bound of L_r */
    const int32_t *context_lens;   /* [B] L_r >= q_len_r */
    const int32_t *query_start_loc;/* [B+1] query rows of r are [qsl[r], qsl[r+1]) */
    const int32_t *page_table;     /* [B][max_blocks] physical block ids */
    int32_t max_blocks;            /* host: row stride of page_table */
    int32_t block_size;            /* host: tokens per block */
} dsa_batch;

/* Indexer key cache: keys [num_blocks][block_size][dim] in `dtype`
 * (DSA_F32 or DSA_E4M3); scales [num_blocks][block_size] fp32 sigma_s >= 0,
 * or NULL for sigma = 1.
 * DSA_MXFP4 keys (OCP Microscaling Formats v1.0: FP4 E2M1 elements, one
 * E8M0 power-of-two scale per 32 elements; dim a multiple of 32): each block
 * is block_size x dim/2 bytes of packed codes (element 2i in the low nibble
 * of byte i) followed by block_size x dim/32 E8M0 bytes (scale b of a token
 * covers its elements [32b, 32b + 32)); the queries are e4m3.  The article's
 * one-launch design names FP4 support as its next step (SemiAnalysis GLM-5.3,
 * "Optimizations", "TileRT"); the format is this library's reading.  The
 * decode step takes such keys through the score rows and dsa_topk's
 * selection (not the candidate-emitting indexer or dsa_decode_step_fused). */
typedef struct {
    const void *keys;
    const float *scales;
    int32_t dtype;
    int32_t dim;
    int32_t num_blocks;   /* blocks in the pool, or 0 if not stated (read only by the debug check) */
} dsa_index_cache;

/* MLA latent cache: kv [num_blocks][block_size][d_latent + d_rope] in
 * `dtype` (DSA_F32, DSA_BF16 or DSA_E4M3); scales [num_blocks][block_size]
 * (one fp32 per token covering all d+r columns; required for DSA_E4M3,
 * must be NULL otherwise). */
typedef struct {
    const void *kv;
    const float *scales;
    int32_t dtype;
    int32_t d_latent;
    int32_t d_rope;
    int32_t num_blocks;   /* blocks in the pool, or 0 if not stated (read only by the debug check) */
} dsa_latent_cache;

/*
 * Lightning-indexer scores (step 1).
 *   q_idx  [T][n_heads_idx][dim], same dtype as the key cache (fp32 or e4m3;
 *          e4m3 for MXFP4 keys; a per-(t,h) query scale is folded into w by
 *          the caller).
 *   w      [T][n_heads_idx] fp32 head weights.
 *   scores [T][ld_scores] fp32: scores[t][s] for s < n_t, and -inf for
 *          n_t <= s < ld_scores (positions a query does not see).
 *          ld_scores >= max_context_len.
 */
int dsa_indexer_scores(const dsa_batch *batch, const dsa_index_cache *cache,
                       const void *q_idx, const float *w, int32_t n_heads_idx,
                       float *scores, int64_t ld_scores, dsa_stream_t stream);

/*
 * Top-K selection (step 2) from materialised scores.
 *   indices [T][k] int32: the min(k, n_t) selected logical positions of row t
 *           in ascending order, then -1 padding.  Selection rule: highest
 *           score first, lower index first among equal scores.  1 <= k <= 4096.
 *   workspace: dsa_workspace_size(DSA_OP_TOPK, batch, k, 0) bytes
 *           (candidate slots for rows longer than 12288 tokens, about 4 bytes
 *           per score; 0 when no row is that long, and NULL is then accepted).
 */
int dsa_topk(const dsa_batch *batch, const float *scores, int64_t ld_scores, int32_t k,
             int32_t *indices, void *workspace, size_t workspace_bytes, dsa_stream_t stream);

/*
 * Sparse MQA-mode MLA (step 3) for decode-sized batches (a few query rows per
 * request); splits each row's selection across workgroups and merges the
 * partial softmaxes by their log-sum-exp.
 *   q       [T][n_heads][d_latent+d_rope]: fp32 for an fp32 cache, bf16 otherwise.
 *   indices [T][k] int32 logical positions; entries < 0 are skipped (the
 *           -1 padding of dsa_topk).  Positions must be < n_t of the row.
 *   out     [T][n_heads][d_latent]: fp32 for an fp32 cache, bf16 otherwise.
 *   lse     [T][n_heads] fp32 natural-log log-sum-exp of the scaled logits,
 *           or NULL.  A row with no valid index gets out = 0, lse = -inf.
 *   workspace: dsa_workspace_size(DSA_OP_MLA_DECODE, batch, k, n_heads).
 */
int dsa_sparse_mla_decode(const dsa_batch *batch, const dsa_latent_cache *cache,
                          const void *q, int32_t n_heads, const int32_t *indices, int32_t k,
                          float softmax_scale, void *out, float *lse,
                          void *workspace, size_t workspace_bytes, dsa_stream_t stream);

/*
 * dsa_sparse_mla_decode over several layers that share one selection (the
 * IndexShare pattern: "IndexShare", the full layer's top-K serves the
 * layers after it), in one call: layer l attends with its own cache
 * caches[l], queries q[l] and outputs out[l] (and lse[l]) over the same
 * `indices`.  The 128-head path runs every layer in one launch (and merges
 * every layer's splits in one more), so the layers' workgroups overlap;
 * other shapes run the layers one after another.  Same results as
 * n_layers calls of dsa_sparse_mla_decode, bit for bit.
 *   caches, q, out: host arrays of n_layers entries (1 <= n_layers <= 4);
 *           every cache has the same dtype, d_latent and d_rope.
 *   lse:    host array of n_layers entries (each may be NULL), or NULL.
 *   workspace: n_layers * dsa_workspace_size(DSA_OP_MLA_DECODE, batch, k,
 *           n_heads) bytes.
 * Errors as dsa_sparse_mla_decode; DSA_ERR_INVALID_ARG for n_layers out of
 * range or NULL arrays, DSA_ERR_UNSUPPORTED for caches of different shapes.
 */
int dsa_sparse_mla_decode_layers(const dsa_batch *batch, const dsa_latent_cache *caches, int32_t n_layers,
                                 const void *const *q, int32_t n_heads, const int32_t *indices, int32_t k,
                                 float softmax_scale, void *const *out, float *const *lse,
                                 void *workspace, size_t workspace_bytes, dsa_stream_t stream);

/*
 * Sparse MQA-mode MLA for prefill-sized batches (many query rows per request,
 * e.g. a 4096-token chunk).  Same arguments and results as the decode entry;
 * each workgroup covers whole selections, so no partial results are merged.
 * Reusing one layer's `indices` with another layer's cache and q is the
 * IndexShare pattern ("IndexShare": cache the top-K at the full layer).
 *   workspace: dsa_workspace_size(DSA_OP_MLA_PREFILL, ...) (may be 0).
 */
int dsa_sparse_mla_prefill(const dsa_batch *batch, const dsa_latent_cache *cache,
                           const void *q, int32_t n_heads, const int32_t *indices, int32_t k,
                           float softmax_scale, void *out, float *lse,
                           void *workspace, size_t workspace_bytes, dsa_stream_t stream);

/*
 * The whole step: indexer scores, top-K and sparse MLA in one call, scores
 * kept in the workspace.  Arguments as in the three calls above.
 *   indices_out  [T][k] or NULL: when given, the selection is also returned
 *                (for reuse by layers that share this layer's indexer).
 *   workspace: dsa_workspace_size(DSA_OP_DECODE_STEP, batch, k, n_heads)
 *   (enough for dsa_decode_step_fused as well).
 */
int dsa_decode_step(const dsa_batch *batch, const dsa_index_cache *index_cache,
                    const void *q_idx, const float *w, int32_t n_heads_idx,
                    const dsa_latent_cache *latent_cache, const void *q_mla, int32_t n_heads,
                    int32_t k, float softmax_scale, void *out, float *lse, int32_t *indices_out,
                    void *workspace, size_t workspace_bytes, dsa_stream_t stream);

/*
 * Measurement variant of dsa_decode_step: the same launches and results,
 * plus DSA_STEP_EVENTS events recorded on `stream` at the step's phase
 * boundaries, so that a caller can time each phase on the stream it runs on:
 *   events[0] before the first launch (so events[0..1] span the top-K bound
 *   sampling, empty when the step takes none), events[1] and events[2] at
 *   the start and end of the lightning indexer (taken by the kernel launch
 *   itself for the persistent decode indexer, so they span the kernel
 *   alone), events[3] after the top-K selection, events[4] after sparse MLA
 *   (and its split combine).
 *   events: DSA_STEP_EVENTS caller-created hipEvent_t handles (as void*);
 *           recording allocates nothing.  n_events >= DSA_STEP_EVENTS, else
 *           DSA_ERR_INVALID_ARG (also for a NULL handle).
 */
#define DSA_STEP_EVENTS 5
int dsa_decode_step_timed(const dsa_batch *batch, const dsa_index_cache *index_cache,
                          const void *q_idx, const float *w, int32_t n_heads_idx,
                          const dsa_latent_cache *latent_cache, const void *q_mla, int32_t n_heads,
                          int32_t k, float softmax_scale, void *out, float *lse, int32_t *indices_out,
                          void *workspace, size_t workspace_bytes, dsa_stream_t stream,
                          void *const *events, int32_t n_events);

/*
 * The same step as one persistent kernel (with a one-workgroup init kernel
 * before it and the merge of split attention after it), following the
 * one-launch decode design of the SemiAnalysis GLM-5.3 article, section
 * "Optimizations" ("TileRT"): workgroups take, in this order, a ready row
 * selection, a ready attention slice, or the next chunk of the key stream,
 * so the selection and attention of requests whose keys are done overlap
 * the key stream of the others.  Same arguments, results (selection exact,
 * output within the tolerances of dsa_decode_step) and workspace
 * (dsa_workspace_size(DSA_OP_DECODE_STEP, ...)) as dsa_decode_step.
 *   Shapes: e4m3 index keys with dim 128 and 16, 32 or 64 indexer heads,
 *   block_size 64, at most 2 query rows a request, bf16 or e4m3 latents of
 *   512 + 64 with 128 MLA heads, softmax_scale != 0, k <= 4096; other
 *   shapes return DSA_ERR_UNSUPPORTED (dsa_decode_step covers them).
 *   events: NULL, or DSA_STEP_EVENTS caller-created hipEvent_t handles (as
 *           void*) recorded on `stream`: events[0] before the first launch,
 *           events[1] and events[2] at the start and end of the persistent
 *           kernel (taken by its launch, so they span the kernel alone),
 *           events[3] after it and events[4] after the merge.  With events,
 *           n_events >= DSA_STEP_EVENTS, else DSA_ERR_INVALID_ARG (also for
 *           a NULL handle).
 *   A wait inside the kernel that gives up (a bound far above any real
 *   step's duration) leaves NaN in every output and lse instead of a result.
 */
int dsa_decode_step_fused(const dsa_batch *batch, const dsa_index_cache *index_cache,
                          const void *q_idx, const float *w, int32_t n_heads_idx,
                          const dsa_latent_cache *latent_cache, const void *q_mla, int32_t n_heads,
                          int32_t k, float softmax_scale, void *out, float *lse, int32_t *indices_out,
                          void *workspace, size_t workspace_bytes, dsa_stream_t stream,
                          void *const *events, int32_t n_events);

/*
 * dsa_decode_step without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  Same arguments (minus the workspace)
 * and the same results as dsa_decode_step.  It allocates nothing: its
 * workspace is a scratch array of DSA_NOALLOC_SCRATCH_BYTES that the library
 * holds on every GPU it runs on until the process ends (its device address is
 * looked up on the first call on each device).
 *   A batch whose dsa_workspace_size(DSA_OP_DECODE_STEP, ...) exceeds the
 *   scratch is rejected with DSA_ERR_TOO_LARGE before anything is launched
 *   (128 MiB covers, e.g., 64 query rows at 128K context, K = 2048, 128 MLA
 *   heads).  Other errors as dsa_decode_step.
 *   All calls on one GPU share that GPU's scratch, which keeps the last
 *   call's contents (the step initialises what it needs): calls that may
 *   overlap on one GPU (different streams, different host threads) race and
 *   must be ordered by the caller.
 */
#define DSA_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
int dsa_decode_step_noalloc(const dsa_batch *batch, const dsa_index_cache *index_cache,
                            const void *q_idx, const float *w, int32_t n_heads_idx,
                            const dsa_latent_cache *latent_cache, const void *q_mla, int32_t n_heads,
                            int32_t k, float softmax_scale, void *out, float *lse, int32_t *indices_out,
                            dsa_stream_t stream);

/* Workspace bytes for `op` (enum dsa_op) with this batch geometry; 0 for an
 * invalid request and for calls that need none (top-K on rows of at most
 * 12288 tokens, prefill MLA without splits).  Host-only, never touches the
 * device. */
size_t dsa_workspace_size(int32_t op, const dsa_batch *batch, int32_t k, int32_t n_heads);

/* Static text for a status code. */
const char *dsa_status_string(int32_t status);

/*
 * Synchronous check of the device-side batch values the entry points trust
 * (the check that DSA_DEBUG adds to every call).  Per request r:
 *   DSA_CHECK_QUERY_START  query_start_loc starts at 0, ends at total_q and
 *                          does not decrease, each q_len_r <= max_q_len;
 *   DSA_CHECK_CONTEXT      q_len_r <= L_r <= max_context_len;
 *   DSA_CHECK_PAGE         the ceil(L_r / block_size) page ids the request
 *                          uses are >= 0 and, when num_blocks > 0, below it;
 *   DSA_CHECK_INDEX        (when indices [total_q][k] is given) every entry
 *                          of row t is < n_t (negative entries are padding).
 * Page ids and indices of a request are checked only when its query range
 * and length hold.  failed (host, may be NULL) receives the OR of the bits
 * that failed.  Waits for `stream`.  Returns DSA_OK, DSA_ERR_BAD_DEVICE_ARG
 * (some check failed), DSA_ERR_INVALID_ARG for host-visible errors,
 * DSA_ERR_UNSUPPORTED while `stream` is being captured, DSA_ERR_LAUNCH.
 */
#define DSA_CHECK_QUERY_START 1u
#define DSA_CHECK_CONTEXT 2u
#define DSA_CHECK_PAGE 4u
#define DSA_CHECK_INDEX 8u
int dsa_check_batch(const dsa_batch *batch, int32_t num_blocks, const int32_t *indices, int32_t k,
                    uint32_t *failed, dsa_stream_t stream);

/* DSA_OK if the current HIP device is gfx950, else DSA_ERR_DEVICE. */
int dsa_check_device(void);

/*
 * Two-tier latent cache (HiSparse design: SemiAnalysis, "Sparse Savings,
 * Persistent Demand: inside GLM-5.3", section "How Sparse Attention Affects
 * DRAM/NAND Memory"; remio.ai, section "HiSparse Move o Histórico Completo
 * para Fora da GPU"): a bounded hot set of latent rows in device memory in front of
 * the full paged latent cache, which stays in pinned host memory.  All
 * buffers are caller-owned device memory:
 *   kv        [capacity][d_latent + d_rope] in the host cache's dtype;
 *   scales    [capacity] fp32 (DSA_E4M3 caches), NULL otherwise;
 *   slot_of   [num_requests][max_context_len] int32: slot of token s of
 *             request r, -1 if not resident;
 *   owner     [capacity] int64: (r << 32) | s of the slot's token, -1 if free;
 *   last_use  [capacity] int32: step of the slot's last use, -1 if never;
 *   clock     [1] int32: the last step (fetches number themselves).
 * The state is bound to one batch layout (num_requests, max_context_len):
 * reset it when that layout changes.
 */
typedef struct {
    void *kv;
    float *scales;
    int32_t capacity;
    int32_t *slot_of;
    int64_t *owner;
    int32_t *last_use;
    int32_t *clock;
} dsa_hot_cache;

/* Empties a hot cache (no token resident, no slot used, clock 0). */
int dsa_hot_cache_reset(const dsa_batch *batch, dsa_hot_cache *hot, dsa_stream_t stream);

/* Workspace bytes of dsa_hot_cache_fetch for this batch, k and capacity (0
 * for an invalid request).  Host-only. */
size_t dsa_hot_cache_workspace_size(const dsa_batch *batch, int32_t k, int32_t capacity);

/*
 * One step of the two-tier cache for a selection `indices` [T][k] (logical
 * positions, -1 padding, as written by dsa_topk / dsa_decode_step): makes
 * every selected token resident in the hot set.
 *  1. selected tokens already resident are hits: their slot's last use
 *     becomes this step (clock + 1);
 *  2. the distinct selected tokens not resident are the misses, in
 *     (request, token) order;
 *  3. victims: the slots not used in this step with the greatest age
 *     (step - last use, saturated at 65535; never used = 65535), ties to the
 *     lower slot, as many as misses; taken as every victim older than the
 *     last one's age in slot order, then those of that age in slot order;
 *  4. miss i moves into victim i: the slot's previous token loses it, the
 *     row (and scale) is read from the host cache (batch->page_table,
 *     block_size layout; `host->kv` and `host->scales` in pinned host memory
 *     that the device can address) and written to the slot.
 * Afterwards sparse MLA over the hot set is dsa_sparse_mla_decode with the
 * batch's page_table = slot_of, max_blocks = max_context_len, block_size = 1,
 * and the latent cache {hot->kv, hot->scales}: the same rows, so the same
 * output as over the full cache.  counts (device int32 [2] or NULL): misses,
 * evictions.  capacity must be >= total_q * k (every selected token of the
 * step fits); DSA_ERR_INVALID_ARG otherwise or for null pointers,
 * DSA_ERR_UNSUPPORTED for a cache whose rows are not a multiple of 16 bytes
 * or exceed 2 KB, DSA_ERR_WORKSPACE for a small workspace.  Asynchronous on `stream`; calls on one hot cache must be
 * ordered on one stream.
 */
int dsa_hot_cache_fetch(const dsa_batch *batch, const dsa_latent_cache *host, const int32_t *indices, int32_t k,
                        dsa_hot_cache *hot, int32_t *counts, void *workspace, size_t workspace_bytes,
                        dsa_stream_t stream);

/*
 * The two phases of dsa_hot_cache_fetch as separate calls (same arguments;
 * dsa_hot_cache_fetch = plan, then copy, with the same workspace):
 *   dsa_hot_cache_plan  steps 1-3: hits (their last use becomes this step),
 *                       the misses and the victims, kept in the workspace;
 *   dsa_hot_cache_copy  step 4: each miss into its victim slot, the rows read
 *                       from host memory; advances the clock, writes counts.
 * For the layer-wise overlap of the same design (while layer N attends over
 * its hot set, later layers' rows are read from host memory): the plans of
 * later layers, short kernels, can run beside a layer's copies, which take
 * a few compute units and the host link.  A copy must follow its own plan on
 * the same workspace, with no other call on that workspace or hot cache in
 * between.  Errors as dsa_hot_cache_fetch.
 */
int dsa_hot_cache_plan(const dsa_batch *batch, const dsa_latent_cache *host, const int32_t *indices, int32_t k,
                       dsa_hot_cache *hot, void *workspace, size_t workspace_bytes, dsa_stream_t stream);
int dsa_hot_cache_copy(const dsa_batch *batch, const dsa_latent_cache *host, const int32_t *indices, int32_t k,
                       dsa_hot_cache *hot, int32_t *counts, void *workspace, size_t workspace_bytes,
                       dsa_stream_t stream);

/* Measurement helper, not a step of the method: the practical HBM read
 * bandwidth that the library's streaming kernels are compared against.
 * dsa_read_probe reads every byte of `buf` (device memory, 16-byte aligned,
 * nbytes a positive multiple of 16, caller-owned) exactly once with 16-byte
 * non-temporal loads, and writes one 32-bit word per workgroup to `sink`
 * (device, caller-owned, at least dsa_read_probe_sink_size() bytes; its
 * contents are meaningless), asynchronously on `stream`; time it with events
 * around the call.  DSA_ERR_INVALID_ARG for a null, misaligned or
 * wrongly sized buffer, DSA_ERR_WORKSPACE for a small sink, DSA_ERR_LAUNCH if
 * the launch fails.  dsa_read_probe_sink_size queries the current device's
 * CU count. */
size_t dsa_read_probe_sink_size(void);
int dsa_read_probe(const void *buf, int64_t nbytes, void *sink, size_t sink_bytes, dsa_stream_t stream);

/* Measurement helper, not a step of the method: the read rate of the
 * decode indexer's access pattern without its arithmetic.  dsa_page_probe
 * reads, for each of the n_pages block ids in `block_ids` (device int32,
 * caller-owned, ids into both pools; the caller keeps them in range),
 * page_bytes at pages + id * page_bytes (device, 16-byte aligned; a
 * multiple of 1024, at most 8192) and scale_bytes at scales + id *
 * scale_bytes (device, 4-byte aligned; 0 to 256, a multiple of 4; scales
 * may be NULL when scale_bytes is 0), with the indexer's grid (two 4-wave
 * workgroups per CU), equal contiguous shares of the list per wave and two
 * pages in flight per wave, and writes one 32-bit word per lane to `sink`
 * (device, caller-owned, at least dsa_page_probe_sink_size() bytes): the
 * XOR of the words that lane read, so the XOR of the whole sink is the XOR
 * of every word read.  Asynchronous on `stream`; time it with events.
 * DSA_ERR_INVALID_ARG for a null pointer, a bad size or a misaligned pool,
 * DSA_ERR_WORKSPACE for a small sink, DSA_ERR_LAUNCH if the launch fails;
 * n_pages = 0 launches nothing. */
size_t dsa_page_probe_sink_size(void);
int dsa_page_probe(const void *pages, int64_t page_bytes, const void *scales, int64_t scale_bytes,
                   const int32_t *block_ids, int32_t n_pages, void *sink, size_t sink_bytes, dsa_stream_t stream);

/* Measurement helper, not a step of the method: the read rate of the
 * 128-head sparse-MLA tile's gather without its arithmetic.  dsa_row_probe
 * reads the n_rows rows listed in `row_ids` (device int32, caller-owned, row
 * ids into the pool; the caller keeps them in range), row id r being
 * row_bytes at base + r * row_bytes (device, 16-byte aligned; row_bytes a
 * multiple of 128, at most 1152: a bf16 latent row of 512 + 64 values), in
 * the tile's launch shape: one 4-wave workgroup per rows_per_wg consecutive
 * entries of the list (a multiple of 32 that divides n_rows), 32-row tiles
 * through a 4-deep LDS ring by direct global-to-LDS transfers, three tiles in
 * flight.  It writes one 32-bit word per workgroup to `sink` (device,
 * caller-owned, at least dsa_row_probe_sink_size(n_rows, rows_per_wg)
 * bytes): the XOR of every 32-bit word of the workgroup's rows.
 * Asynchronous on `stream`; time it with events.  DSA_ERR_INVALID_ARG for a
 * null pointer, a misaligned pool or a bad size, DSA_ERR_WORKSPACE for a
 * small sink, DSA_ERR_LAUNCH if the launch fails; n_rows = 0 launches
 * nothing. */
size_t dsa_row_probe_sink_size(int32_t n_rows, int32_t rows_per_wg);
int dsa_row_probe(const void *base, int64_t row_bytes, const int32_t *row_ids, int32_t n_rows, int32_t rows_per_wg,
                  void *sink, size_t sink_bytes, dsa_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
