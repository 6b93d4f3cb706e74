// C ABI of the DSA step (declared in include/dsa.h): argument validation,
// workspace layout and kernel launches.  No allocation, no synchronisation,
// no state kept between calls.
#include <string.h>

#include <algorithm>
#include <mutex>

#include "dsa.h"
#include "dsa_kernels.h"

using namespace dsa;

namespace {

constexpr size_t ALIGN = 256;

size_t align_up(size_t x) { return (x + ALIGN - 1) / ALIGN * ALIGN; }

int64_t round_up64(int64_t x) { return (x + 63) / 64 * 64; }

bool batch_ok(const dsa_batch* b) {
    return b && b->num_requests >= 1 && b->total_q >= 1 && b->max_q_len >= 1 &&
           b->max_context_len >= 1 && b->max_context_len >= b->max_q_len && b->context_lens &&
           b->query_start_loc && b->page_table && b->block_size >= 1 && b->max_blocks >= 1 &&
           (int64_t)b->max_blocks * b->block_size >= b->max_context_len;
}

Geometry geometry(const dsa_batch* b) {
    Geometry g;
    g.B = b->num_requests;
    g.T = b->total_q;
    g.max_q_len = b->max_q_len;
    g.max_ctx = b->max_context_len;
    g.q_uniform = (int64_t)b->total_q == (int64_t)b->num_requests * b->max_q_len ? b->max_q_len : 0;
    g.ctx = b->context_lens;
    g.qsl = b->query_start_loc;
    g.page_table = b->page_table;
    g.max_blocks = b->max_blocks;
    g.block_size = b->block_size;
    return g;
}

// Workspace pieces (byte offsets from the base, each 256-aligned).
struct TopkLayout { size_t bound, count, cmax, cand, end; int nchunks; };
TopkLayout topk_layout(size_t base, const dsa_batch* b) {
    TopkLayout l;
    l.bound = l.count = l.cmax = l.cand = l.end = base;
    l.nchunks = 0;
    if (b->max_context_len > TOPK_LIST) {
        l.nchunks = (int)(((int64_t)b->max_context_len + TOPK_CHUNK - 1) / TOPK_CHUNK);
        const size_t rc = (size_t)b->total_q * l.nchunks;
        l.count = align_up(base + sizeof(uint32_t) * (size_t)b->total_q);
        l.cmax = align_up(l.count + sizeof(uint32_t) * rc);
        l.cand = align_up(l.cmax + sizeof(uint32_t) * rc);
        l.end = align_up(l.cand + sizeof(uint64_t) * rc * TOPK_CAND_CAP);
    }
    return l;
}

// Split partials: fp16 [T][H][S][512], then (lse, scale) [T][H][S][2].
struct MlaLayout { size_t part_o, part_lse, end; int splits; };
MlaLayout mla_layout(size_t base, const dsa_batch* b, int k, int n_heads, bool prefill, int path) {
    MlaLayout l;
    l.splits = mla_splits(path, b->total_q, n_heads, k, prefill);
    l.part_o = l.part_lse = l.end = base;
    if (l.splits > 1) {
        const size_t th = (size_t)b->total_q * n_heads * l.splits;
        l.part_lse = align_up(base + sizeof(uint16_t) * th * 512);
        l.end = align_up(l.part_lse + 2 * sizeof(float) * th);
    }
    return l;
}

// Largest MLA workspace over the latent dtypes of the fast paths (for size
// queries that do not name the dtype).
size_t mla_layout_max(size_t base, const dsa_batch* b, int k, int n_heads, bool prefill) {
    size_t end = base;
    for (int dt = 0; dt <= 2; ++dt)
        end = std::max(end, mla_layout(base, b, k, n_heads, prefill, mla_path(dt, 512, 64, n_heads)).end);
    return end;
}

// Decode-step workspace: score rows (written by the indexer, or by the
// selection's recompute path), indices, the top-K slots of the score-writing
// path, the candidate lists of the emitting path (bound, count, TOPK_LIST
// composites per query row), then the MLA partials.
struct StepLayout {
    size_t scores, indices, bound, count, cand, mla_base;
    TopkLayout tk; MlaLayout ml; size_t end; int64_t ld;
};
StepLayout step_layout(const dsa_batch* b, int k, int n_heads, int mla_path_id) {
    StepLayout l;
    const size_t T = (size_t)b->total_q;
    l.ld = round_up64(b->max_context_len);
    l.scores = 0;
    l.indices = align_up(sizeof(float) * T * l.ld);
    l.tk = topk_layout(align_up(l.indices + sizeof(int32_t) * T * k), b);
    l.bound = l.tk.end;
    l.count = align_up(l.bound + sizeof(uint32_t) * T);
    l.cand = align_up(l.count + sizeof(uint32_t) * T * ROW_COUNT_STRIDE);
    l.mla_base = align_up(l.cand + sizeof(uint64_t) * T * TOPK_LIST);
    l.ml = mla_layout(l.mla_base, b, k, n_heads, false, mla_path_id);
    l.end = l.ml.end;
    return l;
}

// Fused decode-step workspace: score rows (for rows whose chunk quotas fail),
// indices, candidate lists and counts, the per-row and per-request
// bookkeeping, the ready queue, and the partial slots of split attention.
struct FusedLayout {
    size_t scores, indices, cand, count, excl, req_done, prefix, chunk_req, slot, splits, ctr, rq, part_o, part_lse, end;
    int64_t ld;
    int rq_cap, part_slots;
};
// Partial slots: a pool of 8 per query row plus 32 (so one or two rows can
// always take 16 slices), then a reserve of 2 per row.
constexpr int FUSED_SLOTS_PER_ROW = 8, FUSED_SLOTS_EXTRA = 32, FUSED_SLOTS_RESERVE = 2;
FusedLayout fused_layout(const dsa_batch* b, int k, int n_heads) {
    FusedLayout l;
    const size_t T = (size_t)b->total_q, B = (size_t)b->num_requests;
    l.ld = round_up64(b->max_context_len);
    l.rq_cap = (int)(B + T * FU_MAX_SPLITS);
    l.part_slots = (int)(T * FUSED_SLOTS_PER_ROW + FUSED_SLOTS_EXTRA);
    const size_t slots = (size_t)l.part_slots + FUSED_SLOTS_RESERVE * T;
    l.scores = 0;
    l.indices = align_up(sizeof(float) * T * l.ld);
    l.cand = align_up(l.indices + sizeof(int32_t) * T * k);
    l.count = align_up(l.cand + sizeof(uint64_t) * T * TOPK_LIST);
    l.excl = align_up(l.count + sizeof(uint32_t) * T * ROW_COUNT_STRIDE);
    l.req_done = align_up(l.excl + sizeof(uint64_t) * T);
    l.prefix = align_up(l.req_done + sizeof(uint32_t) * B * ROW_COUNT_STRIDE);
    // chunks of 64 pages of 64 tokens: at most this many per request
    const size_t max_chunks = B * (size_t)((b->max_context_len + 64 * 64 - 1) / (64 * 64));
    l.chunk_req = align_up(l.prefix + sizeof(uint32_t) * (B + 1));
    l.slot = align_up(l.chunk_req + 2 * sizeof(uint32_t) * max_chunks);
    l.splits = align_up(l.slot + sizeof(uint32_t) * T);
    l.ctr = align_up(l.splits + sizeof(uint32_t) * T);
    l.rq = align_up(l.ctr + sizeof(uint32_t) * FC_N);
    l.part_o = align_up(l.rq + 4 * sizeof(uint32_t) * (size_t)l.rq_cap);
    l.part_lse = align_up(l.part_o + sizeof(uint16_t) * 512 * (size_t)n_heads * slots);
    l.end = align_up(l.part_lse + 2 * sizeof(float) * (size_t)n_heads * slots);
    return l;
}

int launch_status(hipError_t e) { return e == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH; }

// Pool size for the debug check's page-id bound: the smaller stated one of
// two caches that share the page table, 0 when neither states it.
int pool_blocks(int a, int b) {
    if (a > 0 && b > 0) return std::min(a, b);
    return a > 0 ? a : (b > 0 ? b : 0);
}

// Workspace of the multi-kernel decode step for any latent dtype.
size_t step_workspace(const dsa_batch* b, int k, int n_heads) {
    size_t end = 0;
    for (int dt = 0; dt <= 2; ++dt) end = std::max(end, step_layout(b, k, n_heads, mla_path(dt, 512, 64, n_heads)).end);
    return end;
}
// Decode-step workspace that serves both entry points (the multi-kernel step
// and the one-launch step).
size_t decode_step_workspace(const dsa_batch* b, int k, int n_heads) {
    return std::max(step_workspace(b, k, n_heads), fused_layout(b, k, n_heads).end);
}

// Indexer arguments that write score rows (no candidate emission).
IndexerArgs indexer_args(const dsa_batch* b, const dsa_index_cache* c, const void* q_idx, const float* w,
                         int n_heads_idx, float* scores, int64_t ld) {
    IndexerArgs a;
    a.g = geometry(b);
    a.keys = c->keys; a.key_scales = c->scales; a.key_dtype = c->dtype; a.dim = c->dim;
    a.q = q_idx; a.w = w; a.n_heads = n_heads_idx;
    a.scores = scores; a.ld = ld;
    a.bound = nullptr; a.row_count = nullptr; a.cand = nullptr; a.k = 0;
    return a;
}

TopkArgs topk_args(const dsa_batch* b, const float* scores, int64_t ld, int k, int32_t* indices, char* base,
                   const TopkLayout& l) {
    TopkArgs a;
    a.g = geometry(b);
    a.scores = scores; a.ld = ld; a.k = k; a.indices = indices;
    a.bound = (uint32_t*)(base + l.bound);
    a.cand_count = (uint32_t*)(base + l.count);
    a.cand_max = (uint32_t*)(base + l.cmax);
    a.cand = (uint64_t*)(base + l.cand);
    a.nchunks = l.nchunks;
    return a;
}

// Top-K limits: one workgroup per row; byte offsets of the scores it reads
// (a row plus two streaming steps) stay below 2^31.
constexpr int64_t TOPK_MAX_CONTEXT = (int64_t)1 << 28;
constexpr int32_t TOPK_MAX_ROWS = 1 << 24;
bool topk_shape_ok(const dsa_batch* b, int k) {
    return k <= TOPK_MAX_K && b->max_context_len <= TOPK_MAX_CONTEXT && b->total_q <= TOPK_MAX_ROWS;
}

int device_arch_ok() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DSA_ERR_DEVICE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return DSA_ERR_DEVICE;
    return strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? DSA_OK : DSA_ERR_DEVICE;
}

}  // namespace

int dsa::device_cu_count() {
    static int cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        cache[dev] = cus;
    }
    return cache[dev];
}

namespace {

int check_device_cached() {
    // Per-device result; the arch of a device never changes.
    static int cache[64];
    static bool known[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return DSA_ERR_DEVICE;
    if (dev < 0 || dev >= 64) return device_arch_ok();
    if (!known[dev]) { cache[dev] = device_arch_ok(); known[dev] = true; }
    return cache[dev];
}

bool index_cache_ok(const dsa_index_cache* c) {
    if (!c || !c->keys || c->dim < 1) return false;
    if (c->dtype == DSA_MXFP4) return c->dim % 32 == 0;
    return c->dtype == DSA_F32 || c->dtype == DSA_E4M3;
}

bool latent_cache_ok(const dsa_latent_cache* c) {
    if (!c || !c->kv || c->d_latent < 1 || c->d_rope < 0) return false;
    if (c->dtype == DSA_E4M3) return c->scales != nullptr;
    return (c->dtype == DSA_F32 || c->dtype == DSA_BF16) && c->scales == nullptr;
}

int validate_indexer(const dsa_batch* b, const dsa_index_cache* c, const void* q, const float* w,
                     int n_heads) {
    if (!batch_ok(b) || !c || !c->keys || !q || !w || n_heads < 1) return DSA_ERR_INVALID_ARG;
    if (!index_cache_ok(c)) return DSA_ERR_UNSUPPORTED;
    if ((int64_t)n_heads * c->dim > 12288) return DSA_ERR_UNSUPPORTED;   // generic path's LDS
    return DSA_OK;
}

int validate_mla(const dsa_batch* b, const dsa_latent_cache* c, const void* q, int n_heads, int k,
                 const void* out) {
    if (!batch_ok(b) || !q || !out || n_heads < 1 || k < 1) return DSA_ERR_INVALID_ARG;
    if (!c || !c->kv) return DSA_ERR_INVALID_ARG;
    if (!latent_cache_ok(c)) return DSA_ERR_UNSUPPORTED;
    if (!mla_fast_path(c->dtype, c->d_latent, c->d_rope, n_heads, b->block_size)) {
        // generic path keeps the selection's rows, the q row and the logits in LDS
        if ((size_t)k * sizeof(int64_t) + (size_t)(c->d_latent + c->d_rope + k) * sizeof(float) > 60 * 1024)
            return DSA_ERR_UNSUPPORTED;
    }
    return DSA_OK;
}

MlaArgs mla_args(const dsa_batch* b, const dsa_latent_cache* c, const void* q, int n_heads,
                 const int32_t* indices, int k, float scale, void* out, float* lse) {
    MlaArgs a;
    a.g = geometry(b);
    a.kv = c->kv; a.kv_scales = c->scales; a.kv_dtype = c->dtype;
    a.d_latent = c->d_latent; a.d_rope = c->d_rope;
    a.q = q; a.n_heads = n_heads;
    a.indices = indices; a.k = k; a.scale = scale;
    a.out = out; a.lse = lse;
    a.part_o = nullptr; a.part_lse = nullptr; a.splits = 1;
    a.n_layers = 1;
    for (int l = 0; l < MLA_MAX_LAYERS; ++l) a.lay[l] = MlaLayer{c->kv, c->scales, q, out, lse};
    return a;
}

// Workspace check for an MLA launch placed at `ws_base` (host only).
int mla_workspace_ok(const dsa_batch* b, const dsa_latent_cache* c, int n_heads, int k, const void* ws,
                     size_t ws_bytes, size_t ws_base, bool prefill) {
    const int path = mla_path(c->dtype, c->d_latent, c->d_rope, n_heads);
    const MlaLayout l = mla_layout(ws_base, b, k, n_heads, prefill, path);
    if (l.splits > 1 && (!ws || l.end > ws_bytes)) return DSA_ERR_WORKSPACE;
    return DSA_OK;
}

int run_mla(const dsa_batch* b, const dsa_latent_cache* c, const void* q, int n_heads,
            const int32_t* indices, int k, float scale, void* out, float* lse, char* ws, size_t ws_bytes,
            size_t ws_base, bool prefill, hipStream_t s) {
    const int path = mla_path(c->dtype, c->d_latent, c->d_rope, n_heads);
    MlaLayout l = mla_layout(ws_base, b, k, n_heads, prefill, path);
    if (l.splits > 1 && (!ws || l.end > ws_bytes)) return DSA_ERR_WORKSPACE;
    MlaArgs a = mla_args(b, c, q, n_heads, indices, k, scale, out, lse);
    a.splits = l.splits;
    if (l.splits > 1) {
        if (!ws) return DSA_ERR_WORKSPACE;
        a.part_o = (uint16_t*)(ws + l.part_o);
        a.part_lse = (float*)(ws + l.part_lse);
    }
    return launch_status(launch_mla(a, prefill, s));
}

}  // namespace

extern "C" {

const char* dsa_status_string(int32_t status) {
    switch (status) {
    case DSA_OK: return "ok";
    case DSA_ERR_INVALID_ARG: return "invalid argument";
    case DSA_ERR_UNSUPPORTED: return "unsupported dtype or shape";
    case DSA_ERR_WORKSPACE: return "workspace too small";
    case DSA_ERR_DEVICE: return "current device is not gfx950";
    case DSA_ERR_LAUNCH: return "kernel launch failed";
    case DSA_ERR_TOO_LARGE: return "batch needs more than the no-allocation entry point's scratch";
    case DSA_ERR_BAD_DEVICE_ARG: return "a device-side size, page id or index is out of range";
    default: return "unknown status";
    }
}

int dsa_check_device(void) { return check_device_cached(); }

int dsa_check_batch(const dsa_batch* b, int32_t num_blocks, const int32_t* indices, int32_t k, uint32_t* failed,
                    dsa_stream_t stream) {
    if (failed) *failed = 0;
    if (!batch_ok(b) || (indices && k < 1)) return DSA_ERR_INVALID_ARG;
    int st = check_device_cached();
    if (st != DSA_OK) return st;
    return run_batch_check(geometry(b), num_blocks, true, indices, k, failed, (hipStream_t)stream);
}

size_t dsa_workspace_size(int32_t op, const dsa_batch* b, int32_t k, int32_t n_heads) {
    if (!batch_ok(b)) return 0;
    switch (op) {
    case DSA_OP_TOPK:
        if (k < 1 || k > TOPK_MAX_K) return 0;
        return topk_layout(0, b).end;   // 0 when no row exceeds TOPK_LIST
    case DSA_OP_MLA_DECODE:
    case DSA_OP_MLA_PREFILL:
        if (k < 1 || n_heads < 1) return 0;
        // the largest over the latent dtypes; the generic path needs none
        return mla_layout_max(0, b, k, n_heads, op == DSA_OP_MLA_PREFILL);
    case DSA_OP_DECODE_STEP:
        if (k < 1 || k > TOPK_MAX_K || n_heads < 1) return 0;
        return decode_step_workspace(b, k, n_heads);
    default:
        return 0;
    }
}

int dsa_indexer_scores(const dsa_batch* b, const dsa_index_cache* c, const void* q_idx, const float* w,
                       int32_t n_heads_idx, float* scores, int64_t ld, dsa_stream_t stream) {
    int st = validate_indexer(b, c, q_idx, w, n_heads_idx);
    if (st != DSA_OK) return st;
    if (!scores || ld < b->max_context_len) return DSA_ERR_INVALID_ARG;
    if ((st = check_device_cached()) != DSA_OK) return st;
    const bool dbg = debug_mode();
    if (dbg && (st = run_batch_check(geometry(b), c->num_blocks, true, nullptr, 0, nullptr, (hipStream_t)stream)))
        return st;
    const IndexerArgs a = indexer_args(b, c, q_idx, w, n_heads_idx, scores, ld);
    hipError_t e = launch_indexer(a, (hipStream_t)stream);
    if (e == hipSuccess) e = launch_score_tail(a, (hipStream_t)stream);
    return debug_finish(dbg, launch_status(e), (hipStream_t)stream);
}

int dsa_topk(const dsa_batch* b, const float* scores, int64_t ld, int32_t k, int32_t* indices,
             void* ws, size_t ws_bytes, dsa_stream_t stream) {
    if (!batch_ok(b) || !scores || !indices || k < 1 || ld < b->max_context_len) return DSA_ERR_INVALID_ARG;
    if (!topk_shape_ok(b, k)) return DSA_ERR_UNSUPPORTED;
    const TopkLayout l = topk_layout(0, b);
    if (l.end > 0 && (!ws || ws_bytes < l.end)) return DSA_ERR_WORKSPACE;
    int st = check_device_cached();
    if (st != DSA_OK) return st;
    const bool dbg = debug_mode();
    if (dbg && (st = run_batch_check(geometry(b), 0, false, nullptr, 0, nullptr, (hipStream_t)stream))) return st;
    const TopkArgs a = topk_args(b, scores, ld, k, indices, (char*)ws, l);
    return debug_finish(dbg, launch_status(launch_topk(a, (hipStream_t)stream)), (hipStream_t)stream);
}

static int mla_entry(const dsa_batch* b, const dsa_latent_cache* c, const void* q, int32_t n_heads,
                     const int32_t* indices, int32_t k, float scale, void* out, float* lse, void* ws,
                     size_t ws_bytes, dsa_stream_t stream, bool prefill) {
    int st = validate_mla(b, c, q, n_heads, k, out);
    if (st != DSA_OK) return st;
    if (!indices) return DSA_ERR_INVALID_ARG;
    if ((st = mla_workspace_ok(b, c, n_heads, k, ws, ws ? ws_bytes : 0, 0, prefill)) != DSA_OK) return st;
    if ((st = check_device_cached()) != DSA_OK) return st;
    const bool dbg = debug_mode();
    if (dbg && (st = run_batch_check(geometry(b), c->num_blocks, true, indices, k, nullptr, (hipStream_t)stream)))
        return st;
    st = run_mla(b, c, q, n_heads, indices, k, scale, out, lse, (char*)ws, ws ? ws_bytes : 0, 0, prefill,
                 (hipStream_t)stream);
    return debug_finish(dbg, st, (hipStream_t)stream);
}

int dsa_sparse_mla_decode(const dsa_batch* b, const dsa_latent_cache* c, const void* q, int32_t n_heads,
                          const int32_t* indices, int32_t k, float scale, void* out, float* lse, void* ws,
                          size_t ws_bytes, dsa_stream_t stream) {
    return mla_entry(b, c, q, n_heads, indices, k, scale, out, lse, ws, ws_bytes, stream, false);
}

int dsa_sparse_mla_decode_layers(const dsa_batch* b, const dsa_latent_cache* caches, int32_t n_layers,
                                 const void* const* q, int32_t n_heads, const int32_t* indices, int32_t k,
                                 float scale, void* const* out, float* const* lse, void* ws, size_t ws_bytes,
                                 dsa_stream_t stream) {
    if (!caches || !q || !out || !indices || n_layers < 1 || n_layers > MLA_MAX_LAYERS) return DSA_ERR_INVALID_ARG;
    int st;
    for (int l = 0; l < n_layers; ++l) {
        if ((st = validate_mla(b, &caches[l], q[l], n_heads, k, out[l])) != DSA_OK) return st;
        if (caches[l].dtype != caches[0].dtype || caches[l].d_latent != caches[0].d_latent ||
            caches[l].d_rope != caches[0].d_rope)
            return DSA_ERR_UNSUPPORTED;
    }
    const dsa_latent_cache* c0 = &caches[0];
    const int path = scale == 0.f ? MLA_PATH_GENERIC : mla_path(c0->dtype, c0->d_latent, c0->d_rope, n_heads);
    // each layer's share: the single-layer decode workspace for this batch
    const size_t per = mla_layout(0, b, k, n_heads, false, mla_path(c0->dtype, c0->d_latent, c0->d_rope, n_heads)).end;
    if (per > 0 && (!ws || ws_bytes < per * n_layers)) return DSA_ERR_WORKSPACE;
    if ((st = check_device_cached()) != DSA_OK) return st;
    hipStream_t s = (hipStream_t)stream;
    const bool dbg = debug_mode();
    if (dbg) {
        int nb = 0;
        for (int l = 0; l < n_layers; ++l) nb = pool_blocks(nb, caches[l].num_blocks);
        if ((st = run_batch_check(geometry(b), nb, true, indices, k, nullptr, s)) != DSA_OK) return st;
    }
    if (path == MLA_PATH_H128) {
        // one launch over every layer (and one merge), the layers' partials
        // side by side: all layers' fp16 partials, then all layers' lse pairs
        MlaArgs a = mla_args(b, c0, q[0], n_heads, indices, k, scale, out[0], lse ? lse[0] : nullptr);
        a.splits = mla_splits(path, b->total_q, n_heads, k, false);
        if (a.splits > 1) {
            const size_t th = (size_t)b->total_q * n_heads * a.splits;
            a.part_o = (uint16_t*)ws;
            a.part_lse = (float*)((char*)ws + align_up(sizeof(uint16_t) * th * 512 * n_layers));
        }
        a.n_layers = n_layers;
        for (int l = 0; l < n_layers; ++l)
            a.lay[l] = MlaLayer{caches[l].kv, caches[l].scales, q[l], out[l], lse ? lse[l] : nullptr};
        st = launch_status(launch_mla(a, false, s));
    } else {
        st = DSA_OK;
        for (int l = 0; l < n_layers && st == DSA_OK; ++l)
            st = run_mla(b, &caches[l], q[l], n_heads, indices, k, scale, out[l], lse ? lse[l] : nullptr,
                         (char*)ws, ws ? ws_bytes : 0, per * l, false, s);
    }
    return debug_finish(dbg, st, s);
}

int dsa_sparse_mla_prefill(const dsa_batch* b, const dsa_latent_cache* c, const void* q, int32_t n_heads,
                           const int32_t* indices, int32_t k, float scale, void* out, float* lse, void* ws,
                           size_t ws_bytes, dsa_stream_t stream) {
    return mla_entry(b, c, q, n_heads, indices, k, scale, out, lse, ws, ws_bytes, stream, true);
}

}  // extern "C"

namespace {

// The decode step; with `ev` (DSA_STEP_EVENTS events) it records ev[0] before
// its first launch, ev[1] and ev[2] at the start and end of the indexer,
// ev[3] after the top-K selection and ev[4] after attention.
int decode_step(const dsa_batch* b, const dsa_index_cache* ic, const void* q_idx, const float* w,
                int32_t n_heads_idx, const dsa_latent_cache* lc, const void* q_mla, int32_t n_heads, int32_t k,
                float scale, void* out, float* lse, int32_t* indices_out, void* ws, size_t ws_bytes,
                dsa_stream_t stream, const hipEvent_t* ev) {
    int st = validate_indexer(b, ic, q_idx, w, n_heads_idx);
    if (st != DSA_OK) return st;
    if ((st = validate_mla(b, lc, q_mla, n_heads, k, out)) != DSA_OK) return st;
    if (!topk_shape_ok(b, k)) return DSA_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    char* base = (char*)ws;
    const StepLayout l = step_layout(b, k, n_heads, mla_path(lc->dtype, lc->d_latent, lc->d_rope, n_heads));
    if (!ws || ws_bytes < l.end) return DSA_ERR_WORKSPACE;
    if ((st = check_device_cached()) != DSA_OK) return st;
    const bool dbg = debug_mode();
    if (dbg && (st = run_batch_check(geometry(b), pool_blocks(ic->num_blocks, lc->num_blocks), true, nullptr, 0,
                                     nullptr, s)))
        return st;
    float* scores = (float*)(base + l.scores);
    int32_t* indices = indices_out ? indices_out : (int32_t*)(base + l.indices);

    const TopkArgs tk = topk_args(b, scores, l.ld, k, indices, base, l.tk);
    IndexerArgs ia = indexer_args(b, ic, q_idx, w, n_heads_idx, scores, l.ld);
    hipError_t e = ev ? hipEventRecord(ev[0], s) : hipSuccess;
    if (e != hipSuccess) return DSA_ERR_LAUNCH;
    if (indexer_emit_ok(ia)) {   // candidates straight from the indexer, no score rows
        ia.bound = (uint32_t*)(base + l.bound);
        ia.row_count = (uint32_t*)(base + l.count);
        ia.cand = (uint64_t*)(base + l.cand);
        ia.k = k;
        e = launch_emit_step(ia, tk, s, ev);
    } else {
        e = launch_indexer(ia, s, ev ? ev + 1 : nullptr);
        if (e == hipSuccess) e = launch_topk(tk, s);
    }
    if (e == hipSuccess && ev) e = hipEventRecord(ev[3], s);
    if (e != hipSuccess) return DSA_ERR_LAUNCH;
    st = run_mla(b, lc, q_mla, n_heads, indices, k, scale, out, lse, base, ws_bytes, l.mla_base, false, s);
    if (st == DSA_OK && ev && hipEventRecord(ev[4], s) != hipSuccess) return DSA_ERR_LAUNCH;
    return debug_finish(dbg, st, s);
}

// The step in one persistent launch (plus its init and merge kernels); with
// `ev` it records ev[0] before the first launch, ev[1] and ev[2] at the start
// and end of the persistent kernel (taken by its launch), ev[3] before the
// merge of split partials and ev[4] after it.
int decode_step_fused(const dsa_batch* b, const dsa_index_cache* ic, const void* q_idx, const float* w,
                      int32_t n_heads_idx, const dsa_latent_cache* lc, const void* q_mla, int32_t n_heads, int32_t k,
                      float scale, void* out, float* lse, int32_t* indices_out, void* ws, size_t ws_bytes,
                      dsa_stream_t stream, const hipEvent_t* ev) {
    int st = validate_indexer(b, ic, q_idx, w, n_heads_idx);
    if (st != DSA_OK) return st;
    if ((st = validate_mla(b, lc, q_mla, n_heads, k, out)) != DSA_OK) return st;
    if (!topk_shape_ok(b, k)) return DSA_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    char* base = (char*)ws;
    const FusedLayout fl = fused_layout(b, k, n_heads);
    IndexerArgs ia = indexer_args(b, ic, q_idx, w, n_heads_idx, (float*)(base + fl.scores), fl.ld);
    ia.k = k;
    MlaArgs ma = mla_args(b, lc, q_mla, n_heads, nullptr, k, scale, out, lse);
    if (!fused_ok(ia, ma)) return DSA_ERR_UNSUPPORTED;
    if (!ws || ws_bytes < fl.end) return DSA_ERR_WORKSPACE;
    if ((st = check_device_cached()) != DSA_OK) return st;
    const bool dbg = debug_mode();
    if (dbg && (st = run_batch_check(geometry(b), pool_blocks(ic->num_blocks, lc->num_blocks), true, nullptr, 0,
                                     nullptr, s)))
        return st;
    FusedArgs f;
    f.indices = indices_out ? indices_out : (int32_t*)(base + fl.indices);
    ia.cand = (uint64_t*)(base + fl.cand);
    ia.row_count = (uint32_t*)(base + fl.count);
    ma.indices = f.indices;
    ma.part_o = (uint16_t*)(base + fl.part_o);
    ma.part_lse = (float*)(base + fl.part_lse);
    f.ia = ia;
    f.ma = ma;
    f.ctr = (uint32_t*)(base + fl.ctr);
    f.chunk_prefix = (uint32_t*)(base + fl.prefix);
    f.chunk_req = (uint32_t*)(base + fl.chunk_req);
    f.req_done = (uint32_t*)(base + fl.req_done);
    f.row_excl = (unsigned long long*)(base + fl.excl);
    f.row_slot = (uint32_t*)(base + fl.slot);
    f.row_splits = (uint32_t*)(base + fl.splits);
    f.rq = (uint32_t*)(base + fl.rq);
    f.rq_cap = fl.rq_cap;
    f.sq_cap = b->num_requests;
    f.part_slots = fl.part_slots;
    hipError_t e = ev ? hipEventRecord(ev[0], s) : hipSuccess;
    if (e == hipSuccess) e = launch_fused(f, s, ev ? ev + 1 : nullptr);
    if (e == hipSuccess && ev) e = hipEventRecord(ev[4], s);
    return debug_finish(dbg, launch_status(e), s);
}

}  // namespace

extern "C" {

int dsa_decode_step(const dsa_batch* b, const dsa_index_cache* ic, const void* q_idx, const float* w,
                    int32_t n_heads_idx, const dsa_latent_cache* lc, const void* q_mla, int32_t n_heads,
                    int32_t k, float scale, void* out, float* lse, int32_t* indices_out, void* ws,
                    size_t ws_bytes, dsa_stream_t stream) {
    return decode_step(b, ic, q_idx, w, n_heads_idx, lc, q_mla, n_heads, k, scale, out, lse, indices_out, ws,
                       ws_bytes, stream, nullptr);
}

int dsa_decode_step_timed(const dsa_batch* b, const dsa_index_cache* ic, const void* q_idx, const float* w,
                          int32_t n_heads_idx, const dsa_latent_cache* lc, const void* q_mla, int32_t n_heads,
                          int32_t k, float scale, void* out, float* lse, int32_t* indices_out, void* ws,
                          size_t ws_bytes, dsa_stream_t stream, void* const* events, int32_t n_events) {
    if (!events || n_events < DSA_STEP_EVENTS) return DSA_ERR_INVALID_ARG;
    hipEvent_t ev[DSA_STEP_EVENTS];
    for (int i = 0; i < DSA_STEP_EVENTS; ++i) {
        if (!events[i]) return DSA_ERR_INVALID_ARG;
        ev[i] = (hipEvent_t)events[i];
    }
    return decode_step(b, ic, q_idx, w, n_heads_idx, lc, q_mla, n_heads, k, scale, out, lse, indices_out, ws,
                       ws_bytes, stream, ev);
}

int dsa_decode_step_fused(const dsa_batch* b, const dsa_index_cache* ic, const void* q_idx, const float* w,
                          int32_t n_heads_idx, const dsa_latent_cache* lc, const void* q_mla, int32_t n_heads,
                          int32_t k, float scale, void* out, float* lse, int32_t* indices_out, void* ws,
                          size_t ws_bytes, dsa_stream_t stream, void* const* events, int32_t n_events) {
    hipEvent_t ev[DSA_STEP_EVENTS];
    if (events) {
        if (n_events < DSA_STEP_EVENTS) return DSA_ERR_INVALID_ARG;
        for (int i = 0; i < DSA_STEP_EVENTS; ++i) {
            if (!events[i]) return DSA_ERR_INVALID_ARG;
            ev[i] = (hipEvent_t)events[i];
        }
    }
    return decode_step_fused(b, ic, q_idx, w, n_heads_idx, lc, q_mla, n_heads, k, scale, out, lse, indices_out, ws,
                             ws_bytes, stream, events ? ev : nullptr);
}

}  // extern "C"

// ---------------------------------------------------------------------------
// No-allocation decode step.  Its workspace is a file-scope device array;
// host code never passes the array's name to a kernel (in host code that
// name is only a stand-in for the symbol): the device address of each GPU's
// copy is looked up once per device with hipGetSymbolAddress and used
// instead.
static __device__ __align__(256) uint8_t scratch[DSA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int NOALLOC_MAX_DEVICES = 64;
std::mutex noalloc_mutex;
void* noalloc_ptr[NOALLOC_MAX_DEVICES];

// Device address of the current device's scratch (looked up on the first
// call on that device, with the device current), or nullptr.
void* noalloc_scratch() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NOALLOC_MAX_DEVICES) return nullptr;
    std::lock_guard<std::mutex> lock(noalloc_mutex);
    if (!noalloc_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
        noalloc_ptr[dev] = p;
    }
    return noalloc_ptr[dev];
}

}  // namespace

extern "C" {

int dsa_decode_step_noalloc(const dsa_batch* b, const dsa_index_cache* ic, const void* q_idx, const float* w,
                            int32_t n_heads_idx, const dsa_latent_cache* lc, const void* q_mla, int32_t n_heads,
                            int32_t k, float scale, void* out, float* lse, int32_t* indices_out,
                            dsa_stream_t stream) {
    int st = validate_indexer(b, ic, q_idx, w, n_heads_idx);
    if (st != DSA_OK) return st;
    if ((st = validate_mla(b, lc, q_mla, n_heads, k, out)) != DSA_OK) return st;
    if (!topk_shape_ok(b, k)) return DSA_ERR_UNSUPPORTED;
    if (step_workspace(b, k, n_heads) > DSA_NOALLOC_SCRATCH_BYTES) return DSA_ERR_TOO_LARGE;
    if ((st = check_device_cached()) != DSA_OK) return st;
    void* ws = noalloc_scratch();
    if (!ws) return DSA_ERR_LAUNCH;
    return decode_step(b, ic, q_idx, w, n_heads_idx, lc, q_mla, n_heads, k, scale, out, lse, indices_out, ws,
                       DSA_NOALLOC_SCRATCH_BYTES, stream, nullptr);
}

}  // extern "C"
