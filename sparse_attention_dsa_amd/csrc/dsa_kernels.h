// Internal definitions shared by the DSA HIP kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dsa {

// ----------------------------------------------------------------- vectors
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// Top-K: largest supported K; rows longer than TOPK_LIST are cut into
// TOPK_CHUNK-score chunks whose candidates fill slots of TOPK_CAND_CAP.
constexpr int TOPK_MAX_K = 4096;
constexpr int TOPK_LIST = 12288;
// Candidate counters of the rows sit one 128-byte line apart: at the end of
// their shares many waves append to the same few rows at once, and counters
// sharing a line would serialise all of those atomics together.
constexpr int ROW_COUNT_STRIDE = 32;
constexpr int TOPK_CHUNK = 8192;
constexpr int TOPK_CAND_CAP = 4096;

// ----------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// OCP e4m3fn code -> fp32, exactly: normal (1+m/8)*2^(e-7), subnormal m*2^-9.
// (The NaN codes 0x7F/0xFF are not produced by the caches and decode to 480.)
__device__ __forceinline__ float e4m3_to_f32(uint32_t code) {
    const uint32_t e = (code >> 3) & 0xFu, m = code & 7u;
    float v = e ? __uint_as_float(((e + 120u) << 23) | (m << 20)) : (float)m * 0x1p-9f;
    return (code & 0x80u) ? -v : v;
}

// Order-preserving map of a float to uint32 (larger float -> larger key);
// -0 is folded onto +0 so that equal scores get equal keys.
__device__ __forceinline__ uint32_t score_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u << 1) == 0u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ------------------------------------------------------------------ MFMA
// D = A(16x128 fp8) * B(128x16 fp8) + C, OCP e4m3 operands, fp32 accumulate.
// Lane l holds row/column (l & 15) of A/B and 32 of the 128 k-values; A and
// B use the same k assignment, so any consistent permutation of k is valid.
__device__ __forceinline__ f32x4 mfma_fp8_16x16x128(i32x8 a, i32x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// D = A(16x32 bf16) * B(32x16 bf16) + C.  Lane l: A row / B column (l & 15),
// k-values 8*(l>>4) .. 8*(l>>4)+7.  C/D: column (l & 15), rows 4*(l>>4)+i.
__device__ __forceinline__ f32x4 mfma_bf16_16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Value held by lane (lane ^ 32), exchanged with v_permlane32_swap (the
// upper half of the first operand trades places with the lower half of the
// second; with both operands x, lane l < 32 finds x[l + 32] in the second
// result and lane l >= 32 finds x[l - 32] in the first), no LDS round trip.
__device__ __forceinline__ float lane_xor32(float x, int lane) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(lane < 32 ? r[1] : r[0]);
}

// Value held by lane (lane ^ 16), by v_permlane16_swap (odd 16-lane rows of
// the first operand trade places with even rows of the second).
__device__ __forceinline__ float lane_xor16(float x, int lane) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float((lane & 16) ? r[0] : r[1]);
}

__device__ __forceinline__ i32x8 join_i32x8(u32x4 lo, u32x4 hi) {
    i32x8 r;
    r[0] = (int)lo[0]; r[1] = (int)lo[1]; r[2] = (int)lo[2]; r[3] = (int)lo[3];
    r[4] = (int)hi[0]; r[5] = (int)hi[1]; r[6] = (int)hi[2]; r[7] = (int)hi[3];
    return r;
}

// Work-item id x through an opaque move.  Values derived from it cannot be
// hoisted out of a persistent kernel's item loop, where they would stay live
// across every kind of item (and spill); each device routine takes it once.
__device__ __forceinline__ int tid_x() {
    int r;
    asm volatile("v_mov_b32 %0, %1" : "=v"(r) : "v"((int)threadIdx.x));
    return r;
}

// Accesses to data that one workgroup hands to another inside a launch.
// Agent-scope atomic accesses are coherent across the device by themselves
// (they do not stop in an XCD's own L2), so a writer that waits for its
// stores (vmcnt 0) before it sets a flag, and a reader that loads the data
// after it has seen the flag, need no L2 write-back or invalidate: those are
// what agent-scope release and acquire add for ordinary accesses, and they
// cost the whole device's streaming bandwidth when issued often.
template <class T>
__device__ __forceinline__ void st_agent(T* p, T v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <class T>
__device__ __forceinline__ T ld_agent(const T* p) {
    return __hip_atomic_load(const_cast<T*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// max(x, 0) for a float that is not a NaN, as a signed-integer max of its
// bits: every negative float, -0 included, has the sign bit set and is below
// 0 as an int32, and every other one keeps its bits.  One integer
// instruction, where fmaxf first canonicalizes an input the compiler cannot
// prove canonical (an MFMA result: a second instruction per element) and
// inline asm would fall outside the compiler's hazard tracking (a VALU read
// of an MFMA result then loses the wait states it needs).
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// ------------------------------------------------ asynchronous LDS fills
// One 64-lane transfer global -> LDS at LDS address m0v (wave-uniform; lane
// l's bytes land at m0v + l * size): 16 B a lane (plain, or streamed: not
// kept in the caches), or 4 B a lane.  Issued by inline asm, so the compiler
// neither counts these transfers nor waits for them before LDS reads (it
// would otherwise wait for every transfer in flight, the prefetched ones
// too); the caller waits for them with wait_vmcnt.  M0 is restored.
__device__ __forceinline__ void dma16(const void* g, uint32_t m0v) {
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "v"(g), "s"(m0v));
}
__device__ __forceinline__ void dma16_stream(const void* g, uint32_t m0v) {
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
                 "global_load_lds_dwordx4 %1, off sc0 nt\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "v"(g), "s"(m0v));
}
__device__ __forceinline__ void dma4(const void* g, uint32_t m0v) {
    uint32_t saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
                 "global_load_lds_dword %1, off\n\ts_mov_b32 m0, %0"
                 : "=&s"(saved) : "v"(g), "s"(m0v));
}
// 32-bit LDS address of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// ------------------------------------------------------ waits and barriers
// Wait until at most N of this wave's vector-memory operations are pending.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that orders LDS traffic only: unlike __syncthreads() it
// does not wait for this wave's outstanding global loads (asynchronous
// transfers in flight), which the callers account for with wait_vmcnt.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ----------------------------------------------------------- batch maps
// Request owning query row t: the largest r with qsl[r] <= t.
__device__ __forceinline__ int find_request(const int32_t* qsl, int B, int t) {
    int lo = 0, hi = B - 1;
    while (lo < hi) {
        int mid = (lo + hi + 1) >> 1;
        if (qsl[mid] <= t) lo = mid; else hi = mid - 1;
    }
    return lo;
}

// Visible-token count of query row t (query j of request r sees [0, L-ql+j]).
__device__ __forceinline__ int visible_count(const int32_t* ctx, const int32_t* qsl, int r, int t) {
    const int ql = qsl[r + 1] - qsl[r];
    return ctx[r] - ql + (t - qsl[r]) + 1;
}

// ------------------------------------------------------- launch helpers
struct Geometry {
    int B, T, max_q_len, max_ctx;
    int q_uniform;          // > 0: every request has exactly this many query rows
    const int32_t* ctx;
    const int32_t* qsl;
    const int32_t* page_table;
    int max_blocks, block_size;
};

// Request of query row t; no lookup when every request has q_uniform rows.
__device__ __forceinline__ int row_request(const Geometry& g, int t) {
    return g.q_uniform > 0 ? t / g.q_uniform : find_request(g.qsl, g.B, t);
}

// Visible-token count of query row t; a single load when the query rows are
// spread uniformly over the requests.
__device__ __forceinline__ int row_visible(const Geometry& g, int t) {
    if (g.q_uniform > 0) {
        const int r = t / g.q_uniform;
        return g.ctx[r] - g.q_uniform + (t - r * g.q_uniform) + 1;
    }
    const int r = find_request(g.qsl, g.B, t);
    return visible_count(g.ctx, g.qsl, r, t);
}

struct IndexerArgs {
    Geometry g;
    const void* keys; const float* key_scales; int key_dtype; int dim;
    const void* q; const float* w; int n_heads;
    float* scores; int64_t ld;
    // candidate emission (fused decode step; cand == nullptr: write scores):
    // per query row, the composites of the scores at or above the key bound
    // go to an unordered list of TOPK_LIST slots instead of the score rows
    uint32_t* bound;         // [T] key bound (written by the sample kernel)
    uint32_t* row_count;     // [T][ROW_COUNT_STRIDE]: candidates appended (may exceed TOPK_LIST)
    uint64_t* cand;          // [T][TOPK_LIST]
    int k;                   // top-K size the bound is drawn for
};

struct TopkArgs {
    Geometry g;
    const float* scores; int64_t ld;
    int k;
    int32_t* indices;        // [T][k] result
    // workspace (rows longer than TOPK_LIST only)
    uint32_t* bound;         // [T] sample key bound
    uint32_t* cand_count;    // [T][nchunks] candidates per chunk
    uint32_t* cand_max;      // [T][nchunks] largest candidate key per chunk
    uint64_t* cand;          // [T][nchunks][TOPK_CAND_CAP] composites in token order
    int nchunks;
};

// Per-layer buffers of a launch over several layers that share one selection
// (layer l > 0 of the 128-head path; layer 0 is MlaArgs' own).
constexpr int MLA_MAX_LAYERS = 4;
struct MlaLayer {
    const void* kv; const float* kv_scales;
    const void* q;
    void* out; float* lse;
};
struct MlaArgs {
    Geometry g;
    const void* kv; const float* kv_scales; int kv_dtype; int d_latent, d_rope;
    const void* q; int n_heads;
    const int32_t* indices; int k;
    float scale;
    void* out; float* lse;
    uint16_t* part_o;                 // split partials: fp16 [layers][T][H][S][d], or nullptr
    float* part_lse;                  // [layers][T][H][S][2]: lse and the partial's scale 2^-k
    int splits;
    int n_layers;                     // >= 1; layers 1 .. n_layers - 1 in lay[]
    MlaLayer lay[MLA_MAX_LAYERS];
};
// The arguments of layer `layer` of a multi-layer launch (the same for 0).
__host__ __device__ inline MlaArgs mla_layer_args(const MlaArgs& a, int layer) {
    MlaArgs b = a;
    if (layer > 0) {
        const MlaLayer& y = a.lay[layer];
        b.kv = y.kv; b.kv_scales = y.kv_scales; b.q = y.q; b.out = y.out; b.lse = y.lse;
        const size_t th = (size_t)a.g.T * a.n_heads * a.splits;
        if (b.part_o) b.part_o += (size_t)layer * th * 512;
        if (b.part_lse) b.part_lse += (size_t)layer * th * 2;
    }
    return b;
}

// The fused decode step's arguments (one persistent launch; see fused.hip).
// Counters in ctr[]: head and tail of the selection queue and of the
// attention queue, the next chunk of the key stream, the attention slices not
// yet finished, an error word, the number of chunks, and the number of
// selection items (requests with query rows).
// Counters that every workgroup updates or polls sit on 128-byte lines of
// their own (a queue's head and tail share one, as they are read together).
enum { FC_SQ_HEAD = 0, FC_SQ_TAIL = 1, FC_MQ_HEAD = 32, FC_MQ_TAIL = 33, FC_TICKET = 64, FC_WORK = 96,
       FC_ERROR = 128, FC_NCHUNKS = 160, FC_NSEL = 161, FC_N = 192 };
enum { RQ_EMPTY = 0, RQ_SEL = 1, RQ_MLA = 2 };
struct FusedArgs {
    IndexerArgs ia;                  // keys, queries, weights, k; cand/row_count: candidate lists;
                                     // scores/ld: rows scored again when a chunk quota failed
    MlaArgs ma;                      // latent cache, MLA queries, out/lse, part_o/part_lse by slot
    int32_t* indices;                // [T][k] selection (ascending, -1 padded)
    uint32_t* ctr;                   // [FC_N]
    uint32_t* chunk_prefix;          // [B] stream position of request r's first chunk
    uint32_t* chunk_req;             // [chunks][2] request and first page of each chunk of the stream
    uint32_t* req_done;              // [B][ROW_COUNT_STRIDE] waves done with the request's pages
    unsigned long long* row_excl;    // [T] largest composite a chunk left out (0: none)
    uint32_t* row_slot;              // [T] first partial slot of the row's slices
    uint32_t* row_splits;            // [T] slices of the row's attention
    uint32_t* rq;                    // [rq_cap][4] queued items: kind, then three words; slots
                                     // [0, sq_cap) the selection queue, the rest the attention queue
    int rq_cap, sq_cap;
    int part_slots;                  // shared partial slots (each: n_heads partials); a
                                     // reserve of 2 per row follows them
};
constexpr int FU_MAX_SPLITS = 16;    // attention slices per row at most
bool fused_ok(const IndexerArgs& ia, const MlaArgs& ma);
// Init kernel, the persistent step (with `ev`: ev[0] and ev[1] its start and
// stop, taken by the launch; ev[2] recorded before the merge), then the merge
// of split partials.
hipError_t launch_fused(const FusedArgs& f, hipStream_t s, const hipEvent_t* ev = nullptr);

// Compute units of the current device (cached per device).
int device_cu_count();

// Launchers (return hipError_t of the last launch).
// With `se`, se[0] and se[1] mark the indexer's start and end (for the
// persistent kernel, taken by its launch itself).
hipError_t launch_indexer(const IndexerArgs& a, hipStream_t s, const hipEvent_t* se = nullptr);
// -inf over every score row's entries past its visible tokens, [n_t, ld).
// MXFP4 index keys (key_dtype 3): the fast kernel's shapes, and its launch.
bool mxfp4_fast(const IndexerArgs& a);
hipError_t launch_indexer_mxfp4(const IndexerArgs& a, hipStream_t s);
hipError_t launch_score_tail(const IndexerArgs& a, hipStream_t s);
// Whether the decode step can take the candidate-emission path for this
// shape (e4m3 keys, dim 128, 16/32/64 heads, 64-token blocks, persistent grid).
bool indexer_emit_ok(const IndexerArgs& a);
hipError_t launch_sample_bound(const IndexerArgs& a, hipStream_t s);
// Sample bound per query row (and zeroed candidate counters), then the
// indexer emitting candidates, then the selection from the candidate lists
// (recomputing a row's scores into a.scores where its bound fails).
// With `ev`, ev[1] and ev[2] mark the start and end of the indexer (the
// measurement variant of the decode step).
hipError_t launch_emit_step(const IndexerArgs& ia, const TopkArgs& ta, hipStream_t s,
                            const hipEvent_t* ev = nullptr);
// Sample bound, chunk compaction, then one selection workgroup per row.
hipError_t launch_topk(const TopkArgs& a, hipStream_t s);
hipError_t launch_mla(const MlaArgs& a, bool prefill, hipStream_t s);

// DSA_DEBUG set in the environment (to anything but "" or "0").
bool debug_mode();
// Checks the batch's device-side values (query starts, context lengths, page
// ids below num_blocks when pages and num_blocks > 0, selection entries below
// their row's visible count when indices != nullptr) and waits for the
// result: DSA_OK, or DSA_ERR_BAD_DEVICE_ARG with the DSA_CHECK_* bits in
// *failed (may be nullptr); DSA_ERR_UNSUPPORTED while `s` is being captured.
int run_batch_check(const Geometry& g, int num_blocks, bool pages, const int32_t* indices, int k,
                    uint32_t* failed, hipStream_t s);
// In debug mode, waits for a successful call's launches and reports a failed
// one as DSA_ERR_LAUNCH; otherwise returns st.
int debug_finish(bool dbg, int st, hipStream_t s);

// Which MLA path serves these shapes, and how many splits it uses.
bool mla_fast_path(int kv_dtype, int d_latent, int d_rope, int n_heads, int block_size);
constexpr int MLA_HEADS_PER_WG = 64;
constexpr int MLA_PATH_GENERIC = 0, MLA_PATH_H64 = 1, MLA_PATH_H128 = 2;
int mla_path(int kv_dtype, int d_latent, int d_rope, int n_heads);
// Partial results per query row (1: no split, no combine pass).
int mla_splits(int path, int T, int n_heads, int k, bool prefill);

}  // namespace dsa
