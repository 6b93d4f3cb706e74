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
    uint32_t* row_count;     // [T] candidates appended (may exceed TOPK_LIST)
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

struct MlaArgs {
    Geometry g;
    const void* kv; const float* kv_scales; int kv_dtype; int d_latent, d_rope;
    const void* q; int n_heads;
    const int32_t* indices; int k;
    float scale;
    void* out; float* lse;
    uint16_t* part_o;                 // split partials: fp16 [T][H][S][d], or nullptr
    float* part_lse;                  // [T][H][S][2]: lse and the partial's scale 2^-k
    int splits;
};

// Compute units of the current device (cached per device).
int device_cu_count();

// Launchers (return hipError_t of the last launch).
// With `se`, se[0] and se[1] mark the indexer's start and end (for the
// persistent kernel, taken by its launch itself).
hipError_t launch_indexer(const IndexerArgs& a, hipStream_t s, const hipEvent_t* se = nullptr);
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

// Which MLA path serves these shapes, and how many splits it uses.
bool mla_fast_path(int kv_dtype, int d_latent, int d_rope, int n_heads, int block_size);
constexpr int MLA_HEADS_PER_WG = 64;
constexpr int MLA_PATH_GENERIC = 0, MLA_PATH_H64 = 1, MLA_PATH_H128 = 2;
int mla_path(int kv_dtype, int d_latent, int d_rope, int n_heads);
// Partial results per query row (1: no split, no combine pass).
int mla_splits(int path, int T, int n_heads, int k, bool prefill);

}  // namespace dsa
