// Lightning-indexer scores on gfx950.
//
// Score of visible token s for query row t (SemiAnalysis GLM-5.3 article,
// "Lightning Indexer"): I[t,s] = sigma_s * sum_h w[t,h] * ReLU(q[t,h,:] . k_s).
// sigma_s (per-token key scale) is applied after the head sum, exact because
// ReLU is positively homogeneous and sigma_s >= 0.
//
// Fast path (e4m3 keys and queries, dim 128, heads a multiple of 16, 64-token
// blocks): per workgroup one request, a group of NQ query rows of it and a
// chunk of its context.  Each wave streams whole 64-token pages of keys
// (8 KB, contiguous) straight into registers and multiplies them against the
// register-resident queries with v_mfma_f32_16x16x128_f8f6f4: heads are the
// M dimension, tokens the N dimension and the full 128-wide key the K
// dimension, so one instruction covers a 16x16 head-token tile.  The ReLU,
// the weighted head sum and the key scale are applied on the accumulators;
// the head sum crosses the four 16-lane groups with three lane exchanges.
// Scores are stored as 256-byte coalesced rows and counted into a per-row
// LDS histogram of the top 12 key bits, which the top-K selection uses to
// find the threshold bucket without a second pass over the scores.
#include "dsa_kernels.h"

namespace dsa {

constexpr int IDX_D = 128;
constexpr int IDX_PAGE = 64;
constexpr int IDX_THREADS = 256;
constexpr int IDX_CHUNK_PAGES = 32;   // 2048 tokens per workgroup

struct KeyPage {
    i32x8 frag[4];   // token 16*nt + (lane & 15), 32 of its 128 bytes
    float scale;     // scale of token (lane) of the page
};

// Lane l loads bytes [16g, 16g+16) and [64+16g, 64+16g+16) of its token,
// g = l >> 4; the query fragments use the same byte assignment.
__device__ __forceinline__ void load_key_page(const uint8_t* __restrict__ keys,
                                              const float* __restrict__ scales, int blk,
                                              int lane, KeyPage& kp) {
    const int g = lane >> 4, col = lane & 15;
    const uint8_t* base = keys + (size_t)blk * (IDX_PAGE * IDX_D);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        const uint8_t* rp = base + (16 * nt + col) * IDX_D + 16 * g;
        u32x4 lo = __builtin_nontemporal_load((const u32x4*)rp);
        u32x4 hi = __builtin_nontemporal_load((const u32x4*)(rp + 64));
        kp.frag[nt] = join_i32x8(lo, hi);
    }
    kp.scale = scales ? scales[(size_t)blk * IDX_PAGE + lane] : 1.0f;
}

// part[nt] holds, for token 16*nt + (lane & 15), the partial head sum of this
// lane's 16-lane group g.  Returns the full sum for token `lane` of the page.
__device__ __forceinline__ float head_sum_transpose(const float part[4], int lane) {
    const int b1 = (lane >> 5) & 1, b0 = (lane >> 4) & 1;
    const float send0 = b1 ? part[0] : part[2];
    const float send1 = b1 ? part[1] : part[3];
    const float keep0 = b1 ? part[2] : part[0];
    const float keep1 = b1 ? part[3] : part[1];
    const float a0 = keep0 + __shfl_xor(send0, 32);
    const float a1 = keep1 + __shfl_xor(send1, 32);
    const float send = b0 ? a0 : a1;
    const float keep = b0 ? a1 : a0;
    return keep + __shfl_xor(send, 16);
}

template <int NQ, int HT, bool HIST>
__global__ __launch_bounds__(IDX_THREADS) void indexer_fp8_mfma(IndexerArgs a, int qgroups,
                                                                int chunk_tokens) {
    const Geometry& G = a.g;
    const int r = blockIdx.y / qgroups, qg = blockIdx.y % qgroups;
    const int L = G.ctx[r];
    const int qs = G.qsl[r], ql = G.qsl[r + 1] - qs;
    const int j0 = qg * NQ;
    if (j0 >= ql) return;
    const int nq = min(NQ, ql - j0);
    const int n_last = L - ql + j0 + nq;          // visible count of the group's last row
    const int tok0 = blockIdx.x * chunk_tokens;
    if (tok0 >= n_last) return;
    const int tok1 = min(n_last, tok0 + chunk_tokens);

    __shared__ uint32_t hist[HIST ? NQ : 1][HIST ? HIST_BINS : 1];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, col = lane & 15;
    constexpr bool use_hist = HIST;
    if (use_hist)
        for (int i = tid; i < NQ * HIST_BINS; i += IDX_THREADS) (&hist[0][0])[i] = 0u;

    // Register-resident queries (A operand: head 16*ht + col) and weights of
    // the four accumulator rows this lane owns (heads 16*ht + 4g + i).
    i32x8 qf[NQ][HT];
    float wv[NQ][HT][4];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const int t = qs + j0 + min(j, nq - 1);
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const uint8_t* qp = (const uint8_t*)a.q + ((size_t)t * a.n_heads + 16 * ht + col) * IDX_D + 16 * g;
            qf[j][ht] = join_i32x8(*(const u32x4*)qp, *(const u32x4*)(qp + 64));
#pragma unroll
            for (int i = 0; i < 4; ++i) wv[j][ht][i] = a.w[(size_t)t * a.n_heads + 16 * ht + 4 * g + i];
        }
    }
    if (use_hist) __syncthreads();

    const int32_t* pt = G.page_table + (size_t)r * G.max_blocks;
    const uint8_t* keys = (const uint8_t*)a.keys;
    const int page1 = (tok1 + IDX_PAGE - 1) / IDX_PAGE;
    int pg = tok0 / IDX_PAGE + wave;
    KeyPage cur;
    if (pg < page1) load_key_page(keys, a.key_scales, pt[pg], lane, cur);
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};

    for (; pg < page1; pg += 4) {
        KeyPage nxt;
        const bool more = pg + 4 < page1;
        if (more) load_key_page(keys, a.key_scales, pt[pg + 4], lane, nxt);
        const int pos = pg * IDX_PAGE + lane;
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            if (j < nq) {
                float part[4];
#pragma unroll
                for (int nt = 0; nt < 4; ++nt) {
                    float acc = 0.f;
#pragma unroll
                    for (int ht = 0; ht < HT; ++ht) {
                        const f32x4 c = mfma_fp8_16x16x128(qf[j][ht], cur.frag[nt], zero);
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc += wv[j][ht][i] * fmaxf(c[i], 0.f);
                    }
                    part[nt] = acc;
                }
                const float s = head_sum_transpose(part, lane) * cur.scale;
                const int t = qs + j0 + j;
                const int n_j = L - ql + j0 + j + 1;
                if (pos < n_j) {
                    a.scores[(size_t)t * a.ld + pos] = s;
                    if (use_hist) atomicAdd(&hist[j][score_key(s) >> HIST_SHIFT], 1u);
                }
            }
        }
        if (more) cur = nxt;
    }

    if (use_hist) {
        __syncthreads();
        for (int j = 0; j < nq; ++j) {
            uint32_t* gh = a.hist + (size_t)(qs + j0 + j) * HIST_BINS;
            for (int b = tid; b < HIST_BINS; b += IDX_THREADS) {
                const uint32_t v = hist[j][b];
                if (v) atomicAdd(gh + b, v);
            }
        }
    }
}

// Generic path: any head count / dim, fp32 or e4m3 keys and queries, any block
// size.  One thread per (query row, token); the query and weights sit in LDS.
__global__ __launch_bounds__(256) void indexer_generic(IndexerArgs a) {
    const Geometry& G = a.g;
    const int t = blockIdx.y;
    const int r = find_request(G.qsl, G.B, t);
    const int n = visible_count(G.ctx, G.qsl, r, t);
    const int H = a.n_heads, D = a.dim;
    extern __shared__ float smem[];
    float* qv = smem;            // [H][D]
    float* wv = smem + H * D;    // [H]
    const bool f8 = a.key_dtype == 2;
    for (int i = threadIdx.x; i < H * D; i += blockDim.x) {
        const size_t off = (size_t)t * H * D + i;
        qv[i] = f8 ? e4m3_to_f32(((const uint8_t*)a.q)[off]) : ((const float*)a.q)[off];
    }
    for (int i = threadIdx.x; i < H; i += blockDim.x) wv[i] = a.w[(size_t)t * H + i];
    __syncthreads();
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= n) return;
    const int bs = G.block_size;
    const size_t row = (size_t)G.page_table[(size_t)r * G.max_blocks + s / bs] * bs + s % bs;
    float total = 0.f;
    for (int h = 0; h < H; ++h) {
        float dot = 0.f;
        for (int d = 0; d < D; ++d) {
            const size_t off = row * D + d;
            const float k = f8 ? e4m3_to_f32(((const uint8_t*)a.keys)[off]) : ((const float*)a.keys)[off];
            dot = fmaf(qv[h * D + d], k, dot);
        }
        total = fmaf(wv[h], fmaxf(dot, 0.f), total);
    }
    const float sc = a.key_scales ? a.key_scales[row] : 1.f;
    const float score = sc * total;
    a.scores[(size_t)t * a.ld + s] = score;
    if (a.hist) atomicAdd(a.hist + (size_t)t * HIST_BINS + (score_key(score) >> HIST_SHIFT), 1u);
}

template <int NQ, int HT>
static hipError_t launch_fp8(const IndexerArgs& a, hipStream_t s) {
    const int qgroups = (a.g.max_q_len + NQ - 1) / NQ;
    const int chunk_tokens = IDX_CHUNK_PAGES * IDX_PAGE;
    dim3 grid((a.g.max_ctx + chunk_tokens - 1) / chunk_tokens, a.g.B * qgroups);
    if (a.hist)
        hipLaunchKernelGGL((indexer_fp8_mfma<NQ, HT, true>), grid, dim3(IDX_THREADS), 0, s, a, qgroups, chunk_tokens);
    else
        hipLaunchKernelGGL((indexer_fp8_mfma<NQ, HT, false>), grid, dim3(IDX_THREADS), 0, s, a, qgroups, chunk_tokens);
    return hipGetLastError();
}

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t s) {
    const bool fast = a.key_dtype == 2 && a.dim == IDX_D && a.g.block_size == IDX_PAGE &&
                      (a.n_heads == 64 || a.n_heads == 32 || a.n_heads == 16);
    if (fast) {
        const bool two = a.g.max_q_len >= 2;
        switch (a.n_heads) {
        case 64: return two ? launch_fp8<2, 4>(a, s) : launch_fp8<1, 4>(a, s);
        case 32: return two ? launch_fp8<2, 2>(a, s) : launch_fp8<1, 2>(a, s);
        default: return two ? launch_fp8<2, 1>(a, s) : launch_fp8<1, 1>(a, s);
        }
    }
    dim3 grid((a.g.max_ctx + 255) / 256, a.g.T);
    const size_t shm = sizeof(float) * ((size_t)a.n_heads * a.dim + a.n_heads);
    hipLaunchKernelGGL(indexer_generic, grid, dim3(256), shm, s, a);
    return hipGetLastError();
}

}  // namespace dsa
