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

// Scores of one 64-token page for the NQ query rows: 16 MFMAs per row (heads x
// tokens x full key), ReLU, head weights, head sum across the lane groups, key
// scale.  Lane l returns the score of token l of the page.
template <int NQ, int HT>
__device__ __forceinline__ void page_scores(const i32x8 (&qf)[NQ][HT], const float (&wv)[NQ][HT][4],
                                            const i32x8 (&kf)[4], float ksc, int lane, int nq,
                                            float (&out)[NQ]) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        if (j < nq) {
            float part[4];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                float acc = 0.f;
#pragma unroll
                for (int ht = 0; ht < HT; ++ht) {
                    const f32x4 c = mfma_fp8_16x16x128(qf[j][ht], kf[nt], zero);
#pragma unroll
                    for (int i = 0; i < 4; ++i) acc += wv[j][ht][i] * fmaxf(c[i], 0.f);
                }
                part[nt] = acc;
            }
            out[j] = head_sum_transpose(part, lane) * ksc;
        } else {
            out[j] = 0.f;
        }
    }
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

    for (; pg < page1; pg += 4) {
        KeyPage nxt;
        const bool more = pg + 4 < page1;
        if (more) load_key_page(keys, a.key_scales, pt[pg + 4], lane, nxt);
        const int pos = pg * IDX_PAGE + lane;
        float ps[NQ];
        page_scores<NQ, HT>(qf, wv, cur.frag, cur.scale, lane, nq, ps);
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            if (j < nq) {
                const float s = ps[j];
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


// ---------------------------------------------------------------------------
// LDS-ring variant: each wave streams its pages through a private ring of
// DMA_DEPTH page slots in LDS with global_load_lds_dwordx4 (one fully
// coalesced 1 KB transfer per instruction, no registers held while in flight).
// Within a page slot the 16-byte units of token t are XOR-permuted by
// page_swz(t) so that the MFMA fragment reads of 16 tokens hit distinct banks.
// Scores stay in registers until the wave's pages are done: global stores in
// the loop would share the vector-memory counter the ring waits on.
#ifndef IDX_DMA_DEPTH
#define IDX_DMA_DEPTH 2
#endif
#ifndef IDX_DMA_PPW
#define IDX_DMA_PPW 4
#endif
constexpr int DMA_DEPTH = IDX_DMA_DEPTH;     // pages in flight per wave
constexpr int DMA_PPW = IDX_DMA_PPW;         // pages per wave per workgroup
constexpr int DMA_OPS_PER_PAGE = 9;          // 8 x 1 KB of keys + 256 B of scales

__device__ __forceinline__ int page_swz(int t) { return (t ^ (t >> 3)) & 7; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    if constexpr (N == 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    else if constexpr (N == 9) asm volatile("s_waitcnt vmcnt(9)" ::: "memory");
    else if constexpr (N == 18) asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
    else if constexpr (N == 27) asm volatile("s_waitcnt vmcnt(27)" ::: "memory");
    else static_assert(N == 0, "unsupported vmcnt");
}

template <int NQ, int HT, bool HIST>
__global__ __launch_bounds__(IDX_THREADS) void indexer_fp8_dma(IndexerArgs a, int qgroups) {
    const Geometry& G = a.g;
    const int r = blockIdx.y / qgroups, qg = blockIdx.y % qgroups;
    const int L = G.ctx[r];
    const int qs = G.qsl[r], ql = G.qsl[r + 1] - qs;
    const int j0 = qg * NQ;
    if (j0 >= ql) return;
    const int nq = min(NQ, ql - j0);
    const int n_last = L - ql + j0 + nq;
    constexpr int CHUNK = 4 * DMA_PPW * IDX_PAGE;
    const int tok0 = blockIdx.x * CHUNK;
    if (tok0 >= n_last) return;
    const int tok1 = min(n_last, tok0 + CHUNK);

    __shared__ __attribute__((aligned(16))) uint8_t kbuf[4][DMA_DEPTH][IDX_PAGE * IDX_D];
    __shared__ __attribute__((aligned(16))) float sbuf[4][DMA_DEPTH][IDX_PAGE];
    __shared__ uint32_t hist[HIST ? NQ : 1][HIST ? HIST_BINS / 2 : 1];   // two 16-bit counts per word
    const int tid = threadIdx.x, lane = tid & 63;
    // wave index in a scalar register: page ids then come from scalar loads,
    // which do not touch the vector-memory counter the ring waits on
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, col = lane & 15;
    if constexpr (HIST)
        for (int i = tid; i < NQ * HIST_BINS / 2; i += IDX_THREADS) (&hist[0][0])[i] = 0u;

    const int32_t* pt = G.page_table + (size_t)r * G.max_blocks;
    const uint8_t* keys = (const uint8_t*)a.keys;
    const bool has_scale = a.key_scales != nullptr;
    const int pfirst = tok0 / IDX_PAGE + wave;               // wave's page i is pfirst + 4 i
    const int page1 = (tok1 + IDX_PAGE - 1) / IDX_PAGE;
    const int npw = pfirst < page1 ? min(DMA_PPW, (page1 - pfirst + 3) / 4) : 0;

    // physical blocks of the wave's pages, read before the ring starts
    int blks[DMA_PPW];
#pragma unroll
    for (int i = 0; i < DMA_PPW; ++i) blks[i] = i < npw ? __builtin_amdgcn_readfirstlane(pt[pfirst + 4 * i]) : 0;
    auto issue = [&](int i) {   // DMA page i of this wave into ring slot i % DMA_DEPTH
        const int blk = blks[i];
        const uint8_t* src = keys + (size_t)blk * (IDX_PAGE * IDX_D);
        uint8_t* dst = &kbuf[wave][i % DMA_DEPTH][0];
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            const int U = 64 * c + lane, t = U >> 3, u = (U & 7) ^ page_swz(t);
            __builtin_amdgcn_global_load_lds((const void*)(src + t * IDX_D + 16 * u), (lds_ptr_t)(dst + 1024 * c),
                                             16, 0, 0);
        }
        const void* ssrc = has_scale ? (const void*)(a.key_scales + (size_t)blk * IDX_PAGE + lane)
                                     : (const void*)(src + 4 * lane);
        __builtin_amdgcn_global_load_lds(ssrc, (lds_ptr_t)&sbuf[wave][i % DMA_DEPTH][0], 4, 0, 0);
    };
#pragma unroll
    for (int d = 0; d < DMA_DEPTH; ++d)
        if (d < npw) issue(d);

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
    if constexpr (HIST) __syncthreads();

    float sc[NQ][DMA_PPW];
#pragma unroll
    for (int i = 0; i < DMA_PPW; ++i) {
#pragma unroll
        for (int j = 0; j < NQ; ++j) sc[j][i] = 0.f;
        if (i < npw) {
            // page i has landed once at most the younger pages' transfers are pending
            if (i + DMA_DEPTH - 1 < npw) wait_vmcnt<DMA_OPS_PER_PAGE * (DMA_DEPTH - 1)>();
            else wait_vmcnt<0>();
            const uint8_t* pb = &kbuf[wave][i % DMA_DEPTH][0];
            i32x8 kf[4];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int t = 16 * nt + col;
                const u32x4 lo = *(const u32x4*)(pb + t * IDX_D + 16 * (g ^ page_swz(t)));
                const u32x4 hi = *(const u32x4*)(pb + t * IDX_D + 16 * ((4 + g) ^ page_swz(t)));
                kf[nt] = join_i32x8(lo, hi);
            }
            const float ksc = has_scale ? sbuf[wave][i % DMA_DEPTH][lane] : 1.f;
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // slot read before it is refilled
            if (i + DMA_DEPTH < npw) issue(i + DMA_DEPTH);
            float ps[NQ];
            page_scores<NQ, HT>(qf, wv, kf, ksc, lane, nq, ps);
#pragma unroll
            for (int j = 0; j < NQ; ++j) sc[j][i] = ps[j];
        }
    }
    // Stores and histogram counts after the ring has drained (LDS atomics
    // issued while transfers are pending would make the compiler wait on them).
    // (histogram first: its barrier then has no stores to wait for)
    if constexpr (HIST) {
#pragma unroll
        for (int i = 0; i < DMA_PPW; ++i) {
            const int pos = (pfirst + 4 * i) * IDX_PAGE + lane;
#pragma unroll
            for (int j = 0; j < NQ; ++j) {
                const int n_j = L - ql + j0 + j + 1;
                if (i < npw && j < nq && pos < n_j) {
                    const uint32_t b = score_key(sc[j][i]) >> HIST_SHIFT;
                    atomicAdd(&hist[j][b >> 1], 1u << (16 * (b & 1)));
                }
            }
        }
        __syncthreads();
        for (int j = 0; j < nq; ++j) {
            uint32_t* gh = a.hist + (size_t)(qs + j0 + j) * HIST_BINS;
            for (int w = tid; w < HIST_BINS / 2; w += IDX_THREADS) {
                const uint32_t v = hist[j][w];
                if (v & 0xFFFFu) atomicAdd(gh + 2 * w, v & 0xFFFFu);
                if (v >> 16) atomicAdd(gh + 2 * w + 1, v >> 16);
            }
        }
    }
#pragma unroll
    for (int i = 0; i < DMA_PPW; ++i) {
        const int pos = (pfirst + 4 * i) * IDX_PAGE + lane;
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            const int n_j = L - ql + j0 + j + 1;
            if (i < npw && j < nq && pos < n_j) a.scores[(size_t)(qs + j0 + j) * a.ld + pos] = sc[j][i];
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

#ifndef IDX_USE_DMA
#define IDX_USE_DMA 1
#endif

template <int NQ, int HT>
static hipError_t launch_fp8(const IndexerArgs& a, hipStream_t s) {
    const int qgroups = (a.g.max_q_len + NQ - 1) / NQ;
    if (IDX_USE_DMA) {
        const int chunk = 4 * DMA_PPW * IDX_PAGE;
        dim3 grid((a.g.max_ctx + chunk - 1) / chunk, a.g.B * qgroups);
        if (a.hist)
            hipLaunchKernelGGL((indexer_fp8_dma<NQ, HT, true>), grid, dim3(IDX_THREADS), 0, s, a, qgroups);
        else
            hipLaunchKernelGGL((indexer_fp8_dma<NQ, HT, false>), grid, dim3(IDX_THREADS), 0, s, a, qgroups);
        return hipGetLastError();
    }
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
