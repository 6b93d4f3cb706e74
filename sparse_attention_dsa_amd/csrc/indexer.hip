// Lightning-indexer scores on gfx950.
//
// Score of visible token s for query row t (SemiAnalysis GLM-5.3 article,
// "Lightning Indexer"): I[t,s] = sigma_s * sum_h w[t,h] * ReLU(q[t,h,:] . k_s).
// sigma_s (per-token key scale) is applied after the head sum, exact because
// ReLU is positively homogeneous and sigma_s >= 0.
//
// Fast path (e4m3 keys and queries, dim 128, 16/32/64 heads, 64-token blocks).
// Keys are streamed once, a 64-token page (8 KB, contiguous) at a time, and
// multiplied against register-resident queries with
// v_mfma_f32_16x16x128_f8f6f4: heads are the M dimension, tokens the N
// dimension and the whole 128-wide key the K dimension, so one instruction
// covers a 16x16 head-token tile and a page takes 16 per query row.  ReLU,
// head weights and the key scale are applied on the accumulators; the head sum
// crosses the four 16-lane groups with three lane exchanges, leaving lane l
// with the score of token l of the page.
//
// Two launch shapes:
//   persistent  (decode-sized batches) a fixed grid, two workgroups per CU;
//               all (request, query group) page ranges are concatenated and
//               each wave streams an equal contiguous share, so every wave
//               does the same work with no per-chunk start-up;
//   chunked     one workgroup per (request, query group, 1024-token chunk),
//               pages fed by an LDS ring of asynchronous transfers.
#include <hip/hip_ext.h>

#include "indexer_dev.h"
#include "topk_dev.h"

namespace dsa {

// ---------------------------------------------------------------------------
// LDS-ring variant: each wave streams its pages through a private ring of
// DMA_DEPTH page slots in LDS with global_load_lds_dwordx4 (one fully
// coalesced 1 KB transfer per instruction, no registers held while in flight).
// Within a page slot the 16-byte units of token t are XOR-permuted by
// page_swz(t) so that the MFMA fragment reads of 16 tokens hit distinct banks.
// Scores stay in registers until the wave's pages are done: global stores in
// the loop would share the vector-memory counter the ring waits on.
constexpr int DMA_DEPTH = 2;                 // pages in flight per wave
constexpr int DMA_PPW = 4;                   // pages per wave per workgroup
constexpr int DMA_OPS_PER_PAGE = 9;          // 8 x 1 KB of keys + 256 B of scales
constexpr int DMA_AUX = 3;                   // cache policy of the key transfers (sc0 nt: streamed once)

typedef __attribute__((address_space(3))) void* lds_ptr_t;

template <int NQ, int HT>
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
    const int tid = threadIdx.x, lane = tid & 63;
    // wave index in a scalar register: page ids then come from scalar loads,
    // which do not touch the vector-memory counter the ring waits on
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, col = lane & 15;

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
                                             16, 0, DMA_AUX);
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
    // scores are stored after the ring has drained (stores share the counter it waits on)
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


// ---------------------------------------------------------------------------
// Query-blocked variant for long query chunks (chunked prefill), where the
// indexer is a dense fp8 product with a causal epilogue.  A workgroup owns
// PF_QB query rows of one request (PF_QW per wave, queries and weights in
// registers) and a range of PF_CHUNK pages.  Each page (8 KB of keys and
// 256 B of scales) enters an LDS ring once per workgroup, by asynchronous
// transfers split evenly over the waves, and is read by every wave, so a key
// byte brought from L2 feeds PF_QB query rows.  Workgroups are numbered
// page-range-major: the ones resident together work on the same pages.
//
// Every wave issues the same transfers for every page (its 1 KB key units and
// the page's scales) and one score store per query row and page (buffer stores whose descriptors
// are sized to each row's visible count, so positions past it are dropped),
// which keeps the vector-memory counts of the ring's waits exact.
// Scores of one page for PF_QW query rows with the MFMAs of the next token
// tile in flight while the current one's results are reduced (two sets of
// accumulators), so the matrix core does not wait for the vector ALU.
template <int NQ, int HT>
__device__ __forceinline__ void page_scores_ilp(const i32x8 (&qf)[NQ][HT], const float (&wv)[NQ][HT][4],
                                                const i32x8 (&kf)[4], float ksc, int lane, float (&out)[NQ]) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 c[2][NQ][HT];
    float part[NQ][4];
#pragma unroll
    for (int j = 0; j < NQ; ++j)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) c[0][j][ht] = mfma_fp8_16x16x128(qf[j][ht], kf[0], zero);
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
        if (nt + 1 < 4) {
#pragma unroll
            for (int j = 0; j < NQ; ++j)
#pragma unroll
                for (int ht = 0; ht < HT; ++ht)
                    c[(nt + 1) & 1][j][ht] = mfma_fp8_16x16x128(qf[j][ht], kf[nt + 1], zero);
        }
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            float acc = 0.f;
#pragma unroll
            for (int ht = 0; ht < HT; ++ht)
#pragma unroll
                for (int i = 0; i < 4; ++i) acc = fmaf(wv[j][ht][i], relu(c[nt & 1][j][ht][i]), acc);
            part[j][nt] = acc;
        }
    }
#pragma unroll
    for (int j = 0; j < NQ; ++j) out[j] = head_sum_transpose(part[j], lane) * ksc;
}

constexpr int PF_WAVES = 4;
constexpr int PF_QW = 2;                       // query rows per wave
constexpr int PF_QB = PF_WAVES * PF_QW;        // query rows per workgroup
constexpr int PF_KU = 8 / PF_WAVES;            // 1 KB key units each wave moves per page
constexpr int PF_OPS = PF_KU + 1;              // transfers per wave per page (keys, scales)
constexpr int PF_CHUNK = 128;                  // pages per workgroup
constexpr int PF_RING = 4;                     // page slots
constexpr int PF_MIN_Q = 8;                    // longest query chunk from which it is used

template <int HT>
__global__ __launch_bounds__(PF_WAVES * 64) __attribute__((amdgpu_waves_per_eu(2)))
void indexer_fp8_prefill(IndexerArgs a, int qblocks) {
    const Geometry& G = a.g;
    const int r = blockIdx.x / qblocks, jb = blockIdx.x % qblocks;
    const int qs = G.qsl[r], ql = G.qsl[r + 1] - qs;
    const int j0 = jb * PF_QB;
    if (j0 >= ql) return;
    const int L = G.ctx[r];
    const int n_last = L - ql + min(ql, j0 + PF_QB);      // visible tokens of the block's last row
    const int p0 = blockIdx.y * PF_CHUNK;
    const int np_all = (n_last + IDX_PAGE - 1) / IDX_PAGE;
    if (p0 >= np_all) return;
    const int np = min(PF_CHUNK, np_all - p0);

    // a slot: the page's keys, then four copies of its 64 scales
    constexpr int SLOT = IDX_PAGE * IDX_D + 16 * IDX_PAGE;
    __shared__ __attribute__((aligned(16))) uint8_t kbuf[PF_RING][SLOT];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, col = lane & 15;

    // this wave's query rows; a row past the request repeats its last row
    // and stores nothing
    const int jw = j0 + PF_QW * wave;
    const int nq = min(PF_QW, ql - jw);
    i32x8 qf[PF_QW][HT];
    float wv[PF_QW][HT][4];
    __amdgpu_buffer_rsrc_t orow[PF_QW];
#pragma unroll
    for (int j = 0; j < PF_QW; ++j) {
        const int jj = min(jw + j, ql - 1);
        const int t = qs + jj;
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const uint8_t* qp = (const uint8_t*)a.q + ((size_t)t * a.n_heads + 16 * ht + col) * IDX_D + 16 * g;
            qf[j][ht] = join_i32x8(*(const u32x4*)qp, *(const u32x4*)(qp + 64));
#pragma unroll
            for (int i = 0; i < 4; ++i) wv[j][ht][i] = a.w[(size_t)t * a.n_heads + 16 * ht + 4 * g + i];
        }
        const int nvis = j < nq ? L - ql + jj + 1 : 0;
        orow[j] = __builtin_amdgcn_make_buffer_rsrc((void*)(a.scores + (size_t)t * a.ld), 0, 4 * nvis, 0x00020000);
    }
    // physical block of chunk page 64b + l in lane l of blkv[b]
    const int32_t* pt = G.page_table + (size_t)r * G.max_blocks;
    int blkv[PF_CHUNK / 64];
#pragma unroll
    for (int b = 0; b < PF_CHUNK / 64; ++b) blkv[b] = 64 * b + lane < np ? pt[p0 + 64 * b + lane] : 0;
    // consume the loads above here, so that no wait for them lands inside
    // the ring (whose waits count only its own transfers and stores)
#pragma unroll
    for (int j = 0; j < PF_QW; ++j)
#pragma unroll
        for (int ht = 0; ht < HT; ++ht) {
            const u32x4 lo = (u32x4)__builtin_shufflevector(qf[j][ht], qf[j][ht], 0, 1, 2, 3);
            const u32x4 hi = (u32x4)__builtin_shufflevector(qf[j][ht], qf[j][ht], 4, 5, 6, 7);
            asm volatile("" ::"v"(lo), "v"(hi));
#pragma unroll
            for (int i = 0; i < 4; ++i) asm volatile("" ::"v"(wv[j][ht][i]));
        }
#pragma unroll
    for (int b = 0; b < PF_CHUNK / 64; ++b) asm volatile("" ::"v"(blkv[b]));

    const uint8_t* keys = (const uint8_t*)a.keys;
    const bool has_scale = a.key_scales != nullptr;
    // chunk page p into the slot at dst: key units 2w, 2w+1 and the page's
    // 64 scales (every wave writes the same scale values)
    auto issue = [&](int p, uint8_t* dst) {
        int bv = blkv[0];
#pragma unroll
        for (int b = 1; b < PF_CHUNK / 64; ++b) bv = (p >> 6) == b ? blkv[b] : bv;
        const int blk = __builtin_amdgcn_readlane(bv, p & 63);
        const uint8_t* src = keys + (size_t)blk * (IDX_PAGE * IDX_D);
#pragma unroll
        for (int c = 0; c < PF_KU; ++c) {
            const int U = 64 * (PF_KU * wave + c) + lane, t = U >> 3, u = (U & 7) ^ page_swz(t);
            __builtin_amdgcn_global_load_lds((const void*)(src + t * IDX_D + 16 * u),
                                             (lds_ptr_t)(dst + 1024 * (PF_KU * wave + c)), 16, 0, DMA_AUX);
        }
        // the 256 B of scales as 16-byte units: lane l moves unit l & 15, so
        // the slot holds four copies
        const uint8_t* ssrc = has_scale ? (const uint8_t*)(a.key_scales + (size_t)blk * IDX_PAGE) : src;
        __builtin_amdgcn_global_load_lds((const void*)(ssrc + 16 * (lane & 15)),
                                         (lds_ptr_t)(dst + IDX_PAGE * IDX_D), 16, 0, 0);
    };
#pragma unroll
    for (int d = 0; d < PF_RING - 1; ++d)
        if (d < np) issue(d, &kbuf[d][0]);

    for (int p = 0; p < np; ++p) {
        // page p's transfers of this wave are done once at most the younger
        // operations are pending: in steady state the stores of the three
        // previous pages and the transfers of the next two; before that, at
        // least the next two pages' transfers
        if (p >= PF_RING - 1 && p + 2 < np) wait_vmcnt<3 * PF_QW + 2 * PF_OPS>();
        else if (p + 2 < np) wait_vmcnt<2 * PF_OPS>();
        else wait_vmcnt<0>();
        lds_barrier();   // every wave's part of page p landed; the slot of page p - 1 is free
        // the slot read and the slot refilled are passed as __restrict__
        // pointers: the compiler then knows the transfers in flight cannot
        // alias the reads and does not wait for them before each read
        auto body = [&](const uint8_t* __restrict__ pb, uint8_t* __restrict__ dst) {
            if (p + PF_RING - 1 < np) issue(p + PF_RING - 1, dst);
            i32x8 kf[4];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int t = 16 * nt + col;
                const u32x4 lo = *(const u32x4*)(pb + t * IDX_D + 16 * (g ^ page_swz(t)));
                const u32x4 hi = *(const u32x4*)(pb + t * IDX_D + 16 * ((4 + g) ^ page_swz(t)));
                kf[nt] = join_i32x8(lo, hi);
            }
            const float ksc = has_scale ? ((const float*)(pb + IDX_PAGE * IDX_D))[lane] : 1.f;
            float ps[PF_QW];
            page_scores_ilp<PF_QW, HT>(qf, wv, kf, ksc, lane, ps);
            const int voff = 4 * ((p0 + p) * IDX_PAGE + lane);
#pragma unroll
            for (int j = 0; j < PF_QW; ++j)
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ps[j]), orow[j], voff, 0, 0);
        };
        const int nx = (p + PF_RING - 1) % PF_RING;
        body(&kbuf[p % PF_RING][0], &kbuf[nx][0]);
    }
}

template <int HT>
static hipError_t launch_fp8_prefill(const IndexerArgs& a, hipStream_t s) {
    const int qblocks = (a.g.max_q_len + PF_QB - 1) / PF_QB;
    const int chunks = ((a.g.max_ctx + IDX_PAGE - 1) / IDX_PAGE + PF_CHUNK - 1) / PF_CHUNK;
    hipLaunchKernelGGL(indexer_fp8_prefill<HT>, dim3(a.g.B * qblocks, chunks), dim3(PF_WAVES * 64), 0, s, a,
                       qblocks);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Persistent variant for decode batches: the work is the concatenation of all
// (request, query group) page ranges; a fixed grid of workgroups splits it
// into equal contiguous shares, one per wave, so every wave streams the same
// number of pages with no per-chunk start-up and no tail imbalance.  Pages
// arrive through the staged register ring (contiguous 1 KB loads, relaid
// through the wave's LDS buffer); queries and weights are reloaded when a
// wave's share crosses into the next request.
constexpr int PER_PF = 2;                  // pages in flight per wave
constexpr int PER_MAX_ITEMS = 4096;        // (request, query group) pairs per launch
constexpr int PER_WG_PER_CU = 2;
constexpr int PER_MIN_PAGES = 2;       // pages per wave at least when emitting (small batches)

// EMIT: instead of storing the scores, each wave stages the composites of its
// scores at or above the row's key bound in LDS and appends them to the row's
// candidate list with one atomic per flush (at a request change, when the
// stage fills, and at the end of the share).  The stage is double-buffered
// and a flush completes one page later: the atomic's returned base is used
// only then, so waiting for it never drains the page ring.
template <int NQ>
constexpr int stage_cap() { return NQ == 1 ? 256 : 128; }   // per wave, query row and half

template <int NQ, int HT, bool EMIT>
__global__ __launch_bounds__(IDX_THREADS) __attribute__((amdgpu_waves_per_eu(2)))
void indexer_fp8_persistent(IndexerArgs a, int qgroups) {
    const Geometry& G = a.g;
    const int n_items = G.B * qgroups;
    __shared__ int item_off[PER_MAX_ITEMS + 1];
    __shared__ int scan_tmp[IDX_THREADS];
    __shared__ __attribute__((aligned(16))) uint8_t pbuf[4][IDX_PAGE * IDX_D];
    constexpr int STAGE_CAP = stage_cap<NQ>();
    __shared__ uint64_t stage[EMIT ? 4 : 1][EMIT ? NQ : 1][EMIT ? 2 : 1][EMIT ? STAGE_CAP : 1];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, col = lane & 15;

    // pages of each item (visible count of the group's last row), prefix-summed
    auto item_pages = [&](int it) -> int {
        const int r = it / qgroups, qg = it % qgroups;
        const int qs = G.qsl[r], ql = G.qsl[r + 1] - qs;
        const int j0 = qg * NQ;
        if (j0 >= ql) return 0;
        const int n_last = G.ctx[r] - ql + j0 + min(NQ, ql - j0);
        return n_last > 0 ? (n_last + IDX_PAGE - 1) / IDX_PAGE : 0;
    };
    const int per = (n_items + IDX_THREADS - 1) / IDX_THREADS;
    const int i0 = min(n_items, tid * per), i1 = min(n_items, i0 + per);
    int local = 0;
    for (int it = i0; it < i1; ++it) local += item_pages(it);
    scan_tmp[tid] = local;
    __syncthreads();
    for (int off = 1; off < IDX_THREADS; off <<= 1) {
        const int v = tid >= off ? scan_tmp[tid - off] : 0;
        __syncthreads();
        scan_tmp[tid] += v;
        __syncthreads();
    }
    int run = scan_tmp[tid] - local;
    for (int it = i0; it < i1; ++it) { item_off[it] = run; run += item_pages(it); }
    if (tid == IDX_THREADS - 1) item_off[n_items] = scan_tmp[tid];
    __syncthreads();

    const int P = item_off[n_items];
    const int nwaves = gridDim.x * 4;
    const int gw = blockIdx.x * 4 + wave;
    const int p0 = (int)(((long long)P * gw) / nwaves), p1 = (int)(((long long)P * (gw + 1)) / nwaves);
    if (p0 >= p1) return;
    auto find_item = [&](int p) -> int {   // largest it with item_off[it] <= p and pages > 0
        int lo = 0, hi = n_items - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (item_off[mid] <= p) lo = mid; else hi = mid - 1;
        }
        while (item_off[lo + 1] <= p) ++lo;
        return lo;
    };
    const uint8_t* keys = (const uint8_t*)a.keys;

    // Page-table entries and item ids of the share, resolved 64 pages at a
    // time (lane l: page base + l) one batch ahead, so no page waits on a
    // page-table load; the cursors read them with v_readlane.
    auto load_batch = [&](int base, int& blk_v, int& item_v) {
        const int p = base + lane;
        int it = 0, blk = 0;
        if (p < p1) {
            it = find_item(p);
            blk = G.page_table[(size_t)(it / qgroups) * G.max_blocks + (p - item_off[it])];
        }
        blk_v = blk;
        item_v = it;
    };
    int bb = p0, cblk, citem, nblk = 0, nitem = 0;
    load_batch(bb, cblk, citem);
    if (bb + 64 < p1) load_batch(bb + 64, nblk, nitem);
    auto blk_of = [&](int q) -> int {   // q in [bb, bb + 128)
        const int d = q - bb;
        return d < 64 ? __builtin_amdgcn_readlane(cblk, d) : __builtin_amdgcn_readlane(nblk, d - 64);
    };

    // The loop body is straight-line for the memory system: every slot
    // issues a page (past the share it re-reads the share's last page) and
    // stores its scores through buffer stores whose out-of-range lanes are
    // dropped, so the compiler's load counting stays exact and the ring of
    // PER_PF pages is never drained early.
    const auto clampp = [&](int q) { return q < p1 ? q : p1 - 1; };
    int iss_p = p0;
    auto issue_next = [&](RawPage& dst) {
        load_raw_page(keys, a.key_scales, blk_of(clampp(iss_p)), iss_p < p1, lane, dst);
        ++iss_p;
    };
    RawPage ring[PER_PF];
#pragma unroll
    for (int d = 0; d < PER_PF; ++d) issue_next(ring[d]);

    // compute cursor state: current item's queries, output rows
    int cur_it = -1, cur_base = 0;
    i32x8 qf[NQ][HT];
    float wv[NQ][HT][4];
    __amdgpu_buffer_rsrc_t orow[NQ];   // score row of each query, sized to its visible count
    // EMIT state per query row of the item: row index, visible count, bound,
    // staged count (all wave-uniform)
    // stage half in use, staged count; pending flush: count, half, row and the
    // atomic's returned base (lane 0)
    int trow[NQ], nvis[NQ], nst[NQ], half[NQ], pn[NQ], ph[NQ], prow[NQ];
    uint32_t pbase[NQ];
    float xf[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        trow[j] = 0; nvis[j] = 0; nst[j] = 0; half[j] = 0; pn[j] = 0; ph[j] = 0; prow[j] = 0; pbase[j] = 0u;
        xf[j] = 0.f;
    }
    auto complete = [&](int j) {   // copy a pending flush's entries to the row's list
        if (pn[j] == 0) return;
        const uint32_t base = (uint32_t)__builtin_amdgcn_readlane((int)pbase[j], 0);
        uint64_t* dst = a.cand + (size_t)prow[j] * TOPK_LIST;
        for (int i = lane; i < pn[j]; i += 64)
            if (base + (uint32_t)i < (uint32_t)TOPK_LIST) dst[base + i] = stage[wave][j][ph[j]][i];
        pn[j] = 0;
    };
    auto flush = [&](int j) {      // reserve list space; the copy happens in complete()
        complete(j);
        if (nst[j] == 0) return;
        if (lane == 0) pbase[j] = atomicAdd(&a.row_count[(size_t)trow[j] * ROW_COUNT_STRIDE], (uint32_t)nst[j]);
        pn[j] = nst[j];
        ph[j] = half[j];
        prow[j] = trow[j];
        half[j] ^= 1;
        nst[j] = 0;
    };
    auto load_item = [&](int it) {
        cur_it = it;
        cur_base = __builtin_amdgcn_readfirstlane(item_off[it]);
        const int r = it / qgroups;
        const int qg = it % qgroups;
        const int qs = __builtin_amdgcn_readfirstlane(G.qsl[r]);
        const int ql = __builtin_amdgcn_readfirstlane(G.qsl[r + 1]) - qs;
        const int L = __builtin_amdgcn_readfirstlane(G.ctx[r]);
        const int j0 = qg * NQ, nq = min(NQ, ql - j0);
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            const int t = qs + j0 + min(j, nq - 1);
            const int n_j = j < nq ? L - ql + j0 + j + 1 : 0;
            if constexpr (EMIT) {
                trow[j] = t;
                nvis[j] = n_j;
                xf[j] = key_floor(a.bound[t]);
            } else {
                orow[j] = __builtin_amdgcn_make_buffer_rsrc(a.scores + (size_t)t * a.ld, 0, 4 * max(n_j, 0),
                                                            0x00020000);
            }
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                const uint8_t* qp = (const uint8_t*)a.q + ((size_t)t * a.n_heads + 16 * ht + col) * IDX_D + 16 * g;
                qf[j][ht] = join_i32x8(*(const u32x4*)qp, *(const u32x4*)(qp + 64));
#pragma unroll
                for (int i = 0; i < 4; ++i) wv[j][ht][i] = a.w[(size_t)t * a.n_heads + 16 * ht + 4 * g + i];
            }
        }
        // Use every reloaded value here: the wait for these loads then sits
        // in this (rare) branch, and the page ring's waits after it stay exact.
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
#pragma unroll
            for (int ht = 0; ht < HT; ++ht) {
                asm volatile("" ::"v"(qf[j][ht][0]), "v"(qf[j][ht][4]));
#pragma unroll
                for (int i = 0; i < 4; ++i) asm volatile("" ::"v"(wv[j][ht][i]));
            }
            if constexpr (EMIT) asm volatile("" ::"v"(xf[j]));
        }
    };
    uint8_t* pb = &pbuf[wave][0];
    const int wt = lane >> 3, wu = lane & 7;
    for (int base = p0; base < p1; base += PER_PF) {
#pragma unroll
        for (int sl = 0; sl < PER_PF; ++sl) {
            const int p = base + sl;
            const int pc = clampp(p);
            if (pc == bb + 64) {   // next batch becomes current; resolve the one after
                bb += 64;
                cblk = nblk;
                citem = nitem;
                if (bb + 64 < p1) load_batch(bb + 64, nblk, nitem);
            }
            const int it = __builtin_amdgcn_readlane(citem, pc - bb);
            if (it != cur_it) {
                if constexpr (EMIT) {
#pragma unroll
                    for (int j = 0; j < NQ; ++j) flush(j);
                }
                load_item(it);
            }
            RawPage& cur = ring[sl];
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const int t = 8 * c + wt;
                *(u32x4*)(pb + t * IDX_D + 16 * (wu ^ page_swz(t))) = cur.v[c];
            }
            i32x8 kf[4];
#pragma unroll
            for (int nt = 0; nt < 4; ++nt) {
                const int t = 16 * nt + col;
                const u32x4 lo = *(const u32x4*)(pb + t * IDX_D + 16 * (g ^ page_swz(t)));
                const u32x4 hi = *(const u32x4*)(pb + t * IDX_D + 16 * ((4 + g) ^ page_swz(t)));
                kf[nt] = join_i32x8(lo, hi);
            }
            const float ksc = a.key_scales ? cur.scale : 1.0f;
            issue_next(cur);
            float ps[NQ];
            page_scores<NQ, HT>(qf, wv, kf, ksc, lane, NQ, ps);
            // out-of-range offsets (past the row's visible count, or a page past
            // the share) are dropped by the buffer range check
            const int pos = (pc - cur_base) * IDX_PAGE + lane;
            if constexpr (EMIT) {
#pragma unroll
                for (int j = 0; j < NQ; ++j) {
                    complete(j);   // a flush issued one page ago
                    const bool keep = p < p1 && pos < nvis[j] && ps[j] >= xf[j];
                    const unsigned long long mk = __ballot(keep);
                    if (mk != 0ull) {
                        const unsigned long long below = lane ? (mk & ((1ull << lane) - 1ull)) : 0ull;
                        if (keep)
                            stage[wave][j][half[j]][nst[j] + __popcll(below)] = composite(score_key(ps[j]), pos);
                        nst[j] += __popcll(mk);
                        if (nst[j] > STAGE_CAP - 64) flush(j);
                    }
                }
            } else {
                const int voff = p < p1 ? 4 * pos : 0x7FFFFFF0;
#pragma unroll
                for (int j = 0; j < NQ; ++j)
                    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ps[j]), orow[j], voff, 0, 0);
            }
        }
    }
    if constexpr (EMIT) {
        // every row's last reservation in flight before waiting for any:
        // at the end of the shares many waves append to the same few rows
#pragma unroll
        for (int j = 0; j < NQ; ++j) complete(j);
#pragma unroll
        for (int j = 0; j < NQ; ++j) flush(j);
#pragma unroll
        for (int j = 0; j < NQ; ++j) complete(j);
    }
}

// ---------------------------------------------------------------------------
// Sample bound for candidate emission: one 1024-thread workgroup per query
// row scores the row's strided sample of tokens (same MFMA page scoring, 16
// tokens per fragment) and writes the key bound the indexer filters with.  It
// also zeroes the row's candidate counter.  Rows of at most TOPK_LIST tokens
// take every token (bound 0).
constexpr int SB_THREADS = 1024;
constexpr int SB_BATCH = 4;                                        // key fragments in flight per lane

template <int HT>
__global__ __launch_bounds__(SB_THREADS) void indexer_sample_bound(IndexerArgs a) {
    const Geometry& G = a.g;
    const int t = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    i32x8 qf[HT];
    float wv[HT][4];
    load_query<HT>(a, t, lane, qf, wv);   // in flight while the row's length arrives
    const int n = row_visible(G, t);
    if (tid == 0) a.row_count[(size_t)t * ROW_COUNT_STRIDE] = 0u;
    if (n <= TOPK_LIST) {
        if (tid == 0) a.bound[t] = 0u;
        return;
    }
    __shared__ uint32_t skeys[TK_SAMPLE_MAX];
    __shared__ uint32_t h[256], res;
    __shared__ uint32_t red[2][SB_THREADS / 64];
    const int r = G.q_uniform > 0 ? t / G.q_uniform : find_request(G.qsl, G.B, t);
    const int32_t* pt = G.page_table + (size_t)r * G.max_blocks;
    const int m = sample_size(n);
    const int per_wave = m / (SB_THREADS / 64);          // 64 .. 256 samples
    const int nfrag = per_wave / 16;
    const int nrun = m / 16;
    // The sample is m / 16 runs of 16 consecutive tokens at evenly spaced,
    // 16-aligned starts, so a run lies in one page: one page-table entry and
    // one contiguous 2 KB of keys.  Fragment f of wave w is run w nfrag + f,
    // lane (g, col) taking its token col (sample i0 + 16 f); four fragments
    // in flight at a time (1024 threads leave 128 registers a lane).
    const int i0 = wave * per_wave + (lane & 15);
    const int last = (n - 16) & ~15;
    for (int f0 = 0; f0 < nfrag; f0 += SB_BATCH) {
        int blk[SB_BATCH], row[SB_BATCH];
#pragma unroll
        for (int b = 0; b < SB_BATCH; ++b) {
            const int run = wave * nfrag + min(f0 + b, nfrag - 1);
            const int start = min((int)((long long)run * n / nrun) & ~15, last);
            blk[b] = pt[start / IDX_PAGE];
            row[b] = start % IDX_PAGE + (lane & 15);
        }
        i32x8 kf[SB_BATCH];
        float ksc[SB_BATCH];
#pragma unroll
        for (int b = 0; b < SB_BATCH; ++b) {
            kf[b] = load_key_fragment(a, blk[b], row[b], lane);
            ksc[b] = a.key_scales ? a.key_scales[(size_t)blk[b] * IDX_PAGE + row[b]] : 1.f;
        }
#pragma unroll
        for (int b = 0; b < SB_BATCH; ++b) {
            const float sc = token_head_sum<HT>(qf, wv, kf[b]) * ksc[b];
            if (lane < 16 && f0 + b < nfrag) skeys[i0 + 16 * (f0 + b)] = score_key(sc);
        }
    }
    lds_barrier();
    const uint32_t x = sample_key_bound<SB_THREADS>(skeys, m, n, (uint32_t)a.k, h, red, &res);
    if (tid == 0) a.bound[t] = x;
}

// FP4 E2M1 code (low 4 bits) and E8M0 scale byte to float (OCP Microscaling
// Formats v1.0: E2M1 has exponent bias 1 and one mantissa bit, exponent 0 is
// subnormal; E8M0 is 2^(e - 127), 255 is NaN).
__device__ __forceinline__ float e2m1_to_f32(uint32_t c) {
    const uint32_t e = (c >> 1) & 3u, m = c & 1u;
    const float mag = e == 0u ? 0.5f * (float)m : __uint_as_float((126u + e) << 23) * (1.0f + 0.5f * (float)m);
    return (c & 8u) ? -mag : mag;
}
__device__ __forceinline__ float e8m0_to_f32(uint32_t e) {
    if (e == 255u) return __builtin_nanf("");
    return e == 0u ? __uint_as_float(0x00400000u) : __uint_as_float(e << 23);
}

// Generic path: any head count / dim, fp32, e4m3 or MXFP4 keys (fp32 or e4m3
// queries), any block size.  One thread per (query row, token); the query and
// weights sit in LDS.
constexpr int GEN_MAX_D4 = 32;   // fp32 key rows held in registers: up to 128 elements
__global__ __launch_bounds__(256) void indexer_generic(IndexerArgs a) {
    const Geometry& G = a.g;
    const int t = blockIdx.y;
    const int r = find_request(G.qsl, G.B, t);
    const int n = visible_count(G.ctx, G.qsl, r, t);
    const int H = a.n_heads, D = a.dim;
    extern __shared__ float smem[];
    float* qv = smem;            // [H][D]
    float* wv = smem + H * D;    // [H]
    const bool f8 = a.key_dtype == 2 || a.key_dtype == 3;   // e4m3 queries
    const bool f4 = a.key_dtype == 3;
    for (int i = threadIdx.x; i < H * D; i += blockDim.x) {
        const size_t off = (size_t)t * H * D + i;
        qv[i] = f8 ? e4m3_to_f32(((const uint8_t*)a.q)[off]) : ((const float*)a.q)[off];
    }
    for (int i = threadIdx.x; i < H; i += blockDim.x) wv[i] = a.w[(size_t)t * H + i];
    __syncthreads();
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= n) return;
    const int bs = G.block_size;
    const size_t blk = (size_t)G.page_table[(size_t)r * G.max_blocks + s / bs];
    const size_t row = blk * bs + s % bs;
    // MXFP4: this token's codes and block scales inside its block
    const uint8_t* f4c = (const uint8_t*)a.keys + blk * bs * (size_t)(D / 2 + D / 32) + (size_t)(s % bs) * (D / 2);
    const uint8_t* f4e = (const uint8_t*)a.keys + blk * bs * (size_t)(D / 2 + D / 32) + (size_t)bs * (D / 2) +
                         (size_t)(s % bs) * (D / 32);
    float total = 0.f;
    if (a.key_dtype == 0 && (D & 3) == 0 && D <= 4 * GEN_MAX_D4) {
        // fp32 keys of at most 128 elements: the token's row in registers by
        // 16-byte loads all issued at once, then every head's dot product
        // from them (same order of additions as below)
        const f32x4* kr = (const f32x4*)((const float*)a.keys + row * D);
        const int d4n = D >> 2;
        f32x4 kv[GEN_MAX_D4];
#pragma unroll
        for (int i = 0; i < GEN_MAX_D4; ++i) kv[i] = i < d4n ? kr[i] : (f32x4){0.f, 0.f, 0.f, 0.f};
        for (int h = 0; h < H; ++h) {
            const float* qh = qv + h * D;
            float dot = 0.f;
#pragma unroll
            for (int i = 0; i < GEN_MAX_D4; ++i) {
                if (i < d4n) {
                    dot = fmaf(qh[4 * i], kv[i][0], dot);
                    dot = fmaf(qh[4 * i + 1], kv[i][1], dot);
                    dot = fmaf(qh[4 * i + 2], kv[i][2], dot);
                    dot = fmaf(qh[4 * i + 3], kv[i][3], dot);
                }
            }
            total = fmaf(wv[h], fmaxf(dot, 0.f), total);
        }
    } else {
        for (int h = 0; h < H; ++h) {
            float dot = 0.f;
            for (int d = 0; d < D; ++d) {
                const size_t off = row * D + d;
                float k;
                if (f4) k = e2m1_to_f32((uint32_t)(f4c[d >> 1] >> (4 * (d & 1)))) * e8m0_to_f32(f4e[d >> 5]);
                else k = f8 ? e4m3_to_f32(((const uint8_t*)a.keys)[off]) : ((const float*)a.keys)[off];
                dot = fmaf(qv[h * D + d], k, dot);
            }
            total = fmaf(wv[h], fmaxf(dot, 0.f), total);
        }
    }
    const float sc = a.key_scales ? a.key_scales[row] : 1.f;
    const float score = sc * total;
    a.scores[(size_t)t * a.ld + s] = score;
}

// Generic path kernel above; launch policy below.
template <int NQ, int HT>
static hipError_t launch_fp8(const IndexerArgs& a, hipStream_t s, const hipEvent_t* se) {
    const int qgroups = (a.g.max_q_len + NQ - 1) / NQ;
    if (a.g.B * qgroups <= PER_MAX_ITEMS) {
        // Emitting into candidate lists, small batches take at most as many
        // workgroups as give each wave PER_MIN_PAGES of the largest page
        // count the batch can have (a host-known bound): every wave with
        // pages makes one final reservation on its rows' counters, and on a
        // single row 512 of them on one line cost more than the pages.
        const long long pmax = (long long)a.g.B * qgroups * ((a.g.max_ctx + IDX_PAGE - 1) / IDX_PAGE);
        const long long full = (long long)device_cu_count() * PER_WG_PER_CU;
        const long long need = (pmax + 4 * PER_MIN_PAGES - 1) / (4 * PER_MIN_PAGES);
        const dim3 grid((unsigned)(a.cand ? std::max(1LL, std::min(full, need)) : full));
        if (se) {   // start and stop events taken by the launch itself: the kernel's own duration
            if (a.cand)
                hipExtLaunchKernelGGL((indexer_fp8_persistent<NQ, HT, true>), grid, dim3(IDX_THREADS), 0, s, se[0],
                                      se[1], 0, a, qgroups);
            else
                hipExtLaunchKernelGGL((indexer_fp8_persistent<NQ, HT, false>), grid, dim3(IDX_THREADS), 0, s, se[0],
                                      se[1], 0, a, qgroups);
        } else if (a.cand) {
            hipLaunchKernelGGL((indexer_fp8_persistent<NQ, HT, true>), grid, dim3(IDX_THREADS), 0, s, a, qgroups);
        } else {
            hipLaunchKernelGGL((indexer_fp8_persistent<NQ, HT, false>), grid, dim3(IDX_THREADS), 0, s, a, qgroups);
        }
        return hipGetLastError();
    }
    if (se) {
        const hipError_t e = hipEventRecord(se[0], s);
        if (e != hipSuccess) return e;
    }
    const int chunk = 4 * DMA_PPW * IDX_PAGE;
    dim3 grid((a.g.max_ctx + chunk - 1) / chunk, a.g.B * qgroups);
    hipLaunchKernelGGL((indexer_fp8_dma<NQ, HT>), grid, dim3(IDX_THREADS), 0, s, a, qgroups);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess && se ? hipEventRecord(se[1], s) : e;
}

bool indexer_emit_ok(const IndexerArgs& a) {
    const int qg = (a.g.max_q_len + 1) / 2;
    const int items = a.g.B * (a.g.max_q_len >= 2 ? qg : a.g.max_q_len);
    // batches with long query chunks take the query-blocked indexer, which
    // writes score rows (launch_indexer + launch_topk)
    return a.key_dtype == 2 && a.dim == IDX_D && a.g.block_size == IDX_PAGE &&
           (a.n_heads == 64 || a.n_heads == 32 || a.n_heads == 16) && items <= PER_MAX_ITEMS &&
           a.g.max_q_len < PF_MIN_Q;
}

hipError_t launch_sample_bound(const IndexerArgs& a, hipStream_t s) {
    switch (a.n_heads) {
    case 64: hipLaunchKernelGGL(indexer_sample_bound<4>, dim3(a.g.T), dim3(SB_THREADS), 0, s, a); break;
    case 32: hipLaunchKernelGGL(indexer_sample_bound<2>, dim3(a.g.T), dim3(SB_THREADS), 0, s, a); break;
    default: hipLaunchKernelGGL(indexer_sample_bound<1>, dim3(a.g.T), dim3(SB_THREADS), 0, s, a); break;
    }
    return hipGetLastError();
}

// -inf over the part of each score row past its visible tokens, [n_t, ld):
// workgroup (x, t) covers an eighth of row t's tail with 16-byte stores.
constexpr int TAIL_SPLIT = 8;
__global__ __launch_bounds__(256) void score_tail_fill(IndexerArgs a) {
    const int t = blockIdx.y;
    const int n = row_visible(a.g, t);
    const int64_t tail = a.ld - n;
    if (tail <= 0) return;
    float* row = a.scores + (size_t)t * a.ld;
    const int64_t per = (tail + TAIL_SPLIT - 1) / TAIL_SPLIT;
    const int64_t b0 = n + per * blockIdx.x, b1 = min<int64_t>(a.ld, b0 + per);
    const float ninf = -__builtin_inff();
    int64_t i = b0 + threadIdx.x;
    // scalar stores up to a 16-byte boundary of the row, then float4 stores
    const int64_t head = min<int64_t>(b1, (b0 + 3) & ~(int64_t)3);
    if (i < head) row[i] = ninf;
    const bool aligned = (reinterpret_cast<uintptr_t>(row) & 15u) == 0u;
    if (aligned) {
        for (int64_t v = head + 4 * (int64_t)threadIdx.x; v + 4 <= b1; v += 4 * 256)
            *(f32x4*)(row + v) = (f32x4){ninf, ninf, ninf, ninf};
        for (int64_t v = max(head, b1 & ~(int64_t)3) + threadIdx.x; v < b1; v += 256) row[v] = ninf;
    } else {
        for (int64_t v = head + threadIdx.x; v < b1; v += 256) row[v] = ninf;
    }
}

hipError_t launch_score_tail(const IndexerArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(score_tail_fill, dim3(TAIL_SPLIT, a.g.T), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_indexer(const IndexerArgs& a, hipStream_t s, const hipEvent_t* se) {
    if (a.key_dtype == 3 && mxfp4_fast(a)) {
        hipError_t e = se ? hipEventRecord(se[0], s) : hipSuccess;
        if (e == hipSuccess) e = launch_indexer_mxfp4(a, s);
        return e == hipSuccess && se ? hipEventRecord(se[1], s) : e;
    }
    const bool fast = a.key_dtype == 2 && a.dim == IDX_D && a.g.block_size == IDX_PAGE &&
                      (a.n_heads == 64 || a.n_heads == 32 || a.n_heads == 16);
    if (fast && a.g.max_q_len < PF_MIN_Q) {
        const bool two = a.g.max_q_len >= 2;
        switch (a.n_heads) {
        case 64: return two ? launch_fp8<2, 4>(a, s, se) : launch_fp8<1, 4>(a, s, se);
        case 32: return two ? launch_fp8<2, 2>(a, s, se) : launch_fp8<1, 2>(a, s, se);
        default: return two ? launch_fp8<2, 1>(a, s, se) : launch_fp8<1, 1>(a, s, se);
        }
    }
    hipError_t e = se ? hipEventRecord(se[0], s) : hipSuccess;
    if (e != hipSuccess) return e;
    if (fast) {
        switch (a.n_heads) {
        case 64: e = launch_fp8_prefill<4>(a, s); break;
        case 32: e = launch_fp8_prefill<2>(a, s); break;
        default: e = launch_fp8_prefill<1>(a, s); break;
        }
    } else {
        dim3 grid((a.g.max_ctx + 255) / 256, a.g.T);
        const size_t shm = sizeof(float) * ((size_t)a.n_heads * a.dim + a.n_heads);
        hipLaunchKernelGGL(indexer_generic, grid, dim3(256), shm, s, a);
        e = hipGetLastError();
    }
    return e == hipSuccess && se ? hipEventRecord(se[1], s) : e;
}

}  // namespace dsa
