// Top-K token selection on gfx950 without a global sort.
//
// Rule (SemiAnalysis GLM-5.3 article, "Lightning Indexer"): keep the K
// highest-scoring visible tokens, or every visible token when a query sees K
// or fewer; equal scores go to the lower token index.
//
// Each score maps to an order-preserving 32-bit key.  Selection runs in three
// kernels per query row:
//   hist   (only when the indexer did not already build it) counts keys per
//          bucket of their top 12 bits into a per-row histogram;
//   filter each workgroup re-derives the threshold bucket b* from the
//          histogram (the bucket holding the K-th largest key), then streams
//          its chunk of the row: tokens above b* are selected outright and
//          tokens in b* are appended to a candidate list; appends are
//          aggregated per wavefront (one atomic per wave);
//   refine one workgroup per row resolves the candidates exactly with an
//          MSB-first radix select over the composite key
//          (low 20 key bits, ~index) -- unique per token, so the lowest-index
//          tie rule falls out of the order -- then sorts the row's K indices
//          ascending in LDS (bitonic) and writes them with -1 padding.
#include "dsa_kernels.h"

namespace dsa {

constexpr int TK_THREADS = 256;
constexpr int TK_CHUNK = 16384;        // scores per filter / hist workgroup
constexpr int RF_THREADS = 512;

__global__ void zero_u32(uint32_t* __restrict__ p, size_t n) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    const size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n; i += stride) p[i] = 0u;
}

hipError_t launch_zero_u32(uint32_t* p, size_t n, hipStream_t s) {
    if (n == 0) return hipSuccess;
    const size_t blocks = min((n + 255) / 256, (size_t)4096);
    hipLaunchKernelGGL(zero_u32, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

__global__ __launch_bounds__(TK_THREADS) void topk_hist(TopkArgs a) {
    const Geometry& G = a.g;
    const int t = blockIdx.y;
    const int r = find_request(G.qsl, G.B, t);
    const int n = visible_count(G.ctx, G.qsl, r, t);
    if (n <= a.k) return;
    const int c0 = blockIdx.x * TK_CHUNK;
    if (c0 >= n) return;
    const int c1 = min(n, c0 + TK_CHUNK);
    __shared__ uint32_t h[HIST_BINS];
    for (int i = threadIdx.x; i < HIST_BINS; i += TK_THREADS) h[i] = 0u;
    __syncthreads();
    const float* row = a.scores + (size_t)t * a.ld;
    for (int s = c0 + threadIdx.x; s < c1; s += TK_THREADS)
        atomicAdd(&h[score_key(row[s]) >> HIST_SHIFT], 1u);
    __syncthreads();
    uint32_t* gh = a.hist + (size_t)t * HIST_BINS;
    for (int i = threadIdx.x; i < HIST_BINS; i += TK_THREADS)
        if (h[i]) atomicAdd(gh + i, h[i]);
}

// Threshold bucket of a row: the bucket b with count(> b) < k <= count(>= b).
// Every thread returns b and count(> b).  256 threads, 16 buckets each.
__device__ void find_threshold_bucket(const uint32_t* __restrict__ gh, int k, uint32_t* sh_scan,
                                      int& bucket, uint32_t& above) {
    static_assert(HIST_BINS == 16 * TK_THREADS, "bucket split");
    const int tid = threadIdx.x;
    const int hi = HIST_BINS - 16 * tid;   // this thread covers [hi-16, hi), highest first
    const u32x4* src = (const u32x4*)(gh + hi - 16);
    uint32_t c[16];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        u32x4 x = src[v];
        c[4 * v] = x[0]; c[4 * v + 1] = x[1]; c[4 * v + 2] = x[2]; c[4 * v + 3] = x[3];
    }
    uint32_t sum = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) sum += c[i];
    // inclusive scan over threads in descending-bucket order
    sh_scan[tid] = sum;
    __syncthreads();
    for (int off = 1; off < TK_THREADS; off <<= 1) {
        uint32_t v = tid >= off ? sh_scan[tid - off] : 0u;
        __syncthreads();
        sh_scan[tid] += v;
        __syncthreads();
    }
    const uint32_t incl = sh_scan[tid];
    const uint32_t excl = incl - sum;
    __syncthreads();
    if (excl < (uint32_t)k && incl >= (uint32_t)k) {
        uint32_t cum = excl;
        for (int i = 15; i >= 0; --i) {
            if (cum + c[i] >= (uint32_t)k) {
                sh_scan[0] = (uint32_t)(hi - 16 + i);
                sh_scan[1] = cum;
                break;
            }
            cum += c[i];
        }
    }
    __syncthreads();
    bucket = (int)sh_scan[0];
    above = sh_scan[1];
    __syncthreads();
}

// Appends `flag` lanes to a per-row list with one atomic per wavefront;
// returns this lane's slot (valid only where flag is set).
__device__ __forceinline__ uint32_t wave_append(bool flag, uint32_t* counter) {
    const unsigned long long mask = __ballot(flag);
    if (mask == 0ull) return 0u;
    const int lane = threadIdx.x & 63;
    const int leader = __ffsll((long long)mask) - 1;
    uint32_t base = 0u;
    if (lane == leader) base = atomicAdd(counter, (uint32_t)__popcll(mask));
    base = __shfl(base, leader);
    const unsigned long long below = lane ? (mask & ((1ull << lane) - 1ull)) : 0ull;
    return base + (uint32_t)__popcll(below);
}

__global__ __launch_bounds__(TK_THREADS) void topk_filter(TopkArgs a) {
    const Geometry& G = a.g;
    const int t = blockIdx.y;
    const int r = find_request(G.qsl, G.B, t);
    const int n = visible_count(G.ctx, G.qsl, r, t);
    if (n <= a.k) return;
    const int c0 = blockIdx.x * TK_CHUNK;
    if (c0 >= n) return;
    const int c1 = min(n, c0 + TK_CHUNK);
    __shared__ uint32_t sh_scan[TK_THREADS];
    int bucket;
    uint32_t above;
    find_threshold_bucket(a.hist + (size_t)t * HIST_BINS, a.k, sh_scan, bucket, above);
    TopkCounters* cnt = a.counters + t;
    if (blockIdx.x == 0 && threadIdx.x == 0) cnt->bucket = (uint32_t)bucket;
    const float* row = a.scores + (size_t)t * a.ld;
    int32_t* sel = a.indices + (size_t)t * a.k;
    int32_t* cand = a.cand + (size_t)t * TOPK_CAND_CAP;
    for (int base = c0; base < c1; base += TK_THREADS) {
        const int s = base + threadIdx.x;
        const bool valid = s < c1;
        const int b = valid ? (int)(score_key(row[s]) >> HIST_SHIFT) : -1;
        const bool is_sel = b > bucket, is_cand = b == bucket;
        const uint32_t ps = wave_append(is_sel, &cnt->above);
        if (is_sel && ps < (uint32_t)a.k) sel[ps] = s;
        const uint32_t pc = wave_append(is_cand, &cnt->cand);
        if (is_cand && pc < (uint32_t)TOPK_CAND_CAP) cand[pc] = s;
    }
}

// Composite selection key of a threshold-bucket token: the 20 key bits below
// the bucket bits, then the complemented index (so lower index ranks higher).
__device__ __forceinline__ uint64_t composite(uint32_t key, int s) {
    return ((uint64_t)(key & ((1u << HIST_SHIFT) - 1u)) << 32) | (uint64_t)(~(uint32_t)s);
}

__global__ __launch_bounds__(RF_THREADS) void topk_refine(TopkArgs a) {
    const Geometry& G = a.g;
    const int t = blockIdx.x;
    const int r = find_request(G.qsl, G.B, t);
    const int n = visible_count(G.ctx, G.qsl, r, t);
    const int K = a.k;
    int32_t* out = a.indices + (size_t)t * K;
    const int tid = threadIdx.x;
    if (n <= K) {      // dense: every visible token, in order
        for (int i = tid; i < K; i += RF_THREADS) out[i] = i < n ? i : -1;
        return;
    }
    __shared__ int32_t list[TOPK_MAX_K];
    __shared__ uint32_t h256[256];
    __shared__ uint32_t sh_state[4];
    const TopkCounters* cnt = a.counters + t;
    const uint32_t above = cnt->above, ncand = cnt->cand;
    const uint32_t bucket = cnt->bucket;
    const bool from_list = ncand <= (uint32_t)TOPK_CAND_CAP;
    const int32_t* cand = a.cand + (size_t)t * TOPK_CAND_CAP;
    const float* row = a.scores + (size_t)t * a.ld;
    const int scan_n = from_list ? (int)ncand : n;

    // MSB-first radix select: find the `need`-th largest composite key.
    uint32_t need = (uint32_t)K - above;
    uint64_t prefix = 0;
    int shift = 48;
    for (;; shift -= 8) {
        for (int i = tid; i < 256; i += RF_THREADS) h256[i] = 0u;
        __syncthreads();
        for (int i = tid; i < scan_n; i += RF_THREADS) {
            const int s = from_list ? cand[i] : i;
            const uint32_t key = score_key(row[s]);
            if (!from_list && (key >> HIST_SHIFT) != bucket) continue;
            const uint64_t ck = composite(key, s);
            if ((ck >> (shift + 8)) == prefix) atomicAdd(&h256[(ck >> shift) & 255u], 1u);
        }
        __syncthreads();
        if (tid == 0) {
            uint32_t cum = 0;
            int d = 255;
            for (; d > 0; --d) {
                if (cum + h256[d] >= need) break;
                cum += h256[d];
            }
            sh_state[0] = (uint32_t)d;
            sh_state[1] = need - cum;                 // still needed inside bucket d
            sh_state[2] = h256[d] == need - cum ? 1u : 0u;
        }
        __syncthreads();
        const uint32_t d = sh_state[0];
        need = sh_state[1];
        const bool done = sh_state[2] != 0u || shift == 0;
        prefix = (prefix << 8) | d;
        __syncthreads();
        if (done) break;
    }

    // Gather: filter's selections [0, above) plus the refined ones.
    for (int i = tid; i < (int)above; i += RF_THREADS) list[i] = out[i];
    if (tid == 0) sh_state[3] = 0u;
    __syncthreads();
    for (int i = tid; i < scan_n; i += RF_THREADS) {
        const int s = from_list ? cand[i] : i;
        const uint32_t key = score_key(row[s]);
        if (!from_list && (key >> HIST_SHIFT) != bucket) continue;
        if ((composite(key, s) >> shift) >= prefix) {
            const uint32_t p = atomicAdd(&sh_state[3], 1u);
            if (above + p < (uint32_t)K) list[above + p] = s;
        }
    }
    __syncthreads();

    // Ascending bitonic sort of the K indices (padded to a power of two).
    int P = 1;
    while (P < K) P <<= 1;
    for (int i = K + tid; i < P; i += RF_THREADS) list[i] = 0x7FFFFFFF;
    __syncthreads();
    for (int size = 2; size <= P; size <<= 1) {
        for (int stride = size >> 1; stride > 0; stride >>= 1) {
            for (int i = tid; i < P / 2; i += RF_THREADS) {
                const int lo = 2 * i - (i & (stride - 1));
                const int hi = lo + stride;
                const bool asc = (lo & size) == 0;
                const int x = list[lo], y = list[hi];
                if ((x > y) == asc) { list[lo] = y; list[hi] = x; }
            }
            __syncthreads();
        }
    }
    for (int i = tid; i < K; i += RF_THREADS) out[i] = list[i];
}

hipError_t launch_topk_hist(const TopkArgs& a, hipStream_t s) {
    dim3 grid((a.g.max_ctx + TK_CHUNK - 1) / TK_CHUNK, a.g.T);
    hipLaunchKernelGGL(topk_hist, grid, dim3(TK_THREADS), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_topk_select(const TopkArgs& a, hipStream_t s) {
    dim3 grid((a.g.max_ctx + TK_CHUNK - 1) / TK_CHUNK, a.g.T);
    hipLaunchKernelGGL(topk_filter, grid, dim3(TK_THREADS), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(topk_refine, dim3(a.g.T), dim3(RF_THREADS), 0, s, a);
    return hipGetLastError();
}

}  // namespace dsa
