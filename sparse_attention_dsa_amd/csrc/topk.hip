// Top-K token selection on gfx950 without a global sort.
//
// Rule (SemiAnalysis GLM-5.3 article, "Lightning Indexer"): keep the K
// highest-scoring visible tokens, or every visible token when a query sees K
// or fewer; equal scores go to the lower token index.
//
// Scores are ranked by an order-preserving 32-bit key; the composite key
// (score key, then the complemented token index) is unique per token and puts
// the lower index first among equal scores, so "the K largest composite keys"
// is exactly the selection the rule asks for.
//
// Two kernels, one streaming pass over the scores:
//   candidate pass   rows longer than SEL_LIST are cut into TOPK_CHUNK-score
//                    chunks, one 256-thread workgroup each.  Every workgroup of
//                    a row draws the same strided sample of the row and takes a
//                    key bound X that, for any ordering that is not adversarial
//                    to the stride, has well over K scores of the row above it
//                    (the sample rank sits six binomial standard deviations
//                    past the expected rank of the K-th score).  It then writes
//                    its chunk's bitmap of "score >= X" as whole words, one
//                    ballot per 64 scores: one compare per score, no atomics.
//   selection        one 1024-thread workgroup per row compacts the bitmap into
//                    an LDS list of composite keys in ascending token order
//                    (short rows load all their scores instead).  If the list
//                    holds at least K entries it contains the whole top K; the
//                    K-th largest composite T* is found with a histogram over
//                    buckets spread across the list's key range, then an exact
//                    pass over the threshold bucket.  The entries >= T* are
//                    written out in list order.  When the sample bound fails
//                    (fewer than K candidates, or more than the list holds) the
//                    same selection runs over the whole row from memory.
#include "dsa_kernels.h"

namespace dsa {

constexpr int TK_THREADS = 256;                        // candidate pass
constexpr int TK_PER_LANE = TOPK_CHUNK / TK_THREADS;   // scores per lane
constexpr int TK_WAVE_SPAN = 64 * TK_PER_LANE;         // contiguous scores per wave
constexpr int TK_SAMPLE = 1024;                        // sample per 128K scores of row
constexpr int TK_SAMPLE_MAX = 4096;
constexpr int TK_SAMPLE_BINS = 256;
static_assert(TK_PER_LANE == 32, "each lane ends up holding one bitmap word of its wave");

constexpr int SEL_THREADS = 1024;                      // selection
constexpr int SEL_WAVES = SEL_THREADS / 64;
constexpr int SEL_LIST = 12288;                        // candidates held in LDS
constexpr int SEL_BINS = 4096;
constexpr int SEL_MEMBERS = 4096;                      // threshold-bucket members sorted directly
static_assert(SEL_LIST > TOPK_MAX_K, "short rows go straight to the list");
static_assert(SEL_BINS == 4 * SEL_THREADS, "four buckets per thread in the threshold scan");

// Order-preserving map's inverse for ">=" tests on floats: for finite v,
// score_key(v) >= x  <=>  v >= key_floor(x)  (x a key of a finite float or
// the unused key below +0; keys at or below that of -inf admit everything).
__device__ __forceinline__ float key_floor(uint32_t x) {
    if (x <= 0x007FFFFFu) return -__builtin_inff();
    if (x >= 0x80000000u) return __uint_as_float(x & 0x7FFFFFFFu);
    return __uint_as_float(~x);
}

__device__ __forceinline__ uint64_t composite(uint32_t key, int s) {
    return ((uint64_t)key << 32) | (uint64_t)(~(uint32_t)s);
}
__device__ __forceinline__ int composite_index(uint64_t ck) { return (int)(~(uint32_t)(ck & 0xFFFFFFFFull)); }
__device__ __forceinline__ uint32_t composite_key(uint64_t ck) { return (uint32_t)(ck >> 32); }

// Bucket of key x in a map of `bins` buckets starting at lo, 2^shift keys
// wide; keys outside clamp to the end buckets (monotonic in x).
__device__ __forceinline__ uint32_t bucket_of(uint32_t x, uint32_t lo, uint32_t shift, uint32_t bins) {
    if (x <= lo) return 0u;
    const uint32_t b = (x - lo) >> shift;
    return b < bins ? b : bins - 1u;
}
__device__ __forceinline__ uint32_t range_shift(uint32_t lo, uint32_t hi, uint32_t bins) {
    uint32_t sh = 0;
    while (((hi - lo) >> sh) >= bins) ++sh;
    return sh;
}

// Exclusive prefix sum over the 64 lanes of a wave; *total gets the wave sum.
__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t v, uint32_t* total) {
    const int lane = threadIdx.x & 63;
    uint32_t x = v;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
        const uint32_t y = __shfl_up(x, off);
        if (lane >= off) x += y;
    }
    *total = __shfl(x, 63);
    return x - v;
}

// Exclusive prefix sum over the workgroup (wsum: one slot per wave).
template <int WAVES>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t wt;
    const uint32_t wex = wave_excl_scan(v, &wt);
    if (lane == 0) wsum[wave] = wt;
    __syncthreads();
    uint32_t ex = wex, tot = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
        const uint32_t x = wsum[w];
        ex += w < wave ? x : 0u;
        tot += x;
    }
    __syncthreads();
    *total = tot;
    return ex;
}

// LDS counter increment; one atomic per wave when all active lanes share the
// bucket (rows of equal scores would otherwise serialize on one address).
__device__ __forceinline__ void lds_count(uint32_t* h, uint32_t bin, bool active) {
    const unsigned long long act = __ballot(active);
    if (act == 0ull) return;
    const int lane = threadIdx.x & 63;
    const int first = __ffsll((long long)act) - 1;
    const uint32_t b0 = (uint32_t)__shfl((int)bin, first);
    if (__ballot(active && bin == b0) == act) {
        if (lane == first) atomicAdd(&h[b0], (uint32_t)__popcll(act));
    } else if (active) {
        atomicAdd(&h[bin], 1u);
    }
}

// ---------------------------------------------------------------------------
// Candidate pass.
__global__ __launch_bounds__(TK_THREADS) void topk_candidates(TopkArgs a) {
    const int t = blockIdx.x, c = blockIdx.y;
    const int n = row_visible(a.g, t);
    const int c0 = c * TOPK_CHUNK;
    if (n <= SEL_LIST || c0 >= n) return;
    const int K = a.k;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const float* row = a.scores + (size_t)t * a.ld;
    __shared__ uint32_t h[TK_SAMPLE_BINS];
    __shared__ uint32_t red[2][TK_THREADS / 64];
    __shared__ uint32_t bound;

    // the row's sample (identical in every chunk of the row), then the chunk;
    // positions past the row read as NaN, which fails every ">=" test
    const int m = TK_SAMPLE * min(TK_SAMPLE_MAX / TK_SAMPLE, (n + 131071) / 131072);
    const int ns = m / TK_THREADS;
    float smp[TK_SAMPLE_MAX / TK_THREADS];
#pragma unroll
    for (int i = 0; i < TK_SAMPLE_MAX / TK_THREADS; ++i)
        if (i < ns) smp[i] = row[(int)((long long)(tid + i * TK_THREADS) * n / m)];
    const int w0 = c0 + wave * TK_WAVE_SPAN;
    float v[TK_PER_LANE];
#pragma unroll
    for (int j = 0; j < TK_PER_LANE; ++j) {
        const int s = w0 + j * 64 + lane;
        v[j] = s < n ? row[s] : __builtin_nanf("");
    }
    h[tid] = 0u;
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
#pragma unroll
    for (int i = 0; i < TK_SAMPLE_MAX / TK_THREADS; ++i)
        if (i < ns) {
            const uint32_t k = score_key(smp[i]);
            mn = min(mn, k);
            mx = max(mx, k);
        }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        mn = min(mn, (uint32_t)__shfl_xor((int)mn, off));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
    }
    if (lane == 0) { red[0][wave] = mn; red[1][wave] = mx; }
    __syncthreads();
    uint32_t lo = red[0][0], hi = red[1][0];
#pragma unroll
    for (int w = 1; w < TK_THREADS / 64; ++w) { lo = min(lo, red[0][w]); hi = max(hi, red[1][w]); }
    const uint32_t sh = range_shift(lo, hi, TK_SAMPLE_BINS);
#pragma unroll
    for (int i = 0; i < TK_SAMPLE_MAX / TK_THREADS; ++i)
        if (i < ns) atomicAdd(&h[bucket_of(score_key(smp[i]), lo, sh, TK_SAMPLE_BINS)], 1u);
    __syncthreads();
    // Sample rank r: the expected rank of the K-th score plus six standard
    // deviations of a binomial count, plus a margin.  X = lower key bound of the
    // highest bucket whose cumulative count (from the top) reaches r.
    if (wave == 0) {
        const float q = (float)K / (float)n, mq = (float)m * q;
        const uint32_t r = (uint32_t)ceilf(mq + 6.f * sqrtf(mq * (1.f - q))) + 8u;
        uint32_t c4[4], sum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) { c4[j] = h[TK_SAMPLE_BINS - 1 - 4 * lane - j]; sum += c4[j]; }
        uint32_t tot;
        const uint32_t ex = wave_excl_scan(sum, &tot);
        if (lane == 0 && tot < r) bound = 0u;   // the sample never reaches r: take everything
        if (ex < r && ex + sum >= r) {
            uint32_t cum = ex;
            for (int j = 0; j < 4; ++j) {
                cum += c4[j];
                if (cum >= r) {
                    const uint32_t b = (uint32_t)(TK_SAMPLE_BINS - 1 - 4 * lane - j);
                    bound = b == 0u ? 0u : lo + (b << sh);
                    break;
                }
            }
        }
    }
    __syncthreads();
    const float xf = key_floor(bound);

    // Step j covers scores w0 + 64j .. +63: bitmap words 2j and 2j+1 of this
    // wave, which end up in lanes 2j and 2j+1.
    uint32_t word = 0u;
#pragma unroll
    for (int j = 0; j < TK_PER_LANE; ++j) {
        const unsigned long long mk = __ballot(v[j] >= xf);
        if (lane == 2 * j) word = (uint32_t)mk;
        if (lane == 2 * j + 1) word = (uint32_t)(mk >> 32);
    }
    if (w0 + 32 * lane < n) a.bitmap[(size_t)t * a.bitmap_ld + (w0 >> 5) + lane] = word;
}

// ---------------------------------------------------------------------------
// Selection.
struct SelShared {
    uint64_t list[SEL_LIST];
    union {
        uint32_t hist[SEL_BINS];
        uint64_t members[SEL_MEMBERS];
    } r;
    uint32_t wsum[SEL_WAVES];
    uint32_t red[2][SEL_WAVES];
    uint32_t st[8];
};

// The K-th largest composite key over source entries i < count (get(i, ck)
// fetches entry i); count >= K.  Called by the whole workgroup.
template <class Get>
__device__ uint64_t kth_composite(int count, uint32_t K, const Get& get, SelShared& S) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // 1. key range of the entries
    uint32_t mn = 0xFFFFFFFFu, mx = 0u;
    for (int i = tid; i < count; i += SEL_THREADS) {
        const uint32_t k = composite_key(get(i));
        mn = min(mn, k);
        mx = max(mx, k);
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        mn = min(mn, (uint32_t)__shfl_xor((int)mn, off));
        mx = max(mx, (uint32_t)__shfl_xor((int)mx, off));
    }
    if (lane == 0) { S.red[0][wave] = mn; S.red[1][wave] = mx; }
    for (int i = tid; i < SEL_BINS; i += SEL_THREADS) S.r.hist[i] = 0u;
    __syncthreads();
    uint32_t lo = S.red[0][0], hi = S.red[1][0];
#pragma unroll
    for (int w = 1; w < SEL_WAVES; ++w) { lo = min(lo, S.red[0][w]); hi = max(hi, S.red[1][w]); }
    const uint32_t sh = range_shift(lo, hi, SEL_BINS);

    // 2. histogram over SEL_BINS buckets spread across [lo, hi]
    for (int base = 0; base < count; base += SEL_THREADS) {
        const int i = base + tid;
        const bool ok = i < count;
        const uint32_t b = ok ? bucket_of(composite_key(get(i)), lo, sh, SEL_BINS) : 0u;
        lds_count(S.r.hist, b, ok);
    }
    __syncthreads();

    // 3. threshold bucket b*: count(> b*) < K <= count(>= b*); thread i owns
    // buckets 4095-4i .. 4092-4i
    uint32_t c4[4], sum = 0;
#pragma unroll
    for (int j = 0; j < 4; ++j) { c4[j] = S.r.hist[SEL_BINS - 1 - 4 * tid - j]; sum += c4[j]; }
    uint32_t tot;
    const uint32_t ex = block_excl_scan<SEL_WAVES>(sum, S.wsum, &tot);
    if (ex < K && ex + sum >= K) {
        uint32_t cum = ex;
        for (int j = 0; j < 4; ++j) {
            if (cum + c4[j] >= K) {
                S.st[0] = (uint32_t)(SEL_BINS - 1 - 4 * tid - j);
                S.st[1] = cum;
                S.st[2] = c4[j];
                break;
            }
            cum += c4[j];
        }
    }
    if (tid == 0) S.st[3] = 0u;
    __syncthreads();
    const uint32_t bstar = S.st[0], need = K - S.st[1], nb = S.st[2];
    __syncthreads();   // the histogram space is reused below

    if (nb <= (uint32_t)SEL_MEMBERS) {
        // 4a. the threshold bucket's members: descending bitonic sort
        for (int base = 0; base < count; base += SEL_THREADS) {
            const int i = base + tid;
            uint64_t ck = 0;
            bool mem = false;
            if (i < count) {
                ck = get(i);
                mem = bucket_of(composite_key(ck), lo, sh, SEL_BINS) == bstar;
            }
            const unsigned long long mk = __ballot(mem);
            if (mk) {
                const int first = __ffsll((long long)mk) - 1;
                uint32_t pos = 0;
                if (lane == first) pos = atomicAdd(&S.st[3], (uint32_t)__popcll(mk));
                const unsigned long long below = lane ? (mk & ((1ull << lane) - 1ull)) : 0ull;
                pos = (uint32_t)__shfl((int)pos, first) + (uint32_t)__popcll(below);
                if (mem) S.r.members[pos] = ck;
            }
        }
        __syncthreads();
        int P = 1;
        while (P < (int)nb) P <<= 1;
        for (int i = (int)nb + tid; i < P; i += SEL_THREADS) S.r.members[i] = 0ull;   // sorts last
        __syncthreads();
        for (int size = 2; size <= P; size <<= 1) {
            for (int stride = size >> 1; stride > 0; stride >>= 1) {
                for (int i = tid; i < P / 2; i += SEL_THREADS) {
                    const int l0 = 2 * i - (i & (stride - 1));
                    const int l1 = l0 + stride;
                    const bool desc = (l0 & size) == 0;
                    const uint64_t x = S.r.members[l0], y = S.r.members[l1];
                    if ((x < y) == desc) { S.r.members[l0] = y; S.r.members[l1] = x; }
                }
                __syncthreads();
            }
        }
        const uint64_t kth = S.r.members[need - 1];
        __syncthreads();
        return kth;
    }

    // 4b. many ties: MSB-first radix select of the need-th largest member
    // composite, 8 bits at a time (unique keys: settled by the last digit)
    uint32_t* h256 = S.r.hist;
    uint32_t rem = need;
    uint64_t prefix = 0;
    for (int d = 56; d >= 0; d -= 8) {
        if (tid < 256) h256[tid] = 0u;
        __syncthreads();
        for (int base = 0; base < count; base += SEL_THREADS) {
            const int i = base + tid;
            uint64_t ck = 0;
            bool ok = false;
            if (i < count) {
                ck = get(i);
                ok = bucket_of(composite_key(ck), lo, sh, SEL_BINS) == bstar &&
                     (d == 56 || (ck >> (d + 8)) == prefix);
            }
            lds_count(h256, (uint32_t)(ck >> d) & 255u, ok);
        }
        __syncthreads();
        if (wave == 0) {
            uint32_t cc[4], s4 = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) { cc[j] = h256[255 - 4 * lane - j]; s4 += cc[j]; }
            uint32_t t4;
            const uint32_t e4 = wave_excl_scan(s4, &t4);
            if (e4 < rem && e4 + s4 >= rem) {
                uint32_t cum = e4;
                for (int j = 0; j < 4; ++j) {
                    if (cum + cc[j] >= rem) { S.st[4] = (uint32_t)(255 - 4 * lane - j); S.st[5] = rem - cum; break; }
                    cum += cc[j];
                }
            }
        }
        __syncthreads();
        prefix = (prefix << 8) | S.st[4];
        rem = S.st[5];
        __syncthreads();
    }
    return prefix;
}

// Writes the source entries with composite >= kth, in source order (which is
// ascending token order); exactly K of them.
template <class Get>
__device__ void write_selected(int count, uint64_t kth, uint32_t K, const Get& get, int32_t* out, SelShared& S) {
    const int tid = threadIdx.x;
    const int per = (count + SEL_THREADS - 1) / SEL_THREADS;
    const int i0 = min(count, tid * per), i1 = min(count, i0 + per);
    uint32_t nsel = 0;
    for (int i = i0; i < i1; ++i) nsel += get(i) >= kth ? 1u : 0u;
    uint32_t tot;
    uint32_t pos = block_excl_scan<SEL_WAVES>(nsel, S.wsum, &tot);
    for (int i = i0; i < i1; ++i) {
        const uint64_t ck = get(i);
        if (ck >= kth) {
            if (pos < K) out[pos] = composite_index(ck);
            ++pos;
        }
    }
}

__global__ __launch_bounds__(SEL_THREADS) void topk_select(TopkArgs a) {
    const int t = blockIdx.x;
    const int n = row_visible(a.g, t);
    const uint32_t K = (uint32_t)a.k;
    const int tid = threadIdx.x;
    int32_t* out = a.indices + (size_t)t * K;
    if (n <= (int)K) {   // every visible token, then -1 padding
        for (int i = tid; i < (int)K; i += SEL_THREADS) out[i] = i < n ? i : -1;
        return;
    }
    __shared__ SelShared S;
    const float* row = a.scores + (size_t)t * a.ld;
    int count = 0;
    if (n <= SEL_LIST) {
        for (int i = tid; i < n; i += SEL_THREADS) S.list[i] = composite(score_key(row[i]), i);
        count = n;
    } else {
        // compact the candidate bitmap: positions by a block scan of popcounts
        const uint32_t* bm = a.bitmap + (size_t)t * a.bitmap_ld;
        const int words = (n + 31) >> 5;
        const int per = (words + SEL_THREADS - 1) / SEL_THREADS;
        const int w0 = min(words, tid * per), w1 = min(words, w0 + per);
        uint32_t nb = 0;
        for (int w = w0; w < w1; ++w) nb += __popc(bm[w]);
        uint32_t tot;
        uint32_t pos = block_excl_scan<SEL_WAVES>(nb, S.wsum, &tot);
        count = (int)tot;
        if (count >= (int)K && count <= SEL_LIST) {
            for (int w = w0; w < w1; ++w) {
                uint32_t bits = bm[w];
                while (bits) {
                    const int b = __ffs(bits) - 1;
                    bits &= bits - 1u;
                    S.list[pos++] = (uint64_t)(w * 32 + b);
                }
            }
            __syncthreads();
            constexpr int G = SEL_LIST / SEL_THREADS;
            float sv[G];
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const int i = tid + j * SEL_THREADS;
                sv[j] = i < count ? row[(int)S.list[i]] : 0.f;
            }
#pragma unroll
            for (int j = 0; j < G; ++j) {
                const int i = tid + j * SEL_THREADS;
                if (i < count) S.list[i] = composite(score_key(sv[j]), (int)S.list[i]);
            }
        } else {
            count = -1;   // the sample bound failed for this row
        }
    }
    __syncthreads();
    if (count >= 0) {
        auto get = [&](int i) -> uint64_t { return S.list[i]; };
        const uint64_t kth = kth_composite(count, K, get, S);
        write_selected(count, kth, K, get, out, S);
    } else {
        auto get = [&](int i) -> uint64_t { return composite(score_key(row[i]), i); };
        const uint64_t kth = kth_composite(n, K, get, S);
        write_selected(n, kth, K, get, out, S);
    }
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
    if (a.g.max_ctx > SEL_LIST) {
        const dim3 grid(a.g.T, (a.g.max_ctx + TOPK_CHUNK - 1) / TOPK_CHUNK);
        hipLaunchKernelGGL(topk_candidates, grid, dim3(TK_THREADS), 0, s, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(topk_select, dim3(a.g.T), dim3(SEL_THREADS), 0, s, a);
    return hipGetLastError();
}

}  // namespace dsa
