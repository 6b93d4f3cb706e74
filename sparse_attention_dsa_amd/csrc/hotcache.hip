// Two-tier latent cache on gfx950: a bounded hot set of latent rows in HBM in
// front of the full history, which stays in pinned host memory (the HiSparse
// design: SemiAnalysis, "Sparse Savings, Persistent Demand: inside GLM-5.3",
// section "How Sparse Attention Affects DRAM/NAND Memory"; remio.ai, section
// "HiSparse Move o Histórico Completo para Fora da GPU" -- an LRU-like device
// cache that loads the tokens a top-K selection misses from host DRAM and
// evicts the least recently used ones).  The output of sparse MLA is unchanged:
// the selected rows are the same bytes, only their placement differs, and the
// MLA reads them through a token-granular slot table (page table with one
// token per block).
//
// Policy, per fetch (one step; the step counter lives on the device):
//  1. every selected token that is resident is a hit: its slot's last use
//     becomes this step;
//  2. the distinct selected tokens that are not resident are the misses,
//     listed in (request, token) order;
//  3. the victims are the M slots (M = number of misses) not used in this
//     step that were used least recently: a never-used slot ranks before any
//     used one, otherwise the earlier last use first, equal ranks to the
//     lower slot.  Ages are exact 32-bit step counts (never capped): the
//     M-th oldest age is found by a two-level selection, first over the high
//     16 bits of the ages, then over the low 16 bits within that bucket;
//  4. each miss moves into one victim (the misses in order take every victim
//     older than the M-th one in slot order, then those of its age in slot
//     order; which victim a miss takes does not change the resident set or
//     any slot's age): the victim's previous token loses its slot, the row
//     (and its e4m3 scale) is copied from host memory by the GPU (zero-copy
//     reads of pinned memory), and the slot's last use becomes this step.
// The capacity is at least T x K (every distinct selected token of a step
// fits), so there are always enough slots not used in the step.
#include "dsa_kernels.h"
#include "topk_dev.h"
#include "dsa.h"

#include <algorithm>

namespace dsa {

constexpr int HC_THREADS = 256;
constexpr int HC_WAVES = HC_THREADS / 64;
constexpr int HC_PER = 4;                         // items per thread in the scans
constexpr int HC_ITEMS = HC_THREADS * HC_PER;     // items per workgroup in the scans
constexpr int HC_AGE_BINS = 65536;             // one 16-bit half of an age
constexpr int HC_COARSE = 256;                 // coarse bins of a level: the half's top 8 bits
constexpr int HC_HIST_WORDS = 2 * (HC_AGE_BINS + HC_COARSE);

// scalars in the workspace: misses, slots older than a*, a*, how many of age
// a* are taken, evictions, this step, victims, the high half of a* and the
// count of slots whose high half is above it
enum { HS_MISSES = 0, HS_OLDER = 1, HS_AGE = 2, HS_NEED = 3, HS_EVICT = 4, HS_STEP = 5, HS_VICTIMS = 6,
       HS_HI = 7, HS_OLDER_HI = 8, HS_N = 16 };

struct HotArgs {
    Geometry g;
    int k;
    const int32_t* indices;
    int32_t* slot_of;        // [B][maxctx]
    int64_t* owner;          // [capacity]
    int32_t* last_use;       // [capacity]
    int32_t* clock;          // [1]
    int capacity, maxctx, wpr;
    uint32_t* scal;          // [HS_N]
    uint32_t* hist;          // [2][HC_AGE_BINS]: high halves, then low halves within one high bucket;
                             // then [2][HC_COARSE]: the same counts by the half's top 8 bits
    uint32_t* bitmap;        // [B][wpr]
    uint32_t* wsum;          // per-workgroup word sums, then offsets
    uint32_t* csum;          // per-workgroup (older, equal) counts, then offsets
    int64_t* miss;           // [T k]
    int32_t* victims;        // [T k]
    const uint8_t* host_kv;
    const float* host_scales;
    const int32_t* host_pt;  // the batch's page table (host cache layout)
    uint8_t* hot_kv;
    float* hot_scales;
    int row_bytes;
    int32_t* counts;         // [2] misses, evictions (or null)
};

// Age of a slot not used in this step: steps since its last use, minus one
// (0 for a slot used in the previous step); a never-used slot gets `step`,
// above every used slot's age (last uses are steps >= 1).
__device__ __forceinline__ uint32_t slot_age(int32_t lu, int step) {
    return lu < 0 ? (uint32_t)step : (uint32_t)(step - lu - 1);
}

// Clears the per-step scalars, age histogram and miss bitmap, and fixes this
// step's number (device clock + 1).
__global__ __launch_bounds__(HC_THREADS) void hc_clear(HotArgs a, int64_t nwords) {
    const int64_t i = (int64_t)blockIdx.x * HC_THREADS + threadIdx.x;
    if (i < HS_N) a.scal[i] = i == HS_STEP ? (uint32_t)(*a.clock + 1) : 0u;
    if (i < HC_HIST_WORDS) a.hist[i] = 0u;
    if (i < nwords) a.bitmap[i] = 0u;
}

// Hits stamp their slot; misses set their bit in the request's bitmap.
__global__ __launch_bounds__(HC_THREADS) void hc_mark(HotArgs a) {
    const int t = blockIdx.y, j = blockIdx.x * HC_THREADS + threadIdx.x;
    if (j >= a.k) return;
    const int s = a.indices[(size_t)t * a.k + j];
    if (s < 0 || s >= a.maxctx) return;
    const int r = row_request(a.g, t);
    const int slot = a.slot_of[(size_t)r * a.maxctx + s];
    if (slot >= 0 && slot < a.capacity) a.last_use[slot] = (int32_t)a.scal[HS_STEP];
    else atomicOr(&a.bitmap[(size_t)r * a.wpr + (s >> 5)], 1u << (s & 31));
}

// Per-workgroup population count of HC_ITEMS consecutive items (bitmap words,
// or (older, equal) slot flags).
__global__ __launch_bounds__(HC_THREADS) void hc_count_words(HotArgs a, int64_t nwords) {
    __shared__ uint32_t wsum[HC_WAVES];
    const int64_t w0 = (int64_t)blockIdx.x * HC_ITEMS + HC_PER * threadIdx.x;
    uint32_t c = 0;
#pragma unroll
    for (int u = 0; u < HC_PER; ++u)
        if (w0 + u < nwords) c += __popc(a.bitmap[w0 + u]);
    uint32_t tot;
    block_excl_scan<HC_WAVES>(c, wsum, &tot);
    if (threadIdx.x == 0) a.wsum[blockIdx.x] = tot;
}

__global__ __launch_bounds__(HC_THREADS) void hc_count_slots(HotArgs a) {
    __shared__ uint32_t wsum[HC_WAVES];
    const int step = (int)a.scal[HS_STEP];
    const uint32_t astar = a.scal[HS_AGE];
    const int64_t s0 = (int64_t)blockIdx.x * HC_ITEMS + HC_PER * threadIdx.x;
    uint32_t older = 0, equal = 0;
#pragma unroll
    for (int u = 0; u < HC_PER; ++u) {
        if (s0 + u >= a.capacity) break;
        const int32_t lu = a.last_use[s0 + u];
        if (lu == step) continue;
        const uint32_t age = slot_age(lu, step);
        older += age > astar;
        equal += age == astar;
    }
    uint32_t to, te;
    block_excl_scan<HC_WAVES>(older, wsum, &to);
    block_excl_scan<HC_WAVES>(equal, wsum, &te);
    if (threadIdx.x == 0) {
        a.csum[2 * blockIdx.x] = to;
        a.csum[2 * blockIdx.x + 1] = te;
    }
}

// One workgroup: exclusive prefix sums, in place, of `n` counts spaced by
// `stride` (components 0 .. stride-1 scanned independently); the totals go to
// out[0 .. stride-1].
__global__ __launch_bounds__(HC_THREADS) void hc_scan(uint32_t* v, int n, int stride, uint32_t* out) {
    __shared__ uint32_t wsum[HC_WAVES];
    for (int c = 0; c < stride; ++c) {
        uint32_t carry = 0;
        for (int base = 0; base < n; base += HC_THREADS) {
            const int i = base + threadIdx.x;
            const uint32_t x = i < n ? v[(size_t)i * stride + c] : 0u;
            uint32_t tot;
            const uint32_t ex = block_excl_scan<HC_WAVES>(x, wsum, &tot);
            if (i < n) v[(size_t)i * stride + c] = carry + ex;
            carry += tot;
        }
        if (threadIdx.x == 0) out[c] = carry;
    }
}

// The misses in (request, token) order.
__global__ __launch_bounds__(HC_THREADS) void hc_write_misses(HotArgs a, int64_t nwords) {
    __shared__ uint32_t wsum[HC_WAVES];
    const int64_t w0 = (int64_t)blockIdx.x * HC_ITEMS + HC_PER * threadIdx.x;
    uint32_t words[HC_PER], c = 0;
#pragma unroll
    for (int u = 0; u < HC_PER; ++u) {
        words[u] = w0 + u < nwords ? a.bitmap[w0 + u] : 0u;
        c += __popc(words[u]);
    }
    uint32_t tot;
    uint32_t pos = a.wsum[blockIdx.x] + block_excl_scan<HC_WAVES>(c, wsum, &tot);
#pragma unroll
    for (int u = 0; u < HC_PER; ++u) {
        uint32_t m = words[u];
        const int64_t w = w0 + u;
        const int r = (int)(w / a.wpr), sb = 32 * (int)(w % a.wpr);
        while (m) {
            const int b = __builtin_ctz(m);
            m &= m - 1;
            a.miss[pos++] = ((int64_t)r << 32) | (uint32_t)(sb + b);
        }
    }
}

// Age histogram of the slots not used in this step, one 16-bit half at a
// time.  Level 0 counts the high halves of all their ages; level 1 counts
// the low halves of the ages whose high half is scal[HS_HI].  The common
// bins (high half 0 at level 0; recent ages and the never-used age at level
// 1) are counted in LDS and flushed once per workgroup; the other ones go to
// the global histogram, one count per run of equal bins among a thread's
// HC_RUN slots.
constexpr int HC_RUN = 32;
constexpr int HC_COPY_WGS = 64;   // workgroups of the row copies
constexpr int HC_LDS_BINS = 4096;
__global__ __launch_bounds__(HC_THREADS) void hc_age_hist(HotArgs a, int level) {
    __shared__ uint32_t h[HC_LDS_BINS + 1];                   // last bin: the never-used age (level 1)
    __shared__ uint32_t hc[HC_COARSE];
    for (int i = threadIdx.x; i <= HC_LDS_BINS; i += HC_THREADS) h[i] = 0u;
    for (int i = threadIdx.x; i < HC_COARSE; i += HC_THREADS) hc[i] = 0u;
    __syncthreads();
    const int step = (int)a.scal[HS_STEP];
    const uint32_t hi = a.scal[HS_HI];
    const uint32_t never = (uint32_t)step;                    // age of a never-used slot
    const bool never_here = level == 1 && (never >> 16) == hi;
    uint32_t* gh = a.hist + (level ? HC_AGE_BINS : 0);
    // the workgroup covers HC_THREADS * HC_RUN consecutive slots; lane-
    // consecutive loads (coalesced), each thread HC_RUN slots HC_THREADS apart
    const int64_t s0 = (int64_t)blockIdx.x * HC_THREADS * HC_RUN + threadIdx.x;
    int cur = -1;
    uint32_t n = 0;
    for (int u = 0; u < HC_RUN; ++u) {
        const int64_t slot = s0 + (int64_t)u * HC_THREADS;
        bool elig = slot < a.capacity;
        uint32_t age = 0;
        if (elig) {
            const int32_t lu = a.last_use[slot];
            age = slot_age(lu, step);
            elig = lu != step && (level == 0 || (age >> 16) == hi);
        }
        const int bin = level ? (int)(age & 0xFFFFu) : (int)(age >> 16);
        const bool is_never = never_here && age == never;
        const bool in_lds = elig && (is_never || bin < HC_LDS_BINS);
        // one LDS atomic per wave when its lanes share the bin (the usual case)
        lds_count(h, is_never ? (uint32_t)HC_LDS_BINS : (uint32_t)min(bin, HC_LDS_BINS - 1), in_lds);
        lds_count(hc, (uint32_t)bin >> 8, elig);
        if (!elig || in_lds) continue;
        if (bin != cur) {
            if (n) atomicAdd(&gh[cur], n);
            cur = bin;
            n = 0;
        }
        ++n;
    }
    if (n) atomicAdd(&gh[cur], n);
    __syncthreads();
    for (int i = threadIdx.x; i < HC_LDS_BINS; i += HC_THREADS)
        if (h[i]) atomicAdd(&gh[i], h[i]);
    if (threadIdx.x == 0 && h[HC_LDS_BINS]) atomicAdd(&gh[never & 0xFFFFu], h[HC_LDS_BINS]);
    uint32_t* gc = a.hist + 2 * HC_AGE_BINS + (level ? HC_COARSE : 0);
    for (int i = threadIdx.x; i < HC_COARSE; i += HC_THREADS)
        if (hc[i]) atomicAdd(&gc[i], hc[i]);
}

// One workgroup, per level: the bucket holding the M-th oldest eligible slot
// (scanning from the oldest bucket down).  Level 0 records the high half and
// the count of slots in older high buckets; level 1 completes a* = (high <<
// 16) | low, the number of eligible slots older than a*, and how many of age
// a* are taken.
__global__ __launch_bounds__(HC_THREADS) void hc_pick(HotArgs a, int level) {
    static_assert(HC_THREADS == HC_COARSE && HC_AGE_BINS == 256 * HC_COARSE, "one coarse bin a thread");
    __shared__ uint32_t wsum[HC_WAVES];
    __shared__ uint32_t s_cb, s_cum;
    const uint32_t M = a.scal[HS_MISSES];
    const uint32_t* h = a.hist + (level ? HC_AGE_BINS : 0);
    const uint32_t* hcs = a.hist + 2 * HC_AGE_BINS + (level ? HC_COARSE : 0);
    const uint32_t base = level ? a.scal[HS_OLDER_HI] : 0u;
    if (threadIdx.x == 0) s_cb = 0xFFFFFFFFu;
    // coarse bins oldest first (thread i: coarse bin 255 - i), then the 256
    // bins of the one where the count reaches `want`
    const uint32_t c = hcs[HC_COARSE - 1 - threadIdx.x];
    uint32_t tot;
    const uint32_t ex = block_excl_scan<HC_WAVES>(c, wsum, &tot);
    if (level == 0 && threadIdx.x == 0) a.scal[HS_VICTIMS] = min(M, tot);
    const uint32_t want = min(M, level ? a.scal[HS_VICTIMS] : tot);   // fewer only if the capacity contract is broken
    if (want == 0u) {
        if (threadIdx.x == 0) {
            a.scal[HS_HI] = 0xFFFFu;
            a.scal[HS_AGE] = 0xFFFFFFFFu;   // no slot is that old
            a.scal[HS_OLDER] = 0u;
            a.scal[HS_NEED] = 0u;
        }
        return;
    }
    if (base + ex < want && base + ex + c >= want) {
        s_cb = HC_COARSE - 1 - threadIdx.x;
        s_cum = base + ex;
    }
    __syncthreads();
    const uint32_t cb = s_cb;
    if (cb >= (uint32_t)HC_COARSE) return;   // counts inconsistent with `want`: nothing chosen
    const uint32_t bin = 256u * cb + 255u - threadIdx.x;
    const uint32_t hb = h[bin];
    uint32_t tot2;
    const uint32_t cum = s_cum + block_excl_scan<HC_WAVES>(hb, wsum, &tot2);
    if (cum < want && cum + hb >= want) {
        if (level == 0) {
            a.scal[HS_HI] = bin;
            a.scal[HS_OLDER_HI] = cum;
        } else {
            a.scal[HS_AGE] = (a.scal[HS_HI] << 16) | bin;
            a.scal[HS_OLDER] = cum;
            a.scal[HS_NEED] = want - cum;
        }
    }
}

// The victims: every eligible slot older than a* (slot order), then the first
// `need` of age a* (slot order).
__global__ __launch_bounds__(HC_THREADS) void hc_write_victims(HotArgs a) {
    __shared__ uint32_t wsum[HC_WAVES];
    const int step = (int)a.scal[HS_STEP];
    const uint32_t astar = a.scal[HS_AGE];
    const uint32_t n_older = a.scal[HS_OLDER], need = a.scal[HS_NEED];
    const int64_t s0 = (int64_t)blockIdx.x * HC_ITEMS + HC_PER * threadIdx.x;
    uint32_t fo = 0, fe = 0;   // flag bits per item
#pragma unroll
    for (int u = 0; u < HC_PER; ++u) {
        if (s0 + u >= a.capacity) break;
        const int32_t lu = a.last_use[s0 + u];
        if (lu == step) continue;
        const uint32_t age = slot_age(lu, step);
        fo |= (age > astar ? 1u : 0u) << u;
        fe |= (age == astar ? 1u : 0u) << u;
    }
    uint32_t to, te;
    uint32_t po = a.csum[2 * blockIdx.x] + block_excl_scan<HC_WAVES>(__popc(fo), wsum, &to);
    uint32_t pe = a.csum[2 * blockIdx.x + 1] + block_excl_scan<HC_WAVES>(__popc(fe), wsum, &te);
#pragma unroll
    for (int u = 0; u < HC_PER; ++u) {
        if ((fo >> u) & 1u) a.victims[po++] = (int32_t)(s0 + u);
        if ((fe >> u) & 1u) {
            if (pe < need) a.victims[n_older + pe] = (int32_t)(s0 + u);
            ++pe;
        }
    }
}

// One row of up to 2 KB by one wave, every load issued before the first store
// (host reads are long round trips).
__device__ __forceinline__ void copy_row(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst, int bytes,
                                         int lane) {
    const int o0 = 16 * lane, o1 = 16 * (lane + 64);
    u32x4 v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
    if (o0 < bytes) v0 = *(const u32x4*)(src + o0);
    if (o1 < bytes) v1 = *(const u32x4*)(src + o1);
    if (o0 < bytes) *(u32x4*)(dst + o0) = v0;
    if (o1 < bytes) *(u32x4*)(dst + o1) = v1;
}

// Returns (in lane 0) whether the victim held a token.
__device__ __forceinline__ uint32_t hc_assign_one(const HotArgs& a, uint32_t i, int step, int lane) {
    const int64_t rs = a.miss[i];
    const int r = (int)(rs >> 32), s = (int)(rs & 0xFFFFFFFF);
    const int v = a.victims[i];
    uint32_t evicted = 0u;
    if (lane == 0) {
        const int64_t old = a.owner[v];
        if (old >= 0) {
            const int orq = (int)(old >> 32), osl = (int)(old & 0xFFFFFFFF);
            if (orq < a.g.B && osl < a.maxctx) a.slot_of[(size_t)orq * a.maxctx + osl] = -1;
            evicted = 1u;
        }
        a.owner[v] = rs;
        a.last_use[v] = step;
        a.slot_of[(size_t)r * a.maxctx + s] = v;
    }
    const int bs = a.g.block_size;
    const int64_t row = (int64_t)a.host_pt[(size_t)r * a.g.max_blocks + s / bs] * bs + s % bs;
    copy_row(a.host_kv + row * a.row_bytes, a.hot_kv + (int64_t)v * a.row_bytes, a.row_bytes, lane);
    if (a.hot_scales && lane == 0) a.hot_scales[v] = a.host_scales[row];
    return evicted;
}

// Per miss, one wave: evict the victim's token, claim the slot, copy the row
// (and scale) from host memory.  A fixed number of workgroups (HC_COPY_WGS)
// takes the misses in turn: enough rows in flight for the host link, while
// the other compute units stay free for kernels that run beside the copy
// (the next layer's attention).
__global__ __launch_bounds__(HC_THREADS) void hc_assign(HotArgs a) {
    const int lane = threadIdx.x & 63;
    const uint32_t M = a.scal[HS_MISSES], nv = a.scal[HS_VICTIMS];
    const int step = (int)a.scal[HS_STEP];
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        *a.clock = step;
        if (a.counts) a.counts[0] = (int32_t)M;
    }
    const uint32_t n = min(M, nv), nw = gridDim.x * HC_WAVES;
    uint32_t evicted = 0u;   // counted per wave, added once: thousands of misses, one counter
    for (uint32_t i = blockIdx.x * HC_WAVES + (threadIdx.x >> 6); i < n; i += nw)
        evicted += hc_assign_one(a, i, step, lane);
    if (lane == 0 && evicted) atomicAdd(&a.scal[HS_EVICT], evicted);
}

__global__ void hc_finish(HotArgs a) {
    if (a.counts) a.counts[1] = (int32_t)a.scal[HS_EVICT];
}

// Resets a hot cache to empty: no token resident, no slot used, clock 0.
__global__ __launch_bounds__(HC_THREADS) void hc_reset(int32_t* slot_of, int64_t n_map, int64_t* owner,
                                                       int32_t* last_use, int capacity, int32_t* clock) {
    const int64_t i = (int64_t)blockIdx.x * HC_THREADS + threadIdx.x;
    if (i < n_map) slot_of[i] = -1;
    if (i < capacity) { owner[i] = -1; last_use[i] = -1; }
    if (i == 0) *clock = 0;
}

struct HotLayout {
    size_t scal, hist, bitmap, wsum, csum, miss, victims, end;
    int64_t nwords;
    int nwg_words, nwg_slots;
};

HotLayout hot_layout(const dsa_batch* b, int k, int capacity) {
    HotLayout l;
    const int wpr = (b->max_context_len + 31) / 32;
    l.nwords = (int64_t)b->num_requests * wpr;
    l.nwg_words = (int)((l.nwords + HC_ITEMS - 1) / HC_ITEMS);
    l.nwg_slots = (capacity + HC_ITEMS - 1) / HC_ITEMS;
    auto al = [](size_t x) { return (x + 255) / 256 * 256; };
    l.scal = 0;
    l.hist = al(l.scal + sizeof(uint32_t) * HS_N);
    l.bitmap = l.hist + sizeof(uint32_t) * HC_HIST_WORDS;   // contiguous with hist: one clear
    l.wsum = al(l.bitmap + sizeof(uint32_t) * (size_t)l.nwords);
    l.csum = al(l.wsum + sizeof(uint32_t) * ((size_t)l.nwg_words + 1));
    l.miss = al(l.csum + sizeof(uint32_t) * (2 * (size_t)l.nwg_slots + 2));
    l.victims = al(l.miss + sizeof(int64_t) * (size_t)b->total_q * k);
    l.end = al(l.victims + sizeof(int32_t) * (size_t)b->total_q * k);
    return l;
}

}  // namespace dsa

namespace {

bool hot_ok(const dsa_hot_cache* h) {
    return h && h->kv && h->slot_of && h->owner && h->last_use && h->clock && h->capacity >= 1;
}

int latent_row_bytes(const dsa_latent_cache* c) {
    const int W = c->d_latent + c->d_rope;
    return c->dtype == DSA_F32 ? 4 * W : c->dtype == DSA_BF16 ? 2 * W : W;
}

}  // namespace

extern "C" {

size_t dsa_hot_cache_workspace_size(const dsa_batch* batch, int32_t k, int32_t capacity) {
    if (!batch || batch->num_requests < 1 || batch->total_q < 1 || batch->max_context_len < 1 || k < 1 ||
        capacity < 1)
        return 0;
    return dsa::hot_layout(batch, k, capacity).end;
}

int dsa_hot_cache_reset(const dsa_batch* batch, dsa_hot_cache* hot, dsa_stream_t stream) {
    if (!batch || batch->num_requests < 1 || batch->max_context_len < 1 || !hot_ok(hot)) return DSA_ERR_INVALID_ARG;
    if (const int st = dsa_check_device(); st != DSA_OK) return st;
    const int64_t n_map = (int64_t)batch->num_requests * batch->max_context_len;
    const int64_t n = std::max<int64_t>(n_map, hot->capacity);
    hipLaunchKernelGGL(dsa::hc_reset, dim3((unsigned)((n + dsa::HC_THREADS - 1) / dsa::HC_THREADS)),
                       dim3(dsa::HC_THREADS), 0, (hipStream_t)stream, hot->slot_of, n_map, hot->owner, hot->last_use,
                       hot->capacity, hot->clock);
    return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH;
}

// Phases of a fetch: the plan (hits, misses, victims) and the copy (misses
// into victims, rows from host memory, clock and counts).
enum { HOT_PLAN = 1, HOT_COPY = 2 };

static int hot_cache_run(const dsa_batch* b, const dsa_latent_cache* host, const int32_t* indices, int32_t k,
                         dsa_hot_cache* hot, int32_t* counts, void* workspace, size_t workspace_bytes,
                         dsa_stream_t stream, int phases) {
    using namespace dsa;
    if (!b || b->num_requests < 1 || b->total_q < 1 || b->max_q_len < 1 || b->max_context_len < 1 ||
        !b->context_lens || !b->query_start_loc || !b->page_table || b->block_size < 1 || b->max_blocks < 1 ||
        (int64_t)b->max_blocks * b->block_size < b->max_context_len || !host || !host->kv || !indices || k < 1 ||
        !hot_ok(hot))
        return DSA_ERR_INVALID_ARG;
    if (!(host->dtype == DSA_F32 || host->dtype == DSA_BF16 || host->dtype == DSA_E4M3) || host->d_latent < 1 ||
        host->d_rope < 0 || (host->dtype == DSA_E4M3) != (host->scales != nullptr) ||
        (host->dtype == DSA_E4M3) != (hot->scales != nullptr))
        return DSA_ERR_UNSUPPORTED;
    const int row_bytes = latent_row_bytes(host);
    if (row_bytes % 16 || row_bytes > 2048) return DSA_ERR_UNSUPPORTED;
    if ((int64_t)hot->capacity < (int64_t)b->total_q * k) return DSA_ERR_INVALID_ARG;
    const HotLayout l = hot_layout(b, k, hot->capacity);
    if (!workspace || workspace_bytes < l.end) return DSA_ERR_WORKSPACE;
    if (const int st = dsa_check_device(); st != DSA_OK) return st;

    uint8_t* base = (uint8_t*)workspace;
    HotArgs a;
    a.g.B = b->num_requests;
    a.g.T = b->total_q;
    a.g.max_q_len = b->max_q_len;
    a.g.max_ctx = b->max_context_len;
    a.g.q_uniform = (int64_t)b->total_q == (int64_t)b->num_requests * b->max_q_len ? b->max_q_len : 0;
    a.g.ctx = b->context_lens;
    a.g.qsl = b->query_start_loc;
    a.g.page_table = b->page_table;
    a.g.max_blocks = b->max_blocks;
    a.g.block_size = b->block_size;
    a.k = k;
    a.indices = indices;
    a.slot_of = hot->slot_of;
    a.owner = hot->owner;
    a.last_use = hot->last_use;
    a.clock = hot->clock;
    a.capacity = hot->capacity;
    a.maxctx = b->max_context_len;
    a.wpr = (b->max_context_len + 31) / 32;
    a.scal = (uint32_t*)(base + l.scal);
    a.hist = (uint32_t*)(base + l.hist);
    a.bitmap = (uint32_t*)(base + l.bitmap);
    a.wsum = (uint32_t*)(base + l.wsum);
    a.csum = (uint32_t*)(base + l.csum);
    a.miss = (int64_t*)(base + l.miss);
    a.victims = (int32_t*)(base + l.victims);
    a.host_kv = (const uint8_t*)host->kv;
    a.host_scales = host->scales;
    a.host_pt = b->page_table;
    a.hot_kv = (uint8_t*)hot->kv;
    a.hot_scales = hot->scales;
    a.row_bytes = row_bytes;
    a.counts = counts;

    hipStream_t s = (hipStream_t)stream;
    const bool dbg = debug_mode();
    if (dbg && (phases & HOT_PLAN)) {
        if (const int st = run_batch_check(a.g, host->num_blocks, true, indices, k, nullptr, s); st != DSA_OK)
            return st;
    }
    if (phases & HOT_PLAN) {
    const int64_t nclear = std::max<int64_t>(HC_HIST_WORDS, l.nwords);
    hipLaunchKernelGGL(hc_clear, dim3((unsigned)((nclear + HC_THREADS - 1) / HC_THREADS)), dim3(HC_THREADS), 0, s, a,
                       l.nwords);
    hipLaunchKernelGGL(hc_mark, dim3((k + HC_THREADS - 1) / HC_THREADS, b->total_q), dim3(HC_THREADS), 0, s, a);
    hipLaunchKernelGGL(hc_count_words, dim3(l.nwg_words), dim3(HC_THREADS), 0, s, a, l.nwords);
    hipLaunchKernelGGL(hc_scan, dim3(1), dim3(HC_THREADS), 0, s, a.wsum, l.nwg_words, 1, a.scal + HS_MISSES);
    hipLaunchKernelGGL(hc_write_misses, dim3(l.nwg_words), dim3(HC_THREADS), 0, s, a, l.nwords);
    const int64_t runs = ((int64_t)hot->capacity + HC_RUN - 1) / HC_RUN;
    const dim3 hgrid((unsigned)((runs + HC_THREADS - 1) / HC_THREADS));
    for (int level = 0; level < 2; ++level) {
        hipLaunchKernelGGL(hc_age_hist, hgrid, dim3(HC_THREADS), 0, s, a, level);
        hipLaunchKernelGGL(hc_pick, dim3(1), dim3(HC_THREADS), 0, s, a, level);
    }
    hipLaunchKernelGGL(hc_count_slots, dim3(l.nwg_slots), dim3(HC_THREADS), 0, s, a);
    hipLaunchKernelGGL(hc_scan, dim3(1), dim3(HC_THREADS), 0, s, a.csum, l.nwg_slots, 2,
                       a.csum + 2 * (size_t)l.nwg_slots);
    hipLaunchKernelGGL(hc_write_victims, dim3(l.nwg_slots), dim3(HC_THREADS), 0, s, a);
    }
    if (phases & HOT_COPY) {
        const int64_t tk = (int64_t)b->total_q * k;
        hipLaunchKernelGGL(hc_assign, dim3((unsigned)std::min<int64_t>(HC_COPY_WGS, (tk + HC_WAVES - 1) / HC_WAVES)),
                           dim3(HC_THREADS), 0, s, a);
        hipLaunchKernelGGL(hc_finish, dim3(1), dim3(1), 0, s, a);
    }
    return debug_finish(dbg, hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH, s);
}

int dsa_hot_cache_fetch(const dsa_batch* b, const dsa_latent_cache* host, const int32_t* indices, int32_t k,
                        dsa_hot_cache* hot, int32_t* counts, void* workspace, size_t workspace_bytes,
                        dsa_stream_t stream) {
    return hot_cache_run(b, host, indices, k, hot, counts, workspace, workspace_bytes, stream, HOT_PLAN | HOT_COPY);
}

int dsa_hot_cache_plan(const dsa_batch* b, const dsa_latent_cache* host, const int32_t* indices, int32_t k,
                       dsa_hot_cache* hot, void* workspace, size_t workspace_bytes, dsa_stream_t stream) {
    return hot_cache_run(b, host, indices, k, hot, nullptr, workspace, workspace_bytes, stream, HOT_PLAN);
}

int dsa_hot_cache_copy(const dsa_batch* b, const dsa_latent_cache* host, const int32_t* indices, int32_t k,
                       dsa_hot_cache* hot, int32_t* counts, void* workspace, size_t workspace_bytes,
                       dsa_stream_t stream) {
    return hot_cache_run(b, host, indices, k, hot, counts, workspace, workspace_bytes, stream, HOT_COPY);
}

}  // extern "C"
