// Device helpers of the top-K selection (gfx950): order-preserving keys,
// composite (key, ~index) ranks, DPP wave scans and reductions, LDS-only
// barriers, and the sample bound.
#pragma once

#include "dsa_kernels.h"

namespace dsa {

// Sample of a long row: TK_SAMPLE positions per 128K tokens, at most
// TK_SAMPLE_MAX, taken as m / 16 runs of 16 consecutive positions at evenly
// spaced starts (each kernel that draws one states its starts).
constexpr int TK_SAMPLE = 1024;
constexpr int TK_SAMPLE_MAX = 4096;
__device__ __forceinline__ int sample_size(int n) { return TK_SAMPLE * min(TK_SAMPLE_MAX / TK_SAMPLE, (n + 131071) / 131072); }

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

// ---------------------------------------------------------------- wave ops
// Cross-lane steps use DPP (row shifts within 16-lane rows, then row
// broadcasts), which run at ALU latency instead of through the LDS crossbar.
constexpr int DPP_ROW_SHR1 = 0x111, DPP_ROW_SHR2 = 0x112, DPP_ROW_SHR4 = 0x114, DPP_ROW_SHR8 = 0x118;
constexpr int DPP_ROW_BCAST15 = 0x142, DPP_ROW_BCAST31 = 0x143;

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    v += __builtin_amdgcn_update_dpp(0u, v, DPP_ROW_SHR1, 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0u, v, DPP_ROW_SHR2, 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0u, v, DPP_ROW_SHR4, 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0u, v, DPP_ROW_SHR8, 0xF, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0u, v, DPP_ROW_BCAST15, 0xA, 0xF, false);
    v += __builtin_amdgcn_update_dpp(0u, v, DPP_ROW_BCAST31, 0xC, 0xF, false);
    return v;
}

// Exclusive prefix sum over the wave; *total gets the wave sum.
__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t v, uint32_t* total) {
    const uint32_t inc = wave_incl_scan(v);
    *total = (uint32_t)__builtin_amdgcn_readlane((int)inc, 63);
    return inc - v;
}

// Wave-wide minimum and maximum (uniform results).  Lanes whose DPP source
// lies outside their row keep their own value.
__device__ __forceinline__ void wave_min_max(uint32_t& mn, uint32_t& mx) {
#define DSA_MINMAX_STEP(ctrl, rmask)                                                               \
    mn = min(mn, (uint32_t)__builtin_amdgcn_update_dpp((int)mn, (int)mn, ctrl, rmask, 0xF, false)); \
    mx = max(mx, (uint32_t)__builtin_amdgcn_update_dpp((int)mx, (int)mx, ctrl, rmask, 0xF, false));
    DSA_MINMAX_STEP(DPP_ROW_SHR1, 0xF)
    DSA_MINMAX_STEP(DPP_ROW_SHR2, 0xF)
    DSA_MINMAX_STEP(DPP_ROW_SHR4, 0xF)
    DSA_MINMAX_STEP(DPP_ROW_SHR8, 0xF)
    DSA_MINMAX_STEP(DPP_ROW_BCAST15, 0xA)
    DSA_MINMAX_STEP(DPP_ROW_BCAST31, 0xC)
#undef DSA_MINMAX_STEP
    mn = (uint32_t)__builtin_amdgcn_readlane((int)mn, 63);
    mx = (uint32_t)__builtin_amdgcn_readlane((int)mx, 63);
}

// Exclusive prefix sum over the workgroup (wsum: one slot per wave).
template <int WAVES>
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wsum, uint32_t* total) {
    const int tid = tid_x(), lane = tid & 63, wave = tid >> 6;
    uint32_t wt;
    const uint32_t wex = wave_excl_scan(v, &wt);
    if (lane == 0) wsum[wave] = wt;
    lds_barrier();
    uint32_t ex = wex, tot = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
        const uint32_t x = wsum[w];
        ex += w < wave ? x : 0u;
        tot += x;
    }
    lds_barrier();
    *total = tot;
    return ex;
}

// Workgroup-wide minimum and maximum (red: two slots per wave).
template <int WAVES>
__device__ __forceinline__ void block_min_max(uint32_t& mn, uint32_t& mx, uint32_t (*red)[WAVES]) {
    const int tid = tid_x(), lane = tid & 63, wave = tid >> 6;
    wave_min_max(mn, mx);
    if (lane == 0) { red[0][wave] = mn; red[1][wave] = mx; }
    lds_barrier();
    mn = red[0][0];
    mx = red[1][0];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) { mn = min(mn, red[0][w]); mx = max(mx, red[1][w]); }
    lds_barrier();
}

// LDS counter increment; one atomic per wave when all active lanes share the
// bucket (rows of equal scores would otherwise serialize on one address).
__device__ __forceinline__ void lds_count(uint32_t* h, uint32_t bin, bool active) {
    const unsigned long long act = __ballot(active);
    if (act == 0ull) return;
    const int lane = tid_x() & 63;
    const int first = __ffsll((long long)act) - 1;
    const uint32_t b0 = (uint32_t)__builtin_amdgcn_readlane((int)bin, first);
    if (__ballot(active && bin == b0) == act) {
        if (lane == first) atomicAdd(&h[b0], (uint32_t)__popcll(act));
    } else if (active) {
        atomicAdd(&h[bin], 1u);
    }
}

// Key bound of a row of n scores from m sampled keys (skeys[0..m), LDS):
// the lower key bound of the highest of 256 buckets (spread over the sample's
// key range) whose cumulative count from the top reaches the sample rank
// r = m q + 6 sqrt(m q (1-q)) + 8, q = K/n -- the expected sample rank of the
// K-th score plus six binomial standard deviations and a margin.  0 (take
// everything) when the sample never reaches r.  Called by the whole
// workgroup (THREADS threads); h: 256 LDS counters, red: 2 x THREADS/64.
template <int THREADS>
__device__ uint32_t sample_key_bound(const uint32_t* skeys, int m, int n, uint32_t K, uint32_t* h,
                                     uint32_t (*red)[THREADS / 64], uint32_t* result) {
    constexpr int WAVES = THREADS / 64;
    const int tid = tid_x(), lane = tid & 63, wave = tid >> 6;
    for (int i = tid; i < 256; i += THREADS) h[i] = 0u;
    uint32_t lo = 0xFFFFFFFFu, hi = 0u;
    for (int i = tid; i < m; i += THREADS) { lo = min(lo, skeys[i]); hi = max(hi, skeys[i]); }
    block_min_max<WAVES>(lo, hi, red);
    const uint32_t sh = range_shift(lo, hi, 256);
    for (int i = tid; i < m; i += THREADS) atomicAdd(&h[bucket_of(skeys[i], lo, sh, 256)], 1u);
    lds_barrier();
    if (wave == 0) {
        const float q = (float)K / (float)n, mq = (float)m * q;
        const uint32_t r = (uint32_t)ceilf(mq + 6.f * sqrtf(mq * (1.f - q))) + 8u;
        uint32_t c4[4], sum = 0;
#pragma unroll
        for (int j = 0; j < 4; ++j) { c4[j] = h[255 - 4 * lane - j]; sum += c4[j]; }
        uint32_t tot;
        const uint32_t ex = wave_excl_scan(sum, &tot);
        if (lane == 0 && tot < r) *result = 0u;
        if (ex < r && ex + sum >= r) {
            uint32_t cum = ex;
            for (int j = 0; j < 4; ++j) {
                cum += c4[j];
                if (cum >= r) {
                    const uint32_t b = (uint32_t)(255 - 4 * lane - j);
                    *result = b == 0u ? 0u : lo + (b << sh);
                    break;
                }
            }
        }
    }
    lds_barrier();
    return *result;
}

}  // namespace dsa
