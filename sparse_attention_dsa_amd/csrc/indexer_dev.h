// Lightning-indexer page scoring shared by the indexer kernels and the
// top-K selection's recompute path (gfx950).
//
// Score of visible token s for query row t (SemiAnalysis GLM-5.3 article,
// "Lightning Indexer"): I[t,s] = sigma_s * sum_h w[t,h] * ReLU(q[t,h,:] . k_s),
// with e4m3 keys and queries of dim 128, fp32 head weights and key scales.
// v_mfma_f32_16x16x128_f8f6f4 takes heads as the M dimension, tokens as the N
// dimension and the whole 128-wide key as the K dimension.  Lane l = 16g + col
// holds, for head (or token) col of a 16-wide tile, key bytes [16g, 16g+16)
// and [64+16g, 64+16g+16): queries and keys use the same byte assignment, so
// the permutation of k inside the instruction is consistent.
#pragma once

#include "dsa_kernels.h"

namespace dsa {

constexpr int IDX_D = 128;
constexpr int IDX_PAGE = 64;
constexpr int IDX_THREADS = 256;

// XOR permutation of the 16-byte units of token t inside an LDS key page
// (fragment reads of 16 tokens then hit distinct banks).
__device__ __forceinline__ int page_swz(int t) { return (t ^ (t >> 3)) & 7; }

// Staged page loads for the persistent kernel: fully contiguous loads (lane l
// reads bytes [1024c + 16l, +16) of the page, 1 KB per instruction, like a
// plain streaming read) into a register ring, then each page is re-laid
// through a private 8 KB LDS buffer of the wave into the MFMA fragment layout.
struct RawPage {
    u32x4 v[8];      // unit (lane & 7) of token 8c + (lane >> 3), c = 0..7
    float scale;     // scale of token (lane)
};

__device__ __forceinline__ void load_raw_page(const uint8_t* __restrict__ keys, const float* __restrict__ scales,
                                              int blk, bool live, int lane, RawPage& p) {
    // Buffer loads through a descriptor of the page (block id and liveness
    // are wave-uniform).  A slot past the wave's share still issues the same
    // instructions, so the ring's load counting stays exact, but its
    // descriptor holds no records: the range check returns zeros and nothing
    // is read from memory.
    const uint8_t* page = keys + (size_t)blk * (IDX_PAGE * IDX_D);
    const __amdgpu_buffer_rsrc_t rk =
        __builtin_amdgcn_make_buffer_rsrc((void*)page, 0, live ? IDX_PAGE * IDX_D : 0, 0x00020000);
#pragma unroll
    for (int c = 0; c < 8; ++c) p.v[c] = __builtin_amdgcn_raw_buffer_load_b128(rk, 16 * lane + 1024 * c, 0, 2);
    // without scales the load reads the page's own keys; the consumer then
    // uses 1 instead (the same instructions issue either way, and nothing
    // here waits for the load)
    const void* sp = scales ? (const void*)(scales + (size_t)blk * IDX_PAGE) : (const void*)page;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)sp, 0, live ? 4 * IDX_PAGE : 0, 0x00020000);
    p.scale = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, 4 * lane, 0, 0));
}


// part[nt] holds, for token 16*nt + (lane & 15), the partial head sum of this
// lane's 16-lane group g.  Returns the full sum for token `lane` of the page.
__device__ __forceinline__ float head_sum_transpose(const float part[4], int lane) {
    const int b1 = (lane >> 5) & 1, b0 = (lane >> 4) & 1;
    const float send0 = b1 ? part[0] : part[2];
    const float send1 = b1 ? part[1] : part[3];
    const float keep0 = b1 ? part[2] : part[0];
    const float keep1 = b1 ? part[3] : part[1];
    const float a0 = keep0 + lane_xor32(send0, lane);
    const float a1 = keep1 + lane_xor32(send1, lane);
    const float send = b0 ? a0 : a1;
    const float keep = b0 ? a1 : a0;
    return keep + lane_xor16(send, lane);
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
                if constexpr (NQ == 1) {
                    // the tile's MFMAs first (distinct results, issued back to
                    // back), then their weighted ReLU sum in the same order;
                    // two query rows keep one result at a time (registers)
                    f32x4 c[HT];
#pragma unroll
                    for (int ht = 0; ht < HT; ++ht) c[ht] = mfma_fp8_16x16x128(qf[j][ht], kf[nt], zero);
#pragma unroll
                    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc = fmaf(wv[j][ht][i], relu(c[ht][i]), acc);
                } else {
#pragma unroll
                    for (int ht = 0; ht < HT; ++ht) {
                        const f32x4 c = mfma_fp8_16x16x128(qf[j][ht], kf[nt], zero);
#pragma unroll
                        for (int i = 0; i < 4; ++i) acc = fmaf(wv[j][ht][i], relu(c[i]), acc);
                    }
                }
                part[nt] = acc;
            }
            out[j] = head_sum_transpose(part, lane) * ksc;
        } else {
            out[j] = 0.f;
        }
    }
}

// Query fragments and head weights of query row t (HT tiles of 16 heads).
template <int HT>
__device__ __forceinline__ void load_query(const IndexerArgs& a, int t, int lane, i32x8 (&qf)[HT],
                                           float (&wv)[HT][4]) {
    const int g = lane >> 4, col = lane & 15;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) {
        const uint8_t* qp = (const uint8_t*)a.q + ((size_t)t * a.n_heads + 16 * ht + col) * IDX_D + 16 * g;
        qf[ht] = join_i32x8(*(const u32x4*)qp, *(const u32x4*)(qp + 64));
#pragma unroll
        for (int i = 0; i < 4; ++i) wv[ht][i] = a.w[(size_t)t * a.n_heads + 16 * ht + 4 * g + i];
    }
}

// Key fragment of one token (row r of physical block blk) in the MFMA layout.
__device__ __forceinline__ i32x8 load_key_fragment(const IndexerArgs& a, int blk, int r, int lane) {
    const uint8_t* kp = (const uint8_t*)a.keys + ((size_t)blk * IDX_PAGE + r) * IDX_D + 16 * (lane >> 4);
    return join_i32x8(*(const u32x4*)kp, *(const u32x4*)(kp + 64));
}

// Head sum of one query row for the 16 tokens of a fragment: every lane of
// column col returns the ReLU-weighted head sum (before the key scale) of
// token col.
template <int HT>
__device__ __forceinline__ float token_head_sum(const i32x8 (&qf)[HT], const float (&wv)[HT][4], i32x8 kf) {
    const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
    f32x4 c[HT];
#pragma unroll
    for (int ht = 0; ht < HT; ++ht) c[ht] = mfma_fp8_16x16x128(qf[ht], kf, zero);
    float acc = 0.f;
#pragma unroll
    for (int ht = 0; ht < HT; ++ht)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc = fmaf(wv[ht][i], relu(c[ht][i]), acc);
    acc += __shfl_xor(acc, 16);
    acc += __shfl_xor(acc, 32);
    return acc;
}

}  // namespace dsa
