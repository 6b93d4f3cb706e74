// Sparse MQA-mode MLA, 128-head slice (gfx950): the device code shared by the
// standalone sparse-MLA kernels and the fused decode step.
//
// Per query row t and head h (SemiAnalysis GLM-5.3 article, "MLA
// Modifications"): logits z_j = scale * q[t,h,:] . kv[s_j, 0:d+r] over the
// selected tokens s_j, out[t,h,:] = softmax(z) . kv[s_j, 0:d]; K and V are the
// same cached latent row, V being its first d = 512 columns.
//
// A workgroup of 4 waves owns one query row, 128 heads (32 per wave) and a
// contiguous slice of the row's selection, so every selected latent row is
// fetched once per slice and each LDS fragment read feeds 32 heads.  Tiles of
// 32 tokens stream through a ring of LDS buffers by global_load_lds_dwordx4
// (three tiles in flight while one is computed); the physical rows of the
// slice are resolved through the page table once, up front.
//   S^T = K Q^T    v_mfma_f32_32x32x16_bf16: A = 32 token rows of the tile
//                  (LDS), B = 32 heads' queries (registers, 36 k-steps);
//   O^T += V^T P^T  A = V^T fragments by ds_read_b64_tr_b16 from the same
//                  rows, B = probabilities straight from S^T's accumulator
//                  layout (token order inside each 16-token k-step permuted
//                  alike on both sides); O^T (512 x 32 per wave) lives in the
//                  accumulation registers.
// e4m3 latent rows (576 codes + one fp32 scale per token) arrive in an fp8
// staging ring and are widened exactly to bf16 in LDS (every e4m3 value is a
// bf16 value); the token's scale multiplies its logit and its probability.
//
// Softmax in the exp2 domain against a fixed reference per head: the largest
// logit of the first tile with a visible token.  Probabilities are
// exp2(z - ref), at most 2^64 while no later logit exceeds the reference by
// more than 64 (fp32 and bf16 hold that range; O^T = sum p v / sum p does not
// depend on the reference), so the accumulators are never rescaled.  A slice
// where some logit does exceed it is computed again with the largest logit
// seen as the reference.  The logit scale enters as a positive factor: for a
// negative scale the queries' signs are flipped when they are loaded (exact),
// which gives the same logits.  (A zero scale takes the generic path.)
#pragma once

#include "dsa_kernels.h"

namespace dsa {

constexpr int M_DL = 512, M_DR = 64, M_DQK = M_DL + M_DR;
constexpr int M_TILE = 32;                 // selected tokens per tile
constexpr int M_ROW_BYTES = 2 * M_DQK;     // 1152: one bf16 row in LDS
constexpr int M_ROW_UNITS = M_ROW_BYTES / 16;
constexpr int M_TILE_BYTES = M_TILE * M_ROW_BYTES;
constexpr int M_THREADS = 256;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

constexpr int M3_HEADS = 128;
constexpr int M3_NBUF = 4;                             // bf16 ring: tiles in LDS
constexpr int M3_FP8_NBUF = 3;                         // e4m3 staging ring
constexpr int M3_FP8_TILE = M_TILE * M_DQK;            // 18432 B of codes per tile
constexpr int M3_MAX_SLICE = 2048;
constexpr int M3_DMA_PER_WAVE = M_TILE_BYTES / 1024 / 4;    // 9 x 1 KB per wave per tile (bf16)
constexpr int M3_KPF = 3;     // K fragments in flight
constexpr int M3_VPF = 2;     // V^T fragments in flight

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void* lds_vptr;
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

// LDS of one slice.  The bf16 ring holds M3_NBUF tiles; an e4m3 slice uses
// the first two as its widened tiles and the rest of the space as its
// staging ring of codes.
struct MlaSliceLds {
    uint8_t ks[M3_NBUF][M_TILE_BYTES];
    int32_t rows[M3_MAX_SLICE];                 // physical row per slot (0 for padding)
    uint32_t tvalid[M3_MAX_SLICE / M_TILE];     // per tile: bit s = slot s holds a token
    float tscale[M3_FP8_NBUF][2 * M_TILE];      // e4m3: the staged tiles' token scales (twice)
    uint32_t redo;
};
static_assert(2 * M_TILE_BYTES + M3_FP8_NBUF * M3_FP8_TILE <= M3_NBUF * M_TILE_BYTES, "e4m3 staging fits");

// Largest |value| of a lane's accumulators and those of lane (lane ^ 32).
// Magnitudes of non-NaN floats order like their bit patterns read as
// unsigned integers, so the maximum is taken on the bits with the sign
// cleared: integer instructions, where fmaxf would first canonicalize every
// accumulator (a second instruction per value).
__device__ __forceinline__ float max_abs_pair(const f32x16 (&o)[M_DL / 32], int lane) {
    uint32_t m = 0u;
#pragma unroll
    for (int cb = 0; cb < M_DL / 32; ++cb)
#pragma unroll
        for (int e = 0; e < 16; ++e) m = max(m, __float_as_uint(o[cb][e]) & 0x7FFFFFFFu);
    const float a = __uint_as_float(m);
    return fmaxf(a, lane_xor32(a, lane));
}

// Split partials are stored as fp16 with one power-of-two scale per (query
// row, head, slice): the head's largest |value| times 2^k lies in
// [2^14, 2^15), so every value keeps 11 significant bits relative to it and
// none overflows.  The merge multiplies by 2^-k.
__device__ __forceinline__ int part_exponent(float amax) {
    if (!(amax > 0.f)) return 0;
    const int e = (int)((__float_as_uint(amax) >> 23) & 0xFFu) - 126;   // amax in [2^(e-1), 2^e)
    return max(-100, min(100, 15 - e));
}
__device__ __forceinline__ float pow2i(int k) { return __uint_as_float((uint32_t)(127 + k) << 23); }
// Two floats to packed fp16, round to nearest even (one instruction).
__device__ __forceinline__ uint32_t pack_f16x2(float x, float y) {
    typedef _Float16 f16x2_v __attribute__((ext_vector_type(2)));
    const f16x2_v v = {(_Float16)x, (_Float16)y};
    return __builtin_bit_cast(uint32_t, v);
}
// Two finite floats to packed bf16, round to nearest even (one instruction).
__device__ __forceinline__ uint32_t pack_bf16x2(float x, float y) {
    typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
    const bf16x2_v v = {(__bf16)x, (__bf16)y};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// max(a, b, c) in one instruction (fmaxf would first canonicalize every
// input it cannot prove canonical; no NaN reaches these)
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

// Two e4m3 codes (bytes 0 and 1 of w when hi is false, bytes 2 and 3
// otherwise) widened to two packed bf16 values by the hardware conversion
// with a unit scale, exactly: e4m3 normals are (1 + m/8) 2^(e-7), subnormals
// m 2^-9, all representable in bf16.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t e4m3x2_to_bf16x2(uint32_t w, bool hi) {
    const bf16x2_t v = hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, true)
                          : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, false);
    return __builtin_bit_cast(uint32_t, v);
}

// Tile layout in LDS (32 rows of 72 16-byte units, bf16): the 1 KB block
// (r >> 3, u >> 3) sits at 1024 (9 (r >> 3) + (u >> 3)); inside it row r & 7
// takes 128 B and holds its units u & 7 XOR-permuted by r & 7, so that one
// unit of the block's 8 rows covers all banks (the S^T fragment reads run
// at the full LDS rate):
//   tile_off(r, u) = 1024 (9 (r >> 3) + (u >> 3)) + 16 (8 (r & 7) + ((u & 7) ^ (r & 7))).
// bf16 rows: wave w moves rows 8w .. 8w+7; its transfer i covers units
// 8i .. 8i+7 of each, lane l taking row 8w + (l >> 3) and unit
// 8i + ((l & 7) ^ (l >> 3)), which the transfer writes at 16 l of the
// instruction's 1 KB block, i.e. at tile_off.  All nine transfers of a lane
// read the same row, so a tile costs one row id per lane.
__device__ __forceinline__ int tile_off(int r, int u) {
    return 1024 * (9 * (r >> 3) + (u >> 3)) + 16 * (8 * (r & 7) + ((u & 7) ^ (r & 7)));
}

// e4m3 staging layout (32 rows of 36 16-byte units of codes): transfer
// (g, i), g = r >> 4, i = u >> 2, is 1 KB at 1024 (9 g + i), lane l of it
// taking row 16 g + (l >> 2) and unit 4 i + (l & 3).  A lane reads one row
// for all its transfers.
__device__ __forceinline__ int fp8_stage_off(int r, int u) {
    return 1024 * (9 * (r >> 4) + (u >> 2)) + 16 * (4 * (r & 15) + (u & 3));
}

// Result of a slice, per lane: element e of block cb is O^T[32 cb + 8 (e/4) +
// 4 hh + e % 4][head] (unnormalised), with the reference m_ref (log2 domain)
// and the row sum l_tot of the probabilities.
struct MlaAcc {
    f32x16 o[M_DL / 32];
    float m_ref, l_tot;
};

// Slice [j_begin, j_begin + nslots) of query row t's selection `sel` (logical
// positions, -1 skipped) through page-table row `pt`, heads [hbase, hbase +
// 128).  Called by all M_THREADS threads; uses L exclusively until it
// returns.  PIPE (bf16 rows): overlap each tile's softmax with the previous
// tile's PV; it needs more registers than a kernel with other live state
// (the fused step) or the e4m3 widening can spare.
template <bool FP8, bool PIPE = false>
__device__ __forceinline__ void mla_slice(const MlaArgs& a, int t, int hbase, const int32_t* sel, const int32_t* pt,
                                          int nslots, MlaSliceLds& L, MlaAcc& acc) {
    const Geometry& G = a.g;
    const int ntiles = (nslots + M_TILE - 1) / M_TILE;
    const int tid = tid_x(), lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hh = lane >> 5, c32 = lane & 31;
    const uint8_t* kvb = (const uint8_t*)a.kv;
    const float zscale = fabsf(a.scale) * LOG2E;
    const uint32_t qsign = a.scale < 0.f ? 0x80008000u : 0u;

    // The queries first: each wave's 32 heads (one contiguous 36 KB block)
    // into ring buffer `wave` by 1 KB transfers, the 16-byte unit u of head h
    // at 1152 h + 16 (u ^ (h & 7)); each transfer reads 1 KB of the block
    // (units permuted within 128-byte groups), and the fragment reads below
    // (8 lanes, 8 heads, one unit) hit distinct banks.  Their latency
    // overlaps the row chain, whose waits cover them (in-order counter).
    {
        const uint8_t* qblk = (const uint8_t*)a.q + ((size_t)t * a.n_heads + hbase + 32 * wave) * M_ROW_BYTES;
        const uint32_t qdst = lds_addr(&L.ks[wave][0]);
#pragma unroll
        for (int i = 0; i < M_TILE_BYTES / 1024; ++i) {
            const int o = 1024 * i + 16 * lane;
            const int h = o / M_ROW_BYTES, up = (o % M_ROW_BYTES) / 16;
            dma16(qblk + (size_t)h * M_ROW_BYTES + 16 * (up ^ (h & 7)), qdst + 1024u * i);
        }
    }
    // the slice's rows (every selection index load, then every page-table
    // load, so each waits one round trip)
    {
        constexpr int PER = M3_MAX_SLICE / M_THREADS;
        const int bs = G.block_size;
        const bool pow2 = (bs & (bs - 1)) == 0;
        const int bsh = __builtin_ctz((unsigned)bs);
        int sj[PER], blk[PER], slot[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int j = tid + u * M_THREADS;
            sj[u] = j < nslots ? ld_agent(sel + j) : -1;   // may come from this launch
        }
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int s = max(sj[u], 0);
            const int b = pow2 ? s >> bsh : s / bs;
            slot[u] = s - b * bs;
            blk[u] = sj[u] >= 0 ? pt[b] : 0;
        }
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int j = tid + u * M_THREADS;
            const bool ok = sj[u] >= 0;
            if (j < ntiles * M_TILE) L.rows[j] = ok ? blk[u] * bs + slot[u] : 0;
            const unsigned long long m = __ballot(ok);   // 64 slots = two tiles
            if (lane == 0 && j < ntiles * M_TILE) L.tvalid[j / M_TILE] = (uint32_t)m;
            if (lane == 32 && j < ntiles * M_TILE) L.tvalid[j / M_TILE] = (uint32_t)(m >> 32);
        }
    }
    u32x4 qf[M_DQK / 16];   // B operand of S^T = K Q^T, one 16-byte fragment per 16-wide k step
    {
        wait_vmcnt<0>();   // this wave's query transfers (the row chain has waited for them already)
        const uint8_t* qb = &L.ks[wave][0] + c32 * M_ROW_BYTES;
#pragma unroll
        for (int ks = 0; ks < M_DQK / 16; ++ks)
            qf[ks] = *(const u32x4*)(qb + 16 * ((2 * ks + hh) ^ (c32 & 7))) ^ qsign;
    }
    __syncthreads();   // rows and tile masks written; every wave's queries read (the ring is free)

    // per-wave transfers of one tile (bf16: 9 x 1 KB into ring buffer b;
    // e4m3: the wave's 5 or 4 staging transfers into staging slot b, and for
    // wave 1 a fifth: the tile's 32 token scales, 4 B per lane, lanes 32..63
    // repeating lanes 0..31)
    constexpr int FP8_OPS = 5;                 // transfers of waves 0, 1 and 2 (wave 3: 4)
    const int dma_col = FP8 ? 16 * (lane & 3) : 16 * ((lane & 7) ^ (lane >> 3));
    const int f8_g = wave >> 1, f8_i0 = (wave & 1) ? 5 : 0, f8_n = (wave & 1) ? 4 : 5;
    const bool f8_sc = wave == 1;
    const int f8_ops = f8_n + (f8_sc ? 1 : 0);
    uint8_t* const f8_stage = &L.ks[0][0] + 2 * M_TILE_BYTES;
    auto tile_row = [&](int tile) -> int {
        return FP8 ? L.rows[M_TILE * tile + 16 * f8_g + (lane >> 2)] : L.rows[M_TILE * tile + 8 * wave + (lane >> 3)];
    };
    auto scale_src = [&](int tile) -> const float* { return a.kv_scales + L.rows[M_TILE * tile + (lane & 31)]; };
    auto issue = [&](int tile, int b) {
        const int row = tile_row(tile);
        if constexpr (!FP8) {
            const uint8_t* src = kvb + (size_t)row * M_ROW_BYTES + dma_col;
            const uint32_t dst = lds_addr(&L.ks[b][0] + 1024 * M3_DMA_PER_WAVE * wave);
#pragma unroll
            for (int i = 0; i < M3_DMA_PER_WAVE; ++i) dma16(src + 128 * i, dst + 1024u * i);
        } else {
            const uint8_t* src = kvb + (size_t)row * M_DQK + 64 * f8_i0 + dma_col;
            const uint32_t dst = lds_addr(f8_stage + M3_FP8_TILE * b + 1024 * (9 * f8_g + f8_i0));
#pragma unroll
            for (int i = 0; i < FP8_OPS; ++i)
                if (i < f8_n) dma16(src + 64 * i, dst + 1024u * i);
            if (f8_sc) dma4(scale_src(tile), lds_addr(&L.tscale[b][0]));
        }
    };
    constexpr int NRING = FP8 ? M3_FP8_NBUF : M3_NBUF;
    // e4m3: staging slot -> widened tile (two buffers), 9 units of 8 columns a thread
    auto widen = [&](int slot, int b) {
        const uint8_t* st8 = f8_stage + M3_FP8_TILE * slot;
        uint8_t* dst = &L.ks[b][0];
#pragma unroll
        for (int i = 0; i < M_TILE * M_ROW_UNITS / M_THREADS; ++i) {
            const int U = tid + M_THREADS * i;
            const int r = U / M_ROW_UNITS, u = U % M_ROW_UNITS;   // bf16 unit u = codes [8u, 8u + 8)
            const u32x2 c = *(const u32x2*)(st8 + fp8_stage_off(r, u >> 1) + 8 * (u & 1));
            u32x4 o;
            o[0] = e4m3x2_to_bf16x2(c[0], false);
            o[1] = e4m3x2_to_bf16x2(c[0], true);
            o[2] = e4m3x2_to_bf16x2(c[1], false);
            o[3] = e4m3x2_to_bf16x2(c[1], true);
            *(u32x4*)(dst + tile_off(r, u)) = o;
        }
    };

    // per-lane LDS offsets: unit 8m + e of row r is at the offset of unit e
    // plus 1024 m, so fragment reads are few bases plus immediates
    int qk_base[4];       // S^T A operand: row c32, unit 2ks + hh; [ks % 4], + 1024 (ks / 4)
    {
        const int rb = 9216 * (c32 >> 3) + 128 * (c32 & 7), sw = c32 & 7;
#pragma unroll
        for (int m = 0; m < 4; ++m) qk_base[m] = rb + 16 * ((2 * m + hh) ^ sw);
    }
    // V^T A operand by transposing reads: in 16-lane group g4 (hh = g4 >> 1,
    // column half 16(g4 & 1)), source lane s = 4jj + q points at token
    // 16kk + 8rd + 4hh + jj, columns 32cb + 16(g4 & 1) + 4q .. +3 (unit
    // 4cb + v, v = 2(g4 & 1) + (q >> 1)), and destination lane d receives
    // column d of the half, tokens jj = 0..3.
    // (token 16kk + 8rd + tl, tl = 4hh + jj < 8: block row 2kk + rd, row tl
    // inside it, so kk and rd enter as the immediate 9216 (2kk + rd))
    int pv_base[2];   // [cb & 1], + 9216 (2kk + rd) + 1024 (cb / 2)
    {
        const int s16 = lane & 15, jj = s16 >> 2, q = s16 & 3;
        const int v = 2 * ((lane >> 4) & 1) + (q >> 1);
        const int tl = 4 * hh + jj;
#pragma unroll
        for (int c1 = 0; c1 < 2; ++c1) pv_base[c1] = 128 * tl + 16 * ((4 * c1 + v) ^ tl) + 8 * (q & 1);
    }

    f32x16* oacc = acc.o;
    float m_ref = -INFINITY, m_seen = -INFINITY, l_run = 0.f;
    bool overflow = false;

    // Masks the slots of tile i that hold no token (their logits take no part).
    auto mask_tile = [&](f32x16& st, uint32_t vmask) {
        const uint32_t vm = vmask >> (4 * hh);
#pragma unroll
        for (int e = 0; e < 16; ++e) st[e] = (vm >> (8 * (e >> 2) + (e & 3))) & 1u ? st[e] : -INFINITY;
    };
    // Softmax of tile i's (masked, and for e4m3 scaled) logits against the
    // fixed reference: the probabilities as the PV operand (bf16) and the
    // running row sum.  Element e of this lane: token 8(e/4) + 4hh + e%4,
    // head c32; e4m3: the tokens' scales also multiply their probabilities
    // (V rows are unscaled codes).
    auto softmax = [&](f32x16& st, int i, bf16x8 (&pb)[2]) {
        const float* tsl = &L.tscale[i % M3_FP8_NBUF][4 * hh];
        // the tile's largest logit (zscale > 0) and the fixed reference
        float tmax = max3f(max3f(max3f(st[0], st[1], st[2]), max3f(st[3], st[4], st[5]),
                                 max3f(st[6], st[7], st[8])),
                           max3f(st[9], st[10], st[11]), max3f(st[12], st[13], fmaxf(st[14], st[15])));
        tmax *= zscale;
        tmax = fmaxf(tmax, lane_xor32(tmax, lane));
        m_seen = fmaxf(m_seen, tmax);
        if (m_ref == -INFINITY) m_ref = tmax;   // first visible token of this head
        overflow |= tmax > m_ref + 64.f;
        // before the first visible token (m_ref = -inf in all lanes of the
        // wave, whose heads share their tokens) every probability is 0
        const float mre = m_ref == -INFINITY ? INFINITY : m_ref;
        float p[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) p[e] = __builtin_amdgcn_exp2f(fmaf(st[e], zscale, -mre));
        {
            float s8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) s8[e] = p[e] + p[e + 8];
#pragma unroll
            for (int e = 0; e < 4; ++e) s8[e] += s8[e + 4];
            l_run += (s8[0] + s8[2]) + (s8[1] + s8[3]);
        }
        if constexpr (FP8) {
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                const f32x4 sc4 = *(const f32x4*)(tsl + 8 * e4);
#pragma unroll
                for (int e = 0; e < 4; ++e) p[4 * e4 + e] *= sc4[e];
            }
        }
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e) pb[kk][e] = (__bf16)p[8 * kk + e];
    };
    // O^T += V^T P^T over tile buffer Kb: V^T fragments (two transposing
    // reads each) read M3_VPF MFMAs ahead; the 16 accumulators rotate
    // between dependent updates
    auto pv = [&](const uint8_t* Kb, const bf16x8 (&pb)[2]) {
        constexpr int NV = 2 * (M_DL / 32);
        auto vread = [&](int n, s16x4& v0, s16x4& v1) {
            const int kk = n / (M_DL / 32), cb = n % (M_DL / 32);
            v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4_ptr)(Kb + pv_base[cb & 1] + 9216 * (2 * kk) + 1024 * (cb >> 1)));
            v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4_ptr)(Kb + pv_base[cb & 1] + 9216 * (2 * kk + 1) + 1024 * (cb >> 1)));
        };
        s16x4 vb0[M3_VPF], vb1[M3_VPF];
#pragma unroll
        for (int j = 0; j < M3_VPF; ++j) vread(j, vb0[j], vb1[j]);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * M3_VPF, 0);
#pragma unroll
        for (int n = 0; n < NV; ++n) {
            const int kk = n / (M_DL / 32), cb = n % (M_DL / 32);
            const s16x4 v0 = vb0[n % M3_VPF], v1 = vb1[n % M3_VPF];
            u32x4 va;
            va[0] = (uint16_t)v0[0] | ((uint32_t)(uint16_t)v0[1] << 16);
            va[1] = (uint16_t)v0[2] | ((uint32_t)(uint16_t)v0[3] << 16);
            va[2] = (uint16_t)v1[0] | ((uint32_t)(uint16_t)v1[1] << 16);
            va[3] = (uint16_t)v1[2] | ((uint32_t)(uint16_t)v1[3] << 16);
            oacc[cb] = mfma_bf16_32x32x16(as_bf16x8(va), pb[kk], oacc[cb]);
            if (n + M3_VPF < NV) vread(n + M3_VPF, vb0[n % M3_VPF], vb1[n % M3_VPF]);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // then its two reads
        }
    };
    // PV of the previous tile (buffer Kb, probabilities pbp) with the
    // softmax of the current tile (logits sc, tile index ic, result pbc) in
    // the same stretch of code: its vector instructions are scheduled
    // between the MFMAs, which do not depend on them.
    auto pv_soft = [&](const uint8_t* Kb, const bf16x8 (&pbp)[2], f32x16& sc, int ic, bf16x8 (&pbc)[2]) {
        constexpr int NV = 2 * (M_DL / 32);
        auto vread = [&](int n, s16x4& v0, s16x4& v1) {
            const int kk = n / (M_DL / 32), cb = n % (M_DL / 32);
            v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4_ptr)(Kb + pv_base[cb & 1] + 9216 * (2 * kk) + 1024 * (cb >> 1)));
            v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4_ptr)(Kb + pv_base[cb & 1] + 9216 * (2 * kk + 1) + 1024 * (cb >> 1)));
        };
        s16x4 vb0[M3_VPF], vb1[M3_VPF];
#pragma unroll
        for (int j = 0; j < M3_VPF; ++j) vread(j, vb0[j], vb1[j]);
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * M3_VPF, 0);
        __builtin_amdgcn_sched_barrier(0);
        softmax(sc, ic, pbc);
#pragma unroll
        for (int n = 0; n < NV; ++n) {
            const int kk = n / (M_DL / 32), cb = n % (M_DL / 32);
            const s16x4 v0 = vb0[n % M3_VPF], v1 = vb1[n % M3_VPF];
            u32x4 va;
            va[0] = (uint16_t)v0[0] | ((uint32_t)(uint16_t)v0[1] << 16);
            va[1] = (uint16_t)v0[2] | ((uint32_t)(uint16_t)v0[3] << 16);
            va[2] = (uint16_t)v1[0] | ((uint32_t)(uint16_t)v1[1] << 16);
            va[3] = (uint16_t)v1[2] | ((uint32_t)(uint16_t)v1[3] << 16);
            oacc[cb] = mfma_bf16_32x32x16(as_bf16x8(va), pbp[kk], oacc[cb]);
            if (n + M3_VPF < NV) vread(n + M3_VPF, vb0[n % M3_VPF], vb1[n % M3_VPF]);
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);   // its two reads
        }
    };
    // S^T of the tile in buffer Kb: K fragments read M3_KPF steps ahead of
    // their MFMA.  With dma, this wave's transfers of another tile (source
    // row dsrc, destination ddst) are spread over the MFMAs, one after every
    // fourth, so that issuing them never holds up the matrix core for long.
    auto qk = [&](const uint8_t* Kb, bool dma, const uint8_t* dsrc, uint8_t* ddst, f32x16& st) {
        constexpr int NK = M_DQK / 16;
        u32x4 kb[M3_KPF];
#pragma unroll
        for (int j = 0; j < M3_KPF; ++j) kb[j] = *(const u32x4*)(Kb + qk_base[j & 3] + 1024 * (j >> 2));
        __builtin_amdgcn_sched_group_barrier(0x100, M3_KPF, 0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < NK; ++ks) {
            if (ks == 0) st = mfma_bf16_32x32x16(as_bf16x8(kb[0]), as_bf16x8(qf[0]), f32x16{});
            else st = mfma_bf16_32x32x16(as_bf16x8(kb[ks % M3_KPF]), as_bf16x8(qf[ks]), st);
            if (ks + M3_KPF < NK) {
                const int kn = ks + M3_KPF;
                kb[ks % M3_KPF] = *(const u32x4*)(Kb + qk_base[kn & 3] + 1024 * (kn >> 2));
            }
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // then one LDS read
            const int di = ks >> 2;
            if (dma && (ks & 3) == 1 && di < (FP8 ? FP8_OPS : M3_DMA_PER_WAVE) && (!FP8 || di < f8_n)) {
                // dma16 is not counted by the compiler: it puts no wait for
                // it before the fragment reads of tile i, which use another
                // buffer (the loop's own vector-memory waits count these
                // transfers)
                dma16(dsrc + (FP8 ? 64 : 128) * di, lds_addr(ddst + 1024 * di));
            }
        }
    };

    for (int pass = 0;; ++pass) {
#pragma unroll
    for (int cb = 0; cb < M_DL / 32; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[cb][i] = 0.f;
    l_run = 0.f;
    overflow = false;
    if (tid == 0) L.redo = 0u;

    if constexpr (PIPE) {
        // Software-pipelined over tiles: tile i's S^T, then tile i's softmax
        // on the vector unit while the MFMAs of tile i-1's PV run.  Ring use
        // at step i: tile i-1 (PV), tile i (S^T), tile i+1 in flight, tile
        // i+2 issued during tile i's S^T into the buffer tile i-2 has left.
        static_assert(!FP8, "e4m3 rows take the one-tile-at-a-time loop (the pipelined one spills)");
#pragma unroll
        for (int b = 0; b < 2; ++b)
            if (b < ntiles) issue(b, b);
        bf16x8 pb_prev[2];
        for (int i = 0; i < ntiles; ++i) {
            // tile i landed (tile i+1's transfers may be outstanding), and
            // every wave is done with tile i-2's buffer
            if (i + 1 < ntiles) wait_vmcnt<M3_DMA_PER_WAVE>();
            else wait_vmcnt<0>();
            lds_barrier();
            const uint8_t* Kb = &L.ks[i % M3_NBUF][0];
            const uint32_t vmask = L.tvalid[i];
            f32x16 st;
            bf16x8 pb[2];
            {
                const int nt = i + 2;
                if (nt < ntiles) {
                    const int srow = tile_row(nt);
                    qk(Kb, true, kvb + (size_t)srow * M_ROW_BYTES + dma_col,
                       &L.ks[nt % M3_NBUF][0] + 1024 * M3_DMA_PER_WAVE * wave, st);
                } else {
                    qk(Kb, false, nullptr, nullptr, st);
                }
            }
            if (vmask != 0xFFFFFFFFu) mask_tile(st, vmask);
            if (i == 0) softmax(st, i, pb);
            else pv_soft(&L.ks[(i - 1) % M3_NBUF][0], pb_prev, st, i, pb);
            pb_prev[0] = pb[0];
            pb_prev[1] = pb[1];
        }
        if (ntiles > 0) pv(&L.ks[(ntiles - 1) % M3_NBUF][0], pb_prev);
    } else {
        // One tile at a time: S^T, softmax, PV; up to NRING - 1 tiles in
        // flight, the next one's transfers spread over the S^T MFMAs.
#pragma unroll
        for (int b = 0; b < NRING - 1; ++b)
            if (b < ntiles) issue(b, b);
        for (int i = 0; i < ntiles; ++i) {
            // this wave's transfers of tile i are done once at most the ones
            // of the (up to NRING - 2) later tiles already issued are outstanding
            const int later = min(NRING - 2, ntiles - 1 - i);
            if constexpr (!FP8) {
                if (later >= 2) wait_vmcnt<2 * M3_DMA_PER_WAVE>();
                else if (later == 1) wait_vmcnt<M3_DMA_PER_WAVE>();
                else wait_vmcnt<0>();
            } else {
                if (later >= 1) { if (f8_ops == FP8_OPS) wait_vmcnt<FP8_OPS>(); else wait_vmcnt<FP8_OPS - 1>(); }
                else wait_vmcnt<0>();
            }
            lds_barrier();   // everyone's part of tile i landed; tile i-1's buffer is free
            const uint8_t* Kb;
            if constexpr (FP8) {
                widen(i % M3_FP8_NBUF, i & 1);
                lds_barrier();   // tile i widened
                Kb = &L.ks[i & 1][0];
            } else {
                Kb = &L.ks[i % M3_NBUF][0];
            }
            const uint32_t vmask = L.tvalid[i];   // tokens present in the tile (bit per slot)

            // S^T, with the transfers of tile i + NRING - 1 (into the buffer
            // or staging slot tile i - 1 has left)
            f32x16 st;
            bf16x8 pb[2];
            {
                const int nt = i + NRING - 1;
                const bool iss = nt < ntiles;
                const int ntc = min(nt, ntiles - 1);
                const int srow = tile_row(ntc);
                const uint8_t* dsrc = FP8 ? kvb + (size_t)srow * M_DQK + 64 * f8_i0 + dma_col
                                          : kvb + (size_t)srow * M_ROW_BYTES + dma_col;
                uint8_t* ddst = FP8 ? f8_stage + M3_FP8_TILE * (nt % M3_FP8_NBUF) + 1024 * (9 * f8_g + f8_i0)
                                    : &L.ks[nt % M3_NBUF][0] + 1024 * M3_DMA_PER_WAVE * wave;
                if (iss) {
                    qk(Kb, true, dsrc, ddst, st);
                    if constexpr (FP8) {
                        if (f8_sc) dma4(scale_src(ntc), lds_addr(&L.tscale[nt % M3_FP8_NBUF][0]));
                    }
                } else {
                    qk(Kb, false, dsrc, ddst, st);
                }
            }
            if constexpr (FP8) {   // the tokens' scales multiply their logits
                const float* tsl = &L.tscale[i % M3_FP8_NBUF][4 * hh];
#pragma unroll
                for (int e4 = 0; e4 < 4; ++e4) {
                    const f32x4 sc4 = *(const f32x4*)(tsl + 8 * e4);
#pragma unroll
                    for (int e = 0; e < 4; ++e) st[4 * e4 + e] *= sc4[e];
                }
            }
            if (vmask != 0xFFFFFFFFu) mask_tile(st, vmask);
            softmax(st, i, pb);
            pv(Kb, pb);
        }
    }
    // the whole workgroup agrees on a second pass (it shares the barriers)
    if (__ballot(overflow) && lane == 0) L.redo = 1u;
    __syncthreads();
    if (pass > 0 || L.redo == 0u) break;
    m_ref = m_seen;
    __syncthreads();
    }
    acc.m_ref = m_ref;
    acc.l_tot = l_run + lane_xor32(l_run, lane);
}

// Output of a finished slice, staged through LDS so that every global store
// writes one whole 1 KB head row.  Each wave owns 32 KB of the (now idle)
// ring: its 32 heads x 512 columns of 16-bit values, row c (head) at 1024 c.
// The 16-byte unit u of row c sits at unit u ^ c, its two 8-byte halves
// swapped when bit 3 of c is set, so that the lanes of a 16-lane group write
// distinct banks and a row is read back by 64 lanes without conflicts.
template <bool HALF>   // HALF: fp16 values, else bf16
__device__ __forceinline__ void mla_stage_rows(const MlaAcc& acc, float sc, MlaSliceLds& L) {
    const int tid = tid_x(), lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, c = lane & 31;
    uint8_t* base = &L.ks[0][0] + 32768 * wave + 1024 * c + 8 * (hh ^ ((c >> 3) & 1));
#pragma unroll
    for (int cb = 0; cb < M_DL / 32; ++cb)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) {
            const float x0 = acc.o[cb][4 * e4] * sc, x1 = acc.o[cb][4 * e4 + 1] * sc;
            const float x2 = acc.o[cb][4 * e4 + 2] * sc, x3 = acc.o[cb][4 * e4 + 3] * sc;
            u32x2 w;
            if constexpr (HALF) {
                w[0] = pack_f16x2(x0, x1);
                w[1] = pack_f16x2(x2, x3);
            } else {
                w[0] = pack_bf16x2(x0, x1);
                w[1] = pack_bf16x2(x2, x3);
            }
            const int u = 4 * cb + e4;   // 16-byte unit of the row: columns 8u .. 8u + 7
            *(u32x2*)(base + 16 * (u ^ c)) = w;
        }
}

// Stores the wave's 32 staged rows: row j (head hfirst + j of the wave) to
// dst + row_stride * j, 16 bytes a lane.
__device__ __forceinline__ void mla_flush_rows(const MlaSliceLds& L, uint16_t* dst, size_t row_stride) {
    const int tid = tid_x(), lane = tid & 63, wave = tid >> 6;
    const uint8_t* base = &L.ks[0][0] + 32768 * wave;
#pragma unroll 8
    for (int j = 0; j < 32; ++j) {
        u32x4 v = *(const u32x4*)(base + 1024 * j + 16 * (lane ^ j));
        if ((j >> 3) & 1) v = (u32x4){v[2], v[3], v[0], v[1]};
        *(u32x4*)(dst + row_stride * j + 8 * lane) = v;
    }
}

// Normalised bf16 output and natural-log lse of a finished slice that covers
// the whole selection.  Called by the whole workgroup after mla_slice (which
// ends with a barrier, so the ring is idle).
__device__ __forceinline__ void mla_store_final(const MlaArgs& a, int t, int hbase, const MlaAcc& acc,
                                                MlaSliceLds& L) {
    const int tid = tid_x(), lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, head = hbase + 32 * wave + (lane & 31);
    const bool empty = acc.l_tot == 0.f;
    const float inv = empty ? 0.f : 1.f / acc.l_tot;
    mla_stage_rows<false>(acc, inv, L);
    if (a.lse && hh == 0)
        a.lse[(size_t)t * a.n_heads + head] = empty ? -INFINITY : (acc.m_ref + log2f(acc.l_tot)) * LN2;
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's rows written (a wave reads only its own)
    mla_flush_rows(L, (uint16_t*)a.out + ((size_t)t * a.n_heads + hbase + 32 * wave) * M_DL, M_DL);
}

// A slice's normalised partial output as fp16 with its power-of-two scale,
// and its natural-log lse: head hbase + i of the slice goes to partial index
// pfirst + pstride i (partial p: part_o[p][512], part_lse[p][2]).
__device__ __forceinline__ void mla_store_partial_at(const MlaArgs& a, size_t pfirst, size_t pstride,
                                                     const MlaAcc& acc, MlaSliceLds& L) {
    const int tid = tid_x(), lane = tid & 63, wave = tid >> 6;
    const int hh = lane >> 5, hl = 32 * wave + (lane & 31);
    const bool empty = acc.l_tot == 0.f;
    const float inv = empty ? 0.f : 1.f / acc.l_tot;
    const float lse_nat = empty ? -INFINITY : (acc.m_ref + log2f(acc.l_tot)) * LN2;
    // the head's values sit in lanes c32 and c32 + 32
    const float amax = max_abs_pair(acc.o, lane);
    const int k = part_exponent(amax * inv);
    mla_stage_rows<true>(acc, inv * pow2i(k), L);
    const size_t pidx = pfirst + pstride * hl;
    if (hh == 0) {
        a.part_lse[2 * pidx] = lse_nat;
        a.part_lse[2 * pidx + 1] = pow2i(-k);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // this wave's rows written
    mla_flush_rows(L, a.part_o + (pfirst + pstride * 32 * wave) * M_DL, pstride * M_DL);
}

// ... at partial index ((t * H + head) * S + sp) (slices of a row adjacent).
__device__ __forceinline__ void mla_store_partial(const MlaArgs& a, int t, int hbase, int sp, const MlaAcc& acc,
                                                  MlaSliceLds& L) {
    const int S = a.splits;
    mla_store_partial_at(a, ((size_t)t * a.n_heads + hbase) * S + sp, (size_t)S, acc, L);
}

// Merge of split partials by their log-sum-exp, by one wave, for HP heads:
// slice s of head h is partial p0 + h hs + s ps (part_o row and part_lse
// pair), and lane l accumulates the head's output columns 8l .. 8l + 7 into
// acc[h] (normalised); lse[h] is the natural-log lse (-inf when every slice
// is empty).  Up to NS slices of every head go through registers, with all
// their loads issued before any arithmetic (one memory round trip); more
// slices are merged NS at a time.  The sums run in slice order, so the
// result depends on neither NS nor HP.
template <int NS, int HP = 1>
__device__ __forceinline__ void merge_partials(const uint16_t* part_o, const float* part_lse, size_t p0, size_t hs,
                                               size_t ps, int S, int lane, float (&acc)[HP][8], float (&lse)[HP]) {
    float mx[HP], den[HP];
#pragma unroll
    for (int h = 0; h < HP; ++h) {
        mx[h] = -INFINITY;
        den[h] = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] = 0.f;
        if (S > NS)
            for (int s = 0; s < S; ++s) mx[h] = fmaxf(mx[h], part_lse[2 * (p0 + h * hs + (size_t)s * ps)]);
    }
    for (int s0 = 0; s0 < S; s0 += NS) {
        f32x2 pl[HP][NS];
        u32x4 v[HP][NS];
#pragma unroll
        for (int h = 0; h < HP; ++h)
#pragma unroll
            for (int u = 0; u < NS; ++u)
                if (s0 + u < S) pl[h][u] = *(const f32x2*)(part_lse + 2 * (p0 + h * hs + (size_t)(s0 + u) * ps));
#pragma unroll
        for (int h = 0; h < HP; ++h)
#pragma unroll
            for (int u = 0; u < NS; ++u)
                if (s0 + u < S)
                    v[h][u] = *(const u32x4*)(part_o + (p0 + h * hs + (size_t)(s0 + u) * ps) * M_DL + 8 * lane);
#pragma unroll
        for (int h = 0; h < HP; ++h) {
            if (S <= NS)
#pragma unroll
                for (int u = 0; u < NS; ++u)
                    if (u < S) mx[h] = fmaxf(mx[h], pl[h][u][0]);
            if (mx[h] == -INFINITY) continue;
#pragma unroll
            for (int u = 0; u < NS; ++u) {
                if (s0 + u < S) {
                    const float wgt = __expf(pl[h][u][0] - mx[h]);
                    den[h] += wgt;
                    const float ws = wgt * pl[h][u][1];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const uint16_t b = (uint16_t)(v[h][u][i >> 1] >> (16 * (i & 1)));
                        acc[h][i] += ws * (float)__builtin_bit_cast(_Float16, b);
                    }
                }
            }
        }
    }
#pragma unroll
    for (int h = 0; h < HP; ++h) {
        if (mx[h] == -INFINITY) {
            lse[h] = -INFINITY;
            continue;
        }
        const float inv = 1.f / den[h];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[h][i] *= inv;
        lse[h] = mx[h] + logf(den[h]);
    }
}

// merge_partials with the register depth picked from S (the splits of a
// decode row are a power of two, at most 16 for K = 2048).
template <int HP = 1>
__device__ __forceinline__ void merge_partials_any(const uint16_t* part_o, const float* part_lse, size_t p0,
                                                   size_t hs, size_t ps, int S, int lane, float (&acc)[HP][8],
                                                   float (&lse)[HP]) {
    if (S <= 4) merge_partials<4, HP>(part_o, part_lse, p0, hs, ps, S, lane, acc, lse);
    else if (S <= 8) merge_partials<8, HP>(part_o, part_lse, p0, hs, ps, S, lane, acc, lse);
    else merge_partials<16, HP>(part_o, part_lse, p0, hs, ps, S, lane, acc, lse);
}

}  // namespace dsa
