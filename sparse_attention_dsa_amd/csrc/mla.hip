// Sparse MQA-mode MLA on gfx950.
//
// Per query row t and head h (SemiAnalysis GLM-5.3 article, "MLA
// Modifications"): logits z_j = scale * q[t,h,:] . kv[s_j, 0:d+r] over the
// selected tokens s_j, out[t,h,:] = softmax(z) . kv[s_j, 0:d]; K and V are the
// same cached latent row, V being its first d columns.
//
// Fast path (d = 512, r = 64, bf16 or e4m3 latent, heads a multiple of 64): a
// workgroup owns one query row, 64 heads (16 per wave) and a contiguous slice
// of the row's selection, processed in tiles of 32 selected tokens.  A tile's
// latent rows are gathered through the page table into one row-major LDS
// buffer (1152 B per row; the 16-byte units of row r are XOR-permuted by
// ks_swz(r) so that fragment reads of 16 rows hit distinct banks):
//   * bf16 latent: async global_load_lds_dwordx4 transfers (one fully
//     coalesced 1 KB segment per instruction) into a double buffer -- tile
//     i+1 is in flight while tile i is computed, without holding registers;
//   * e4m3 latent: register loads widened exactly to bf16 (e4m3 values are
//     bf16-representable), the per-token scale applied to logits and
//     probabilities.
// Logits S^T = K Q^T use the LDS rows as the A operand (k = latent dim) and
// register-resident queries as the B operand.  S^T's accumulator layout is
// exactly the B-operand layout P^T needs for O^T = V^T P^T (token order inside
// a 32-token step permuted consistently on both sides), so probabilities never
// leave registers.  The V^T operand is read from the same row-major buffer
// with ds_read_b64_tr_b16, which transposes 16-bit elements across each
// 16-lane group.  Each lane's O^T accumulators belong to one head, so the
// online-softmax rescale is a per-lane scalar.  Decode rows split their
// selection across workgroups and a second kernel merges the partial results
// by their log-sum-exp; prefill rows have enough parallelism without it.
#include "mla_dev.h"

namespace dsa {

// Slot order inside a 32-token tile: k-slot 8g + j of lane group g holds token
// slot_token(g, j); lane group g's logit accumulators hold tokens 4g..4g+3 of
// the first 16-token half and 16+4g..16+4g+3 of the second.
__device__ __forceinline__ int slot_token(int g, int j) {
    return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4);
}

// XOR permutation of the 16-byte units inside row r (within aligned groups of
// 8 units; 72 units per row).
__device__ __forceinline__ int ks_swz(int r) { return (r ^ (r >> 3)) & 7; }

// Byte offset in a tile buffer of logical 16-byte unit u of row r.
__device__ __forceinline__ int ks_off(int r, int u) { return r * M_ROW_BYTES + 16 * (u ^ ks_swz(r)); }

// 8 latent columns [8u, 8u+8) of an e4m3 cache row widened exactly to bf16.
__device__ __forceinline__ u32x4 load_e4m3_unit(const uint8_t* kv, int row, int u) {
    const u32x2 v = *(const u32x2*)(kv + (size_t)row * M_DQK + 8 * u);
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t w = v[i >> 1] >> (16 * (i & 1));
        const uint32_t b0 = __float_as_uint(e4m3_to_f32(w & 0xFFu)) >> 16;
        const uint32_t b1 = __float_as_uint(e4m3_to_f32((w >> 8) & 0xFFu)) >> 16;
        o[i] = b0 | (b1 << 16);
    }
    return o;
}

template <bool FP8, bool SPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(M_THREADS, M_THREADS), amdgpu_waves_per_eu(2, 2)))
void mla_bf16_mfma(MlaArgs a, int slice) {
    const Geometry& G = a.g;
    const int hgroups = a.n_heads / MLA_HEADS_PER_WG;
    const int t = blockIdx.x / hgroups, hg = blockIdx.x % hgroups;
    const int sp = blockIdx.y;
    const int r = find_request(G.qsl, G.B, t);
    const int j_begin = sp * slice;
    const int j_end = min(a.k, j_begin + slice);

    // double buffer; each unrolled half names its buffer with a constant index,
    // so the compiler can tell the buffer being read from the one an
    // asynchronous transfer is filling (and folds the choice into offsets)
    __shared__ __attribute__((aligned(16))) uint8_t Ks[FP8 ? 1 : 2][M_TILE_BYTES];
    __shared__ int32_t rows[3][M_TILE];          // physical rows of tiles i, i+1, i+2 (-1: none)
    __shared__ float tscale[FP8 ? 3 : 1][M_TILE];  // e4m3 per-token scales of those rows

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int g = lane >> 4, col = lane & 15;
    const int head = hg * MLA_HEADS_PER_WG + wave * 16 + col;

    const int32_t* sel = a.indices + (size_t)t * a.k;
    const int32_t* pt = G.page_table + (size_t)r * G.max_blocks;
    const int nslots = max(0, j_end - j_begin);
    const int ntiles = (nslots + M_TILE - 1) / M_TILE;
    auto stage_rows = [&](int b, int tile) {     // threads < M_TILE: row ids (+ scales) of a tile
        const int j = tile * M_TILE + tid;
        int row = -1;
        if (j < nslots) {
            const int s = sel[j_begin + j];
            if (s >= 0) row = pt[s / G.block_size] * G.block_size + s % G.block_size;
        }
        rows[b][tid] = row;
        if constexpr (FP8) tscale[b][tid] = row >= 0 ? a.kv_scales[row] : 0.f;
    };
    // bf16: one tile's rows into a buffer, 9 coalesced 1 KB transfers per wave
    auto issue = [&](uint8_t* dst, const int32_t* trow) {
        // recomputed per tile on purpose: hoisting these offsets out of the tile
        // loop costs more registers than the few instructions that make them
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int i = 0; i < M_TILE_BYTES / 16 / M_THREADS; ++i) {
            const int U = (wave * (M_TILE_BYTES / 16 / M_THREADS) + i) * 64 + ln;   // LDS unit
            const int rr = U / M_ROW_UNITS, pu = U % M_ROW_UNITS;
            const int u = pu ^ ks_swz(rr);                                       // logical unit
            const int row = trow[rr];
            const uint8_t* src = (const uint8_t*)a.kv + (size_t)(row < 0 ? 0 : row) * M_ROW_BYTES + 16 * u;
            __builtin_amdgcn_global_load_lds((const void*)src,
                                             (lds_vptr)(dst + 1024 * (wave * (M_TILE_BYTES / 16 / M_THREADS) + i)),
                                             16, 0, 0);
        }
    };
    // e4m3: one tile's rows widened to bf16 into the single buffer (synchronous)
    auto gather_fp8 = [&](const int32_t* trow) {
        for (int U = tid; U < M_TILE * M_ROW_UNITS; U += M_THREADS) {
            const int rr = U / M_ROW_UNITS, u = U % M_ROW_UNITS;
            const int row = trow[rr];
            const u32x4 v = row >= 0 ? load_e4m3_unit((const uint8_t*)a.kv, row, u) : (u32x4){0u, 0u, 0u, 0u};
            *(u32x4*)(&Ks[0][0] + ks_off(rr, u)) = v;
        }
    };

    // Queries: B operand of S^T = K Q^T, one 16-byte fragment per 32-wide k step.
    u32x4 qf[M_DQK / 32];
    {
        const uint16_t* qp = (const uint16_t*)a.q + ((size_t)t * a.n_heads + head) * M_DQK + 8 * g;
#pragma unroll
        for (int ks = 0; ks < M_DQK / 32; ++ks) qf[ks] = *(const u32x4*)(qp + 32 * ks);
    }
    f32x4 oacc[M_DL / 16];
#pragma unroll
    for (int ct = 0; ct < M_DL / 16; ++ct) oacc[ct] = (f32x4){0.f, 0.f, 0.f, 0.f};
    float m_run = -INFINITY, l_run = 0.f;
    const float zscale = a.scale * LOG2E;

    // Per-lane LDS offsets.  XOR-ing a unit index with ks_swz(r) < 8 only
    // touches its low 3 bits, so every fragment read is one of a few per-lane
    // bases plus a compile-time immediate (128 B per 8 units).
    int qk_base[2][2];                   // [token half][k-step parity]
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
        const int rr = 16 * tt + col;
        qk_base[tt][0] = rr * M_ROW_BYTES + 16 * (g ^ ks_swz(rr));
        qk_base[tt][1] = rr * M_ROW_BYTES + 16 * ((4 + g) ^ ks_swz(rr));
    }
    // V^T fragments by transposing reads: source lane s of a 16-lane group
    // points at token slot_token(g, s/4 + 4h), columns c0+4(s%4)..+3; this lane
    // then receives 4 tokens of column c0 + col.
    int pv_base[2][4];                   // [h][column-tile mod 4]
    {
        const int cq = 4 * (col & 3);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int tok = slot_token(g, (col >> 2) + 4 * h);
#pragma unroll
            for (int m = 0; m < 4; ++m)
                pv_base[h][m] = tok * M_ROW_BYTES + 16 * ((2 * m + (cq >> 3)) ^ ks_swz(tok)) + 2 * (cq & 7);
        }
    }

    // One tile from an LDS buffer: logits and online softmax (returns the
    // bf16 probabilities in the P^T operand layout), then PV.
    auto logits_softmax = [&](const uint8_t* Kb, int slot) -> bf16x8 {
        const int32_t* trow = rows[slot];
        float x[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int ks = 0; ks < M_DQK / 32; ++ks) {
                const u32x4 kfrag = *(const u32x4*)(Kb + qk_base[tt][ks & 1] + 128 * (ks >> 1));
                s = mfma_bf16_16x16x32(as_bf16x8(kfrag), as_bf16x8(qf[ks]), s);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = 16 * tt + 4 * g + i;
                float zs = zscale;
                if constexpr (FP8) zs *= tscale[slot][tok];
                x[tt][i] = trow[tok] >= 0 ? s[i] * zs : -INFINITY;
            }
        }
        float tmax = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                           fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);
        float p[2][4];
        float psum = 0.f, alpha = 1.f;
        if (m_new != -INFINITY) {
            alpha = __builtin_amdgcn_exp2f(m_run - m_new);
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    p[tt][i] = __builtin_amdgcn_exp2f(x[tt][i] - m_new);
                    psum += p[tt][i];
                }
        } else {
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) p[tt][i] = 0.f;
        }
        psum += __shfl_xor(psum, 16);
        psum += __shfl_xor(psum, 32);
        l_run = l_run * alpha + psum;
        m_run = m_new;
        if (alpha != 1.f) {
#pragma unroll
            for (int ct = 0; ct < M_DL / 16; ++ct) oacc[ct] *= alpha;
        }
        if constexpr (FP8) {   // V rows are unscaled codes: fold each token's scale into p
#pragma unroll
            for (int tt = 0; tt < 2; ++tt)
#pragma unroll
                for (int i = 0; i < 4; ++i) p[tt][i] *= tscale[slot][16 * tt + 4 * g + i];
        }
        u32x4 pb;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int tt = m >> 1, i = 2 * (m & 1);
            pb[m] = f32_to_bf16(p[tt][i]) | (f32_to_bf16(p[tt][i + 1]) << 16);
        }
        return as_bf16x8(pb);
    };
    auto pv = [&](const uint8_t* Kb, bf16x8 pbf) {
#pragma unroll
        for (int ct = 0; ct < M_DL / 16; ++ct) {
            const s16x4 v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4_ptr)(Kb + pv_base[0][ct & 3] + 128 * (ct >> 2)));
            const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                (lds_s16x4_ptr)(Kb + pv_base[1][ct & 3] + 128 * (ct >> 2)));
            u32x4 va;
            va[0] = (uint16_t)v0[0] | ((uint32_t)(uint16_t)v0[1] << 16);
            va[1] = (uint16_t)v0[2] | ((uint32_t)(uint16_t)v0[3] << 16);
            va[2] = (uint16_t)v1[0] | ((uint32_t)(uint16_t)v1[1] << 16);
            va[3] = (uint16_t)v1[2] | ((uint32_t)(uint16_t)v1[3] << 16);
            oacc[ct] = mfma_bf16_16x16x32(as_bf16x8(va), pbf, oacc[ct]);
        }
    };

    if (tid < M_TILE) {
        stage_rows(0, 0);
        stage_rows(1, 1);
    }
    __syncthreads();
    if constexpr (!FP8) {
        // Row ids are staged by wave 0 two tiles ahead with a two-tile chain
        // (the index of tile i+3 and the page-table entry of tile i+2 are
        // loaded at the top of tile i, the row id written at its end), so no
        // staging load is waited for while a tile's transfers are in flight.
        const bool stager = tid < M_TILE;
        auto sel_of = [&](int tile) { const int j = tile * M_TILE + tid; return j < nslots ? sel[j_begin + j] : -1; };
        int sidx_q = stager ? sel_of(2) : -1;    // index for tile i+2
        if (ntiles > 0) issue(&Ks[0][0], rows[0]);
        for (int i = 0; i < ntiles; ++i) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();                       // tile i landed; the other buffer is free
            int blk = 0, sidx_n = -1;
            if (stager) {
                if (sidx_q >= 0) blk = pt[sidx_q / G.block_size];
                sidx_n = sel_of(i + 3);
            }
            if (i + 1 < ntiles) issue(&Ks[((i + 1) & 1) % (FP8 ? 1 : 2)][0], rows[(i + 1) % 3]);
            const uint8_t* cur = &Ks[(i & 1) % (FP8 ? 1 : 2)][0];
            pv(cur, logits_softmax(cur, i % 3));
            if (stager) {
                rows[(i + 2) % 3][tid] = sidx_q < 0 ? -1 : blk * G.block_size + sidx_q % G.block_size;
                sidx_q = sidx_n;
            }
        }
    } else {
        for (int i = 0; i < ntiles; ++i) {
            gather_fp8(rows[i % 3]);
            __syncthreads();
            if (tid < M_TILE) stage_rows((i + 2) % 3, i + 2);
            pv(&Ks[0][0], logits_softmax(&Ks[0][0], i % 3));
            __syncthreads();
        }
    }

    // ---- epilogue: lane holds O^T[c = 16ct + 4g + i][head]
    const bool empty = l_run == 0.f;
    const float inv = empty ? 0.f : 1.f / l_run;
    const float lse_nat = empty ? -INFINITY : (m_run + log2f(l_run)) * LN2;
    if (SPLIT) {
        // the head's values sit in lanes col, col + 16, col + 32, col + 48
        // (the magnitudes' maximum on their bits, as in max_abs_pair)
        uint32_t amb = 0u;
#pragma unroll
        for (int ct = 0; ct < M_DL / 16; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) amb = max(amb, __float_as_uint(oacc[ct][i]) & 0x7FFFFFFFu);
        float amax = __uint_as_float(amb);
        amax = fmaxf(amax, __shfl_xor(amax, 16));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        const int k = part_exponent(amax * inv);
        const float sc = inv * pow2i(k);
        const size_t pidx = ((size_t)t * a.n_heads + head) * a.splits + sp;
        uint16_t* po = a.part_o + pidx * M_DL;
#pragma unroll
        for (int ct = 0; ct < M_DL / 16; ++ct) {
            const f32x4 o = oacc[ct] * sc;
            u32x2 w;
            w[0] = pack_f16x2(o[0], o[1]);
            w[1] = pack_f16x2(o[2], o[3]);
            *(u32x2*)(po + 16 * ct + 4 * g) = w;
        }
        if (g == 0) {
            a.part_lse[2 * pidx] = lse_nat;
            a.part_lse[2 * pidx + 1] = pow2i(-k);
        }
    } else {
        uint16_t* op = (uint16_t*)a.out + ((size_t)t * a.n_heads + head) * M_DL;
#pragma unroll
        for (int ct = 0; ct < M_DL / 16; ++ct) {
            const f32x4 o = oacc[ct] * inv;
            u32x2 w;
            w[0] = f32_to_bf16(o[0]) | (f32_to_bf16(o[1]) << 16);
            w[1] = f32_to_bf16(o[2]) | (f32_to_bf16(o[3]) << 16);
            *(u32x2*)(op + 16 * ct + 4 * g) = w;
        }
        if (a.lse && g == 0) a.lse[(size_t)t * a.n_heads + head] = lse_nat;
    }
}

// Merge split partials: out = sum_s e^{lse_s - L} o_s with L = log-sum-exp.
// One wave per HP adjacent (query row, head) pairs (T H is even), each
// pair's slices adjacent, so a wave's loads are HP S contiguous partial rows;
// NS slices are held in registers.  The launch picks NS from S, and two pairs
// a wave up to 8 slices, one beyond (the register count, and with it the
// occupancy, follows the split count).
template <int NS, int HP>
__global__ __launch_bounds__(256) void mla_combine(MlaArgs a0) {
    const MlaArgs a = mla_layer_args(a0, blockIdx.y);
    const int lane = threadIdx.x & 63;
    const size_t th0 = ((size_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * HP;   // first (t, h) of the wave
    if (th0 >= (size_t)a.g.T * a.n_heads) return;
    const int S = a.splits;
    float acc[HP][8], lse[HP];
    merge_partials<NS, HP>(a.part_o, a.part_lse, th0 * S, (size_t)S, 1, S, lane, acc, lse);
#pragma unroll
    for (int h = 0; h < HP; ++h) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = f32_to_bf16(acc[h][2 * i]) | (f32_to_bf16(acc[h][2 * i + 1]) << 16);
        *(u32x4*)((uint16_t*)a.out + (th0 + h) * M_DL + 8 * lane) = w;
        if (a.lse && lane == 0) a.lse[th0 + h] = lse[h];
    }
}

static void launch_combine(const MlaArgs& a, hipStream_t s) {
    const int pairs = a.g.T * a.n_heads;
    if (a.splits <= 4)
        hipLaunchKernelGGL((mla_combine<4, 2>), dim3((pairs / 2 + 3) / 4, a.n_layers), dim3(256), 0, s, a);
    else if (a.splits <= 8)
        hipLaunchKernelGGL((mla_combine<8, 2>), dim3((pairs / 2 + 3) / 4, a.n_layers), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((mla_combine<16, 1>), dim3((pairs + 3) / 4, a.n_layers), dim3(256), 0, s, a);
}

// Generic path: any dims and head counts, fp32 / bf16 / e4m3 latent.  One
// workgroup per (query row, head); logits and probabilities in LDS.
constexpr int GEN_MAX_W4 = 32;     // fp32 latent rows held in registers: up to 128 values
constexpr int GEN_PV_BATCH = 16;   // value rows in flight per thread in the PV sum
__global__ __launch_bounds__(256) void mla_generic(MlaArgs a) {
    const Geometry& G = a.g;
    const int t = blockIdx.x / a.n_heads, h = blockIdx.x % a.n_heads;
    const int r = find_request(G.qsl, G.B, t);
    const int W = a.d_latent + a.d_rope, D = a.d_latent;
    extern __shared__ int64_t smem64[];
    int64_t* rows = smem64;                       // [k] physical row of each slot (-1: padding)
    float* qv = (float*)(smem64 + a.k);           // [W]
    float* z = qv + W;                            // [k]
    __shared__ float red[256];
    const bool f32 = a.kv_dtype == 0;
    const int32_t* sel = a.indices + (size_t)t * a.k;
    const int32_t* pt = G.page_table + (size_t)r * G.max_blocks;
    const int bs = G.block_size;
    for (int c = threadIdx.x; c < W; c += blockDim.x) {
        const size_t off = ((size_t)t * a.n_heads + h) * W + c;
        qv[c] = f32 ? ((const float*)a.q)[off] : bf16_to_f32(((const uint16_t*)a.q)[off]);
    }
    // the selection's rows through the page table, once
    for (int j = threadIdx.x; j < a.k; j += blockDim.x) {
        const int s = sel[j];
        rows[j] = s >= 0 ? (int64_t)pt[s / bs] * bs + s % bs : -1;
    }
    __syncthreads();
    auto elem = [&](int64_t row, int c) -> float {
        const size_t off = (size_t)row * W + c;
        if (a.kv_dtype == 0) return ((const float*)a.kv)[off];
        if (a.kv_dtype == 1) return bf16_to_f32(((const uint16_t*)a.kv)[off]);
        return e4m3_to_f32(((const uint8_t*)a.kv)[off]) * a.kv_scales[row];
    };
    // fp32 rows of at most 128 values whose sizes are multiples of 4: rows
    // read by 16-byte loads all in flight at once (same order of additions)
    const bool vec = f32 && (W & 3) == 0 && (D & 3) == 0 && W <= 4 * GEN_MAX_W4;
    float lmax = -INFINITY;
    for (int j = threadIdx.x; j < a.k; j += blockDim.x) {
        const int64_t row = rows[j];
        float zj = -INFINITY;
        if (row >= 0) {
            float dot = 0.f;
            if (vec) {
                const f32x4* kr = (const f32x4*)((const float*)a.kv + (size_t)row * W);
                const int w4 = W >> 2;
                f32x4 kv[GEN_MAX_W4];
#pragma unroll
                for (int i = 0; i < GEN_MAX_W4; ++i) kv[i] = i < w4 ? kr[i] : (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int i = 0; i < GEN_MAX_W4; ++i) {
                    if (i < w4) {
                        dot = fmaf(qv[4 * i], kv[i][0], dot);
                        dot = fmaf(qv[4 * i + 1], kv[i][1], dot);
                        dot = fmaf(qv[4 * i + 2], kv[i][2], dot);
                        dot = fmaf(qv[4 * i + 3], kv[i][3], dot);
                    }
                }
            } else {
#pragma unroll 8
                for (int c = 0; c < W; ++c) dot = fmaf(qv[c], elem(row, c), dot);
            }
            zj = dot * a.scale;
        }
        z[j] = zj;
        lmax = fmaxf(lmax, zj);
    }
    red[threadIdx.x] = lmax;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (threadIdx.x < off) red[threadIdx.x] = fmaxf(red[threadIdx.x], red[threadIdx.x + off]);
        __syncthreads();
    }
    const float mx = red[0];
    __syncthreads();
    float lsum = 0.f;
    for (int j = threadIdx.x; j < a.k; j += blockDim.x) {
        const float p = mx == -INFINITY || rows[j] < 0 ? 0.f : __expf(z[j] - mx);
        z[j] = p;
        lsum += p;
    }
    red[threadIdx.x] = lsum;
    __syncthreads();
    for (int off = 128; off > 0; off >>= 1) {
        if (threadIdx.x < off) red[threadIdx.x] += red[threadIdx.x + off];
        __syncthreads();
    }
    const float den = red[0];
    const float inv = den > 0.f ? 1.f / den : 0.f;
    if (vec) {
        // 4 value columns a thread (D <= 128: at most 32 column groups), the
        // selection split over 256 / (D / 4) groups of threads, GEN_PV_BATCH
        // rows in flight per thread; the groups' sums are added in group order
        __shared__ f32x4 part[256];
        const int nc4 = D >> 2, groups = 256 / nc4;
        const int c4 = threadIdx.x % nc4, g = threadIdx.x / nc4;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (g < groups) {
            for (int j0 = g; j0 < a.k; j0 += groups * GEN_PV_BATCH) {
                f32x4 v[GEN_PV_BATCH];
                float p[GEN_PV_BATCH];
#pragma unroll
                for (int u = 0; u < GEN_PV_BATCH; ++u) {
                    const int j = j0 + u * groups;
                    const int64_t row = j < a.k ? rows[j] : -1;   // padding has p = 0: read row 0
                    p[u] = j < a.k ? z[j] : 0.f;
                    v[u] = ((const f32x4*)((const float*)a.kv + (size_t)(row < 0 ? 0 : row) * W))[c4];
                }
#pragma unroll
                for (int u = 0; u < GEN_PV_BATCH; ++u) {
                    acc[0] = fmaf(p[u], v[u][0], acc[0]);
                    acc[1] = fmaf(p[u], v[u][1], acc[1]);
                    acc[2] = fmaf(p[u], v[u][2], acc[2]);
                    acc[3] = fmaf(p[u], v[u][3], acc[3]);
                }
            }
        }
        part[threadIdx.x] = acc;
        __syncthreads();
        for (int c = threadIdx.x; c < D; c += blockDim.x) {
            float sum = 0.f;
            for (int gg = 0; gg < groups; ++gg) sum += part[gg * nc4 + (c >> 2)][c & 3];
            ((float*)a.out)[((size_t)t * a.n_heads + h) * D + c] = sum * inv;
        }
    } else
    for (int c = threadIdx.x; c < D; c += blockDim.x) {
        float acc = 0.f;
#pragma unroll 8
        for (int j = 0; j < a.k; ++j) {
            const int64_t row = rows[j];   // padding has p = 0: read row 0 instead
            acc = fmaf(z[j], elem(row < 0 ? 0 : row, c), acc);
        }
        const size_t off = ((size_t)t * a.n_heads + h) * D + c;
        if (f32) ((float*)a.out)[off] = acc * inv;
        else ((uint16_t*)a.out)[off] = (uint16_t)f32_to_bf16(acc * inv);
    }
    if (a.lse && threadIdx.x == 0)
        a.lse[(size_t)t * a.n_heads + h] = den > 0.f ? mx + logf(den) : -INFINITY;
}

// ---------------------------------------------------------------------------
// 128-head path (bf16 or e4m3 latent, d = 512, r = 64, heads a multiple of
// 128): one workgroup per (query row, 128 heads, slice of the selection),
// the slice computed by mla_slice (mla_dev.h).  With several slices per row,
// each stores its normalised partial (fp16 with a power-of-two scale) and
// its log-sum-exp at its slice index, and mla_combine merges them.
template <bool FP8>
__global__ __attribute__((amdgpu_flat_work_group_size(M_THREADS, M_THREADS), amdgpu_waves_per_eu(1, 1)))
void mla_h128(MlaArgs a0, int slice) {
    const MlaArgs a = mla_layer_args(a0, blockIdx.z);
    const Geometry& G = a.g;
    const int hgroups = a.n_heads / M3_HEADS;
    const int unit = blockIdx.x;
    const int t = unit / hgroups, hg = unit % hgroups;
    const int sp = blockIdx.y, S = a.splits;
    const int j_begin = sp * slice;
    const int nslots = max(0, min(a.k, j_begin + slice) - j_begin);
    __shared__ MlaSliceLds L;
    const int r = row_request(G, t);
    MlaAcc acc;
    mla_slice<FP8, !FP8>(a, t, hg * M3_HEADS, a.indices + (size_t)t * a.k + j_begin,
                   G.page_table + (size_t)r * G.max_blocks, nslots, L, acc);
    if (S == 1) mla_store_final(a, t, hg * M3_HEADS, acc, L);
    else mla_store_partial(a, t, hg * M3_HEADS, sp, acc, L);
}

// Which kernel serves an MLA call.
int mla_path(int kv_dtype, int d_latent, int d_rope, int n_heads) {
    if (d_latent != M_DL || d_rope != M_DR) return MLA_PATH_GENERIC;
    if ((kv_dtype == 1 || kv_dtype == 2) && n_heads % M3_HEADS == 0) return MLA_PATH_H128;
    if ((kv_dtype == 1 || kv_dtype == 2) && n_heads % MLA_HEADS_PER_WG == 0) return MLA_PATH_H64;
    return MLA_PATH_GENERIC;
}

bool mla_fast_path(int kv_dtype, int d_latent, int d_rope, int n_heads, int block_size) {
    (void)block_size;
    return mla_path(kv_dtype, d_latent, d_rope, n_heads) != MLA_PATH_GENERIC;
}

constexpr int MLA_MIN_SLICE = 128;   // fewest selected tokens per split
// Splits per query row.  Decode: enough workgroups to cover the chip, at
// least 128 selected tokens per split; the 128-head path also keeps each
// slice within its row-id buffer.
int mla_splits(int path, int T, int n_heads, int k, bool prefill) {
    if (path == MLA_PATH_GENERIC) return 1;
    const int min_s = path == MLA_PATH_H128 ? (k + M3_MAX_SLICE - 1) / M3_MAX_SLICE : 1;
    if (prefill) return min_s;
    const int per_row = n_heads / (path == MLA_PATH_H128 ? M3_HEADS : MLA_HEADS_PER_WG);
    const int units = T * per_row;
    const int target = path == MLA_PATH_H128 ? device_cu_count() : 2 * device_cu_count();
    int s = 1;
    while (units * s < target && k / (2 * s) >= MLA_MIN_SLICE) s <<= 1;
    return max(s, min_s);
}

hipError_t launch_mla(const MlaArgs& a, bool prefill, hipStream_t s) {
    // a zero logit scale takes the generic kernel (the 128-head tile folds
    // the scale's sign into the queries and needs it nonzero)
    const int path = a.scale == 0.f ? MLA_PATH_GENERIC : mla_path(a.kv_dtype, a.d_latent, a.d_rope, a.n_heads);
    if (path == MLA_PATH_H128) {
        const int S = a.splits;
        int slice = (a.k + S - 1) / S;
        slice = (slice + M_TILE - 1) / M_TILE * M_TILE;
        if (slice > M3_MAX_SLICE) return hipErrorInvalidValue;
        const dim3 grid(a.g.T * (a.n_heads / M3_HEADS), S, a.n_layers);
        if (a.kv_dtype == 2) hipLaunchKernelGGL(mla_h128<true>, grid, dim3(M_THREADS), 0, s, a, slice);
        else hipLaunchKernelGGL(mla_h128<false>, grid, dim3(M_THREADS), 0, s, a, slice);
        hipError_t e = hipGetLastError();
        if (e == hipSuccess && S > 1) {
            launch_combine(a, s);
            e = hipGetLastError();
        }
        return e;
    }
    if (a.n_layers != 1) return hipErrorInvalidValue;   // several layers: the 128-head path only
    if (path == MLA_PATH_H64) {
        const int hgroups = a.n_heads / MLA_HEADS_PER_WG;
        const bool split = a.splits > 1;
        const int S = split ? a.splits : 1;
        int slice = (a.k + S - 1) / S;
        slice = (slice + M_TILE - 1) / M_TILE * M_TILE;
        dim3 grid(a.g.T * hgroups, S);
        const bool fp8 = a.kv_dtype == 2;
        if (split) {
            if (fp8) hipLaunchKernelGGL((mla_bf16_mfma<true, true>), grid, dim3(M_THREADS), 0, s, a, slice);
            else hipLaunchKernelGGL((mla_bf16_mfma<false, true>), grid, dim3(M_THREADS), 0, s, a, slice);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            launch_combine(a, s);
        } else {
            if (fp8) hipLaunchKernelGGL((mla_bf16_mfma<true, false>), grid, dim3(M_THREADS), 0, s, a, slice);
            else hipLaunchKernelGGL((mla_bf16_mfma<false, false>), grid, dim3(M_THREADS), 0, s, a, slice);
        }
        return hipGetLastError();
    }
    if (path != MLA_PATH_GENERIC) return hipErrorInvalidValue;
    const size_t shm = sizeof(int64_t) * (size_t)a.k + sizeof(float) * ((size_t)a.d_latent + a.d_rope + a.k);
    hipLaunchKernelGGL(mla_generic, dim3(a.g.T * a.n_heads), dim3(256), shm, s, a);
    return hipGetLastError();
}

}  // namespace dsa
