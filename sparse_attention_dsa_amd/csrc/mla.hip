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

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Split partials are stored as fp16 with one power-of-two scale per (query
// row, head, slice): the head's largest |value| times 2^k lies in
// [2^14, 2^15), so every value keeps 11 significant bits relative to it and
// none overflows.  The combine multiplies by 2^-k.
__device__ __forceinline__ int part_exponent(float amax) {
    if (!(amax > 0.f)) return 0;
    const int e = (int)((__float_as_uint(amax) >> 23) & 0xFFu) - 126;   // amax in [2^(e-1), 2^e)
    return max(-100, min(100, 15 - e));
}
__device__ __forceinline__ float pow2i(int k) { return __uint_as_float((uint32_t)(127 + k) << 23); }
__device__ __forceinline__ uint32_t pack_f16x2(float x, float y) {
    const _Float16 hx = (_Float16)x, hy = (_Float16)y;
    return (uint32_t)__builtin_bit_cast(uint16_t, hx) | ((uint32_t)__builtin_bit_cast(uint16_t, hy) << 16);
}

typedef __attribute__((address_space(3))) void* lds_vptr;
typedef __attribute__((address_space(3))) s16x4* lds_s16x4_ptr;

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
        float amax = 0.f;
#pragma unroll
        for (int ct = 0; ct < M_DL / 16; ++ct)
#pragma unroll
            for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(oacc[ct][i]));
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
__global__ __launch_bounds__(256) void mla_combine(MlaArgs a) {
    const int lane = threadIdx.x & 63;
    const size_t th = (size_t)blockIdx.x * 4 + (threadIdx.x >> 6);   // (t, h), one wave each
    if (th >= (size_t)a.g.T * a.n_heads) return;
    const int S = a.splits;
    const float* pl = a.part_lse + 2 * th * S;   // per slice: lse, 2^-k
    const uint16_t* po = a.part_o + th * S * M_DL + 8 * lane;
    float mx = -INFINITY;
    for (int s = 0; s < S; ++s) mx = fmaxf(mx, pl[2 * s]);
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
    if (mx != -INFINITY) {
        for (int s0 = 0; s0 < S; s0 += 4) {
            u32x4 h[4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
                if (s0 + u < S) h[u] = *(const u32x4*)(po + (size_t)(s0 + u) * M_DL);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (s0 + u >= S) break;
                const float wgt = __expf(pl[2 * (s0 + u)] - mx);
                den += wgt;
                const float ws = wgt * pl[2 * (s0 + u) + 1];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const uint16_t b = (uint16_t)(h[u][i >> 1] >> (16 * (i & 1)));
                    acc[i] += ws * (float)__builtin_bit_cast(_Float16, b);
                }
            }
        }
        const float inv = 1.f / den;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] *= inv;
    }
    uint16_t* op = (uint16_t*)a.out + th * M_DL + 8 * lane;
    u32x4 w;
#pragma unroll
    for (int i = 0; i < 4; ++i) w[i] = f32_to_bf16(acc[2 * i]) | (f32_to_bf16(acc[2 * i + 1]) << 16);
    *(u32x4*)op = w;
    if (a.lse && lane == 0) a.lse[th] = mx == -INFINITY ? -INFINITY : mx + logf(den);
}

// Generic path: any dims and head counts, fp32 / bf16 / e4m3 latent.  One
// workgroup per (query row, head); logits and probabilities in LDS.
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
    float lmax = -INFINITY;
    for (int j = threadIdx.x; j < a.k; j += blockDim.x) {
        const int64_t row = rows[j];
        float zj = -INFINITY;
        if (row >= 0) {
            float dot = 0.f;
#pragma unroll 8
            for (int c = 0; c < W; ++c) dot = fmaf(qv[c], elem(row, c), dot);
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
// 128-head path (bf16 latent, d = 512, r = 64, heads a multiple of 128): a
// workgroup owns one query row, 128 heads (32 per wave) and a slice of the
// row's selection, so every selected latent row is fetched once per slice
// and each LDS fragment read feeds 32 heads.  Tiles of 32 tokens stream
// through a 4-deep ring of LDS buffers by global_load_lds_dwordx4 (three
// tiles in flight while one is computed); the physical row ids of the whole
// slice are resolved through the page table once, up front.
//   S^T = K Q^T    v_mfma_f32_32x32x16_bf16: A = 32 token rows of the tile
//                  (LDS), B = 32 heads' queries (registers, 36 k-steps);
//   O^T += V^T P^T  A = V^T fragments by ds_read_b64_tr_b16 from the same
//                  rows, B = probabilities straight from S^T's accumulator
//                  layout (token order inside each 16-token k-step permuted
//                  alike on both sides); O^T (512 x 32 per wave) lives in
//                  accumulation registers.
// Softmax in the exp2 domain against a fixed reference per head: the max of
// the first tile with a visible token.  Probabilities are exp2(z - ref), at
// most 2^64 when no later logit exceeds the reference by more than 64 (fp32
// and bf16 hold that range, and O^T = sum p v / sum p does not depend on the
// reference), so the 256 accumulation registers are never rescaled.  A slice
// where some logit does exceed it is computed again with the largest logit
// seen as the reference.
constexpr int M3_HEADS = 128;
constexpr int M3_NBUF = 4;
constexpr int M3_MAX_SLICE = 2048;
constexpr int M3_DMA_PER_WAVE = M_TILE_BYTES / 1024 / 4;    // 9 x 1 KB per wave per tile
constexpr int M3_KPF = 4;     // K fragments in flight
constexpr int M3_VPF = 3;     // V^T fragments in flight
typedef float f32x16 __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16 mfma_bf16_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 32-bit LDS address of a pointer into a __shared__ array
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)p;
}

// max(a, b, c) in one instruction (fmaxf would first canonicalize every
// input it cannot prove canonical; no NaN reaches these)
__device__ __forceinline__ float max3f(float a, float b, float c) {
    float r;
    asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
    return r;
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier that orders LDS traffic only: unlike __syncthreads() it
// does not wait for this wave's outstanding global loads (the ring's
// transfers in flight), which the loop accounts for with wait_vmcnt.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <bool SPLIT>
__global__ __attribute__((amdgpu_flat_work_group_size(M_THREADS, M_THREADS), amdgpu_waves_per_eu(1, 1)))
void mla_h128(MlaArgs a, int slice) {
    const Geometry& G = a.g;
    const int hgroups = a.n_heads / M3_HEADS;
    const int unit = blockIdx.x;
    const int t = unit / hgroups, hg = unit % hgroups;
    const int sp = blockIdx.y;
    const int j_begin = sp * slice;
    const int nslots = max(0, min(a.k, j_begin + slice) - j_begin);
    const int ntiles = (nslots + M_TILE - 1) / M_TILE;

    __shared__ __attribute__((aligned(1024))) uint8_t Ks[M3_NBUF][M_TILE_BYTES];
    __shared__ int32_t rows[M3_MAX_SLICE];                 // physical row per slot (0 for padding)
    __shared__ uint32_t tvalid[M3_MAX_SLICE / M_TILE];     // per tile: bit s = slot s holds a token

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int hh = lane >> 5, c32 = lane & 31;
    const int head = hg * M3_HEADS + wave * 32 + c32;

    // queries first (needed last), then the slice's rows: every selection
    // index load, then every page-table load, so each waits one round trip
    u32x4 qf[M_DQK / 16];
    {
        const uint16_t* qp = (const uint16_t*)a.q + ((size_t)t * a.n_heads + head) * M_DQK + 8 * hh;
#pragma unroll
        for (int ks = 0; ks < M_DQK / 16; ++ks) qf[ks] = *(const u32x4*)(qp + 16 * ks);
    }
    {
        constexpr int PER = M3_MAX_SLICE / M_THREADS;
        const int r = row_request(G, t);
        const int32_t* sel = a.indices + (size_t)t * a.k + j_begin;
        const int32_t* pt = G.page_table + (size_t)r * G.max_blocks;
        const int bs = G.block_size;
        const bool pow2 = (bs & (bs - 1)) == 0;
        const int bsh = __builtin_ctz((unsigned)bs);
        int sj[PER], blk[PER], slot[PER];
#pragma unroll
        for (int u = 0; u < PER; ++u) {
            const int j = tid + u * M_THREADS;
            sj[u] = j < nslots ? sel[j] : -1;
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
            if (j < ntiles * M_TILE) rows[j] = ok ? blk[u] * bs + slot[u] : 0;
            const unsigned long long m = __ballot(ok);   // 64 slots = two tiles
            if (lane == 0 && j < ntiles * M_TILE) tvalid[j / M_TILE] = (uint32_t)m;
            if (lane == 32 && j < ntiles * M_TILE) tvalid[j / M_TILE] = (uint32_t)(m >> 32);
        }
    }
    __syncthreads();

    // Tile layout in LDS (32 rows of 72 16-byte units): the 1 KB block
    // (r >> 3, u >> 3) sits at 1024 (9 (r >> 3) + (u >> 3)); inside it row
    // r & 7 takes 128 B and holds its units u & 7 XOR-permuted by r & 7, so
    // that one unit of the block's 8 rows covers all banks:
    //   tile_off(r, u) = 1024 (9 (r >> 3) + (u >> 3)) + 16 (8 (r & 7) + ((u & 7) ^ (r & 7))).
    // Wave w moves rows 8w .. 8w+7: its instruction i covers units 8i .. 8i+7
    // of each, lane l taking row 8w + (l >> 3) and unit 8i + ((l & 7) ^ (l >> 3)),
    // which the transfer writes at 16 l of the instruction's 1 KB block, i.e.
    // at tile_off.  All nine instructions of a lane read the same row, so a
    // tile costs one row id per lane and immediate offsets.
    static_assert(M_TILE == 32 && M_THREADS == 256 && M_ROW_UNITS == 72 && M3_DMA_PER_WAVE == 9,
                  "tile layout: 4 waves x 8 rows, 9 blocks of 8 units per row");
    const int dma_col = 16 * ((lane & 7) ^ (lane >> 3));
    auto issue = [&](int tile, int b) {
        const int row = rows[M_TILE * tile + 8 * wave + (lane >> 3)];
        const uint8_t* src = (const uint8_t*)a.kv + (size_t)row * M_ROW_BYTES + dma_col;
        uint8_t* dst = &Ks[b][0] + 1024 * M3_DMA_PER_WAVE * wave;
#pragma unroll
        for (int i = 0; i < M3_DMA_PER_WAVE; ++i)
            __builtin_amdgcn_global_load_lds((const void*)(src + 128 * i), (lds_vptr)(dst + 1024 * i), 16, 0, 0);
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
    int pv_base[2][2][2];   // [kk][rd][cb & 1], + 1024 (cb / 2)
    {
        const int s16 = lane & 15, jj = s16 >> 2, q = s16 & 3;
        const int v = 2 * ((lane >> 4) & 1) + (q >> 1);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int rd = 0; rd < 2; ++rd) {
                const int tok = 16 * kk + 8 * rd + 4 * hh + jj;
#pragma unroll
                for (int c1 = 0; c1 < 2; ++c1)
                    pv_base[kk][rd][c1] = 9216 * (tok >> 3) + 128 * (tok & 7) + 16 * ((4 * c1 + v) ^ (tok & 7)) +
                                          8 * (q & 1);
            }
    }

    __shared__ uint32_t redo;
    f32x16 oacc[M_DL / 32];
    float m_ref = -INFINITY, m_seen = -INFINITY, l_run = 0.f;
    const float zscale = a.scale * LOG2E;

    for (int pass = 0;; ++pass) {
#pragma unroll
    for (int cb = 0; cb < M_DL / 32; ++cb)
#pragma unroll
        for (int i = 0; i < 16; ++i) oacc[cb][i] = 0.f;
    l_run = 0.f;
    bool overflow = false;
    if (tid == 0) redo = 0u;

#pragma unroll
    for (int b = 0; b < M3_NBUF - 1; ++b)
        if (b < ntiles) issue(b, b);

    for (int i = 0; i < ntiles; ++i) {
        // this wave's transfers of tile i are done once at most the ones of
        // the (up to two) later tiles already issued are outstanding
        const int later = min(M3_NBUF - 2, ntiles - 1 - i);
        if (later >= 2) wait_vmcnt<2 * M3_DMA_PER_WAVE>();
        else if (later == 1) wait_vmcnt<M3_DMA_PER_WAVE>();
        else wait_vmcnt<0>();
        lds_barrier();   // everyone's part of tile i landed; tile i-1's buffer is free
        const uint8_t* Kb = &Ks[i % M3_NBUF][0];

        const uint32_t vmask = tvalid[i];   // tokens present in the tile (bit per slot)

        // S^T: K fragments read M3_KPF steps ahead of their MFMA; the nine
        // transfers of tile i+3 (into the buffer tile i-1 has left) are
        // spread over the MFMAs, one after every fourth, so that issuing them
        // never holds up the matrix core for long
        f32x16 st;
        {
            constexpr int NK = M_DQK / 16;
            const int nt = i + M3_NBUF - 1;
            const bool iss = nt < ntiles;
            const uint8_t* dsrc = (const uint8_t*)a.kv +
                                  (size_t)rows[M_TILE * min(nt, ntiles - 1) + 8 * wave + (lane >> 3)] * M_ROW_BYTES +
                                  dma_col;
            auto qk = [&](const uint8_t* kbuf, uint8_t* dst, bool dma) {
                u32x4 kb[M3_KPF];
#pragma unroll
                for (int j = 0; j < M3_KPF; ++j) kb[j] = *(const u32x4*)(kbuf + qk_base[j & 3] + 1024 * (j >> 2));
                __builtin_amdgcn_sched_group_barrier(0x100, M3_KPF, 0);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int ks = 0; ks < NK; ++ks) {
                    if (ks == 0) st = mfma_bf16_32x32x16(as_bf16x8(kb[0]), as_bf16x8(qf[0]), f32x16{});
                    else st = mfma_bf16_32x32x16(as_bf16x8(kb[ks % M3_KPF]), as_bf16x8(qf[ks]), st);
                    if (ks + M3_KPF < NK) {
                        const int kn = ks + M3_KPF;
                        kb[ks % M3_KPF] = *(const u32x4*)(kbuf + qk_base[kn & 3] + 1024 * (kn >> 2));
                    }
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // then one LDS read
                    if (dma && (ks & 3) == 1) {
                        // Issued by inline asm: the compiler does not track it as an
                        // LDS write, so it puts no wait for it before the fragment
                        // reads of tile i, which use another buffer (the loop's own
                        // vector-memory waits count these transfers).  M0 holds the
                        // LDS address and is restored afterwards; no immediate
                        // offset, which the LDS destination would include as well.
                        const uint32_t m0v = lds_addr(dst + 1024 * (ks >> 2));
                        const uint8_t* gsrc = dsrc + 128 * (ks >> 2);
                        uint32_t saved;
                        asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\t"
                                     "global_load_lds_dwordx4 %1, off\n\ts_mov_b32 m0, %0"
                                     : "=&s"(saved) : "v"(gsrc), "s"(m0v));
                    }
                }
            };
            uint8_t* ddst = &Ks[nt % M3_NBUF][0] + 1024 * M3_DMA_PER_WAVE * wave;
            if (iss) qk(Kb, ddst, true);
            else qk(Kb, ddst, false);
        }
        // element e of this lane: token 8(e/4) + 4hh + e%4, head c32.
        // The tile's largest logit comes from the raw scores' extreme in the
        // direction of the scale's sign, slots without a token excluded (the
        // tiles with padding only); probabilities are exp2(s * zscale - ref)
        // by one fused multiply-add, zero for those slots.
        const bool full = vmask == 0xFFFFFFFFu;
        float ext;
        if (zscale >= 0.f) {
            float sm[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) sm[e] = st[e];
            if (!full) {
#pragma unroll
                for (int e = 0; e < 16; ++e)
                    sm[e] = (vmask >> (8 * (e >> 2) + 4 * hh + (e & 3))) & 1u ? sm[e] : -INFINITY;
            }
            ext = fmaxf(max3f(max3f(sm[0], sm[1], sm[2]), max3f(sm[3], sm[4], sm[5]), max3f(sm[6], sm[7], sm[8])),
                        max3f(max3f(sm[9], sm[10], sm[11]), max3f(sm[12], sm[13], sm[14]), sm[15]));
        } else {
            ext = INFINITY;
#pragma unroll
            for (int e = 0; e < 16; ++e)
                if (full || ((vmask >> (8 * (e >> 2) + 4 * hh + (e & 3))) & 1u)) ext = fminf(ext, st[e]);
        }
        float tmax = vmask ? ext * zscale : -INFINITY;
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
        if (!full) {
#pragma unroll
            for (int e = 0; e < 16; ++e)
                p[e] = (vmask >> (8 * (e >> 2) + 4 * hh + (e & 3))) & 1u ? p[e] : 0.f;
        }
        {
            float s8[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) s8[e] = p[e] + p[e + 8];
#pragma unroll
            for (int e = 0; e < 4; ++e) s8[e] += s8[e + 4];
            l_run += (s8[0] + s8[2]) + (s8[1] + s8[3]);
        }
        bf16x8 pb[2];
#pragma unroll
        for (int kk = 0; kk < 2; ++kk)
#pragma unroll
            for (int e = 0; e < 8; ++e) pb[kk][e] = (__bf16)p[8 * kk + e];

        // O^T += V^T P^T: V^T fragments (two transposing reads each) read
        // M3_VPF MFMAs ahead; the 16 accumulators rotate between dependent updates
        {
            constexpr int NV = 2 * (M_DL / 32);
            auto vread = [&](int n, s16x4& v0, s16x4& v1) {
                const int kk = n / (M_DL / 32), cb = n % (M_DL / 32);
                v0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4_ptr)(Kb + pv_base[kk][0][cb & 1] + 1024 * (cb >> 1)));
                v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (lds_s16x4_ptr)(Kb + pv_base[kk][1][cb & 1] + 1024 * (cb >> 1)));
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
        }
    }
    // the whole workgroup agrees on a second pass (it shares the barriers)
    if (__ballot(overflow) && lane == 0) redo = 1u;
    __syncthreads();
    if (pass > 0 || redo == 0u) break;
    m_ref = m_seen;
    __syncthreads();
    }
    const float m_run = m_ref;

    // ---- epilogue: element e of block cb is O^T[32cb + 8(e/4) + 4hh + e%4][head]
    const float l_tot = l_run + lane_xor32(l_run, lane);
    const bool empty = l_tot == 0.f;
    const float inv = empty ? 0.f : 1.f / l_tot;
    const float lse_nat = empty ? -INFINITY : (m_run + log2f(l_tot)) * LN2;
    if (SPLIT) {
        // the head's values sit in lanes c32 and c32 + 32
        float amax = 0.f;
#pragma unroll
        for (int cb = 0; cb < M_DL / 32; ++cb)
#pragma unroll
            for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(oacc[cb][e]));
        amax = fmaxf(amax, __shfl_xor(amax, 32));
        const int k = part_exponent(amax * inv);
        const float sc = inv * pow2i(k);
        const size_t pidx = ((size_t)t * a.n_heads + head) * a.splits + sp;
        uint16_t* po = a.part_o + pidx * M_DL;
#pragma unroll
        for (int cb = 0; cb < M_DL / 32; ++cb)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                u32x2 w;
                w[0] = pack_f16x2(oacc[cb][4 * e4] * sc, oacc[cb][4 * e4 + 1] * sc);
                w[1] = pack_f16x2(oacc[cb][4 * e4 + 2] * sc, oacc[cb][4 * e4 + 3] * sc);
                *(u32x2*)(po + 32 * cb + 8 * e4 + 4 * hh) = w;
            }
        if (hh == 0) {
            a.part_lse[2 * pidx] = lse_nat;
            a.part_lse[2 * pidx + 1] = pow2i(-k);
        }
    } else {
        uint16_t* op = (uint16_t*)a.out + ((size_t)t * a.n_heads + head) * M_DL;
#pragma unroll
        for (int cb = 0; cb < M_DL / 32; ++cb)
#pragma unroll
            for (int e4 = 0; e4 < 4; ++e4) {
                u32x2 w;
                w[0] = f32_to_bf16(oacc[cb][4 * e4] * inv) | (f32_to_bf16(oacc[cb][4 * e4 + 1] * inv) << 16);
                w[1] = f32_to_bf16(oacc[cb][4 * e4 + 2] * inv) | (f32_to_bf16(oacc[cb][4 * e4 + 3] * inv) << 16);
                *(u32x2*)(op + 32 * cb + 8 * e4 + 4 * hh) = w;
            }
        if (a.lse && hh == 0) a.lse[(size_t)t * a.n_heads + head] = lse_nat;
    }
}

// Which kernel serves an MLA call.
int mla_path(int kv_dtype, int d_latent, int d_rope, int n_heads) {
    if (d_latent != M_DL || d_rope != M_DR) return MLA_PATH_GENERIC;
    if (kv_dtype == 1 && n_heads % M3_HEADS == 0) return MLA_PATH_H128;
    if ((kv_dtype == 1 || kv_dtype == 2) && n_heads % MLA_HEADS_PER_WG == 0) return MLA_PATH_H64;
    return MLA_PATH_GENERIC;
}

bool mla_fast_path(int kv_dtype, int d_latent, int d_rope, int n_heads, int block_size) {
    (void)block_size;
    return mla_path(kv_dtype, d_latent, d_rope, n_heads) != MLA_PATH_GENERIC;
}

#ifndef MLA_MIN_SLICE
#define MLA_MIN_SLICE 128
#endif
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
    const int path = mla_path(a.kv_dtype, a.d_latent, a.d_rope, a.n_heads);
    if (path == MLA_PATH_H128) {
        const int S = a.splits;
        int slice = (a.k + S - 1) / S;
        slice = (slice + M_TILE - 1) / M_TILE * M_TILE;
        if (slice > M3_MAX_SLICE) return hipErrorInvalidValue;
        const dim3 grid(a.g.T * (a.n_heads / M3_HEADS), S);
        if (S > 1) {
            hipLaunchKernelGGL(mla_h128<true>, grid, dim3(M_THREADS), 0, s, a, slice);
            const hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL(mla_combine, dim3((a.g.T * a.n_heads + 3) / 4), dim3(256), 0, s, a);
        } else {
            hipLaunchKernelGGL(mla_h128<false>, grid, dim3(M_THREADS), 0, s, a, slice);
        }
        return hipGetLastError();
    }
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
            hipLaunchKernelGGL(mla_combine, dim3((a.g.T * a.n_heads + 3) / 4), dim3(256), 0, s, a);
        } else {
            if (fp8) hipLaunchKernelGGL((mla_bf16_mfma<true, false>), grid, dim3(M_THREADS), 0, s, a, slice);
            else hipLaunchKernelGGL((mla_bf16_mfma<false, false>), grid, dim3(M_THREADS), 0, s, a, slice);
        }
        return hipGetLastError();
    }
    const size_t shm = sizeof(int64_t) * (size_t)a.k + sizeof(float) * ((size_t)a.d_latent + a.d_rope + a.k);
    hipLaunchKernelGGL(mla_generic, dim3(a.g.T * a.n_heads), dim3(256), shm, s, a);
    return hipGetLastError();
}

}  // namespace dsa
