// Sparse MQA-mode MLA on gfx950.
//
// Per query row t and head h (SemiAnalysis GLM-5.3 article, "MLA
// Modifications"): logits z_j = scale * q[t,h,:] . kv[s_j, 0:d+r] over the
// selected tokens s_j, out[t,h,:] = softmax(z) . kv[s_j, 0:d]; K and V are the
// same cached latent row, V being its first d columns.
//
// Fast path (d = 512, r = 64, 64-token blocks, bf16 or e4m3 latent, heads a
// multiple of 64): a workgroup owns one query row, 64 heads (16 per wave) and
// a contiguous slice of the row's selection.  Tiles of 32 selected tokens are
// gathered through the page table into LDS twice:
//   Ks  [32][576+8]  row-major, the A operand of S^T = K Q^T (k = latent dim);
//   Vt  [512][32]    transposed with an XOR swizzle, the A operand of
//                    O^T = V^T P^T (k = token).  The 8x8 bf16 transposes are
//                    done in registers between the global loads and the
//                    LDS stores.
// Queries stay in registers as the B operand of the logit MFMAs.  Computing
// S^T rather than S leaves each lane with one head and eight tokens, which is
// exactly the B-operand layout P^T needs for the PV MFMAs (the token order
// inside a 32-token step is permuted consistently on both sides), so the
// probabilities never leave registers.  Online softmax in the exp2 domain;
// each lane's O^T accumulators all belong to its own head, so the running
// rescale is a per-lane scalar.  Decode rows split their selection across
// workgroups and a second kernel merges the partial results by their
// log-sum-exp; prefill rows have enough parallelism without splitting.
#include "dsa_kernels.h"

namespace dsa {

constexpr int M_DL = 512, M_DR = 64, M_DQK = M_DL + M_DR;
constexpr int M_TILE = 32;                 // selected tokens per tile
constexpr int M_KS_STRIDE = M_DQK + 8;     // bf16 elements per Ks row (16 B pad)
constexpr int M_THREADS = 256;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;

// Slot order inside a 32-token tile: B-operand slot 8g + j of P^T holds the
// logit of token pi(g, j), where lane group g got tokens 4g..4g+3 from the
// first 16-token logit tile and 16+4g..16+4g+3 from the second.
__device__ __forceinline__ int slot_token(int g, int j) {
    return j < 4 ? 4 * g + j : 16 + 4 * g + (j - 4);
}

// 16-byte unit of row c of Vt that holds slot group g (XOR swizzle keeps the
// reads of 8 or 16 consecutive rows on distinct bank groups).
__device__ __forceinline__ int vt_unit(int c, int g) {
    return g ^ (((c >> 1) ^ (c >> 2)) & 3);
}

// Loads 8 latent columns [8*c8, 8*c8+8) of a cache row as 8 bf16 (16 bytes).
template <bool FP8>
__device__ __forceinline__ u32x4 load_cols8(const void* kv, const float* scales, int row, int c8) {
    if (!FP8) {
        return *(const u32x4*)((const uint16_t*)kv + (size_t)row * M_DQK + 8 * c8);
    } else {
        const u32x2 v = *(const u32x2*)((const uint8_t*)kv + (size_t)row * M_DQK + 8 * c8);
        const float sc = scales[row];
        u32x4 o;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t w = v[i >> 1] >> (16 * (i & 1));
            const float x0 = e4m3_to_f32(w & 0xFFu) * sc;
            const float x1 = e4m3_to_f32((w >> 8) & 0xFFu) * sc;
            o[i] = f32_to_bf16(x0) | (f32_to_bf16(x1) << 16);
        }
        return o;
    }
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

    __shared__ __attribute__((aligned(16))) uint16_t Ks[M_TILE * M_KS_STRIDE];
    __shared__ __attribute__((aligned(16))) uint16_t Vt[M_DL * M_TILE];
    __shared__ int32_t rows[2][M_TILE];   // physical rows of the current / next tile (-1: none)

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 4, col = lane & 15;
    const int head = hg * MLA_HEADS_PER_WG + wave * 16 + col;

    const int32_t* sel = a.indices + (size_t)t * a.k;
    const int32_t* pt = G.page_table + (size_t)r * G.max_blocks;
    const int nslots = max(0, j_end - j_begin);
    auto row_of = [&](int j) -> int32_t {     // slot j of the slice
        if (j >= nslots) return -1;
        const int s = sel[j_begin + j];
        return s < 0 ? -1 : pt[s / G.block_size] * G.block_size + s % G.block_size;
    };
    if (tid < M_TILE) rows[0][tid] = row_of(tid);

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
    __syncthreads();

    // Gather roles: V part -> token group gv (slots 8gv..8gv+7), column chunk cv.
    const int gv = tid & 3, cv = tid >> 2;             // cv in [0, 64)
    const int rope_tok = tid >> 3, rope_c8 = 64 + (tid & 7);

    for (int j0 = 0, buf = 0; j0 < nslots; j0 += M_TILE, buf ^= 1) {
        const int32_t* trow = rows[buf];
        // ---- gather tile into LDS, four tokens of the slot group at a time
#pragma unroll
        for (int half = 0; half < 2; ++half) {
            u32x4 v[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int row = trow[slot_token(gv, 4 * half + jj)];
                v[jj] = row >= 0 ? load_cols8<FP8>(a.kv, a.kv_scales, row, cv) : (u32x4){0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                *(u32x4*)(Ks + slot_token(gv, 4 * half + jj) * M_KS_STRIDE + 8 * cv) = v[jj];
            // 4x8 transpose: column cc of the chunk, these four slots in order.
#pragma unroll
            for (int cc = 0; cc < 8; ++cc) {
                const int sh = 16 * (cc & 1), w = cc >> 1;
                u32x2 o;
#pragma unroll
                for (int m = 0; m < 2; ++m) {
                    const uint32_t lo = (v[2 * m][w] >> sh) & 0xFFFFu;
                    const uint32_t hi = (v[2 * m + 1][w] >> sh) & 0xFFFFu;
                    o[m] = lo | (hi << 16);
                }
                const int c = 8 * cv + cc;
                *(u32x2*)(Vt + c * M_TILE + 8 * vt_unit(c, gv) + 4 * half) = o;
            }
        }
        {
            const int rrow = trow[rope_tok];
            const u32x4 vr = rrow >= 0 ? load_cols8<FP8>(a.kv, a.kv_scales, rrow, rope_c8)
                                       : (u32x4){0u, 0u, 0u, 0u};
            *(u32x4*)(Ks + rope_tok * M_KS_STRIDE + 8 * rope_c8) = vr;
        }
        __syncthreads();

        // ---- logits S^T for two 16-token halves: lane holds tokens 16tt+4g+i of head `col`
        float x[2][4];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            f32x4 s = {0.f, 0.f, 0.f, 0.f};
            const uint16_t* kp = Ks + (16 * tt + col) * M_KS_STRIDE + 8 * g;
#pragma unroll
            for (int ks = 0; ks < M_DQK / 32; ++ks)
                s = mfma_bf16_16x16x32(as_bf16x8(*(const u32x4*)(kp + 32 * ks)), as_bf16x8(qf[ks]), s);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tok = 16 * tt + 4 * g + i;
                const bool ok = trow[tok] >= 0;
                x[tt][i] = ok ? s[i] * zscale : -INFINITY;
            }
        }
        // ---- online softmax (per head = per lane column; reduce over the 4 lane groups)
        float tmax = fmaxf(fmaxf(fmaxf(x[0][0], x[0][1]), fmaxf(x[0][2], x[0][3])),
                           fmaxf(fmaxf(x[1][0], x[1][1]), fmaxf(x[1][2], x[1][3])));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
        const float m_new = fmaxf(m_run, tmax);
        float p[2][4];
        float psum = 0.f;
        float alpha = 1.f;
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
        u32x4 pb;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const int tt = m >> 1, i = 2 * (m & 1);
            pb[m] = f32_to_bf16(p[tt][i]) | (f32_to_bf16(p[tt][i + 1]) << 16);
        }
        // ---- O^T += V^T P^T
        const bf16x8 pbf = as_bf16x8(pb);
#pragma unroll
        for (int ct = 0; ct < M_DL / 16; ++ct) {
            const int c = 16 * ct + col;
            const u32x4 va = *(const u32x4*)(Vt + c * M_TILE + 8 * vt_unit(c, g));
            oacc[ct] = mfma_bf16_16x16x32(as_bf16x8(va), pbf, oacc[ct]);
        }
        if (tid < M_TILE) rows[buf ^ 1][tid] = row_of(j0 + M_TILE + tid);
        __syncthreads();
    }

    // ---- epilogue: lane holds O^T[c = 16ct + 4g + i][head]
    const bool empty = l_run == 0.f;
    const float inv = empty ? 0.f : 1.f / l_run;
    const float lse_nat = empty ? -INFINITY : (m_run + log2f(l_run)) * LN2;
    if (SPLIT) {
        float* po = a.part_o + (((size_t)t * a.n_heads + head) * a.splits + sp) * M_DL;
#pragma unroll
        for (int ct = 0; ct < M_DL / 16; ++ct)
            *(f32x4*)(po + 16 * ct + 4 * g) = oacc[ct] * inv;
        if (g == 0) a.part_lse[((size_t)t * a.n_heads + head) * a.splits + sp] = lse_nat;
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
__global__ __launch_bounds__(128) void mla_combine(MlaArgs a) {
    const size_t th = blockIdx.x;             // (t, h)
    const int c4 = threadIdx.x;               // 4 columns each
    const int S = a.splits;
    const float* pl = a.part_lse + th * S;
    float mx = -INFINITY;
    for (int s = 0; s < S; ++s) mx = fmaxf(mx, pl[s]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float den = 0.f;
    if (mx != -INFINITY) {
        for (int s = 0; s < S; ++s) {
            const float wgt = __expf(pl[s] - mx);
            den += wgt;
            acc += wgt * *(const f32x4*)(a.part_o + (th * S + s) * M_DL + 4 * c4);
        }
        acc *= 1.f / den;
    }
    uint16_t* op = (uint16_t*)a.out + th * M_DL + 4 * c4;
    u32x2 w;
    w[0] = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
    w[1] = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
    *(u32x2*)op = w;
    if (a.lse && c4 == 0) a.lse[th] = mx == -INFINITY ? -INFINITY : mx + logf(den);
}

// Generic path: any dims and head counts, fp32 / bf16 / e4m3 latent.  One
// workgroup per (query row, head); logits and probabilities in LDS.
__global__ __launch_bounds__(256) void mla_generic(MlaArgs a) {
    const Geometry& G = a.g;
    const int t = blockIdx.x / a.n_heads, h = blockIdx.x % a.n_heads;
    const int r = find_request(G.qsl, G.B, t);
    const int W = a.d_latent + a.d_rope, D = a.d_latent;
    extern __shared__ float smem[];
    float* qv = smem;            // [W]
    float* z = smem + W;         // [k]
    __shared__ float red[256];
    const bool f32 = a.kv_dtype == 0;
    for (int c = threadIdx.x; c < W; c += blockDim.x) {
        const size_t off = ((size_t)t * a.n_heads + h) * W + c;
        qv[c] = f32 ? ((const float*)a.q)[off] : bf16_to_f32(((const uint16_t*)a.q)[off]);
    }
    __syncthreads();
    auto elem = [&](int64_t row, int c) -> float {
        const size_t off = (size_t)row * W + c;
        if (a.kv_dtype == 0) return ((const float*)a.kv)[off];
        if (a.kv_dtype == 1) return bf16_to_f32(((const uint16_t*)a.kv)[off]);
        return e4m3_to_f32(((const uint8_t*)a.kv)[off]) * a.kv_scales[row];
    };
    const int32_t* sel = a.indices + (size_t)t * a.k;
    const int32_t* pt = G.page_table + (size_t)r * G.max_blocks;
    const int bs = G.block_size;
    float lmax = -INFINITY;
    for (int j = threadIdx.x; j < a.k; j += blockDim.x) {
        const int s = sel[j];
        float zj = -INFINITY;
        if (s >= 0) {
            const int64_t row = (int64_t)pt[s / bs] * bs + s % bs;
            float dot = 0.f;
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
        const float p = mx == -INFINITY ? 0.f : __expf(z[j] - mx);
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
        for (int j = 0; j < a.k; ++j) {
            const int s = sel[j];
            if (s < 0) continue;
            acc = fmaf(z[j], elem((int64_t)pt[s / bs] * bs + s % bs, c), acc);
        }
        const size_t off = ((size_t)t * a.n_heads + h) * D + c;
        if (f32) ((float*)a.out)[off] = acc * inv;
        else ((uint16_t*)a.out)[off] = (uint16_t)f32_to_bf16(acc * inv);
    }
    if (a.lse && threadIdx.x == 0)
        a.lse[(size_t)t * a.n_heads + h] = den > 0.f ? mx + logf(den) : -INFINITY;
}

bool mla_fast_path(int kv_dtype, int d_latent, int d_rope, int n_heads, int block_size) {
    (void)block_size;
    return (kv_dtype == 1 || kv_dtype == 2) && d_latent == M_DL && d_rope == M_DR &&
           n_heads % MLA_HEADS_PER_WG == 0;
}

// Splits per decode row: enough workgroups to cover the chip (~2 per CU),
// at least 128 selected tokens per split.
int mla_decode_splits(int T, int n_heads, int k) {
    const int units = T * (n_heads / MLA_HEADS_PER_WG);
    int s = 1;
    while (units * s < 512 && k / (2 * s) >= 128) s <<= 1;
    return s;
}

hipError_t launch_mla(const MlaArgs& a, bool prefill, hipStream_t s) {
    if (mla_fast_path(a.kv_dtype, a.d_latent, a.d_rope, a.n_heads, a.g.block_size)) {
        const int hgroups = a.n_heads / MLA_HEADS_PER_WG;
        const bool split = !prefill && a.splits > 1;
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
            hipLaunchKernelGGL(mla_combine, dim3(a.g.T * a.n_heads), dim3(M_DL / 4), 0, s, a);
        } else {
            if (fp8) hipLaunchKernelGGL((mla_bf16_mfma<true, false>), grid, dim3(M_THREADS), 0, s, a, slice);
            else hipLaunchKernelGGL((mla_bf16_mfma<false, false>), grid, dim3(M_THREADS), 0, s, a, slice);
        }
        return hipGetLastError();
    }
    const size_t shm = sizeof(float) * ((size_t)a.d_latent + a.d_rope + a.k);
    hipLaunchKernelGGL(mla_generic, dim3(a.g.T * a.n_heads), dim3(256), shm, s, a);
    return hipGetLastError();
}

}  // namespace dsa
