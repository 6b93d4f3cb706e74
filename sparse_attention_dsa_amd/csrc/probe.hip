// Streaming-read probe: the practical HBM read bandwidth of this device, the
// ceiling the HBM-bound kernels of the library are compared against.  Every
// byte of a buffer is read once with 16-byte non-temporal loads by a grid of 8
// workgroups per CU, each streaming one contiguous range; each workgroup folds
// what it read into one word (so the loads cannot be dropped) and writes it.
#include "dsa_kernels.h"
#include "dsa.h"

namespace dsa {

constexpr int PR_THREADS = 256;
constexpr int PR_UNROLL = 8;

__global__ __launch_bounds__(PR_THREADS) void stream_read(const uint8_t* __restrict__ buf, int64_t nbytes,
                                                          uint32_t* __restrict__ sink) {
    // workgroup b streams the contiguous range [v0, v1) of 16-byte vectors,
    // 32 KB per step (8 loads in flight per lane, each step's loads contiguous)
    const int64_t nvec = nbytes / 16;
    const int64_t per = (nvec + gridDim.x - 1) / gridDim.x;
    const int64_t v0 = min(nvec, (int64_t)blockIdx.x * per), v1 = min(nvec, v0 + per);
    const u32x4* p = (const u32x4*)buf;
    uint32_t acc = 0u;
    int64_t i = v0 + threadIdx.x;
    for (; i + (PR_UNROLL - 1) * PR_THREADS < v1; i += PR_UNROLL * PR_THREADS) {
        u32x4 v[PR_UNROLL];
#pragma unroll
        for (int u = 0; u < PR_UNROLL; ++u) v[u] = __builtin_nontemporal_load(p + i + u * PR_THREADS);
#pragma unroll
        for (int u = 0; u < PR_UNROLL; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
    }
    for (; i < v1; i += PR_THREADS) {
        const u32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
    }
    __shared__ uint32_t red[PR_THREADS / 64];
    for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        uint32_t x = 0u;
        for (int w = 0; w < PR_THREADS / 64; ++w) x ^= red[w];
        sink[blockIdx.x] = x;
    }
}

int probe_grid() { return 8 * device_cu_count(); }

// Random-page read probe: the pages a block-id list names, read the way the
// persistent indexer reads its key pages (the same grid of 2 four-wave
// workgroups per CU, equal contiguous shares of the list per wave, 2 pages
// in flight per wave, 1 KB non-temporal loads) but with no arithmetic: the
// memory system's rate for that access pattern.  Page b is page_bytes at
// pages + b page_bytes (a multiple of 1 KB, at most 8 KB) plus scale_bytes
// (0 or a multiple of 4, at most 256) at scales + b scale_bytes.  Each lane
// folds what it read into one word; sink[w][lane] for wave w.
constexpr int PP_WG_PER_CU = 2;
constexpr int PP_INFLIGHT = 2;

__global__ __launch_bounds__(256) void page_read(const uint8_t* __restrict__ pages, int page_kb,
                                                 const uint8_t* __restrict__ scales, int scale_bytes,
                                                 const int32_t* __restrict__ blocks, int n, uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int gw = blockIdx.x * 4 + (threadIdx.x >> 6), nw = gridDim.x * 4;
    const int p0 = (int)((long long)n * gw / nw), p1 = (int)((long long)n * (gw + 1) / nw);
    const int64_t pstride = 1024 * (int64_t)page_kb;
    const bool has_sc = 4 * lane < scale_bytes;
    uint32_t acc = 0u;
    for (int p = p0; p < p1; p += PP_INFLIGHT) {
        u32x4 v[PP_INFLIGHT][8];
        uint32_t sc[PP_INFLIGHT];
#pragma unroll
        for (int d = 0; d < PP_INFLIGHT; ++d) {
            const bool live = p + d < p1;
            const int64_t b = live ? blocks[p + d] : 0;
            const uint8_t* src = pages + b * pstride + 16 * lane;
#pragma unroll
            for (int c = 0; c < 8; ++c)
                v[d][c] = live && c < page_kb ? __builtin_nontemporal_load((const u32x4*)(src + 1024 * c))
                                              : (u32x4){0u, 0u, 0u, 0u};
            sc[d] = live && has_sc ? *(const uint32_t*)(scales + b * scale_bytes + 4 * lane) : 0u;
        }
#pragma unroll
        for (int d = 0; d < PP_INFLIGHT; ++d) {
#pragma unroll
            for (int c = 0; c < 8; ++c) acc ^= v[d][c][0] ^ v[d][c][1] ^ v[d][c][2] ^ v[d][c][3];
            acc ^= sc[d];
        }
    }
    sink[(size_t)gw * 64 + lane] = acc;
}

int page_probe_grid() { return PP_WG_PER_CU * device_cu_count(); }

// Row-gather probe: the rows a list names, gathered the way the 128-head
// sparse-MLA tile gathers its slice (one 4-wave workgroup per rows_per_wg
// consecutive list entries, 32-row tiles into a 4-deep LDS ring by
// global_load_lds_dwordx4, wave w moving rows 8w .. 8w + 7 of a tile, lane l
// row 8w + l / 8 and its 16-byte units 8i + (l & 7), three tiles in flight)
// but with no arithmetic: the memory system's rate for that access pattern.
// Each thread folds its share of every tile (read back from LDS) into one
// word; sink[wg] holds the workgroup's XOR.
constexpr int RP_NBUF = 4;
constexpr int RP_TILE_ROWS = 32;
constexpr int RP_MAX_ROW_BYTES = 1152;
template <int XF>   // 1 KB transfers per wave per tile: rows of 128 XF bytes
__global__ __launch_bounds__(256) void row_read(const uint8_t* __restrict__ base, const int32_t* rows,
                                                int rows_per_wg, uint32_t* __restrict__ sink) {
    __shared__ __attribute__((aligned(16))) uint8_t ring[RP_NBUF][RP_TILE_ROWS * RP_MAX_ROW_BYTES];
    __shared__ uint32_t red[4];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int32_t* r = rows + (size_t)blockIdx.x * rows_per_wg;
    const int ntiles = rows_per_wg / RP_TILE_ROWS;
    constexpr int row_bytes = 128 * XF, tile_bytes = RP_TILE_ROWS * row_bytes;
    // lane l's 16-byte unit of transfer i: row 8w + l / 8, unit 8i + (l & 7)
    auto issue = [&](int tile, int b) {
        const int row = r[RP_TILE_ROWS * tile + 8 * wave + (lane >> 3)];
        const uint8_t* src = base + (size_t)row * row_bytes + 16 * (lane & 7);
        const uint32_t dst = lds_addr(&ring[b][0]) + (uint32_t)(8 * row_bytes * wave);
#pragma unroll
        for (int i = 0; i < XF; ++i) dma16(src + 128 * i, dst + 1024u * i);
    };
    for (int b = 0; b < RP_NBUF - 1; ++b)
        if (b < ntiles) issue(b, b);
    uint32_t acc = 0u;
    for (int i = 0; i < ntiles; ++i) {
        // this wave's transfers of tile i are done once at most those of the
        // (up to two) later tiles already issued are pending
        const int later = min(RP_NBUF - 2, ntiles - 1 - i);
        if (later >= 2) wait_vmcnt<2 * XF>();
        else if (later == 1) wait_vmcnt<XF>();
        else wait_vmcnt<0>();
        __syncthreads();   // every wave's part of tile i landed; tile i - 1's buffer is free
        if (i + RP_NBUF - 1 < ntiles) issue(i + RP_NBUF - 1, (i + RP_NBUF - 1) % RP_NBUF);
        const uint8_t* tb = &ring[i % RP_NBUF][0];
        for (int o = 16 * tid; o < tile_bytes; o += 16 * 256) {
            const u32x4 v = *(const u32x4*)(tb + o);
            acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
        }
    }
    for (int off = 32; off > 0; off >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, off);
    if (lane == 0) red[wave] = acc;
    __syncthreads();
    if (tid == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

}  // namespace dsa

extern "C" {

size_t dsa_read_probe_sink_size(void) { return sizeof(uint32_t) * (size_t)dsa::probe_grid(); }

int dsa_read_probe(const void* buf, int64_t nbytes, void* sink, size_t sink_bytes, dsa_stream_t stream) {
    if (!buf || nbytes < 16 || (nbytes & 15) || ((uintptr_t)buf & 15) || !sink) return DSA_ERR_INVALID_ARG;
    if (const int st = dsa_check_device(); st != DSA_OK) return st;
    const int grid = dsa::probe_grid();
    if (sink_bytes < sizeof(uint32_t) * (size_t)grid) return DSA_ERR_WORKSPACE;
    hipLaunchKernelGGL(dsa::stream_read, dim3(grid), dim3(dsa::PR_THREADS), 0, (hipStream_t)stream, (const uint8_t*)buf, nbytes,
                       (uint32_t*)sink);
    return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH;
}

size_t dsa_page_probe_sink_size(void) { return sizeof(uint32_t) * 256 * (size_t)dsa::page_probe_grid(); }

int dsa_page_probe(const void* pages, int64_t page_bytes, const void* scales, int64_t scale_bytes,
                   const int32_t* block_ids, int32_t n_pages, void* sink, size_t sink_bytes, dsa_stream_t stream) {
    if (!pages || !block_ids || !sink || n_pages < 0 || page_bytes < 1024 || page_bytes > 8192 ||
        (page_bytes & 1023) || scale_bytes < 0 || scale_bytes > 256 || (scale_bytes & 3) ||
        (scale_bytes > 0 && !scales) || ((uintptr_t)pages & 15) || ((uintptr_t)scales & 3))
        return DSA_ERR_INVALID_ARG;
    if (const int st = dsa_check_device(); st != DSA_OK) return st;
    const int grid = dsa::page_probe_grid();
    if (sink_bytes < sizeof(uint32_t) * 256 * (size_t)grid) return DSA_ERR_WORKSPACE;
    if (n_pages == 0) return DSA_OK;
    hipLaunchKernelGGL(dsa::page_read, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const uint8_t*)pages,
                       (int)(page_bytes / 1024), (const uint8_t*)scales, (int)scale_bytes, block_ids, n_pages,
                       (uint32_t*)sink);
    return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH;
}

size_t dsa_row_probe_sink_size(int32_t n_rows, int32_t rows_per_wg) {
    return rows_per_wg > 0 ? sizeof(uint32_t) * (size_t)((n_rows + rows_per_wg - 1) / rows_per_wg) : 0;
}
int dsa_row_probe(const void* base, int64_t row_bytes, const int32_t* row_ids, int32_t n_rows, int32_t rows_per_wg,
                  void* sink, size_t sink_bytes, dsa_stream_t stream) {
    if (!base || !row_ids || !sink || ((uintptr_t)base & 15) || row_bytes < 128 || row_bytes % 128 ||
        row_bytes > dsa::RP_MAX_ROW_BYTES || n_rows < 0 || rows_per_wg < dsa::RP_TILE_ROWS ||
        rows_per_wg % dsa::RP_TILE_ROWS || n_rows % rows_per_wg)
        return DSA_ERR_INVALID_ARG;
    if (const int st = dsa_check_device(); st != DSA_OK) return st;
    if (sink_bytes < dsa_row_probe_sink_size(n_rows, rows_per_wg)) return DSA_ERR_WORKSPACE;
    if (n_rows == 0) return DSA_OK;
    const dim3 grid(n_rows / rows_per_wg);
    const hipStream_t s = (hipStream_t)stream;
    const uint8_t* b8 = (const uint8_t*)base;
    uint32_t* sk = (uint32_t*)sink;
    switch (row_bytes / 128) {
    case 1: hipLaunchKernelGGL(dsa::row_read<1>, grid, dim3(256), 0, s, b8, row_ids, rows_per_wg, sk); break;
    case 2: hipLaunchKernelGGL(dsa::row_read<2>, grid, dim3(256), 0, s, b8, row_ids, rows_per_wg, sk); break;
    case 3: hipLaunchKernelGGL(dsa::row_read<3>, grid, dim3(256), 0, s, b8, row_ids, rows_per_wg, sk); break;
    case 4: hipLaunchKernelGGL(dsa::row_read<4>, grid, dim3(256), 0, s, b8, row_ids, rows_per_wg, sk); break;
    case 5: hipLaunchKernelGGL(dsa::row_read<5>, grid, dim3(256), 0, s, b8, row_ids, rows_per_wg, sk); break;
    case 6: hipLaunchKernelGGL(dsa::row_read<6>, grid, dim3(256), 0, s, b8, row_ids, rows_per_wg, sk); break;
    case 7: hipLaunchKernelGGL(dsa::row_read<7>, grid, dim3(256), 0, s, b8, row_ids, rows_per_wg, sk); break;
    case 8: hipLaunchKernelGGL(dsa::row_read<8>, grid, dim3(256), 0, s, b8, row_ids, rows_per_wg, sk); break;
    default: hipLaunchKernelGGL(dsa::row_read<9>, grid, dim3(256), 0, s, b8, row_ids, rows_per_wg, sk); break;
    }
    return hipGetLastError() == hipSuccess ? DSA_OK : DSA_ERR_LAUNCH;
}

}  // extern "C"
