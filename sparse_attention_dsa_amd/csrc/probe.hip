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

}  // extern "C"
