// Synchronous check of the device-side batch values that the entry points
// read (query_start_loc, context_lens, page ids, token indices), for the
// DSA_DEBUG mode and dsa_check_batch.  The step's kernels trust these values
// (a page id beyond the pool or an index beyond a row's visible tokens reads
// outside the caches); this check turns such values into a status code before
// anything else is launched.  The result word is a file-scope device variable
// (nothing is allocated), found per device with hipGetSymbolAddress.
#include <stdlib.h>
#include <string.h>

#include <mutex>

#include "dsa.h"
#include "dsa_kernels.h"

namespace dsa {

constexpr int CHECK_THREADS = 256;

// One workgroup per request r: its query range and context length first, then
// (when those hold) the page ids of its ceil(L_r / block_size) blocks and the
// entries of its rows' selections.
__global__ __launch_bounds__(CHECK_THREADS) void batch_check(Geometry g, int num_blocks, int pages,
                                                             const int32_t* indices, int k, uint32_t* failed) {
    __shared__ int s_qs, s_qe, s_len;
    __shared__ uint32_t s_bad;
    const int r = blockIdx.x;
    if (threadIdx.x == 0) {
        uint32_t bad = 0;
        const int qs = g.qsl[r], qe = g.qsl[r + 1];
        if ((r == 0 && qs != 0) || (r == g.B - 1 && qe != g.T) || qs < 0 || qe < qs || qe > g.T ||
            qe - qs > g.max_q_len)
            bad |= DSA_CHECK_QUERY_START;
        const int len = g.ctx[r];
        if (len < 0 || len > g.max_ctx || (bad == 0 && len < qe - qs)) bad |= DSA_CHECK_CONTEXT;
        s_qs = qs;
        s_qe = qe;
        s_len = len;
        s_bad = bad;
        if (bad) atomicOr(failed, bad);
    }
    __syncthreads();
    if (s_bad) return;
    const int qs = s_qs, nq = s_qe - s_qs, len = s_len;
    uint32_t bad = 0;
    if (pages) {
        const int npg = (len + g.block_size - 1) / g.block_size;   // <= max_blocks (host-checked)
        const int32_t* row = g.page_table + (size_t)r * g.max_blocks;
        for (int i = threadIdx.x; i < npg; i += CHECK_THREADS) {
            const int32_t id = row[i];
            if (id < 0 || (num_blocks > 0 && id >= num_blocks)) bad |= DSA_CHECK_PAGE;
        }
    }
    if (indices) {
        const int64_t n = (int64_t)nq * k;
        for (int64_t e = threadIdx.x; e < n; e += CHECK_THREADS) {
            const int j = (int)(e / k);                       // row qs + j sees len - nq + j + 1 tokens
            if (indices[(size_t)(qs + j) * k + (size_t)(e % k)] >= len - nq + j + 1) bad |= DSA_CHECK_INDEX;
        }
    }
    if (bad) atomicOr(failed, bad);
}

}  // namespace dsa

static __device__ __align__(16) uint32_t check_word[4];

namespace {

constexpr int CHECK_MAX_DEVICES = 64;
std::mutex check_mutex;
void* check_ptr[CHECK_MAX_DEVICES];

// Device address of the current device's result word (looked up once per
// device, with the device current), or nullptr.  Called with check_mutex held.
uint32_t* check_word_ptr() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= CHECK_MAX_DEVICES) return nullptr;
    if (!check_ptr[dev]) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(check_word)) != hipSuccess || !p) return nullptr;
        check_ptr[dev] = p;
    }
    return (uint32_t*)check_ptr[dev];
}

}  // namespace

namespace dsa {

bool debug_mode() {
    const char* v = getenv("DSA_DEBUG");
    return v && v[0] && strcmp(v, "0") != 0;
}

int run_batch_check(const Geometry& g, int num_blocks, bool pages, const int32_t* indices, int k,
                    uint32_t* failed, hipStream_t s) {
    if (failed) *failed = 0;
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(s, &cs) != hipSuccess) return DSA_ERR_LAUNCH;
    if (cs != hipStreamCaptureStatusNone) return DSA_ERR_UNSUPPORTED;   // it waits for the stream
    std::lock_guard<std::mutex> lock(check_mutex);   // one result word per device
    uint32_t* word = check_word_ptr();
    if (!word) return DSA_ERR_LAUNCH;
    uint32_t host = 0;
    if (hipMemsetAsync(word, 0, sizeof(uint32_t), s) != hipSuccess) return DSA_ERR_LAUNCH;
    hipLaunchKernelGGL(batch_check, dim3(g.B), dim3(CHECK_THREADS), 0, s, g, num_blocks, pages ? 1 : 0, indices,
                       indices ? k : 0, word);
    if (hipGetLastError() != hipSuccess) return DSA_ERR_LAUNCH;
    if (hipMemcpyAsync(&host, word, sizeof(uint32_t), hipMemcpyDeviceToHost, s) != hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return DSA_ERR_LAUNCH;
    if (failed) *failed = host;
    return host ? DSA_ERR_BAD_DEVICE_ARG : DSA_OK;
}

int debug_finish(bool dbg, int st, hipStream_t s) {
    if (!dbg || st != DSA_OK) return st;
    if (hipStreamSynchronize(s) != hipSuccess || hipGetLastError() != hipSuccess) return DSA_ERR_LAUNCH;
    return DSA_OK;
}

}  // namespace dsa
