// prefetch.hip -- side-stream weight prefetch.
//
// "Hyper Optimizing Kimi K3 in vLLM", Part 1 section 4 ("Prefetching
// upcoming weights into cache"): while the main stream is in a phase that
// does not use the memory bandwidth, a dedicated kernel on a side stream
// reads the next operator's weights so that they hit in cache when that
// operator runs. On MI355X the cache that can hold an operator's weights is
// the 256 MB memory-side MALL (the L2 is 4 MB per XCD), so the kernel issues
// ordinary (allocating) 128-bit loads over the range; the results feed a
// store that only runs if the data equal a value the host picks, which keeps
// the loads alive without writing anything in practice.
#include "k3_device.h"
#include "k3_internal.h"

namespace k3 {

__device__ uint32_t g_prefetch_sink;

// NT: non-temporal loads (the weight streams' kind) instead of allocating
// ones; k3_stream_read uses them to measure the streaming-read ceiling.
template <int U, bool NT = false>
__global__ void __launch_bounds__(kBlock)
k_prefetch(const u32x4 *__restrict__ p, size_t n, uint32_t never) {
    const size_t stride = (size_t)gridDim.x * kBlock * U;
    uint32_t acc = 0;
    for (size_t base = (size_t)blockIdx.x * kBlock * U + threadIdx.x; base < n; base += stride) {
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const size_t i = base + (size_t)u * kBlock;
            v[u] = i < n ? (NT ? __builtin_nontemporal_load(p + i) : p[i]) : zero16();
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == never)
        g_prefetch_sink = acc;
}

}  // namespace k3

using namespace k3;

extern "C" int k3_prefetch(const void *p, size_t bytes, int cu_budget, void *stream) {
    if (cu_budget < 0)
        return K3_ERR_INVALID_ARG;
    if (bytes == 0)
        return K3_OK;
    if (!p)
        return K3_ERR_INVALID_ARG;
    if (!aligned16(p) || bytes % 16)
        return K3_ERR_UNSUPPORTED;
    const int fv = forced_variant(K3_OP_PREFETCH);
    if (fv != K3_VARIANT_NONE && fv != K3_VARIANT_STREAM)
        return K3_ERR_UNSUPPORTED;
    const size_t n = bytes / 16;
    const size_t per_block = (size_t)kBlock * 8;
    const size_t want = (n + per_block - 1) / per_block;
    const int grid = budget_grid(want > (1u << 30) ? (1 << 30) : (int)want, cu_budget, 1);
    hipStream_t s = (hipStream_t)stream;
    trace_begin(K3_OP_PREFETCH, s);
    k_prefetch<8><<<grid, kBlock, 0, s>>>((const u32x4 *)p, n, 0x9e3779b9u);
    trace_end(K3_OP_PREFETCH, s);
    const int st = launch_status();
    if (st == K3_OK)
        record_dispatch(K3_OP_PREFETCH, K3_VARIANT_STREAM);
    return st;
}

extern "C" int k3_stream_read(const void *p, size_t bytes, void *stream) {
    if (bytes == 0)
        return K3_OK;
    if (!p)
        return K3_ERR_INVALID_ARG;
    if (!aligned16(p) || bytes % 16)
        return K3_ERR_UNSUPPORTED;
    const size_t n = bytes / 16;
    const size_t per_block = (size_t)kBlock * 8;
    const size_t want = (n + per_block - 1) / per_block;
    const int grid = budget_grid(want > (1u << 30) ? (1 << 30) : (int)want, 0, 1);
    k_prefetch<8, true><<<grid, kBlock, 0, (hipStream_t)stream>>>((const u32x4 *)p, n,
                                                                  0x9e3779b9u);
    return launch_status();
}
