// api.cpp -- status strings, version, dispatch record, launch sizing and
// workspace layouts of libk3dec.
#include <atomic>
#include <mutex>

#include "k3_internal.h"

namespace k3 {

namespace {
constexpr int kOps = K3_OP_DENSE_PASS + 1;  // op slots of the dispatch record
std::atomic<int> g_last_variant[kOps];
std::atomic<int> g_forced_variant[kOps];
std::atomic<void *> g_trace_begin[kOps];
std::atomic<void *> g_trace_end[kOps];
std::mutex g_cu_mutex;
int g_cu_count[64];
int g_max_lds[64];
}  // namespace

size_t device_max_lds() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 65536;
    std::lock_guard<std::mutex> lock(g_cu_mutex);
    if (g_max_lds[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) !=
                hipSuccess ||
            n <= 0)
            n = 65536;
        g_max_lds[dev] = n;
    }
    return (size_t)g_max_lds[dev];
}

int device_cu_count() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
        return 256;
    std::lock_guard<std::mutex> lock(g_cu_mutex);
    if (g_cu_count[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        g_cu_count[dev] = n;
    }
    return g_cu_count[dev];
}

int budget_grid(int want, int cu_budget, int per_cu) {
    int cus = device_cu_count();
    if (cu_budget > 0 && cu_budget < cus)
        cus = cu_budget;
    long cap = (long)cus * per_cu;
    long g = want < cap ? want : cap;
    return g < 1 ? 1 : (int)g;
}

void record_dispatch(int op, int variant) {
    if (op >= 0 && op < kOps)
        g_last_variant[op].store(variant);
}

void trace_begin(int op, hipStream_t s) {
    if (op < 0 || op >= kOps)
        return;
    void *ev = g_trace_begin[op].load();
    if (ev)
        (void)hipEventRecord((hipEvent_t)ev, s);
}

void trace_end(int op, hipStream_t s) {
    if (op < 0 || op >= kOps)
        return;
    void *ev = g_trace_end[op].load();
    if (ev)
        (void)hipEventRecord((hipEvent_t)ev, s);
}

int forced_variant(int op) {
    return (op >= 0 && op < kOps) ? g_forced_variant[op].load() : K3_VARIANT_NONE;
}

}  // namespace k3

extern "C" {

const char *k3_status_string(int status) {
    switch (status) {
    case K3_OK: return "K3_OK: success";
    case K3_ERR_INVALID_ARG: return "K3_ERR_INVALID_ARG: NULL pointer, non-positive size or bad leading dimension";
    case K3_ERR_UNSUPPORTED: return "K3_ERR_UNSUPPORTED: shape outside the supported range, misaligned pointer, or forced variant that cannot run the shape";
    case K3_ERR_WORKSPACE: return "K3_ERR_WORKSPACE: workspace NULL or smaller than the size query requires";
    case K3_ERR_HIP: return "K3_ERR_HIP: the HIP runtime reported an error at launch";
    case K3_ERR_SCRATCH: return "K3_ERR_SCRATCH: the shape needs more scratch than the no-alloc entry point holds (K3_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown k3 status";
    }
}

int k3_version(void) { return 10000; }

int k3_get_last_dispatch(int op) {
    return (op >= 0 && op < k3::kOps) ? k3::g_last_variant[op].load() : K3_VARIANT_NONE;
}

int k3_force_variant(int op, int variant) {
    if (op < 0 || op >= k3::kOps || op == K3_OP_DENSE_PASS || variant < K3_VARIANT_NONE ||
        variant > K3_VARIANT_LASTWG)
        return K3_ERR_INVALID_ARG;
    k3::g_forced_variant[op].store(variant);
    return K3_OK;
}

int k3_trace_events(int op, void *begin, void *end) {
    if (op < 0 || op >= k3::kOps || (!begin) != (!end))
        return K3_ERR_INVALID_ARG;
    k3::g_trace_begin[op].store(begin);
    k3::g_trace_end[op].store(end);
    return K3_OK;
}

}  // extern "C"
