// noalloc.hip -- k3_moe_block_noalloc: the MoE block with its scratch memory
// in a fixed device array instead of a caller's workspace, for callers that
// cannot allocate (code under stream capture, serving loops that forbid
// allocation).
//
// `scratch` is a file-scope device array: in host code its name is only a
// host-side stand-in, so the kernels are handed the array's device address,
// looked up once per device (hipGetSymbolAddress) and kept in a table. Each
// device holds its own copy of the array until the process ends.
#include <mutex>

#include "k3_internal.h"

namespace {

__device__ __align__(256) unsigned char scratch[K3_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];  // per device: the array's device address

// The current device's copy of the array, looked up on the first call made
// on that device; nullptr (and no lookup retried this call) on a HIP error.
void *device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
        return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return nullptr;
        }
        g_scratch_ptr[dev] = p;
    }
    return g_scratch_ptr[dev];
}

}  // namespace

extern "C" int k3_moe_block_noalloc(const uint16_t *x, int64_t ldx, int b, int d,
                                    const uint16_t *w_router, const float *bias, int E, int k,
                                    const uint16_t *w_lat, int d_lat, const uint16_t *w13,
                                    const uint16_t *w2, int I, const uint16_t *w13_s,
                                    const uint16_t *w2_s, int I_s, int32_t *topk_ids,
                                    float *topk_w, uint16_t *z, int64_t ldz, float *y_s,
                                    uint16_t *y, void *stream) {
    if (!x)
        return K3_ERR_INVALID_ARG;
    const size_t need = k3_moe_block_workspace_size(b, d, E, k, d_lat, I, I_s);
    if (need == 0)
        return K3_ERR_INVALID_ARG;
    if (need > (size_t)K3_NOALLOC_SCRATCH_BYTES)
        return K3_ERR_SCRATCH;
    void *ws = device_scratch();
    if (!ws)
        return K3_ERR_HIP;
    // the block's kernels need no cleared scratch: every workspace byte they
    // read is written earlier in the same call
    return k3_moe_block(x, ldx, b, d, w_router, bias, E, k, w_lat, d_lat, w13, w2, I, w13_s,
                        w2_s, I_s, topk_ids, topk_w, z, ldz, y_s, y, ws,
                        (size_t)K3_NOALLOC_SCRATCH_BYTES, stream);
}
