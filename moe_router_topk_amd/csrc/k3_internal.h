// k3_internal.h -- host-side helpers shared by the libk3dec entry points.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/k3dec.h"

namespace k3 {

// Compute units on the current device (cached per device).
int device_cu_count();

// Grid size for a kernel that wants `want` workgroups of 256 threads, at most
// `per_cu` resident per compute unit, on min(cu_budget, all) compute units.
int budget_grid(int want, int cu_budget, int per_cu);

// Variant bookkeeping for k3_get_last_dispatch / k3_force_variant.
void record_dispatch(int op, int variant);

// Event pair of k3_trace_events, recorded around an op's main kernel.
void trace_begin(int op, hipStream_t s);
void trace_end(int op, hipStream_t s);
int forced_variant(int op);

inline bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

inline size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

inline int launch_status() {
    return hipGetLastError() == hipSuccess ? K3_OK : K3_ERR_HIP;
}

// Workspace layout of k3_moe_experts (offsets in bytes, 256-byte aligned).
struct MoeWorkspace {
    size_t n_light, n_heavy, light_expert, light_start, light_ntok, heavy_expert, heavy_start,
        heavy_ntok, sorted_token, slot_pos, hbuf, part, total;
};
MoeWorkspace moe_workspace_layout(int b, int E, int k, int I, int d_out);

// Dense launchers defined in dense.hip, shared with the fused MoE block.
bool rls_fits(int b, int d, int E);
void launch_rls(const uint16_t *x, int64_t ldx, int b, int d, const uint16_t *w_router,
                const float *bias, int E, float *logits, const uint16_t *w_lat, int NL,
                uint16_t *z, int64_t ldz, const uint16_t *w13s, int Is, uint16_t *hs,
                hipStream_t s);
void launch_topk(const float *logits, int b, int E, int k, int32_t *ids, float *wts,
                 hipStream_t s);
void launch_dense_bf16(const uint16_t *x, int64_t ldx, int b, const uint16_t *W, int N, int K,
                       uint16_t *y, int64_t ldy, hipStream_t s);
void launch_dense_logits(const uint16_t *x, int64_t ldx, int b, const uint16_t *W, int E, int K,
                         const float *bias, float *logits, hipStream_t s);

}  // namespace k3
