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
// LDS a workgroup may allocate on the current device (bytes).
size_t device_max_lds();

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
// The router+latent+shared pass may normalise its input itself: x =
// RMSNorm(h32) * gamma, written to x_out too when that is not null (one
// token, only where rls_gemv_fits).
// rls_gemv_fits: the pass runs on the 8-row engine for these b (<= 4) tokens.
struct NormIn {
    const float *h32;
    const uint16_t *gamma;
    float eps;
    uint16_t *x_out;
};
bool rls_gemv_fits(int b, int d, int E, int NL, int Is);
void launch_rls(const uint16_t *x, int64_t ldx, int b, int d, const uint16_t *w_router,
                const float *bias, int E, float *logits, const uint16_t *w_lat, int NL,
                uint16_t *z, int64_t ldz, const uint16_t *w13s, int Is, uint16_t *hs,
                hipStream_t s, int cu_budget = 0, const NormIn *norm = nullptr);
// y[t] = RMSNorm(h32[t]) * gamma, bf16, one workgroup per token.
void launch_rmsnorm(const float *h32, int b, int d, const uint16_t *gamma, float eps, uint16_t *y,
                    hipStream_t s);
// One token on the 8-row engine: y[n] = x . W[n] in fp32, n < N (K % 64 == 0).
bool gemv1_f32_fits(int N, int K);
void launch_gemv1_f32(const uint16_t *x, const uint16_t *W, int N, int K, float *y, int cu_budget,
                      hipStream_t s);
void launch_topk(const float *logits, int b, int E, int k, int32_t *ids, float *wts,
                 hipStream_t s);

// The split-K MFMA engine (skinny.hip). Each projection writes fp32 partial
// sums of its K ranges into `part` (sk_partial_bytes(T, rows, K) bytes, rows
// = all output rows of the call) and a small kernel finishes them. K = 0
// gives the bound over every K (for size queries that are not given K).
size_t sk_partial_bytes(int T, int rows, int K);
int sk_ksplit(int K, int T);
int sk_mt(int T);
void sk_proj_bf16(const uint16_t *x, int64_t ldx, int T, const uint16_t *W, int N, int K,
                  uint16_t *y, int64_t ldy, float *part, hipStream_t s);
void sk_proj_f32(const uint16_t *x, int64_t ldx, int T, const uint16_t *W, int N, int K,
                 float *y, int64_t ldy, float *part, int cu_budget, hipStream_t s);
void sk_proj_f32_direct(const uint16_t *x, int64_t ldx, int T, const uint16_t *W, int N, int K,
                        float *y, int64_t ldy, int cu_budget, hipStream_t s);
void sk_router_topk(const uint16_t *x, int64_t ldx, int T, const uint16_t *W, int E, int K,
                    const float *bias, int k, float *logits, int32_t *ids, float *wts,
                    float *part, hipStream_t s);
void sk_router_topk_latent(const uint16_t *x, int64_t ldx, int T, int K, const uint16_t *W_r,
                           int E, const float *bias, int k, float *logits, int32_t *ids,
                           float *wts, const uint16_t *W_lat, int d_lat, uint16_t *z,
                           int64_t ldz, float *part, hipStream_t s);
void sk_router_latent_shared(const uint16_t *x, int64_t ldx, int T, int K, const uint16_t *W_r,
                             int E, const float *bias, int k, float *logits, int32_t *ids,
                             float *wts, const uint16_t *W_lat, int d_lat, uint16_t *z,
                             int64_t ldz, const uint16_t *W13_s, int I_s, uint16_t *hs,
                             float *part, hipStream_t s);
void sk_swiglu(const uint16_t *x, int64_t ldx, int T, int K, const uint16_t *W13, int I,
               uint16_t *hs, float *part, int cu_budget, hipStream_t s);
int sk_oproj_partials(const uint16_t *a, int64_t lda, int T, int K, const uint16_t *W_o, int d,
                      float *part, hipStream_t s);
void sk_oproj_residual(const uint16_t *a, int64_t lda, int T, int K, const uint16_t *W_o, int d,
                       uint16_t *residual, float *h32, float *part, hipStream_t s);

// Batch-1 routed experts (moe_b1.hip). up_b1: routed gate/up + SwiGLU into
// hbuf, k x I values in the pair's own layout ([I / 4][k][4], read only by
// down_b1: launch both or neither); with `topk` the selection from logits
// happens in the kernel (ids/weights written out); with w13s (`shared` in
// up_b1_fits) the shared expert's gate/up rows on xs (d wide) stream first,
// into hs. down_b1: y = bf16(base +
// sum_j w_j w2[ids[j]] . h_j) with base = y_add, or, with w2s, the shared
// expert's down projection of hs (also written to y_s).
bool up_b1_fits(int d, int k, int I, int cu_budget, bool shared = false);
void launch_up_b1(bool topk, const uint16_t *z, int d, const uint16_t *w13, int I, int E, int k,
                  const int32_t *ids_in, const float *logits, int32_t *ids_out, float *w_out,
                  uint16_t *hbuf, int cu_budget, hipStream_t s, const uint16_t *xs = nullptr,
                  const uint16_t *w13s = nullptr, uint16_t *hs = nullptr);
bool down_b1_fits(int k, int I, int d_out, bool shared, int cu_budget);
void launch_down_b1(const uint16_t *hbuf, int I, const uint16_t *w2, int d_out,
                    const int32_t *ids, const float *wts, int k, int E, const float *y_add,
                    const uint16_t *hs, const uint16_t *w2s, float *y_s, uint16_t *y,
                    int cu_budget, hipStream_t s);

}  // namespace k3
