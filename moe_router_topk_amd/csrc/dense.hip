// dense.hip -- skinny dense projections, router scoring + top-k, and the
// output projection with residual add and RMSNorm.
//
// Two GEMV/GEMM engines serve every dense [N x K] weight read here:
//  * dot2: each wave owns whole weight rows and streams them with 128-bit
//    non-temporal loads (up to 16 in flight per lane), multiplying against
//    the T <= 8 token rows with v_dot2c_f32_bf16 and reducing across the
//    wave at the end of a row. Small-batch kernels of "Hyper Optimizing Kimi
//    K3 in vLLM", Part 1 section 1 ("Tune shapes for the workload").
//  * mfma: one workgroup per 16-row tile of W; its four waves split K into
//    quarters and run v_mfma_f32_16x16x32_bf16 with the tokens as the A
//    operand (up to four 16-token tiles) and the weight rows as B, then sum
//    the four partial tiles in LDS in a fixed order. This is the
//    work-splitting kernel the same section uses above batch 2; the split
//    stays inside one workgroup, so no partial sums go through HBM.
#include <math.h>

#include "k3_device.h"
#include "k3_internal.h"

namespace k3 {

// ------------------------------------------------------------------ epilogues
struct EpiBf16 {  // y[t][n] = bf16(s)
    uint16_t *y;
    int64_t ldy;
    __device__ void operator()(int t, int n, float s) const {
        y[(int64_t)t * ldy + n] = f32_to_bf16(s);
    }
};

struct EpiLogits {  // logits[t][e] = s (+ bias[e]), fp32
    float *logits;
    int E;
    const float *bias;
    __device__ void operator()(int t, int n, float s) const {
        logits[(int64_t)t * E + n] = bias ? s + bias[n] : s;
    }
};

struct EpiResidual {  // h = r + s: fp32 copy for the norm, bf16 back into r
    uint16_t *res;
    float *h32;
    int d;
    __device__ void operator()(int t, int n, float s) const {
        const int64_t i = (int64_t)t * d + n;
        const float h = bf16_to_f32(res[i]) + s;
        h32[i] = h;
        res[i] = f32_to_bf16(h);
    }
};

// ------------------------------------------------------------------ dot2 engine
// Wave w owns rows [w * rows_per_wave, ...) of W and takes them R at a time;
// lane l reads 16-byte vectors l, l + 64, ... of each row (U of them in
// flight per row) and the matching vectors of the T token rows.
template <int T, int R, int U, class Epi>
__global__ void __launch_bounds__(kBlock)
k_gemv_dot2(const uint16_t *__restrict__ x, int64_t ldx, int b,
            const uint16_t *__restrict__ W, int N, int K, int rows_per_wave, Epi epi) {
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = blockIdx.x * (kBlock / kWave) + (threadIdx.x / kWave);
    const int r_begin = wave * rows_per_wave;
    const int r_end = min(N, r_begin + rows_per_wave);
    const int nv = K >> 3;
    for (int r = r_begin; r < r_end; r += R) {
        float acc[R][T];
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int t = 0; t < T; ++t)
                acc[i][t] = 0.0f;
        for (int v0 = 0; v0 < nv; v0 += kWave * U) {
            u32x4 w[R][U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = v0 + u * kWave + lane;
#pragma unroll
                for (int i = 0; i < R; ++i)
                    w[i][u] = (v < nv && r + i < r_end)
                                  ? ld_weight16(W + (int64_t)(r + i) * K + (int64_t)v * 8)
                                  : zero16();
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int v = v0 + u * kWave + lane;
                if (v < nv) {
#pragma unroll
                    for (int t = 0; t < T; ++t) {
                        if (t < b) {
                            const u32x4 xv = ld_act16(x + (int64_t)t * ldx + (int64_t)v * 8);
#pragma unroll
                            for (int i = 0; i < R; ++i)
                                acc[i][t] = dot8(w[i][u], xv, acc[i][t]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int i = 0; i < R; ++i)
#pragma unroll
            for (int t = 0; t < T; ++t) {
                if (t < b && r + i < r_end) {
                    const float s = wave_sum(acc[i][t]);
                    if (lane == 0)
                        epi(t, r + i, s);
                }
            }
    }
}

// ------------------------------------------------------------------ mfma engine
// Workgroup per 16-row tile of W (grid-stride over tiles). Wave q handles
// K range [q K/4, (q+1) K/4) in steps of 32; lane l loads B = W[n0 + l%16]
// at k + 8(l/16) (16 bytes) and A = x[m][same k] for m = 16 mt + l%16.
template <int U, class Epi>
__global__ void __launch_bounds__(kBlock)
k_gemm_mfma(const uint16_t *__restrict__ x, int64_t ldx, int b,
            const uint16_t *__restrict__ W, int N, int K, Epi epi) {
    __shared__ float red[4][4][4][kWave];  // [wave][m tile][element][lane]
    const int lane = threadIdx.x & (kWave - 1);
    const int wq = threadIdx.x / kWave;
    const int MT = (b + 15) >> 4;
    const int kq = K >> 2;
    const int k_begin = wq * kq;
    const int k_end = k_begin + kq;
    const int kgrp = (lane >> 4) * 8;
    int64_t aoff[4];
    bool aval[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
        const int m = mt * 16 + (lane & 15);
        aval[mt] = m < b;
        aoff[mt] = (int64_t)(aval[mt] ? m : 0) * ldx;
    }
    const int tiles = (N + 15) >> 4;
    for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const int n = tile * 16 + (lane & 15);
        const bool nval = n < N;
        const uint16_t *wrow = W + (int64_t)(nval ? n : 0) * K;
        f32x4 acc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int ks = k_begin; ks < k_end; ks += 32 * U) {
            u32x4 bfr[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int k = ks + 32 * u + kgrp;
                bfr[u] = (ks + 32 * u < k_end && nval) ? ld_weight16(wrow + k) : zero16();
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (ks + 32 * u < k_end) {
                    const int k = ks + 32 * u + kgrp;
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {
                        if (mt < MT) {
                            const u32x4 a = aval[mt] ? ld_act16(x + aoff[mt] + k) : zero16();
                            acc[mt] = mfma16x16x32(a, bfr[u], acc[mt]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            if (mt < MT)
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    red[wq][mt][i][lane] = acc[mt][i];
        __syncthreads();
        for (int idx = threadIdx.x; idx < MT * 256; idx += kBlock) {
            const int mt = idx >> 8, i = (idx >> 6) & 3, l = idx & 63;
            const float s = red[0][mt][i][l] + red[1][mt][i][l] + red[2][mt][i][l] + red[3][mt][i][l];
            const int m = mt * 16 + 4 * (l >> 4) + i;
            const int nn = tile * 16 + (l & 15);
            if (m < b && nn < N)
                epi(m, nn, s);
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ launchers
template <int T, class Epi>
static void launch_dot2_t(const uint16_t *x, int64_t ldx, int b, const uint16_t *W, int N, int K,
                          Epi epi, int cu_budget, hipStream_t s) {
    // Rows per wave: spread N evenly over the waves of one workgroup per CU.
    const int cus = budget_grid(1 << 30, cu_budget, 1);
    const int waves = cus * (kBlock / kWave);
    const int R = K > 4096 ? 1 : (K > 2048 ? 2 : 4);
    int rpw = (N + waves - 1) / waves;
    rpw = (rpw + R - 1) / R * R;
    const int grid = ((N + rpw - 1) / rpw + 3) / 4;
    if (R == 1)
        k_gemv_dot2<T, 1, 16, Epi><<<grid, kBlock, 0, s>>>(x, ldx, b, W, N, K, rpw, epi);
    else if (R == 2)
        k_gemv_dot2<T, 2, 8, Epi><<<grid, kBlock, 0, s>>>(x, ldx, b, W, N, K, rpw, epi);
    else
        k_gemv_dot2<T, 4, 4, Epi><<<grid, kBlock, 0, s>>>(x, ldx, b, W, N, K, rpw, epi);
}

template <class Epi>
static void launch_dot2(const uint16_t *x, int64_t ldx, int b, const uint16_t *W, int N, int K,
                        Epi epi, int cu_budget, hipStream_t s) {
    if (b <= 1)
        launch_dot2_t<1>(x, ldx, b, W, N, K, epi, cu_budget, s);
    else if (b <= 2)
        launch_dot2_t<2>(x, ldx, b, W, N, K, epi, cu_budget, s);
    else if (b <= 4)
        launch_dot2_t<4>(x, ldx, b, W, N, K, epi, cu_budget, s);
    else
        launch_dot2_t<8>(x, ldx, b, W, N, K, epi, cu_budget, s);
}

template <class Epi>
static void launch_mfma(const uint16_t *x, int64_t ldx, int b, const uint16_t *W, int N, int K,
                        Epi epi, int cu_budget, hipStream_t s) {
    const int tiles = (N + 15) / 16;
    const int grid = budget_grid(tiles, cu_budget, 4);
    k_gemm_mfma<8, Epi><<<grid, kBlock, 0, s>>>(x, ldx, b, W, N, K, epi);
}

// Variant for a dense [N x K] read at batch b: dot2 up to 8 tokens, MFMA
// above (MFMA needs K % 128 == 0 so each wave's K quarter is whole steps).
static int pick_dense_variant(int op, int b, int K) {
    int v = forced_variant(op);
    if (v == K3_VARIANT_NONE)
        v = (b <= 8 || K % 128 != 0) ? K3_VARIANT_DOT2 : K3_VARIANT_MFMA;
    if (v == K3_VARIANT_DOT2 && b > 8)
        return -1;
    if (v == K3_VARIANT_MFMA && K % 128 != 0)
        return -1;
    if (v != K3_VARIANT_DOT2 && v != K3_VARIANT_MFMA)
        return -1;
    return v;
}

template <class Epi>
static void launch_dense(int variant, const uint16_t *x, int64_t ldx, int b, const uint16_t *W,
                         int N, int K, Epi epi, int cu_budget, hipStream_t s) {
    if (variant == K3_VARIANT_DOT2)
        launch_dot2(x, ldx, b, W, N, K, epi, cu_budget, s);
    else
        launch_mfma(x, ldx, b, W, N, K, epi, cu_budget, s);
}

// ------------------------------------------------------------------ top-k
// One wave per token. Lane l holds logits l, l + 64, ...; k rounds of a
// wave-wide argmax under the order (logit desc, index asc) pick the experts;
// lane j keeps the j-th pick. The weights are the softmax over the k picked
// logits (the full softmax renormalised over the selection).
__global__ void __launch_bounds__(kWave)
k_topk_softmax(const float *__restrict__ logits, int E, int k, int32_t *__restrict__ ids,
               float *__restrict__ wts) {
    constexpr int PER = K3_MAX_EXPERTS / kWave;
    const int t = blockIdx.x;
    const int lane = threadIdx.x;
    float v[PER];
    uint32_t taken = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = i * kWave + lane;
        float l = -INFINITY;
        if (e < E)
            l = logits[(int64_t)t * E + e];
        else
            taken |= 1u << i;
        v[i] = (l != l) ? -INFINITY : l;  // NaN never outranks a number
    }
    float sel_v = 0.0f, top = 0.0f;
    int sel_e = 0;
    for (int j = 0; j < k; ++j) {
        float bv = -INFINITY;
        int be = 0x7fffffff;
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            const int e = i * kWave + lane;
            if (!((taken >> i) & 1u) && (v[i] > bv || (v[i] == bv && e < be))) {
                bv = v[i];
                be = e;
            }
        }
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) {
            const float ov = __shfl_xor(bv, m, kWave);
            const int oe = __shfl_xor(be, m, kWave);
            if (ov > bv || (ov == bv && oe < be)) {
                bv = ov;
                be = oe;
            }
        }
        if ((be & (kWave - 1)) == lane)
            taken |= 1u << (be / kWave);
        if (lane == j) {
            sel_v = bv;
            sel_e = be;
        }
        if (j == 0)
            top = bv;
    }
    const float dl = (sel_v == top) ? 0.0f : sel_v - top;
    const float p = lane < k ? expf(dl) : 0.0f;
    const float sum = wave_sum(p);
    if (lane < k) {
        ids[(int64_t)t * k + lane] = sel_e;
        wts[(int64_t)t * k + lane] = p / sum;
    }
}

// ------------------------------------------------------------------ RMSNorm
// One workgroup per token: mean of h^2 over d in fp32 (fixed reduction
// order), then y = h / sqrt(mean + eps) * gamma.
__global__ void __launch_bounds__(kBlock)
k_rmsnorm(const float *__restrict__ h32, int d, const uint16_t *__restrict__ gamma, float eps,
          uint16_t *__restrict__ y) {
    __shared__ float part[kBlock / kWave];
    const int t = blockIdx.x;
    const float *h = h32 + (int64_t)t * d;
    float ss = 0.0f;
    for (int n = threadIdx.x; n < d; n += kBlock)
        ss += h[n] * h[n];
    ss = wave_sum(ss);
    if ((threadIdx.x & (kWave - 1)) == 0)
        part[threadIdx.x / kWave] = ss;
    __syncthreads();
    const float total = (part[0] + part[1]) + (part[2] + part[3]);
    const float inv = 1.0f / sqrtf(total / (float)d + eps);
    for (int n = threadIdx.x; n < d; n += kBlock)
        y[(int64_t)t * d + n] = f32_to_bf16(h[n] * inv * bf16_to_f32(gamma[n]));
}

}  // namespace k3

using namespace k3;

// ------------------------------------------------------------------ entry points
extern "C" int k3_proj_skinny(const uint16_t *x, int64_t ldx, int b, int K, const uint16_t *w,
                              int N, uint16_t *y, int64_t ldy, void *workspace, size_t ws_bytes,
                              void *stream) {
    (void)workspace;
    (void)ws_bytes;
    if (!x || !w || !y)
        return K3_ERR_INVALID_ARG;
    if (b <= 0 || K <= 0 || N <= 0 || ldx < K || ldy < N)
        return K3_ERR_INVALID_ARG;
    if (b > K3_MAX_BATCH || K % 8 || ldx % 8 || !aligned16(x) || !aligned16(w))
        return K3_ERR_UNSUPPORTED;
    const int variant = pick_dense_variant(K3_OP_PROJ_SKINNY, b, K);
    if (variant < 0)
        return K3_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    trace_begin(K3_OP_PROJ_SKINNY, s);
    launch_dense(variant, x, ldx, b, w, N, K, EpiBf16{y, ldy}, 0, s);
    trace_end(K3_OP_PROJ_SKINNY, s);
    const int st = launch_status();
    if (st == K3_OK)
        record_dispatch(K3_OP_PROJ_SKINNY, variant);
    return st;
}

extern "C" int k3_router_topk(const uint16_t *x, int64_t ldx, int b, int d,
                              const uint16_t *w_router, const float *bias, int E, int k,
                              int32_t *topk_ids, float *topk_w, void *workspace, size_t ws_bytes,
                              void *stream) {
    if (!x || !w_router || !topk_ids || !topk_w)
        return K3_ERR_INVALID_ARG;
    if (b <= 0 || d <= 0 || E <= 0 || k <= 0 || ldx < d)
        return K3_ERR_INVALID_ARG;
    if (b > K3_MAX_BATCH || E > K3_MAX_EXPERTS || k > K3_MAX_TOPK || k > E || d % 8 || ldx % 8 ||
        !aligned16(x) || !aligned16(w_router))
        return K3_ERR_UNSUPPORTED;
    if (!workspace || ws_bytes < k3_router_topk_workspace_size(b, E))
        return K3_ERR_WORKSPACE;
    const int variant = pick_dense_variant(K3_OP_ROUTER_TOPK, b, d);
    if (variant < 0)
        return K3_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    float *logits = (float *)workspace;
    trace_begin(K3_OP_ROUTER_TOPK, s);
    launch_dense(variant, x, ldx, b, w_router, E, d, EpiLogits{logits, E, bias}, 0, s);
    trace_end(K3_OP_ROUTER_TOPK, s);
    k_topk_softmax<<<b, kWave, 0, s>>>(logits, E, k, topk_ids, topk_w);
    const int st = launch_status();
    if (st == K3_OK)
        record_dispatch(K3_OP_ROUTER_TOPK, variant);
    return st;
}

extern "C" int k3_oproj_residual(const uint16_t *a, int64_t lda, int b, int K,
                                 const uint16_t *w_o, int d, uint16_t *residual,
                                 const uint16_t *gamma, float eps, uint16_t *y_norm,
                                 void *workspace, size_t ws_bytes, void *stream) {
    if (!a || !w_o || !residual || !gamma || !y_norm)
        return K3_ERR_INVALID_ARG;
    if (b <= 0 || K <= 0 || d <= 0 || lda < K || !(eps >= 0.0f))
        return K3_ERR_INVALID_ARG;
    if (b > K3_MAX_BATCH || K % 8 || lda % 8 || d % 8 || !aligned16(a) || !aligned16(w_o))
        return K3_ERR_UNSUPPORTED;
    if (!workspace || ws_bytes < k3_oproj_residual_workspace_size(b, K, d))
        return K3_ERR_WORKSPACE;
    const int variant = pick_dense_variant(K3_OP_OPROJ_RESIDUAL, b, K);
    if (variant < 0)
        return K3_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    float *h32 = (float *)workspace;
    trace_begin(K3_OP_OPROJ_RESIDUAL, s);
    launch_dense(variant, a, lda, b, w_o, d, K, EpiResidual{residual, h32, d}, 0, s);
    trace_end(K3_OP_OPROJ_RESIDUAL, s);
    k_rmsnorm<<<b, kBlock, 0, s>>>(h32, d, gamma, eps, y_norm);
    const int st = launch_status();
    if (st == K3_OK)
        record_dispatch(K3_OP_OPROJ_RESIDUAL, variant);
    return st;
}
