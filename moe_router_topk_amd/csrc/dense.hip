// dense.hip -- skinny dense projections, router scoring + top-k, and the
// output projection with residual add and RMSNorm.
//
// Two engines serve the dense [N x K] weight reads here:
//  * dot2 (batch <= 4): the row-streaming engine of k3_device.h -- each wave
//    owns whole weight rows, reads them 1 KB per load instruction with two
//    row buffers in flight, and multiplies against the tokens staged in LDS
//    with v_dot2c_f32_bf16. The small-batch kernels of "Hyper Optimizing
//    Kimi K3 in vLLM", Part 1 section 1 ("Tune shapes for the workload").
//  * mfma (batch > 4): one workgroup per 16-row tile of W; its four waves
//    split K into quarters and run v_mfma_f32_16x16x32_bf16 with the tokens
//    as the A operand (up to four 16-token tiles) and the weight rows as B,
//    then sum the four partial tiles in LDS in a fixed order: the
//    work-splitting kernel the same section uses at larger batch, with the
//    split kept inside one workgroup so no partial sums go through HBM.
//
// Router top-k and RMSNorm need every output of their projection. On the
// dot2 path they run in the projection kernel itself: each workgroup
// publishes its results, a device-scope fence orders them before a counter
// increment, and the workgroup that brings the counter to the grid size
// (after an acquire fence) finishes the job and resets the counter. All
// cross-workgroup sums run in a fixed order, so results are deterministic.
#include <math.h>

#include "k3_device.h"
#include "k3_internal.h"

namespace k3 {

constexpr int kDot2MaxTokens = 4;

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
    __device__ float operator()(int t, int n, float s) const {
        const int64_t i = (int64_t)t * d + n;
        const float h = bf16_to_f32(res[i]) + s;
        h32[i] = h;
        res[i] = f32_to_bf16(h);
        return h;
    }
};

struct EpiResidualStore {  // EpiResidual without the return value
    EpiResidual r;
    __device__ void operator()(int t, int n, float s) const { (void)r(t, n, s); }
};

// Rows per wave so that N rows spread evenly over `waves` waves, rounded up
// to whole RB-row batches.
static inline int rows_per_wave(int N, int waves, int RB) {
    int rpw = (N + waves - 1) / waves;
    return (rpw + RB - 1) / RB * RB;
}

// ------------------------------------------------------------------ dot2 dense
template <int TM, int CB, class Epi>
__global__ void __launch_bounds__(kBlock)
k_dense_dot2(const uint16_t *__restrict__ x, int64_t ldx, int b, const uint16_t *__restrict__ W,
             int N, int K, int rpw, Epi epi) {
    extern __shared__ u32x4 xs[];
    const int nv = K >> 3;
    stage_rows(xs, nv, b, nv, [&](int t) { return x + (int64_t)t * ldx; });
    __syncthreads();
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = blockIdx.x * (kBlock / kWave) + threadIdx.x / kWave;
    const int r0 = wave * rpw, r1 = min(N, r0 + rpw);
    stream_rows<TM, 16 / CB, CB>(
        r0, r1, nv, xs, nv, b, [&](int r) { return W + (int64_t)r * K; },
        [&](int r, int t, float s) {
            if (lane == 0)
                epi(t, r, s);
        });
}

// ------------------------------------------------------------------ top-k
// One wave picks token t's k experts: lane l holds logits l, l + 64, ...;
// k rounds of a wave-wide argmax under the order (logit desc, index asc);
// lane j keeps the j-th pick. The weights are the softmax over the k picked
// logits (the full softmax renormalised over the selection).
__device__ void topk_wave(const float *logits, int E, int k, int32_t *ids, float *wts) {
    constexpr int PER = K3_MAX_EXPERTS / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    float v[PER];
    uint32_t taken = 0;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const int e = i * kWave + lane;
        float l = -INFINITY;
        if (e < E)
            l = logits[e];
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
        ids[lane] = sel_e;
        wts[lane] = p / sum;
    }
}

__global__ void __launch_bounds__(kWave)
k_topk_softmax(const float *__restrict__ logits, int E, int k, int32_t *__restrict__ ids,
               float *__restrict__ wts) {
    const int t = blockIdx.x;
    topk_wave(logits + (int64_t)t * E, E, k, ids + (int64_t)t * k, wts + (int64_t)t * k);
}

// Publish this workgroup's results and count it; true in the one workgroup
// that arrives last, after an acquire fence (all other workgroups' results
// are then visible to its loads).
__device__ bool arrive_last(int *counter) {
    __shared__ int is_last;
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0)
        is_last = atomicAdd(counter, 1) == (int)gridDim.x - 1;
    __syncthreads();
    if (!is_last)
        return false;
    __threadfence();
    return true;
}

// Router logits on the dot2 engine; the last workgroup runs the top-k for
// every token (wave w takes tokens w, w + 4, ...) and resets the counter.
template <int TM, int CB>
__global__ void __launch_bounds__(kBlock)
k_router_dot2(const uint16_t *__restrict__ x, int64_t ldx, int b, const uint16_t *__restrict__ W,
              int E, int d, int rpw, const float *__restrict__ bias, float *logits, int *counter,
              int k, int32_t *__restrict__ ids, float *__restrict__ wts) {
    extern __shared__ u32x4 xs[];
    const int nv = d >> 3;
    stage_rows(xs, nv, b, nv, [&](int t) { return x + (int64_t)t * ldx; });
    __syncthreads();
    const int lane = threadIdx.x & (kWave - 1);
    const int wq = threadIdx.x / kWave;
    const int wave = blockIdx.x * (kBlock / kWave) + wq;
    const int r0 = wave * rpw, r1 = min(E, r0 + rpw);
    stream_rows<TM, 16 / CB, CB>(
        r0, r1, nv, xs, nv, b, [&](int r) { return W + (int64_t)r * d; },
        [&](int r, int t, float s) {
            if (lane == 0)
                logits[(int64_t)t * E + r] = bias ? s + bias[r] : s;
        });
    if (!arrive_last(counter))
        return;
    for (int t = wq; t < b; t += kBlock / kWave)
        topk_wave(logits + (int64_t)t * E, E, k, ids + (int64_t)t * k, wts + (int64_t)t * k);
    if (threadIdx.x == 0)
        atomicExch(counter, 0);
}

// Output projection + residual on the dot2 engine. Lane 0 of each wave keeps
// the running sum of h^2 per token over its rows; the workgroup's four wave
// sums are added in order into ss_part[block][t]; the last workgroup adds the
// ss_part of all workgroups in block order and writes y = h * inv * gamma.
template <int TM, int CB>
__global__ void __launch_bounds__(kBlock)
k_oproj_dot2(const uint16_t *__restrict__ a, int64_t lda, int b, const uint16_t *__restrict__ Wo,
             int d, int K, int rpw, uint16_t *res, const uint16_t *__restrict__ gamma, float eps,
             float *h32, float *ss_part, int *counter, uint16_t *__restrict__ y) {
    extern __shared__ u32x4 xs[];
    __shared__ float wss[kBlock / kWave][TM];
    __shared__ float inv[TM];
    const int nv = K >> 3;
    stage_rows(xs, nv, b, nv, [&](int t) { return a + (int64_t)t * lda; });
    __syncthreads();
    const int lane = threadIdx.x & (kWave - 1);
    const int wq = threadIdx.x / kWave;
    const int wave = blockIdx.x * (kBlock / kWave) + wq;
    const int r0 = wave * rpw, r1 = min(d, r0 + rpw);
    const EpiResidual er{res, h32, d};
    float ss[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t)
        ss[t] = 0.0f;
    stream_rows<TM, 16 / CB, CB>(
        r0, r1, nv, xs, nv, b, [&](int r) { return Wo + (int64_t)r * K; },
        [&](int r, int t, float s) {
            if (lane == 0) {
                const float h = er(t, r, s);
                ss[t] += h * h;
            }
        });
    if (lane == 0)
#pragma unroll
        for (int t = 0; t < TM; ++t)
            wss[wq][t] = ss[t];
    __syncthreads();
    if (threadIdx.x < b)
        ss_part[(int64_t)blockIdx.x * TM + threadIdx.x] =
            (wss[0][threadIdx.x] + wss[1][threadIdx.x]) + (wss[2][threadIdx.x] + wss[3][threadIdx.x]);
    if (!arrive_last(counter))
        return;
    if (wq < b) {  // wave t sums token t's partials: lanes take blocks l, l+64, ...
        float s = 0.0f;
        for (int g = lane; g < (int)gridDim.x; g += kWave)
            s += ss_part[(int64_t)g * TM + wq];
        s = wave_sum(s);
        if (lane == 0)
            inv[wq] = 1.0f / sqrtf(s / (float)d + eps);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < b * d; i += kBlock) {
        const int t = i / d, n = i - t * d;
        y[i] = f32_to_bf16(h32[i] * inv[t] * bf16_to_f32(gamma[n]));
    }
    if (threadIdx.x == 0)
        atomicExch(counter, 0);
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
                            const u32x4 av = aval[mt] ? ld_act16(x + aoff[mt] + k) : zero16();
                            acc[mt] = mfma16x16x32(av, bfr[u], acc[mt]);
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

// One workgroup per token: y = h / sqrt(mean(h^2) + eps) * gamma, the mean in
// fp32 with a fixed reduction order; loads are issued in 16-byte vectors so
// the loop is not latency-bound (d % 4 == 0).
__global__ void __launch_bounds__(kBlock)
k_rmsnorm(const float *__restrict__ h32, int d, const uint16_t *__restrict__ gamma, float eps,
          uint16_t *__restrict__ y) {
    __shared__ float part[kBlock / kWave];
    const int t = blockIdx.x;
    const f32x4 *h = reinterpret_cast<const f32x4 *>(h32 + (int64_t)t * d);
    const int n4 = d >> 2;
    float ss = 0.0f;
#pragma unroll 8
    for (int i = threadIdx.x; i < n4; i += kBlock) {
        const f32x4 v = h[i];
        ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
    }
    ss = wave_sum(ss);
    if ((threadIdx.x & (kWave - 1)) == 0)
        part[threadIdx.x / kWave] = ss;
    __syncthreads();
    const float inv = 1.0f / sqrtf(((part[0] + part[1]) + (part[2] + part[3])) / (float)d + eps);
#pragma unroll 8
    for (int i = threadIdx.x; i < n4; i += kBlock) {
        const f32x4 v = h[i];
        uint16_t *o = y + (int64_t)t * d + 4 * i;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            o[j] = f32_to_bf16(v[j] * inv * bf16_to_f32(gamma[4 * i + j]));
    }
}

// ------------------------------------------------------------------ launchers
// Launch geometry of the dot2 engine: one workgroup (four waves) per compute
// unit by default; each wave streams an even share of the rows.
struct Dot2Geom {
    int grid, rpw, cb;
    size_t lds;
};

static Dot2Geom dot2_geom(int N, int K, int b, int cu_budget) {
    Dot2Geom g;
    g.cb = K > 2048 ? 16 : (K > 512 ? 4 : 1);
    const int rb = 16 / g.cb;
    const int cus = budget_grid(1 << 30, cu_budget, 1);
    g.rpw = rows_per_wave(N, cus * (kBlock / kWave), rb);
    const int waves = (N + g.rpw - 1) / g.rpw;
    g.grid = (waves + 3) / 4;
    g.lds = (size_t)b * K * sizeof(uint16_t);
    return g;
}

// The dot2 engine keeps a whole row in one register buffer (K <= 8192) and
// the b token rows in LDS (at most 64 KB).
static bool dot2_fits(int b, int K) {
    return b <= kDot2MaxTokens && K <= 16 * 512 && (size_t)b * K * 2 <= 65536;
}

template <int TM, class Epi>
static void launch_dense_dot2_t(const uint16_t *x, int64_t ldx, int b, const uint16_t *W, int N,
                                int K, Epi epi, hipStream_t s) {
    const Dot2Geom g = dot2_geom(N, K, b, 0);
    if (g.cb == 16)
        k_dense_dot2<TM, 16, Epi><<<g.grid, kBlock, g.lds, s>>>(x, ldx, b, W, N, K, g.rpw, epi);
    else if (g.cb == 4)
        k_dense_dot2<TM, 4, Epi><<<g.grid, kBlock, g.lds, s>>>(x, ldx, b, W, N, K, g.rpw, epi);
    else
        k_dense_dot2<TM, 1, Epi><<<g.grid, kBlock, g.lds, s>>>(x, ldx, b, W, N, K, g.rpw, epi);
}

template <class Epi>
static void launch_dense(int variant, const uint16_t *x, int64_t ldx, int b, const uint16_t *W,
                         int N, int K, Epi epi, hipStream_t s) {
    if (variant == K3_VARIANT_DOT2) {
        if (b == 1)
            launch_dense_dot2_t<1>(x, ldx, b, W, N, K, epi, s);
        else
            launch_dense_dot2_t<kDot2MaxTokens>(x, ldx, b, W, N, K, epi, s);
    } else {
        const int grid = budget_grid((N + 15) / 16, 0, 4);
        k_gemm_mfma<8, Epi><<<grid, kBlock, 0, s>>>(x, ldx, b, W, N, K, epi);
    }
}

// Variant for a dense [N x K] read at batch b: dot2 while the tokens fit the
// engine, MFMA above (MFMA needs K % 128 == 0 so each K quarter is whole
// 32-wide steps).
static int pick_dense_variant(int op, int b, int K) {
    int v = forced_variant(op);
    if (v == K3_VARIANT_NONE)
        v = dot2_fits(b, K) ? K3_VARIANT_DOT2 : K3_VARIANT_MFMA;
    if (v == K3_VARIANT_DOT2 && !dot2_fits(b, K))
        return -1;
    if (v == K3_VARIANT_MFMA && K % 128 != 0)
        return -1;
    if (v != K3_VARIANT_DOT2 && v != K3_VARIANT_MFMA)
        return -1;
    return v;
}

}  // namespace k3

using namespace k3;

// ------------------------------------------------------------------ workspace layouts
// The completion counter sits at offset 0, where it stays whatever the shape
// of the call, so a workspace reused for other shapes of the same entry
// point still finds it at zero.
namespace {
constexpr size_t kCounterBytes = 256;
size_t oproj_h32_offset() { return kCounterBytes; }
size_t oproj_ss_offset(int b, int d) {
    return kCounterBytes + align_up((size_t)b * d * sizeof(float), 256);
}
size_t router_logits_offset() { return kCounterBytes; }
}  // namespace

extern "C" size_t k3_router_topk_workspace_size(int b, int E) {
    if (b <= 0 || E <= 0)
        return 0;
    return router_logits_offset() + align_up((size_t)b * E * sizeof(float), 256);
}

extern "C" size_t k3_oproj_residual_workspace_size(int b, int K, int d) {
    (void)K;
    if (b <= 0 || d <= 0)
        return 0;
    return oproj_ss_offset(b, d) + align_up((size_t)1024 * kDot2MaxTokens * sizeof(float), 256);
}

extern "C" size_t k3_proj_skinny_workspace_size(int b, int K, int N) {
    (void)b;
    (void)K;
    (void)N;
    return 0;
}

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
    launch_dense(variant, x, ldx, b, w, N, K, EpiBf16{y, ldy}, s);
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
    if (!workspace || ws_bytes < k3_router_topk_workspace_size(b, E) || !aligned16(workspace))
        return K3_ERR_WORKSPACE;
    const int variant = pick_dense_variant(K3_OP_ROUTER_TOPK, b, d);
    if (variant < 0)
        return K3_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    int *counter = (int *)workspace;
    float *logits = (float *)((char *)workspace + router_logits_offset());
    trace_begin(K3_OP_ROUTER_TOPK, s);
    if (variant == K3_VARIANT_DOT2) {
        const Dot2Geom g = dot2_geom(E, d, b, 0);
        if (g.cb == 16 && b == 1)
            k_router_dot2<1, 16><<<g.grid, kBlock, g.lds, s>>>(x, ldx, b, w_router, E, d, g.rpw,
                                                              bias, logits, counter, k, topk_ids,
                                                              topk_w);
        else if (g.cb == 16)
            k_router_dot2<kDot2MaxTokens, 16><<<g.grid, kBlock, g.lds, s>>>(
                x, ldx, b, w_router, E, d, g.rpw, bias, logits, counter, k, topk_ids, topk_w);
        else if (g.cb == 4)
            k_router_dot2<kDot2MaxTokens, 4><<<g.grid, kBlock, g.lds, s>>>(
                x, ldx, b, w_router, E, d, g.rpw, bias, logits, counter, k, topk_ids, topk_w);
        else
            k_router_dot2<kDot2MaxTokens, 1><<<g.grid, kBlock, g.lds, s>>>(
                x, ldx, b, w_router, E, d, g.rpw, bias, logits, counter, k, topk_ids, topk_w);
        trace_end(K3_OP_ROUTER_TOPK, s);
    } else {
        launch_dense(variant, x, ldx, b, w_router, E, d, EpiLogits{logits, E, bias}, s);
        trace_end(K3_OP_ROUTER_TOPK, s);
        k_topk_softmax<<<b, kWave, 0, s>>>(logits, E, k, topk_ids, topk_w);
    }
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
    if (b > K3_MAX_BATCH || K % 8 || lda % 8 || d % 8 || !aligned16(a) || !aligned16(w_o) ||
        !aligned16(residual))
        return K3_ERR_UNSUPPORTED;
    if (!workspace || ws_bytes < k3_oproj_residual_workspace_size(b, K, d) ||
        !aligned16(workspace))
        return K3_ERR_WORKSPACE;
    const int variant = pick_dense_variant(K3_OP_OPROJ_RESIDUAL, b, K);
    if (variant < 0)
        return K3_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    char *ws = (char *)workspace;
    int *counter = (int *)ws;
    float *h32 = (float *)(ws + oproj_h32_offset());
    float *ss_part = (float *)(ws + oproj_ss_offset(b, d));
    trace_begin(K3_OP_OPROJ_RESIDUAL, s);
    if (variant == K3_VARIANT_DOT2) {
        const Dot2Geom g = dot2_geom(d, K, b, 0);
        if (g.grid > 1024)
            return K3_ERR_UNSUPPORTED;
        if (g.cb == 16 && b == 1)
            k_oproj_dot2<1, 16><<<g.grid, kBlock, g.lds, s>>>(a, lda, b, w_o, d, K, g.rpw,
                                                             residual, gamma, eps, h32, ss_part,
                                                             counter, y_norm);
        else if (g.cb == 16)
            k_oproj_dot2<kDot2MaxTokens, 16><<<g.grid, kBlock, g.lds, s>>>(
                a, lda, b, w_o, d, K, g.rpw, residual, gamma, eps, h32, ss_part, counter, y_norm);
        else if (g.cb == 4)
            k_oproj_dot2<kDot2MaxTokens, 4><<<g.grid, kBlock, g.lds, s>>>(
                a, lda, b, w_o, d, K, g.rpw, residual, gamma, eps, h32, ss_part, counter, y_norm);
        else
            k_oproj_dot2<kDot2MaxTokens, 1><<<g.grid, kBlock, g.lds, s>>>(
                a, lda, b, w_o, d, K, g.rpw, residual, gamma, eps, h32, ss_part, counter, y_norm);
        trace_end(K3_OP_OPROJ_RESIDUAL, s);
    } else {
        launch_dense(variant, a, lda, b, w_o, d, K, EpiResidualStore{EpiResidual{residual, h32, d}},
                     s);
        trace_end(K3_OP_OPROJ_RESIDUAL, s);
        k_rmsnorm<<<b, kBlock, 0, s>>>(h32, d, gamma, eps, y_norm);
    }
    const int st = launch_status();
    if (st == K3_OK)
        record_dispatch(K3_OP_OPROJ_RESIDUAL, variant);
    return st;
}
