// dense.hip -- skinny dense projections, router scoring + top-k, and the
// output projection with residual add and RMSNorm.
//
// Two engines serve the dense [N x K] weight reads here:
//  * dot2 (batch <= 4): the row-streaming engine of k3_device.h -- each wave
//    owns whole weight rows, reads them 1 KB per load instruction with two
//    row buffers in flight, and multiplies against the tokens staged in LDS
//    with v_dot2c_f32_bf16. The small-batch kernels of "Hyper Optimizing
//    Kimi K3 in vLLM", Part 1 section 1 ("Tune shapes for the workload").
//  * mfma (batch > 4): the split-K MFMA engine of k3_skinny.h (skinny.hip),
//    whose partial sums a small kernel finishes (bf16 projection, fp32
//    logits, or residual + RMSNorm): the work-splitting kernels the same
//    section uses at larger batch.
//
// Router top-k and RMSNorm need every output of their projection; each runs
// as a small kernel after it. (Finishing them in the last workgroup of the
// projection would need a device-scope release per workgroup, which on this
// multi-XCD part writes back the L2 and drains every load in flight.) All
// sums run in a fixed order, so results are deterministic.
#include <math.h>

#include "k3_device.h"
#include "k3_gemv.h"
#include "k3_internal.h"
#include "k3_skinny.h"

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
    const int lane = threadIdx.x & (kWave - 1);
    const int wave = blockIdx.x * (kBlock / kWave) + wave_in_block();
    const int r0 = wave * rpw, r1 = min(N, r0 + rpw);
    stream_rows<TM, 16 / CB, CB>(
        r0, r1, nv, xs, nv, b, [&](int r) { return W + (int64_t)r * K; },
        [&](int r, int t, float s) {
            if (lane == 0)
                epi(t, r, s);
        },
        [&]() {
            stage_rows(xs, nv, b, nv, [&](int t) { return x + (int64_t)t * ldx; });
            __syncthreads();
        });
}

// ------------------------------------------------------------------ top-k
__global__ void __launch_bounds__(kWave)
k_topk_softmax(const float *__restrict__ logits, int E, int k, int32_t *__restrict__ ids,
               float *__restrict__ wts) {
    const int t = blockIdx.x;
    topk_wave(logits + (int64_t)t * E, E, k, ids + (int64_t)t * k, wts + (int64_t)t * k);
}

// One pass over the staged input x for every row set that reads it: E router
// rows (fp32 logits, + bias), NL latent rows (z, bf16) and, when Is > 0, the
// shared expert's Is gate/up row pairs (h_s = silu(gate) * up, bf16). Wave w
// takes an even share of each set, in that order, in one pipeline; the
// router bias is staged in LDS beside x so the epilogues load nothing from
// global memory behind the weight stream. No workgroup waits for another:
// the top-k runs in the next kernel.
template <int TM, int CB>
__global__ void __launch_bounds__(kBlock)
k_rls_dot2(const uint16_t *__restrict__ x, int64_t ldx, int b, int d,
           const uint16_t *__restrict__ Wr, const float *__restrict__ bias, int E,
           float *__restrict__ logits, const uint16_t *__restrict__ Wl, int NL,
           uint16_t *__restrict__ z, int64_t ldz, const uint16_t *__restrict__ W13s, int Is,
           uint16_t *__restrict__ hs) {
    extern __shared__ u32x4 xs[];
    const int nv = d >> 3;
    float *bs = reinterpret_cast<float *>(xs + b * nv);
    const int lane = threadIdx.x & (kWave - 1);
    const int waves = gridDim.x * (kBlock / kWave);
    const int wave = blockIdx.x * (kBlock / kWave) + wave_in_block();
    int ra, rb, la, lb, sa, sb;
    split_range(E, waves, wave, ra, rb);
    split_range(NL, waves, waves - 1 - wave, la, lb);  // spare latent rows to router-free waves
    split_range(Is, waves, wave, sa, sb);
    const int nr = rb - ra, nrl = nr + (lb - la);
    float gsave[TM];
#pragma unroll
    for (int t = 0; t < TM; ++t)
        gsave[t] = 0.0f;
    stream_rows<TM, (CB == 1 && TM > 1) ? 4 : 16 / CB, CB>(
        0, nrl + 2 * (sb - sa), nv, xs, nv, b,
        [&](int i) {
            if (i < nr)
                return Wr + (int64_t)(ra + i) * d;
            if (i < nrl)
                return Wl + (int64_t)(la + i - nr) * d;
            const int q = i - nrl, j = sa + (q >> 1);
            return W13s + (int64_t)((q & 1) ? Is + j : j) * d;
        },
        [&](int i, int t, float s) {
            if (i < nr) {
                if (lane == 0)
                    logits[(int64_t)t * E + ra + i] = s + bs[ra + i];
            } else if (i < nrl) {
                if (lane == 0)
                    z[(int64_t)t * ldz + la + i - nr] = f32_to_bf16(s);
            } else {
                const int q = i - nrl;
                if ((q & 1) == 0)
                    gsave[t] = s;
                else if (lane == 0)
                    hs[(int64_t)t * Is + sa + (q >> 1)] = f32_to_bf16(silu(gsave[t]) * s);
            }
        },
        [&]() {
            stage_rows(xs, nv, b, nv, [&](int t) { return x + (int64_t)t * ldx; });
            for (int e = threadIdx.x; e < E; e += kBlock)
                bs[e] = bias ? bias[e] : 0.0f;
            __syncthreads();
        });
}

// Output projection + residual on the dot2 engine: h = r + a . Wo^T, written
// as fp32 (for the norm) and bf16 (back into r). The residuals of the
// block's rows are staged in LDS with the activations, so the epilogue loads
// nothing from global memory behind the weight stream. RMSNorm follows in
// its own kernel.
template <int TM, int CB>
__global__ void __launch_bounds__(kBlock)
k_oproj_dot2(const uint16_t *__restrict__ a, int64_t lda, int b, const uint16_t *__restrict__ Wo,
             int d, int K, int rows_blk, uint16_t *res, float *__restrict__ h32) {
    extern __shared__ u32x4 xs[];
    const int nv = K >> 3;
    // the rows split evenly over the workgroups (every compute unit streams
    // the same share), then over the block's waves
    int rblk, rend;
    split_range(d, gridDim.x, blockIdx.x, rblk, rend);
    float *rs = reinterpret_cast<float *>(xs + b * nv);  // [b][rows_blk], rows_blk >= rend - rblk
    const int lane = threadIdx.x & (kWave - 1);
    int q0, q1;
    split_range(rend - rblk, kBlock / kWave, wave_in_block(), q0, q1);
    const int r0 = rblk + q0, r1 = rblk + q1;
    stream_rows<TM, 16 / CB, CB>(
        r0, r1, nv, xs, nv, b, [&](int r) { return Wo + (int64_t)r * K; },
        [&](int r, int t, float s) {
            if (lane == 0) {
                const int64_t i = (int64_t)t * d + r;
                const float h = rs[t * rows_blk + (r - rblk)] + s;
                h32[i] = h;
                res[i] = f32_to_bf16(h);
            }
        },
        [&]() {
            stage_rows(xs, nv, b, nv, [&](int t) { return a + (int64_t)t * lda; });
            for (int i = threadIdx.x; i < b * rows_blk; i += kBlock) {
                const int t = i / rows_blk, r = rblk + (i - t * rows_blk);
                rs[i] = r < rend ? bf16_to_f32(res[(int64_t)t * d + r]) : 0.0f;
            }
            __syncthreads();
        });
}

// One token's RMSNorm by one workgroup: y = h / sqrt(mean(h^2) + eps) *
// gamma, the mean in fp32 with a fixed reduction order (d % 4 == 0,
// d <= 8192). load() issues every load of h and gamma (indexes clamped, no
// branches), finish() waits for them, reduces (one barrier) and hands
// element e of y to out(e, bf16).
constexpr int kNormVec = 8;
struct RmsRow {
    f32x4 v[kNormVec];  // thread i holds elements 4 (i + 256 j) .. + 3
    uint16_t gm[kNormVec][4];
    __device__ __forceinline__ void load_gamma(int d, const uint16_t *__restrict__ gamma) {
        const int n4 = d >> 2;
#pragma unroll
        for (int j = 0; j < kNormVec; ++j) {
            const int i = threadIdx.x + j * kBlock;
            const int ic = i < n4 ? i : 0;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                gm[j][q] = gamma[4 * ic + q];
        }
    }
    __device__ __forceinline__ void load(const float *__restrict__ h32, int d,
                                         const uint16_t *__restrict__ gamma) {
        const f32x4 *h = reinterpret_cast<const f32x4 *>(h32);
        const int n4 = d >> 2;
#pragma unroll
        for (int j = 0; j < kNormVec; ++j) {
            const int i = threadIdx.x + j * kBlock;
            v[j] = h[i < n4 ? i : 0];
        }
        load_gamma(d, gamma);
    }
    template <class Out>
    __device__ __forceinline__ void finish(int d, float eps, Out out) const {
        __shared__ float part[kBlock / kWave];
        const int n4 = d >> 2;
        float ss = 0.0f;
#pragma unroll
        for (int j = 0; j < kNormVec; ++j)
            if (threadIdx.x + j * kBlock < n4)
                ss += v[j].x * v[j].x + v[j].y * v[j].y + v[j].z * v[j].z + v[j].w * v[j].w;
        ss = wave_sum(ss);
        if ((threadIdx.x & (kWave - 1)) == 0)
            part[threadIdx.x / kWave] = ss;
        __syncthreads();
        const float inv =
            1.0f / sqrtf(((part[0] + part[1]) + (part[2] + part[3])) / (float)d + eps);
#pragma unroll
        for (int j = 0; j < kNormVec; ++j) {
            const int i = threadIdx.x + j * kBlock;
            if (i < n4)
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    out(4 * i + q, f32_to_bf16(v[j][q] * inv * bf16_to_f32(gm[j][q])));
        }
    }
};

// One workgroup per token.
__global__ void __launch_bounds__(kBlock)
k_rmsnorm(const float *__restrict__ h32, int d, const uint16_t *__restrict__ gamma, float eps,
          uint16_t *__restrict__ y) {
    const int t = blockIdx.x;
    uint16_t *yt = y + (int64_t)t * d;
    RmsRow rr;
    rr.load(h32 + (int64_t)t * d, d, gamma);
    rr.finish(d, eps, [&](int e, uint16_t v) { yt[e] = v; });
}

// The o-projection's finish fused with the norm, one workgroup per token:
// h = r + the K ranges' fp32 partial sums (added in range order, as
// k_sk_finish adds them), r <- bf16(h), h32 <- h, y = RMSNorm(h) * gamma (as
// k_rmsnorm computes it). part[(ks * T + t) * d + n]; d % 4 == 0.
__global__ void __launch_bounds__(kBlock)
k_oproj_finish_rmsnorm(const float *__restrict__ part, int ks, int T, int d, uint16_t *res,
                       float *__restrict__ h32, const uint16_t *__restrict__ gamma, float eps,
                       uint16_t *__restrict__ y) {
    const int t = blockIdx.x, n4 = d >> 2;
    const int64_t stride = (int64_t)T * d / 4;  // one K range, in 16-byte vectors
    const f32x4 *p = reinterpret_cast<const f32x4 *>(part + (int64_t)t * d);
    uint2 *r = reinterpret_cast<uint2 *>(res + (int64_t)t * d);
    f32x4 *h = reinterpret_cast<f32x4 *>(h32 + (int64_t)t * d);
    RmsRow rr;
    // the K ranges in two halves of kSkMaxSplit / 2 (every load of a half in
    // flight at once), added in range order
    constexpr int HS = kSkMaxSplit / 2;
    f32x4 pv[kNormVec][HS], acc[kNormVec];
    uint2 rv[kNormVec];
#pragma unroll
    for (int j = 0; j < kNormVec; ++j) {
        const int i = threadIdx.x + j * kBlock;
        const int ic = i < n4 ? i : 0;
        rv[j] = r[ic];
#pragma unroll
        for (int q = 0; q < HS; ++q)
            pv[j][q] = p[ic + (q < ks ? q : 0) * stride];
    }
    rr.load_gamma(d, gamma);
#pragma unroll
    for (int j = 0; j < kNormVec; ++j) {
        acc[j] = pv[j][0];
#pragma unroll
        for (int q = 1; q < HS; ++q)
            if (q < ks)
                acc[j] += pv[j][q];
    }
    if (ks > HS) {
#pragma unroll
        for (int j = 0; j < kNormVec; ++j) {
            const int i = threadIdx.x + j * kBlock;
            const int ic = i < n4 ? i : 0;
#pragma unroll
            for (int q = 0; q < HS; ++q)
                pv[j][q] = p[ic + (HS + q < ks ? HS + q : 0) * stride];
        }
#pragma unroll
        for (int j = 0; j < kNormVec; ++j)
#pragma unroll
            for (int q = 0; q < HS; ++q)
                if (HS + q < ks)
                    acc[j] += pv[j][q];
    }
#pragma unroll
    for (int j = 0; j < kNormVec; ++j) {
        f32x4 v = acc[j];
        const uint32_t lo = rv[j].x, hi = rv[j].y;
        v.x += bf16_to_f32((uint16_t)(lo & 0xffffu));
        v.y += bf16_to_f32((uint16_t)(lo >> 16));
        v.z += bf16_to_f32((uint16_t)(hi & 0xffffu));
        v.w += bf16_to_f32((uint16_t)(hi >> 16));
        rr.v[j] = v;
        const int i = threadIdx.x + j * kBlock;
        if (i < n4) {
            h[i] = v;
            r[i] = uint2{(uint32_t)f32_to_bf16(v.x) | ((uint32_t)f32_to_bf16(v.y) << 16),
                         (uint32_t)f32_to_bf16(v.z) | ((uint32_t)f32_to_bf16(v.w) << 16)};
        }
    }
    uint16_t *yt = y + (int64_t)t * d;
    rr.finish(d, eps, [&](int e, uint16_t v) { yt[e] = v; });
}

// ------------------------------------------------------------------ batch 1 (k3_gemv.h)
// Shares of the rows per workgroup and the LDS layout of the 8-row engine:
// x (K / 8 vectors), then the four quarters' partial sums [4][ps_stride],
// then (o-proj) the residuals of the share, for nt tokens.
struct GemvGeom {
    int grid, ps_stride;
    size_t lds;
};

static GemvGeom gemv_geom(int N, int K, bool resid, int cu_budget = 0, int nt = 1) {
    GemvGeom g;
    g.grid = budget_grid(N, cu_budget, 2);
    const int rows = (N + g.grid - 1) / g.grid;
    g.ps_stride = (rows + 7) / 8 * 8;
    g.lds = (size_t)nt * K * 2 + (size_t)(4 + (resid ? 1 : 0)) * nt * g.ps_stride * sizeof(float);
    return g;
}

// The 8-row engine takes K in 64-element pieces.
static bool gemv_fits(int K) { return K % 64 == 0 && K <= 8192; }

// y[t][n] = epi(t, n, x[t] . W[n]) for NT (1..4) tokens, rows ldx apart.
template <int U, int NT, class Epi>
__global__ void __launch_bounds__(kBlock)
k_gemv(const uint16_t *__restrict__ x, int64_t ldx, const uint16_t *__restrict__ W, int N,
       int K, int ps_stride, Epi epi) {
    extern __shared__ u32x4 xs[];  // NT token rows, then ps[4][NT][ps_stride]
    const int nv = K >> 3;
    float *ps = reinterpret_cast<float *>(xs + NT * nv);
    int r0, r1;
    split_range(N, gridDim.x, blockIdx.x, r0, r1);
    GvStage<4> st[NT];  // K <= 8192
    gemv8_stream<U, NT>(
        (r1 - r0 + 7) >> 3, K,
        [&](int g, const uint16_t *&base, int &nr, int &skip) {
            base = W + (int64_t)(r0 + 8 * g) * K;
            nr = min(8, r1 - r0 - 8 * g);
            skip = 0;
        },
        [&](int, int kv, int t) { return xs[t * nv + kv]; }, ps, ps_stride,
        [&]() {
#pragma unroll
            for (int t = 0; t < NT; ++t)
                st[t].load(x + (int64_t)t * ldx, nv);
        },
        [&]() {
#pragma unroll
            for (int t = 0; t < NT; ++t)
                st[t].store(xs + t * nv, nv);
            __syncthreads();
        });
    const int rows = r1 - r0;
    for (int q = threadIdx.x; q < NT * rows; q += kBlock) {
        const int t = q / rows, i = q - t * rows;
        epi(t, r0 + i, gv_total(ps, ps_stride, i, NT, t));
    }
}

// Output projection + residual for NT (1..4) tokens: h = r + a . Wo^T,
// written as fp32 (for the norm) and bf16 (back into r). The share's
// residuals are staged beside a while the first weights load (thread q
// holds residual q of the NT x rows share; NT * rows <= the block size).
template <int U, int NT>
__global__ void __launch_bounds__(kBlock)
k_oproj_gemv(const uint16_t *__restrict__ a, int64_t lda, const uint16_t *__restrict__ Wo,
             int d, int K, int ps_stride, uint16_t *res, float *__restrict__ h32) {
    extern __shared__ u32x4 xs[];  // NT rows of a, ps[4][NT][ps_stride], rs[NT * rows]
    const int nv = K >> 3;
    float *ps = reinterpret_cast<float *>(xs + NT * nv);
    float *rs = ps + 4 * NT * ps_stride;
    int r0, r1;
    split_range(d, gridDim.x, blockIdx.x, r0, r1);
    const int rows = r1 - r0;
    GvStage<4> st[NT];  // K <= 8192
    uint16_t rv = 0;
    gemv8_stream<U, NT>(
        (rows + 7) >> 3, K,
        [&](int g, const uint16_t *&base, int &nr, int &skip) {
            base = Wo + (int64_t)(r0 + 8 * g) * K;
            nr = min(8, rows - 8 * g);
            skip = 0;
        },
        [&](int, int kv, int t) { return xs[t * nv + kv]; }, ps, ps_stride,
        [&]() {
#pragma unroll
            for (int t = 0; t < NT; ++t)
                st[t].load(a + (int64_t)t * lda, nv);
            const int q = min((int)threadIdx.x, NT * rows - 1), t = q / rows;
            rv = res[(int64_t)t * d + r0 + (q - t * rows)];
        },
        [&]() {
#pragma unroll
            for (int t = 0; t < NT; ++t)
                st[t].store(xs + t * nv, nv);
            if ((int)threadIdx.x < NT * rows)
                rs[threadIdx.x] = bf16_to_f32(rv);
            __syncthreads();
        });
    for (int q = threadIdx.x; q < NT * rows; q += kBlock) {
        const int t = q / rows, i = q - t * rows;
        const float h = rs[q] + gv_total(ps, ps_stride, i, NT, t);
        h32[(int64_t)t * d + r0 + i] = h;
        res[(int64_t)t * d + r0 + i] = f32_to_bf16(h);
    }
}

// The pass of NT (1..4) tokens over x for every row set that reads it (as
// k_rls_dot2):
// E router rows (fp32 logits + bias), NL latent rows (z, bf16) and Is shared
// gate/up row pairs (h_s = silu(gate) * up, bf16). The rows form one
// sequence of 8-row groups -- router, latent, then shared pair groups (gate
// rows 4q .. 4q + 3 with up rows Is + 4q .. Is + 4q + 3) -- split evenly
// over the workgroups. Each row is summed in the same order as k_gemv, so
// logits and z match the separate calls bit for bit.
// With NORM (one token) the input is x = RMSNorm(h32) * gamma (as k_rmsnorm
// computes it), normalised by every workgroup while its first weights load;
// workgroup 0 also writes x to x_out when that is not null.
// After the outputs: nothing (NoFinish), or LastTopk.
struct NoFinish {
    __device__ void operator()(const float *, int) const {}
};

// The forced K3_VARIANT_LASTWG of the one-token router: every workgroup
// publishes its logits (agent-scope release fence) and takes a ticket from
// the counter; the holder of the last ticket acquires, resets the counter for
// the next call and selects the token's experts from all E logits, as
// k_topk_softmax does.
struct LastTopk {
    int *counter;  // zero before the launch, zero after it
    int k;
    int32_t *ids;
    float *wts;
    __device__ void operator()(const float *logits, int E) const {
        __shared__ int last;
        __threadfence();
        __syncthreads();
        if (threadIdx.x == 0)
            last = atomicAdd(counter, 1) == (int)gridDim.x - 1;
        __syncthreads();
        if (!last)
            return;
        __threadfence();
        if (threadIdx.x == 0)
            *counter = 0;
        if (threadIdx.x < kWave)
            topk_wave(logits, E, k, ids, wts);
    }
};

template <int U, int NT, bool NORM, class Fin = NoFinish>
__global__ void __launch_bounds__(kBlock)
k_rls_gemv(const uint16_t *__restrict__ x, int64_t ldx, int d, const uint16_t *__restrict__ Wr,
            const float *__restrict__ bias, int E, float *__restrict__ logits,
            const uint16_t *__restrict__ Wl, int NL, uint16_t *__restrict__ z,
            const uint16_t *__restrict__ W13s, int Is, uint16_t *__restrict__ hs,
            int ps_stride, const float *__restrict__ h32, const uint16_t *__restrict__ gamma,
            float eps, uint16_t *__restrict__ x_out, int64_t ldz, Fin fin = Fin{}) {
    extern __shared__ u32x4 xs[];  // NT token rows, then ps[4][NT][ps_stride], then bias
    const int nv = d >> 3;
    float *ps = reinterpret_cast<float *>(xs + NT * nv);
    float *bs = ps + 4 * NT * ps_stride;
    const int Gr = (E + 7) >> 3, Gl = (NL + 7) >> 3, Gs = Is >> 2;
    int g0, g1;
    split_range(Gr + Gl + Gs, gridDim.x, blockIdx.x, g0, g1);
    GvStage<4> st[NT];  // d <= 8192
    RmsRow rr;
    float bv[4];    // router bias, E <= 1024
    gemv8_stream<U, NT>(
        g1 - g0, d,
        [&](int g, const uint16_t *&base, int &nr, int &skip) {
            const int vg = g0 + g;
            skip = 0;
            if (vg < Gr) {
                base = Wr + (int64_t)(8 * vg) * d;
                nr = min(8, E - 8 * vg);
            } else if (vg < Gr + Gl) {
                const int r = 8 * (vg - Gr);
                base = Wl + (int64_t)r * d;
                nr = min(8, NL - r);
            } else {
                base = W13s + (int64_t)(4 * (vg - Gr - Gl)) * d;
                nr = 8;
                skip = Is - 4;
            }
        },
        [&](int, int kv, int t) { return xs[t * nv + kv]; }, ps, ps_stride,
        [&]() {
            if (NORM) {
                rr.load(h32, d, gamma);
            } else {
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    st[t].load(x + (int64_t)t * ldx, nv);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = threadIdx.x + j * kBlock;
                bv[j] = bias ? bias[e < E ? e : 0] : 0.0f;
            }
        },
        [&]() {
            if (NORM) {
                uint16_t *x16 = reinterpret_cast<uint16_t *>(xs);
                const bool pub = x_out && blockIdx.x == 0;
                rr.finish(d, eps, [&](int e, uint16_t v) {
                    x16[e] = v;
                    if (pub)
                        x_out[e] = v;
                });
            } else {
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    st[t].store(xs + t * nv, nv);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int e = threadIdx.x + j * kBlock;
                if (e < E)
                    bs[e] = bv[j];
            }
            __syncthreads();
        });
    const int nrow = 8 * (g1 - g0);
    for (int q = threadIdx.x; q < NT * nrow; q += kBlock) {
        const int t = q / nrow, i = q - t * nrow;
        const int vg = g0 + (i >> 3), r = i & 7;
        if (vg < Gr) {
            const int e = 8 * vg + r;
            if (e < E)
                logits[(int64_t)t * E + e] = gv_total(ps, ps_stride, i, NT, t) + bs[e];
        } else if (vg < Gr + Gl) {
            const int n = 8 * (vg - Gr) + r;
            if (n < NL)
                z[(int64_t)t * ldz + n] = f32_to_bf16(gv_total(ps, ps_stride, i, NT, t));
        } else if (r < 4) {
            hs[(int64_t)t * Is + 4 * (vg - Gr - Gl) + r] =
                f32_to_bf16(silu(gv_total(ps, ps_stride, i, NT, t)) *
                            gv_total(ps, ps_stride, i + 4, NT, t));
        }
    }
    fin(logits, E);
}

static int rls_gemv_ps_stride(int E, int NL, int Is, int grid) {
    const int total = (E + 7) / 8 + (NL + 7) / 8 + Is / 4;
    return 8 * ((total + grid - 1) / grid);
}

// LDS of one 8-row-engine workgroup: two of them per compute unit share its
// 160 KB (and the device's per-workgroup limit applies).
static size_t gemv_lds_cap() {
    const size_t cap = device_max_lds();
    return cap < 81920 ? cap : 81920;
}

// The 8-row engine serves b tokens while their rows (and the partial sums)
// fit gemv_lds_cap(); the o-projection also needs b x rows <= the block size.
static bool gemv_fits_b(int b, int N, int K, bool resid, int cu_budget = 0) {
    if (b < 1 || b > kDot2MaxTokens || !gemv_fits(K))
        return false;
    const GemvGeom g = gemv_geom(N, K, resid, cu_budget, b);
    return g.lds <= gemv_lds_cap() && (!resid || b * g.ps_stride <= kBlock);
}

template <int NT, class Epi>
static void launch_gemv_nt(const uint16_t *x, int64_t ldx, const uint16_t *W, int N, int K,
                           Epi epi, hipStream_t s, int cu_budget) {
    const GemvGeom g = gemv_geom(N, K, false, cu_budget, NT);
    if (gv_unit_pieces(K) == 7)
        k_gemv<7, NT, Epi><<<g.grid, kBlock, g.lds, s>>>(x, ldx, W, N, K, g.ps_stride, epi);
    else
        k_gemv<8, NT, Epi><<<g.grid, kBlock, g.lds, s>>>(x, ldx, W, N, K, g.ps_stride, epi);
}

// y[t][n] = epi(t, n, x[t] . W[n]) for b <= 4 tokens (gemv_fits_b).
template <class Epi>
static void launch_gemv(const uint16_t *x, int64_t ldx, int b, const uint16_t *W, int N, int K,
                        Epi epi, hipStream_t s, int cu_budget = 0) {
    if (b == 1)
        launch_gemv_nt<1>(x, ldx, W, N, K, epi, s, cu_budget);
    else if (b == 2)
        launch_gemv_nt<2>(x, ldx, W, N, K, epi, s, cu_budget);
    else if (b == 3)
        launch_gemv_nt<3>(x, ldx, W, N, K, epi, s, cu_budget);
    else
        launch_gemv_nt<4>(x, ldx, W, N, K, epi, s, cu_budget);
}

template <int NT>
static void launch_oproj_gemv_nt(const uint16_t *a, int64_t lda, const uint16_t *W, int d, int K,
                                 uint16_t *res, float *h32, hipStream_t s) {
    const GemvGeom g = gemv_geom(d, K, true, 0, NT);
    if (gv_unit_pieces(K) == 7)
        k_oproj_gemv<7, NT><<<g.grid, kBlock, g.lds, s>>>(a, lda, W, d, K, g.ps_stride, res, h32);
    else
        k_oproj_gemv<8, NT><<<g.grid, kBlock, g.lds, s>>>(a, lda, W, d, K, g.ps_stride, res, h32);
}

static void launch_oproj_gemv(const uint16_t *a, int64_t lda, int b, const uint16_t *W, int d,
                              int K, uint16_t *res, float *h32, hipStream_t s) {
    if (b == 1)
        launch_oproj_gemv_nt<1>(a, lda, W, d, K, res, h32, s);
    else if (b == 2)
        launch_oproj_gemv_nt<2>(a, lda, W, d, K, res, h32, s);
    else if (b == 3)
        launch_oproj_gemv_nt<3>(a, lda, W, d, K, res, h32, s);
    else
        launch_oproj_gemv_nt<4>(a, lda, W, d, K, res, h32, s);
}

void launch_rmsnorm(const float *h32, int b, int d, const uint16_t *gamma, float eps, uint16_t *y,
                    hipStream_t s) {
    k_rmsnorm<<<b, kBlock, 0, s>>>(h32, d, gamma, eps, y);
}

bool gemv1_f32_fits(int N, int K) { return gemv_fits_b(1, N, K, false); }

// One token, y[n] = x . W[n] in fp32 (the shared expert's down projection).
void launch_gemv1_f32(const uint16_t *x, const uint16_t *W, int N, int K, float *y, int cu_budget,
                      hipStream_t s) {
    launch_gemv(x, K, 1, W, N, K, EpiLogits{y, N, nullptr}, s, cu_budget);
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
    const int cus = budget_grid(1 << 30, cu_budget, 2);
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
static void launch_dense_dot2(const uint16_t *x, int64_t ldx, int b, const uint16_t *W, int N,
                              int K, Epi epi, hipStream_t s) {
    if (gemv_fits_b(b, N, K, false))
        launch_gemv(x, ldx, b, W, N, K, epi, s);
    else if (b == 1)
        launch_dense_dot2_t<1>(x, ldx, b, W, N, K, epi, s);
    else
        launch_dense_dot2_t<kDot2MaxTokens>(x, ldx, b, W, N, K, epi, s);
}

// Variant for a dense [N x K] read at batch b: dot2 while the tokens fit the
// engine, the split-K MFMA engine above.
static int pick_dense_variant(int op, int b, int K) {
    int v = forced_variant(op);
    if (v == K3_VARIANT_NONE)
        v = dot2_fits(b, K) ? K3_VARIANT_DOT2 : K3_VARIANT_MFMA;
    if (v == K3_VARIANT_DOT2 && !dot2_fits(b, K))
        return -1;
    if (v != K3_VARIANT_DOT2 && v != K3_VARIANT_MFMA)
        return -1;
    return v;
}

}  // namespace k3

using namespace k3;

// ------------------------------------------------------------------ workspace layouts
// Each workspace starts with a 256-byte head that no kernel touches; the
// MFMA variants keep the fp32 partial sums of their K ranges after it.
namespace {
constexpr size_t kHeadBytes = 256;
size_t router_logits_offset() { return kHeadBytes; }
size_t router_partial_offset(int b, int E) {
    return kHeadBytes + align_up((size_t)b * E * sizeof(float), 256);
}
size_t oproj_h32_offset() { return kHeadBytes; }
}  // namespace

extern "C" size_t k3_router_topk_workspace_size(int b, int E) {
    if (b <= 0 || E <= 0)
        return 0;
    return router_partial_offset(b, E) + sk_partial_bytes(b, E, 0);
}

extern "C" size_t k3_router_topk_latent_workspace_size(int b, int E, int d_lat) {
    if (b <= 0 || E <= 0 || d_lat <= 0)
        return 0;
    return router_partial_offset(b, E) + sk_partial_bytes(b, E + d_lat, 0);
}

static size_t oproj_part_offset(int b, int d) {
    return kHeadBytes + align_up((size_t)b * d * sizeof(float), 256);
}

extern "C" const float *k3_oproj_residual_h32(const void *workspace) {
    return workspace ? (const float *)((const char *)workspace + oproj_h32_offset()) : nullptr;
}

extern "C" size_t k3_oproj_residual_workspace_size(int b, int K, int d) {
    if (b <= 0 || d <= 0 || K <= 0)
        return 0;
    return oproj_part_offset(b, d) + sk_partial_bytes(b, d, K);
}

extern "C" size_t k3_proj_skinny_workspace_size(int b, int K, int N) {
    if (b <= 0 || N <= 0 || K <= 0)
        return 0;
    return kHeadBytes + sk_partial_bytes(b, N, K);
}

// ------------------------------------------------------------------ launchers
namespace k3 {

bool rls_fits(int b, int d, int E) {
    return dot2_fits(b, d) && (size_t)b * d * 2 + (size_t)E * 4 <= 65536;
}

static size_t rls_gemv_lds(int nt, int d, int E, int NL, int Is, int grid, int &ps_stride) {
    ps_stride = rls_gemv_ps_stride(E, NL, Is, grid);
    return (size_t)nt * d * 2 + ((size_t)4 * nt * ps_stride + E) * sizeof(float);
}

static int rls_gemv_grid(int E, int NL, int Is, int cu_budget) {
    return budget_grid((E + 7) / 8 + (NL + 7) / 8 + Is / 4, cu_budget, 2);
}

bool rls_gemv_fits(int b, int d, int E, int NL, int Is) {
    int ps_stride;
    return b >= 1 && b <= kDot2MaxTokens && gemv_fits(d) && Is % 4 == 0 && d % 4 == 0 &&
           rls_gemv_lds(b, d, E, NL, Is, rls_gemv_grid(E, NL, Is, 0), ps_stride) <= 65536;
}

void launch_rls(const uint16_t *x, int64_t ldx, int b, int d, const uint16_t *w_router,
                const float *bias, int E, float *logits, const uint16_t *w_lat, int NL,
                uint16_t *z, int64_t ldz, const uint16_t *w13s, int Is, uint16_t *hs,
                hipStream_t s, int cu_budget, const NormIn *norm) {
    if (rls_gemv_fits(b, d, E, NL, Is) && (b == 1 || !norm)) {
        const int grid = rls_gemv_grid(E, NL, Is, cu_budget);
        int ps_stride;
        const size_t lds = rls_gemv_lds(b, d, E, NL, Is, grid, ps_stride);
        const float *h32 = norm ? norm->h32 : nullptr;
        const uint16_t *gamma = norm ? norm->gamma : nullptr;
        const float eps = norm ? norm->eps : 0.0f;
        uint16_t *x_out = norm ? norm->x_out : nullptr;
#define K3_RLSG(U_, T_, N_)                                                                    \
    k_rls_gemv<U_, T_, N_><<<grid, kBlock, lds, s>>>(x, ldx, d, w_router, bias, E, logits,     \
                                                      w_lat, NL, z, w13s, Is, hs, ps_stride,   \
                                                      h32, gamma, eps, x_out, ldz)
#define K3_RLSB(U_)                                                                            \
    if (b == 1 && norm)                                                                        \
        K3_RLSG(U_, 1, true);                                                                  \
    else if (b == 1)                                                                           \
        K3_RLSG(U_, 1, false);                                                                 \
    else if (b == 2)                                                                           \
        K3_RLSG(U_, 2, false);                                                                 \
    else if (b == 3)                                                                           \
        K3_RLSG(U_, 3, false);                                                                 \
    else                                                                                       \
        K3_RLSG(U_, 4, false)
        if (gv_unit_pieces(d) == 7) {
            K3_RLSB(7);
        } else {
            K3_RLSB(8);
        }
#undef K3_RLSB
#undef K3_RLSG
        return;
    }
    const int cus = budget_grid(1 << 30, 0, 2);
    const int grid = (NL > 0 || Is > 0) ? cus : (E + kBlock / kWave - 1) / (kBlock / kWave);
    const size_t lds = (size_t)b * d * sizeof(uint16_t) + (size_t)E * sizeof(float);
    const int cb = d > 2048 ? 16 : (d > 512 ? 4 : 1);
#define K3_RLS(TM_, CB_)                                                                       \
    k_rls_dot2<TM_, CB_><<<grid, kBlock, lds, s>>>(x, ldx, b, d, w_router, bias, E, logits,   \
                                                   w_lat, NL, z, ldz, w13s, Is, hs)
    if (b == 1) {
        if (cb == 16)
            K3_RLS(1, 16);
        else if (cb == 4)
            K3_RLS(1, 4);
        else
            K3_RLS(1, 1);
    } else {
        if (cb == 16)
            K3_RLS(kDot2MaxTokens, 16);
        else if (cb == 4)
            K3_RLS(kDot2MaxTokens, 4);
        else
            K3_RLS(kDot2MaxTokens, 1);
    }
#undef K3_RLS
}

// One token's router logits and top-k in one kernel (K3_VARIANT_LASTWG);
// false when the row engine cannot run the shape.
bool launch_router_last(const uint16_t *x, int64_t ldx, int d, const uint16_t *w_router,
                        const float *bias, int E, float *logits, int k, int32_t *ids, float *wts,
                        int *counter, hipStream_t s) {
    if (!rls_gemv_fits(1, d, E, 0, 0))
        return false;
    const int grid = rls_gemv_grid(E, 0, 0, 0);
    int ps_stride;
    const size_t lds = rls_gemv_lds(1, d, E, 0, 0, grid, ps_stride);
    const LastTopk fin{counter, k, ids, wts};
    if (gv_unit_pieces(d) == 7)
        k_rls_gemv<7, 1, false, LastTopk><<<grid, kBlock, lds, s>>>(
            x, ldx, d, w_router, bias, E, logits, nullptr, 0, nullptr, nullptr, 0, nullptr,
            ps_stride, nullptr, nullptr, 0.0f, nullptr, 0, fin);
    else
        k_rls_gemv<8, 1, false, LastTopk><<<grid, kBlock, lds, s>>>(
            x, ldx, d, w_router, bias, E, logits, nullptr, 0, nullptr, nullptr, 0, nullptr,
            ps_stride, nullptr, nullptr, 0.0f, nullptr, 0, fin);
    return true;
}

void launch_topk(const float *logits, int b, int E, int k, int32_t *ids, float *wts,
                 hipStream_t s) {
    k_topk_softmax<<<b, kWave, 0, s>>>(logits, E, k, ids, wts);
}

}  // namespace k3

namespace {

int check_router_args(const uint16_t *x, int64_t ldx, int b, int d, const uint16_t *w_router,
                      int E, int k, const int32_t *ids, const float *wts, void *workspace,
                      size_t ws_bytes, size_t need) {
    if (!x || !w_router || !ids || !wts)
        return K3_ERR_INVALID_ARG;
    if (b <= 0 || d <= 0 || E <= 0 || k <= 0 || ldx < d)
        return K3_ERR_INVALID_ARG;
    if (b > K3_MAX_BATCH || E > K3_MAX_EXPERTS || k > K3_MAX_TOPK || k > E || d % 8 || ldx % 8 ||
        !aligned16(x) || !aligned16(w_router))
        return K3_ERR_UNSUPPORTED;
    if (!workspace || ws_bytes < need || !aligned16(workspace))
        return K3_ERR_WORKSPACE;
    return K3_OK;
}

// dot2 for the router (+ latent) only when the bias fits beside the tokens
int pick_router_variant(int op, int b, int d, int E) {
    int v = pick_dense_variant(op, b, d);
    if (v == K3_VARIANT_DOT2 && !rls_fits(b, d, E)) {
        if (forced_variant(op) == K3_VARIANT_DOT2)
            return -1;
        v = K3_VARIANT_MFMA;
    }
    return v;
}

}  // namespace

// ------------------------------------------------------------------ entry points
extern "C" int k3_proj_skinny(const uint16_t *x, int64_t ldx, int b, int K, const uint16_t *w,
                              int N, uint16_t *y, int64_t ldy, void *workspace, size_t ws_bytes,
                              void *stream) {
    if (!x || !w || !y)
        return K3_ERR_INVALID_ARG;
    if (b <= 0 || K <= 0 || N <= 0 || ldx < K || ldy < N)
        return K3_ERR_INVALID_ARG;
    if (b > K3_MAX_BATCH || K % 8 || ldx % 8 || !aligned16(x) || !aligned16(w))
        return K3_ERR_UNSUPPORTED;
    const int variant = pick_dense_variant(K3_OP_PROJ_SKINNY, b, K);
    if (variant < 0)
        return K3_ERR_UNSUPPORTED;
    if (variant == K3_VARIANT_MFMA &&
        (!workspace || ws_bytes < k3_proj_skinny_workspace_size(b, K, N) || !aligned16(workspace)))
        return K3_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    trace_begin(K3_OP_PROJ_SKINNY, s);
    if (variant == K3_VARIANT_DOT2)
        launch_dense_dot2(x, ldx, b, w, N, K, EpiBf16{y, ldy}, s);
    else
        sk_proj_bf16(x, ldx, b, w, N, K, y, ldy, (float *)((char *)workspace + kHeadBytes), s);
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
    const int chk = check_router_args(x, ldx, b, d, w_router, E, k, topk_ids, topk_w, workspace,
                                      ws_bytes, k3_router_topk_workspace_size(b, E));
    if (chk != K3_OK)
        return chk;
    hipStream_t s = (hipStream_t)stream;
    float *logits = (float *)((char *)workspace + router_logits_offset());
    float *part = (float *)((char *)workspace + router_partial_offset(b, E));
    if (forced_variant(K3_OP_ROUTER_TOPK) == K3_VARIANT_LASTWG) {
        // the counter sits in the workspace head, which no other kernel touches
        if (b != 1)
            return K3_ERR_UNSUPPORTED;
        trace_begin(K3_OP_ROUTER_TOPK, s);
        if (!launch_router_last(x, ldx, d, w_router, bias, E, logits, k, topk_ids, topk_w,
                                (int *)workspace, s))
            return K3_ERR_UNSUPPORTED;
        trace_end(K3_OP_ROUTER_TOPK, s);
        const int st = launch_status();
        if (st == K3_OK)
            record_dispatch(K3_OP_ROUTER_TOPK, K3_VARIANT_LASTWG);
        return st;
    }
    const int variant = pick_router_variant(K3_OP_ROUTER_TOPK, b, d, E);
    if (variant < 0)
        return K3_ERR_UNSUPPORTED;
    trace_begin(K3_OP_ROUTER_TOPK, s);
    if (variant == K3_VARIANT_DOT2) {
        launch_rls(x, ldx, b, d, w_router, bias, E, logits, nullptr, 0, nullptr, 0, nullptr, 0,
                   nullptr, s);
        trace_end(K3_OP_ROUTER_TOPK, s);
        launch_topk(logits, b, E, k, topk_ids, topk_w, s);
    } else {
        sk_router_topk(x, ldx, b, w_router, E, d, bias, k, logits, topk_ids, topk_w, part, s);
        trace_end(K3_OP_ROUTER_TOPK, s);
    }
    const int st = launch_status();
    if (st == K3_OK)
        record_dispatch(K3_OP_ROUTER_TOPK, variant);
    return st;
}

extern "C" int k3_router_topk_latent(const uint16_t *x, int64_t ldx, int b, int d,
                                     const uint16_t *w_router, const float *bias, int E, int k,
                                     const uint16_t *w_lat, int d_lat, int32_t *topk_ids,
                                     float *topk_w, uint16_t *z, int64_t ldz, void *workspace,
                                     size_t ws_bytes, void *stream) {
    if (!w_lat || !z)
        return K3_ERR_INVALID_ARG;
    if (d_lat <= 0 || ldz < d_lat)
        return K3_ERR_INVALID_ARG;
    const int chk = check_router_args(x, ldx, b, d, w_router, E, k, topk_ids, topk_w, workspace,
                                      ws_bytes, k3_router_topk_latent_workspace_size(b, E, d_lat));
    if (chk != K3_OK)
        return chk;
    if (!aligned16(w_lat))
        return K3_ERR_UNSUPPORTED;
    const int variant = pick_router_variant(K3_OP_ROUTER_LATENT, b, d, E);
    if (variant < 0)
        return K3_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    float *logits = (float *)((char *)workspace + router_logits_offset());
    float *part = (float *)((char *)workspace + router_partial_offset(b, E));
    trace_begin(K3_OP_ROUTER_LATENT, s);
    if (variant == K3_VARIANT_DOT2) {
        launch_rls(x, ldx, b, d, w_router, bias, E, logits, w_lat, d_lat, z, ldz, nullptr, 0,
                   nullptr, s);
        trace_end(K3_OP_ROUTER_LATENT, s);
        launch_topk(logits, b, E, k, topk_ids, topk_w, s);
    } else {
        sk_router_topk_latent(x, ldx, b, d, w_router, E, bias, k, logits, topk_ids, topk_w,
                              w_lat, d_lat, z, ldz, part, s);
        trace_end(K3_OP_ROUTER_LATENT, s);
    }
    const int st = launch_status();
    if (st == K3_OK)
        record_dispatch(K3_OP_ROUTER_LATENT, variant);
    return st;
}

extern "C" int k3_oproj_residual(const uint16_t *a, int64_t lda, int b, int K,
                                 const uint16_t *w_o, int d, uint16_t *residual,
                                 const uint16_t *gamma, float eps, uint16_t *y_norm,
                                 void *workspace, size_t ws_bytes, void *stream) {
    if (!a || !w_o || !residual || (y_norm && !gamma))
        return K3_ERR_INVALID_ARG;
    if (b <= 0 || K <= 0 || d <= 0 || lda < K || !(eps >= 0.0f))
        return K3_ERR_INVALID_ARG;
    if (b > K3_MAX_BATCH || K % 8 || lda % 8 || d % 8 || d > 8192 || !aligned16(a) ||
        !aligned16(w_o))
        return K3_ERR_UNSUPPORTED;
    if (!workspace || ws_bytes < k3_oproj_residual_workspace_size(b, K, d) ||
        !aligned16(workspace))
        return K3_ERR_WORKSPACE;
    int variant = pick_dense_variant(K3_OP_OPROJ_RESIDUAL, b, K);
    Dot2Geom g{};
    int rows_blk = 0;
    if (variant == K3_VARIANT_DOT2 && !gemv_fits_b(b, d, K, true)) {
        g = dot2_geom(d, K, b, 0);
        g.grid = budget_grid(d, 0, 2);  // two workgroups per compute unit, even row shares
        rows_blk = (d + g.grid - 1) / g.grid;
        g.lds += (size_t)b * rows_blk * sizeof(float);  // staged residuals
        if (g.lds > 65536) {
            if (forced_variant(K3_OP_OPROJ_RESIDUAL) == K3_VARIANT_DOT2)
                return K3_ERR_UNSUPPORTED;
            variant = K3_VARIANT_MFMA;
        }
    }
    if (variant < 0)
        return K3_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    float *h32 = (float *)((char *)workspace + oproj_h32_offset());
    trace_begin(K3_OP_OPROJ_RESIDUAL, s);
    if (variant == K3_VARIANT_DOT2 && gemv_fits_b(b, d, K, true)) {
        launch_oproj_gemv(a, lda, b, w_o, d, K, residual, h32, s);
        trace_end(K3_OP_OPROJ_RESIDUAL, s);
        if (y_norm)
            k_rmsnorm<<<b, kBlock, 0, s>>>(h32, d, gamma, eps, y_norm);
    } else if (variant == K3_VARIANT_DOT2) {
#define K3_OPROJ(TM_, CB_)                                                                     \
    k_oproj_dot2<TM_, CB_><<<g.grid, kBlock, g.lds, s>>>(a, lda, b, w_o, d, K, rows_blk, \
                                                         residual, h32)
        if (b == 1 && g.cb == 16)
            K3_OPROJ(1, 16);
        else if (b == 1 && g.cb == 4)
            K3_OPROJ(1, 4);
        else if (b == 1)
            K3_OPROJ(1, 1);
        else if (g.cb == 16)
            K3_OPROJ(kDot2MaxTokens, 16);
        else if (g.cb == 4)
            K3_OPROJ(kDot2MaxTokens, 4);
        else
            K3_OPROJ(kDot2MaxTokens, 1);
#undef K3_OPROJ
        trace_end(K3_OP_OPROJ_RESIDUAL, s);
        if (y_norm)
            k_rmsnorm<<<b, kBlock, 0, s>>>(h32, d, gamma, eps, y_norm);
    } else if (y_norm && d % 4 == 0 && d <= 4 * kNormVec * kBlock &&
               sk_ksplit(K, b) <= kSkMaxSplit / 2) {
        // partial sums, then the finish and the norm in one kernel. That
        // kernel gives each token one workgroup, which reads all the token's
        // K-range partials; with more than four ranges the finish spread over
        // every compute unit plus the norm kernel is faster (the chain of
        // projections at 8, 16, 32 tokens: 63.5 -> 61.1, 68.2 -> 66.1,
        // 73.9 -> 72.5 us; with four ranges at 64 tokens the fused kernel
        // was 1.8 us faster). The 8192-wide o-projection of the chain has
        // eight ranges at every token count.
        float *part = (float *)((char *)workspace + oproj_part_offset(b, d));
        const int ks = sk_oproj_partials(a, lda, b, K, w_o, d, part, s);
        k_oproj_finish_rmsnorm<<<b, kBlock, 0, s>>>(part, ks, b, d, residual, h32, gamma, eps,
                                                    y_norm);
        trace_end(K3_OP_OPROJ_RESIDUAL, s);
    } else {
        sk_oproj_residual(a, lda, b, K, w_o, d, residual, h32,
                          (float *)((char *)workspace + oproj_part_offset(b, d)), s);
        trace_end(K3_OP_OPROJ_RESIDUAL, s);
        if (y_norm)
            k_rmsnorm<<<b, kBlock, 0, s>>>(h32, d, gamma, eps, y_norm);
    }
    const int st = launch_status();
    if (st == K3_OK)
        record_dispatch(K3_OP_OPROJ_RESIDUAL, variant);
    return st;
}
