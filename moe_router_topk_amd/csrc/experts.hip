// experts.hip -- routed experts (permutation, grouped SwiGLU gate/up, down
// projection with the weighted combine) and the shared expert.
//
// "Hyper Optimizing Kimi K3 in vLLM", Part 1 section 3 ("Improve MoE
// scheduling and overlap"): the routed experts run after the router and the
// latent projection; the shared expert runs on its own stream beside them.
//
// Layout of the routed work after the permutation: the (token, slot) pairs
// are sorted by expert id, and within an expert by token index. Position p
// of that list has a token sorted_token[p] and a weight sorted_w[p]; active
// expert a (ascending id) owns positions [active_start[a], active_start[a+1]).
// The gate/up kernel writes h for position p into row p of hbuf.
//
// Both expert kernels use bf16 MFMA 16x16x32 tiles: an expert's tokens (at
// most 64, four 16-row tiles, padded with zeros) are the A operand, 16 weight
// rows the B operand. The four waves of a workgroup split the contraction
// into quarters and their partial tiles are summed in LDS in a fixed order.
#include <math.h>

#include "k3_device.h"
#include "k3_internal.h"

namespace k3 {

// Routed work list, read from the workspace the permutation kernel wrote.
struct Routed {
    const int *n_active;
    const int *active_expert;
    const int *active_start;
    const int *sorted_token;
    const float *sorted_w;
    __device__ int count() const { return *n_active; }
    __device__ void expert(int a, int &e, int &p0, int &n) const {
        e = active_expert[a];
        p0 = active_start[a];
        n = active_start[a + 1] - p0;
    }
    __device__ int token(int p) const { return sorted_token[p]; }
    __device__ float weight(int p) const { return sorted_w[p]; }
};

// The shared expert: one expert, every token in order, weight 1.
struct Dense {
    int b;
    __device__ int count() const { return 1; }
    __device__ void expert(int, int &e, int &p0, int &n) const {
        e = 0;
        p0 = 0;
        n = b;
    }
    __device__ int token(int p) const { return p; }
    __device__ float weight(int) const { return 1.0f; }
};

// ------------------------------------------------------------------ permutation
// One workgroup. Each token's chosen experts set bit t in mask[e]; counts are
// the popcounts, so each (expert, token) pair gets exactly one position and
// every position in [0, total) is written. Ids outside [0, E) are dropped.
__global__ void __launch_bounds__(kBlock)
k_moe_permute(const int32_t *__restrict__ ids, const float *__restrict__ w, int b, int k, int E,
              int *n_active, int *active_expert, int *active_start, int *sorted_token,
              float *sorted_w) {
    __shared__ unsigned long long mask[K3_MAX_EXPERTS];
    __shared__ int start[K3_MAX_EXPERTS];
    __shared__ int wave_c[kBlock / kWave], wave_f[kBlock / kWave];
    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1), wq = tid / kWave;
    const int P = b * k;
    for (int e = tid; e < E; e += kBlock)
        mask[e] = 0ull;
    __syncthreads();
    for (int i = tid; i < P; i += kBlock) {
        const int e = ids[i];
        if (e >= 0 && e < E)
            atomicOr(&mask[e], 1ull << (i / k));
    }
    __syncthreads();
    // Exclusive scans of counts and of active flags; thread owns 4 experts.
    constexpr int PER = K3_MAX_EXPERTS / kBlock;
    int c[PER];
    int lc = 0, lf = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int e = tid * PER + q;
        c[q] = e < E ? __popcll(mask[e]) : 0;
        lc += c[q];
        lf += c[q] > 0;
    }
    int sc = lc, sf = lf;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int tc = __shfl_up(sc, off, kWave);
        const int tf = __shfl_up(sf, off, kWave);
        if (lane >= off) {
            sc += tc;
            sf += tf;
        }
    }
    if (lane == kWave - 1) {
        wave_c[wq] = sc;
        wave_f[wq] = sf;
    }
    __syncthreads();
    for (int q = 0; q < wq; ++q) {
        sc += wave_c[q];
        sf += wave_f[q];
    }
    int ec = sc - lc, ef = sf - lf;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int e = tid * PER + q;
        if (e < E) {
            start[e] = ec;
            if (c[q] > 0) {
                active_expert[ef] = e;
                active_start[ef] = ec;
                ++ef;
            }
        }
        ec += c[q];
    }
    if (tid == kBlock - 1) {
        *n_active = sf;
        active_start[sf] = sc;
    }
    __syncthreads();
    for (int i = tid; i < P; i += kBlock) {
        const int e = ids[i];
        if (e >= 0 && e < E) {
            const int t = i / k;
            const int pos = start[e] + __popcll(mask[e] & ((1ull << t) - 1ull));
            sorted_token[pos] = t;
            sorted_w[pos] = w[i];
        }
    }
}

// ------------------------------------------------------------------ gate/up + SwiGLU
// Work item = (active expert a, tile of 16 intermediate columns j). Lane l
// streams gate row j0 + l%16 and up row I + j0 + l%16 of w13[e]; wave q
// covers input range [q d/4, (q+1) d/4). Epilogue: h = silu(g) * u -> bf16.
template <int U, class Route>
__global__ void __launch_bounds__(kBlock)
k_expert_gateup(const uint16_t *__restrict__ z, int64_t ldz, int d, const uint16_t *__restrict__ w13,
                int I, Route rt, uint16_t *__restrict__ hbuf) {
    __shared__ float red[4][2][4][4][kWave];  // [wave][gate/up][m tile][element][lane]
    const int lane = threadIdx.x & (kWave - 1);
    const int wq = threadIdx.x / kWave;
    const int kq = d >> 2;
    const int k_begin = wq * kq, k_end = k_begin + kq;
    const int kgrp = (lane >> 4) * 8;
    const int tiles = I >> 4;
    const int total = rt.count() * tiles;
    for (int item = blockIdx.x; item < total; item += gridDim.x) {
        const int a = item / tiles;
        const int tile = item - a * tiles;
        int e, p0, na;
        rt.expert(a, e, p0, na);
        const int MT = min((na + 15) >> 4, 4);
        const int j = tile * 16 + (lane & 15);
        const uint16_t *grow = w13 + ((int64_t)e * 2 * I + j) * d;
        const uint16_t *urow = grow + (int64_t)I * d;
        int64_t aoff[4];
        bool aval[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            const int m = mt * 16 + (lane & 15);
            aval[mt] = m < na;
            aoff[mt] = aval[mt] ? (int64_t)rt.token(p0 + m) * ldz : 0;
        }
        f32x4 ag[4], au[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
            ag[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            au[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
        for (int ks = k_begin; ks < k_end; ks += 32 * U) {
            u32x4 bg[U], bu[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const bool in = ks + 32 * u < k_end;
                const int k = ks + 32 * u + kgrp;
                bg[u] = in ? ld_weight16(grow + k) : zero16();
                bu[u] = in ? ld_weight16(urow + k) : zero16();
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                if (ks + 32 * u < k_end) {
                    const int k = ks + 32 * u + kgrp;
#pragma unroll
                    for (int mt = 0; mt < 4; ++mt) {
                        if (mt < MT) {
                            const u32x4 av = aval[mt] ? ld_act16(z + aoff[mt] + k) : zero16();
                            ag[mt] = mfma16x16x32(av, bg[u], ag[mt]);
                            au[mt] = mfma16x16x32(av, bu[u], au[mt]);
                        }
                    }
                }
            }
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
            if (mt < MT)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    red[wq][0][mt][i][lane] = ag[mt][i];
                    red[wq][1][mt][i][lane] = au[mt][i];
                }
        __syncthreads();
        for (int idx = threadIdx.x; idx < MT * 256; idx += kBlock) {
            const int mt = idx >> 8, i = (idx >> 6) & 3, l = idx & 63;
            const float g = red[0][0][mt][i][l] + red[1][0][mt][i][l] + red[2][0][mt][i][l] +
                            red[3][0][mt][i][l];
            const float u = red[0][1][mt][i][l] + red[1][1][mt][i][l] + red[2][1][mt][i][l] +
                            red[3][1][mt][i][l];
            const int m = mt * 16 + 4 * (l >> 4) + i;
            if (m < na)
                hbuf[(int64_t)(p0 + m) * I + tile * 16 + (l & 15)] = f32_to_bf16(silu(g) * u);
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ down + combine
// Workgroup per tile of 16 output rows (grid-stride). It walks the active
// experts in ascending id: wave q streams w2[e][r0 + l%16][q I/4 .. (q+1) I/4)
// against the experts' h rows and adds weight * result into its own LDS
// accumulator yacc[q][token][column]; after the last expert the four
// accumulators are summed in a fixed order and handed to `out`.
struct OutCombine {  // y = bf16(y_add + routed)
    uint16_t *y;
    const float *y_add;
    int d;
    __device__ void operator()(int t, int n, float s) const {
        const int64_t i = (int64_t)t * d + n;
        y[i] = f32_to_bf16(y_add ? y_add[i] + s : s);
    }
};

struct OutF32 {  // y_s = s, fp32
    float *y;
    int d;
    __device__ void operator()(int t, int n, float s) const { y[(int64_t)t * d + n] = s; }
};

template <int U, class Route, class Out>
__global__ void __launch_bounds__(kBlock)
k_expert_down(const uint16_t *__restrict__ hbuf, int I, const uint16_t *__restrict__ w2, int d_out,
              Route rt, int b, Out out) {
    __shared__ float yacc[4][K3_MAX_BATCH][16];
    const int lane = threadIdx.x & (kWave - 1);
    const int wq = threadIdx.x / kWave;
    const int kq = I >> 2;
    const int k_begin = wq * kq, k_end = k_begin + kq;
    const int kgrp = (lane >> 4) * 8;
    const int n_act = rt.count();
    const int tiles = d_out >> 4;
    for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        for (int i = lane; i < K3_MAX_BATCH * 16; i += kWave)
            (&yacc[wq][0][0])[i] = 0.0f;
        const int r = tile * 16 + (lane & 15);
        for (int a = 0; a < n_act; ++a) {
            int e, p0, na;
            rt.expert(a, e, p0, na);
            const int MT = min((na + 15) >> 4, 4);
            const uint16_t *wrow = w2 + ((int64_t)e * d_out + r) * I;
            int64_t aoff[4];
            bool aval[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt) {
                const int m = mt * 16 + (lane & 15);
                aval[mt] = m < na;
                aoff[mt] = (int64_t)(aval[mt] ? p0 + m : 0) * I;
            }
            f32x4 acc[4];
#pragma unroll
            for (int mt = 0; mt < 4; ++mt)
                acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
            for (int ks = k_begin; ks < k_end; ks += 32 * U) {
                u32x4 bfr[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int k = ks + 32 * u + kgrp;
                    bfr[u] = (ks + 32 * u < k_end) ? ld_weight16(wrow + k) : zero16();
                }
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    if (ks + 32 * u < k_end) {
                        const int k = ks + 32 * u + kgrp;
#pragma unroll
                        for (int mt = 0; mt < 4; ++mt) {
                            if (mt < MT) {
                                const u32x4 av = aval[mt] ? ld_act16(hbuf + aoff[mt] + k) : zero16();
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
                    for (int i = 0; i < 4; ++i) {
                        const int m = mt * 16 + 4 * (lane >> 4) + i;
                        if (m < na) {
                            const int t = rt.token(p0 + m);
                            yacc[wq][t][lane & 15] += rt.weight(p0 + m) * acc[mt][i];
                        }
                    }
        }
        __syncthreads();
        for (int idx = threadIdx.x; idx < b * 16; idx += kBlock) {
            const int t = idx >> 4, c = idx & 15;
            const float s = (yacc[0][t][c] + yacc[1][t][c]) + (yacc[2][t][c] + yacc[3][t][c]);
            out(t, tile * 16 + c, s);
        }
        __syncthreads();
    }
}

}  // namespace k3

using namespace k3;

// ------------------------------------------------------------------ entry points
extern "C" int k3_moe_experts(const uint16_t *z, int64_t ldz, int b, int d_in,
                              const int32_t *topk_ids, const float *topk_w, int k,
                              const uint16_t *w13, const uint16_t *w2, int E, int I, int d_out,
                              const float *y_add, void *y_add_ready, uint16_t *y, int cu_budget,
                              void *workspace, size_t ws_bytes, void *stream) {
    if (!z || !topk_ids || !topk_w || !w13 || !w2 || !y)
        return K3_ERR_INVALID_ARG;
    if (b <= 0 || d_in <= 0 || k <= 0 || E <= 0 || I <= 0 || d_out <= 0 || ldz < d_in ||
        cu_budget < 0)
        return K3_ERR_INVALID_ARG;
    if (b > K3_MAX_BATCH || k > K3_MAX_TOPK || E > K3_MAX_EXPERTS || I % 128 || d_in % 128 ||
        d_out % 16 || ldz % 8 || !aligned16(z) || !aligned16(w13) || !aligned16(w2))
        return K3_ERR_UNSUPPORTED;
    const int fv = forced_variant(K3_OP_MOE_EXPERTS);
    if (fv != K3_VARIANT_NONE && fv != K3_VARIANT_GROUPED)
        return K3_ERR_UNSUPPORTED;
    const MoeWorkspace L = moe_workspace_layout(b, E, k, I);
    if (!workspace || ws_bytes < L.total)
        return K3_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    char *ws = (char *)workspace;
    Routed rt{(const int *)(ws + L.n_active), (const int *)(ws + L.active_expert),
              (const int *)(ws + L.active_start), (const int *)(ws + L.sorted_token),
              (const float *)(ws + L.sorted_w)};
    uint16_t *hbuf = (uint16_t *)(ws + L.hbuf);
    k_moe_permute<<<1, kBlock, 0, s>>>(topk_ids, topk_w, b, k, E, (int *)(ws + L.n_active),
                                       (int *)(ws + L.active_expert),
                                       (int *)(ws + L.active_start), (int *)(ws + L.sorted_token),
                                       (float *)(ws + L.sorted_w));
    const int max_active = b * k < E ? b * k : E;
    const int g1 = budget_grid(max_active * (I / 16), cu_budget, 4);
    trace_begin(K3_OP_MOE_EXPERTS, s);
    k_expert_gateup<8, Routed><<<g1, kBlock, 0, s>>>(z, ldz, d_in, w13, I, rt, hbuf);
    trace_end(K3_OP_MOE_EXPERTS, s);
    if (y_add_ready && hipStreamWaitEvent(s, (hipEvent_t)y_add_ready, 0) != hipSuccess)
        return K3_ERR_HIP;
    const int g2 = budget_grid(d_out / 16, cu_budget, 2);
    k_expert_down<16, Routed, OutCombine><<<g2, kBlock, 0, s>>>(hbuf, I, w2, d_out, rt, b,
                                                                 OutCombine{y, y_add, d_out});
    const int st = launch_status();
    if (st == K3_OK)
        record_dispatch(K3_OP_MOE_EXPERTS, K3_VARIANT_GROUPED);
    return st;
}

extern "C" int k3_shared_expert(const uint16_t *x, int64_t ldx, int b, int d, const uint16_t *w13,
                                const uint16_t *w2, int I, float *y_s, int cu_budget,
                                void *workspace, size_t ws_bytes, void *stream) {
    if (!x || !w13 || !w2 || !y_s)
        return K3_ERR_INVALID_ARG;
    if (b <= 0 || d <= 0 || I <= 0 || ldx < d || cu_budget < 0)
        return K3_ERR_INVALID_ARG;
    if (b > K3_MAX_BATCH || I % 128 || d % 128 || ldx % 8 || !aligned16(x) || !aligned16(w13) ||
        !aligned16(w2))
        return K3_ERR_UNSUPPORTED;
    const int fv = forced_variant(K3_OP_SHARED_EXPERT);
    if (fv != K3_VARIANT_NONE && fv != K3_VARIANT_MFMA)
        return K3_ERR_UNSUPPORTED;
    if (!workspace || ws_bytes < k3_shared_expert_workspace_size(b, d, I))
        return K3_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    uint16_t *hbuf = (uint16_t *)workspace;
    Dense rt{b};
    const int g1 = budget_grid(I / 16, cu_budget, 4);
    trace_begin(K3_OP_SHARED_EXPERT, s);
    k_expert_gateup<8, Dense><<<g1, kBlock, 0, s>>>(x, ldx, d, w13, I, rt, hbuf);
    trace_end(K3_OP_SHARED_EXPERT, s);
    const int g2 = budget_grid(d / 16, cu_budget, 2);
    k_expert_down<16, Dense, OutF32><<<g2, kBlock, 0, s>>>(hbuf, I, w2, d, rt, b, OutF32{y_s, d});
    const int st = launch_status();
    if (st == K3_OK)
        record_dispatch(K3_OP_SHARED_EXPERT, K3_VARIANT_MFMA);
    return st;
}
