// experts.hip -- routed experts (token-to-expert permutation, grouped SwiGLU
// gate/up, down projection, weighted combine) and the shared expert.
//
// "Hyper Optimizing Kimi K3 in vLLM", Part 1 section 3 ("Improve MoE
// scheduling and overlap"): the routed experts run after the router and the
// latent projection; the shared expert runs on its own stream beside them.
//
// After the permutation the (token, slot) pairs are sorted by expert id and,
// within an expert, by token index; position p of that list holds token
// sorted_token[p], and slot (t, j) sits at position slot_pos[t k + j]. The
// active experts form two lists in ascending id: "light" experts (at most
// kDot2MaxTokens tokens) run on the dot2 row-streaming engine, "heavy" ones
// on bf16 MFMA tiles, where the contraction is dense enough to need them.
// Gate/up writes h for position p into row p of hbuf (bf16); the down
// projection writes position p's output into row p of part (fp32); the
// combine kernel forms y[t] = y_add[t] + sum_j w[t][j] part[slot_pos[t][j]]
// in slot order. At batch 1 the slots are the experts (k distinct ids), so
// no permutation is needed and position p is slot p.
#include <math.h>

#include "k3_device.h"
#include "k3_internal.h"

namespace k3 {

constexpr int kDot2MaxTokens = 4;

// ------------------------------------------------------------------ expert lists
struct ExpertList {  // a compacted list written by the permutation kernel
    const int *n;
    const int *expert, *start, *ntok;
    const int *sorted_token;
    __device__ int count() const { return *n; }
    __device__ void get(int a, int &e, int &p0, int &na) const {
        e = expert[a];
        p0 = start[a];
        na = ntok[a];
    }
    __device__ int token(int p) const { return sorted_token[p]; }
};

struct SlotList {  // batch 1: slot j is expert ids[j], position j, token 0
    const int32_t *ids;
    int k, E;
    __device__ int count() const { return k; }
    __device__ void get(int a, int &e, int &p0, int &na) const {
        e = ids[a];
        p0 = a;
        na = (e >= 0 && e < E) ? 1 : 0;
        if (!na)
            e = 0;
    }
    __device__ int token(int) const { return 0; }
};

struct DenseList {  // the shared expert: one expert, every token in order
    int b;
    __device__ int count() const { return 1; }
    __device__ void get(int, int &e, int &p0, int &na) const {
        e = 0;
        p0 = 0;
        na = b;
    }
    __device__ int token(int p) const { return p; }
};

// ------------------------------------------------------------------ permutation
// One workgroup. Token t's choice of expert e sets bit t of mask[e]; an
// expert's token count is the popcount, so every (expert, token) pair gets
// exactly one position and all positions [0, total) are written. Ids outside
// [0, E) are dropped (slot_pos = -1). Exclusive scans over the experts give
// the positions and the two compacted lists.
__global__ void __launch_bounds__(kBlock)
k_moe_permute(const int32_t *__restrict__ ids, int b, int k, int E, int *n_light,
              int *light_expert, int *light_start, int *light_ntok, int *n_heavy,
              int *heavy_expert, int *heavy_start, int *heavy_ntok, int *sorted_token,
              int *slot_pos) {
    __shared__ unsigned long long mask[K3_MAX_EXPERTS];
    __shared__ int start[K3_MAX_EXPERTS];
    __shared__ int wsum[3][kBlock / kWave];
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
    constexpr int PER = K3_MAX_EXPERTS / kBlock;
    int c[PER];
    int lc = 0, ll = 0, lh = 0;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int e = tid * PER + q;
        c[q] = e < E ? __popcll(mask[e]) : 0;
        lc += c[q];
        ll += (c[q] > 0 && c[q] <= kDot2MaxTokens);
        lh += c[q] > kDot2MaxTokens;
    }
    int sc = lc, sl = ll, sh = lh;  // inclusive scans across the block
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int tc = __shfl_up(sc, off, kWave);
        const int tl = __shfl_up(sl, off, kWave);
        const int th = __shfl_up(sh, off, kWave);
        if (lane >= off) {
            sc += tc;
            sl += tl;
            sh += th;
        }
    }
    if (lane == kWave - 1) {
        wsum[0][wq] = sc;
        wsum[1][wq] = sl;
        wsum[2][wq] = sh;
    }
    __syncthreads();
    for (int q = 0; q < wq; ++q) {
        sc += wsum[0][q];
        sl += wsum[1][q];
        sh += wsum[2][q];
    }
    int ec = sc - lc, el = sl - ll, eh = sh - lh;
#pragma unroll
    for (int q = 0; q < PER; ++q) {
        const int e = tid * PER + q;
        if (e < E) {
            start[e] = ec;
            if (c[q] > 0 && c[q] <= kDot2MaxTokens) {
                light_expert[el] = e;
                light_start[el] = ec;
                light_ntok[el] = c[q];
                ++el;
            } else if (c[q] > kDot2MaxTokens) {
                heavy_expert[eh] = e;
                heavy_start[eh] = ec;
                heavy_ntok[eh] = c[q];
                ++eh;
            }
        }
        ec += c[q];
    }
    if (tid == kBlock - 1) {
        *n_light = sl;
        *n_heavy = sh;
    }
    __syncthreads();
    for (int i = tid; i < P; i += kBlock) {
        const int e = ids[i];
        int pos = -1;
        if (e >= 0 && e < E) {
            const int t = i / k;
            pos = start[e] + __popcll(mask[e] & ((1ull << t) - 1ull));
            sorted_token[pos] = t;
        }
        slot_pos[i] = pos;
    }
}

// ------------------------------------------------------------------ dot2 gate/up
// The (expert, intermediate column) pairs of the list are split evenly over
// the workgroups. A workgroup stages the token rows of each expert segment it
// meets in LDS, its four waves split the segment's columns, and each wave
// streams gate row j then up row I + j (the two row buffers), keeping the
// gate sums until the up sums arrive: h = silu(g) * u -> bf16.
template <int TM, class List>
__global__ void __launch_bounds__(kBlock)
k_gateup_dot2(const uint16_t *__restrict__ z, int64_t ldz, int d,
              const uint16_t *__restrict__ w13, int I, List L, uint16_t *__restrict__ hbuf) {
    extern __shared__ u32x4 xs[];
    const int nv = d >> 3;
    const int lane = threadIdx.x & (kWave - 1);
    const int wq = threadIdx.x / kWave;
    const int total = L.count() * I;
    int g0, g1;
    split_range(total, gridDim.x, blockIdx.x, g0, g1);
    for (int s0 = g0; s0 < g1;) {
        const int a = s0 / I;
        const int s1 = min(g1, (a + 1) * I);
        int e, p0, na;
        L.get(a, e, p0, na);
        __syncthreads();
        stage_rows(xs, nv, na, nv, [&](int t) { return z + (int64_t)L.token(p0 + t) * ldz; });
        __syncthreads();
        if (na > 0) {
            int j0, j1;
            split_range(s1 - s0, kBlock / kWave, wq, j0, j1);
            j0 += s0 - a * I;
            j1 += s0 - a * I;
            const uint16_t *base = w13 + (int64_t)e * 2 * I * d;
            float gsave[TM];
#pragma unroll
            for (int t = 0; t < TM; ++t)
                gsave[t] = 0.0f;
            stream_rows<TM, 1, 16>(
                2 * j0, 2 * j1, nv, xs, nv, na,
                [&](int i) {
                    const int j = i >> 1;
                    return base + (int64_t)((i & 1) ? I + j : j) * d;
                },
                [&](int i, int t, float s) {
                    if ((i & 1) == 0)
                        gsave[t] = s;
                    else if (lane == 0)
                        hbuf[(int64_t)(p0 + t) * I + (i >> 1)] = f32_to_bf16(silu(gsave[t]) * s);
                });
        }
        s0 = s1;
    }
}

// ------------------------------------------------------------------ dot2 down
// The (expert, output row) pairs are split evenly over the workgroups; each
// expert segment stages the experts' h rows in LDS and its waves stream the
// segment's rows of w2[e], four rows per buffer (I <= 2048).
struct OutPart {  // part[p][r] = s
    float *part;
    int d_out;
    __device__ void operator()(int p, int r, float s) const { part[(int64_t)p * d_out + r] = s; }
};

template <int TM, int CB, class List, class Out>
__global__ void __launch_bounds__(kBlock)
k_down_dot2(const uint16_t *__restrict__ hbuf, int I, const uint16_t *__restrict__ w2, int d_out,
            List L, Out out) {
    extern __shared__ u32x4 xs[];
    const int nv = I >> 3;
    const int lane = threadIdx.x & (kWave - 1);
    const int wq = threadIdx.x / kWave;
    const int total = L.count() * d_out;
    int g0, g1;
    split_range(total, gridDim.x, blockIdx.x, g0, g1);
    for (int s0 = g0; s0 < g1;) {
        const int a = s0 / d_out;
        const int s1 = min(g1, (a + 1) * d_out);
        int e, p0, na;
        L.get(a, e, p0, na);
        __syncthreads();
        stage_rows(xs, nv, na, nv, [&](int t) { return hbuf + (int64_t)(p0 + t) * I; });
        __syncthreads();
        if (na > 0) {
            int r0, r1;
            split_range(s1 - s0, kBlock / kWave, wq, r0, r1);
            r0 += s0 - a * d_out;
            r1 += s0 - a * d_out;
            const uint16_t *base = w2 + (int64_t)e * d_out * I;
            stream_rows<TM, 16 / CB, CB>(
                r0, r1, nv, xs, nv, na, [&](int r) { return base + (int64_t)r * I; },
                [&](int r, int t, float s) {
                    if (lane == 0)
                        out(p0 + t, r, s);
                });
        }
        s0 = s1;
    }
}

// ------------------------------------------------------------------ mfma gate/up
// Item = (list entry a, tile of 16 intermediate columns j). Lane l streams
// gate row j0 + l%16 and up row I + j0 + l%16 of w13[e]; wave q covers input
// range [q d/4, (q+1) d/4); the four partial tiles are summed in LDS.
template <int U, class List>
__global__ void __launch_bounds__(kBlock)
k_gateup_mfma(const uint16_t *__restrict__ z, int64_t ldz, int d, const uint16_t *__restrict__ w13,
              int I, List L, uint16_t *__restrict__ hbuf) {
    __shared__ float red[4][2][4][4][kWave];  // [wave][gate/up][m tile][element][lane]
    const int lane = threadIdx.x & (kWave - 1);
    const int wq = threadIdx.x / kWave;
    const int kq = d >> 2;
    const int k_begin = wq * kq, k_end = k_begin + kq;
    const int kgrp = (lane >> 4) * 8;
    const int tiles = I >> 4;
    const int total = L.count() * tiles;
    for (int item = blockIdx.x; item < total; item += gridDim.x) {
        const int a = item / tiles;
        const int tile = item - a * tiles;
        int e, p0, na;
        L.get(a, e, p0, na);
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
            aoff[mt] = aval[mt] ? (int64_t)L.token(p0 + m) * ldz : 0;
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

// ------------------------------------------------------------------ mfma down
// Item = (list entry a, tile of 16 output rows); wave q covers the
// intermediate range [q I/4, (q+1) I/4); output for position p0 + m.
template <int U, class List, class Out>
__global__ void __launch_bounds__(kBlock)
k_down_mfma(const uint16_t *__restrict__ hbuf, int I, const uint16_t *__restrict__ w2, int d_out,
            List L, Out out) {
    __shared__ float red[4][4][4][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int wq = threadIdx.x / kWave;
    const int kq = I >> 2;
    const int k_begin = wq * kq, k_end = k_begin + kq;
    const int kgrp = (lane >> 4) * 8;
    const int tiles = d_out >> 4;
    const int total = L.count() * tiles;
    for (int item = blockIdx.x; item < total; item += gridDim.x) {
        const int a = item / tiles;
        const int tile = item - a * tiles;
        int e, p0, na;
        L.get(a, e, p0, na);
        const int MT = min((na + 15) >> 4, 4);
        const uint16_t *wrow = w2 + ((int64_t)e * d_out + tile * 16 + (lane & 15)) * I;
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
                for (int i = 0; i < 4; ++i)
                    red[wq][mt][i][lane] = acc[mt][i];
        __syncthreads();
        for (int idx = threadIdx.x; idx < MT * 256; idx += kBlock) {
            const int mt = idx >> 8, i = (idx >> 6) & 3, l = idx & 63;
            const float s = (red[0][mt][i][l] + red[1][mt][i][l]) + (red[2][mt][i][l] + red[3][mt][i][l]);
            const int m = mt * 16 + 4 * (l >> 4) + i;
            if (m < na)
                out(p0 + m, tile * 16 + (l & 15), s);
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------------ combine
// y[t][r] = bf16(y_add[t][r] + sum_j w[t][j] * part[pos(t, j)][r]), slots in
// order; pos = slot_pos[t k + j] (or j at batch 1 when ids[j] is valid).
__global__ void __launch_bounds__(kBlock)
k_combine(const float *__restrict__ part, int d_out, const int *__restrict__ slot_pos,
          const int32_t *__restrict__ ids, int E, const float *__restrict__ topk_w, int b, int k,
          const float *__restrict__ y_add, uint16_t *__restrict__ y) {
    const int i = blockIdx.x * kBlock + threadIdx.x;
    if (i >= b * d_out)
        return;
    const int t = i / d_out, r = i - t * d_out;
    float s = y_add ? y_add[i] : 0.0f;
    for (int j = 0; j < k; ++j) {
        int pos;
        if (slot_pos) {
            pos = slot_pos[t * k + j];
        } else {
            const int e = ids[j];
            pos = (e >= 0 && e < E) ? j : -1;
        }
        if (pos >= 0)
            s += topk_w[t * k + j] * part[(int64_t)pos * d_out + r];
    }
    y[i] = f32_to_bf16(s);
}

}  // namespace k3

using namespace k3;

// ------------------------------------------------------------------ workspace layout
namespace k3 {
MoeWorkspace moe_workspace_layout(int b, int E, int k, int I, int d_out) {
    const size_t A = 256;
    const size_t P = (size_t)b * k;
    const size_t cap = P < (size_t)E ? P : (size_t)E;
    MoeWorkspace w;
    size_t o = 0;
    auto take = [&](size_t bytes) {
        const size_t at = o;
        o = align_up(o + bytes, A);
        return at;
    };
    w.n_light = take(sizeof(int));
    w.n_heavy = take(sizeof(int));
    w.light_expert = take(cap * sizeof(int));
    w.light_start = take(cap * sizeof(int));
    w.light_ntok = take(cap * sizeof(int));
    w.heavy_expert = take(cap * sizeof(int));
    w.heavy_start = take(cap * sizeof(int));
    w.heavy_ntok = take(cap * sizeof(int));
    w.sorted_token = take(P * sizeof(int));
    w.slot_pos = take(P * sizeof(int));
    w.hbuf = take(P * (size_t)I * sizeof(uint16_t));
    w.part = take(P * (size_t)d_out * sizeof(float));
    w.total = o;
    return w;
}
}  // namespace k3

extern "C" size_t k3_moe_experts_workspace_size(int b, int d_in, int E, int k, int I, int d_out) {
    (void)d_in;
    if (b <= 0 || E <= 0 || k <= 0 || I <= 0 || d_out <= 0)
        return 0;
    return moe_workspace_layout(b, E, k, I, d_out).total;
}

extern "C" size_t k3_shared_expert_workspace_size(int b, int d, int I) {
    (void)d;
    if (b <= 0 || I <= 0)
        return 0;
    return align_up((size_t)b * I * sizeof(uint16_t), 256);
}

// ------------------------------------------------------------------ launchers
namespace {

int dot2_grid(int cu_budget) { return budget_grid(1 << 30, cu_budget, 1); }

template <class List>
void launch_gateup_dot2(int tm, const uint16_t *z, int64_t ldz, int d, const uint16_t *w13, int I,
                        List L, uint16_t *hbuf, int cu_budget, hipStream_t s) {
    const size_t lds = (size_t)tm * d * sizeof(uint16_t);
    const int grid = dot2_grid(cu_budget);
    if (tm == 1)
        k_gateup_dot2<1, List><<<grid, kBlock, lds, s>>>(z, ldz, d, w13, I, L, hbuf);
    else
        k_gateup_dot2<kDot2MaxTokens, List><<<grid, kBlock, lds, s>>>(z, ldz, d, w13, I, L, hbuf);
}

template <class List, class Out>
void launch_down_dot2(int tm, const uint16_t *hbuf, int I, const uint16_t *w2, int d_out, List L,
                      Out out, int cu_budget, hipStream_t s) {
    const size_t lds = (size_t)tm * I * sizeof(uint16_t);
    const int grid = dot2_grid(cu_budget);
    const int cb = I > 2048 ? 16 : (I > 512 ? 4 : 1);
#define K3_DOWN(TM_, CB_) \
    k_down_dot2<TM_, CB_, List, Out><<<grid, kBlock, lds, s>>>(hbuf, I, w2, d_out, L, out)
    if (tm == 1) {
        if (cb == 16)
            K3_DOWN(1, 16);
        else if (cb == 4)
            K3_DOWN(1, 4);
        else
            K3_DOWN(1, 1);
    } else {
        if (cb == 16)
            K3_DOWN(kDot2MaxTokens, 16);
        else if (cb == 4)
            K3_DOWN(kDot2MaxTokens, 4);
        else
            K3_DOWN(kDot2MaxTokens, 1);
    }
#undef K3_DOWN
}

}  // namespace

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
        d_in > 8192 || I > 8192 || d_out % 16 || ldz % 8 || !aligned16(z) || !aligned16(w13) ||
        !aligned16(w2))
        return K3_ERR_UNSUPPORTED;
    const int fv = forced_variant(K3_OP_MOE_EXPERTS);
    if (fv != K3_VARIANT_NONE && fv != K3_VARIANT_GROUPED)
        return K3_ERR_UNSUPPORTED;
    const MoeWorkspace L = moe_workspace_layout(b, E, k, I, d_out);
    if (!workspace || ws_bytes < L.total || !aligned16(workspace))
        return K3_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    char *ws = (char *)workspace;
    uint16_t *hbuf = (uint16_t *)(ws + L.hbuf);
    float *part = (float *)(ws + L.part);
    const OutPart out{part, d_out};
    const int *slot_pos = nullptr;
    trace_begin(K3_OP_MOE_EXPERTS, s);
    if (b == 1) {
        const SlotList sl{topk_ids, k, E};
        launch_gateup_dot2(1, z, ldz, d_in, w13, I, sl, hbuf, cu_budget, s);
        trace_end(K3_OP_MOE_EXPERTS, s);
        if (y_add_ready && hipStreamWaitEvent(s, (hipEvent_t)y_add_ready, 0) != hipSuccess)
            return K3_ERR_HIP;
        launch_down_dot2(1, hbuf, I, w2, d_out, sl, out, cu_budget, s);
    } else {
        int *n_light = (int *)(ws + L.n_light), *n_heavy = (int *)(ws + L.n_heavy);
        const ExpertList light{n_light, (int *)(ws + L.light_expert), (int *)(ws + L.light_start),
                               (int *)(ws + L.light_ntok), (int *)(ws + L.sorted_token)};
        const ExpertList heavy{n_heavy, (int *)(ws + L.heavy_expert), (int *)(ws + L.heavy_start),
                               (int *)(ws + L.heavy_ntok), (int *)(ws + L.sorted_token)};
        slot_pos = (const int *)(ws + L.slot_pos);
        k_moe_permute<<<1, kBlock, 0, s>>>(
            topk_ids, b, k, E, n_light, (int *)(ws + L.light_expert), (int *)(ws + L.light_start),
            (int *)(ws + L.light_ntok), n_heavy, (int *)(ws + L.heavy_expert),
            (int *)(ws + L.heavy_start), (int *)(ws + L.heavy_ntok), (int *)(ws + L.sorted_token),
            (int *)(ws + L.slot_pos));
        launch_gateup_dot2(kDot2MaxTokens, z, ldz, d_in, w13, I, light, hbuf, cu_budget, s);
        const bool any_heavy = b > kDot2MaxTokens;
        if (any_heavy) {
            const int max_heavy = (b * k) / (kDot2MaxTokens + 1);
            const int g = budget_grid((max_heavy < E ? max_heavy : E) * (I / 16), cu_budget, 4);
            k_gateup_mfma<8, ExpertList><<<g, kBlock, 0, s>>>(z, ldz, d_in, w13, I, heavy, hbuf);
        }
        trace_end(K3_OP_MOE_EXPERTS, s);
        launch_down_dot2(kDot2MaxTokens, hbuf, I, w2, d_out, light, out, cu_budget, s);
        if (any_heavy) {
            const int max_heavy = (b * k) / (kDot2MaxTokens + 1);
            const int g = budget_grid((max_heavy < E ? max_heavy : E) * (d_out / 16), cu_budget, 4);
            k_down_mfma<16, ExpertList, OutPart><<<g, kBlock, 0, s>>>(hbuf, I, w2, d_out, heavy,
                                                                     out);
        }
        if (y_add_ready && hipStreamWaitEvent(s, (hipEvent_t)y_add_ready, 0) != hipSuccess)
            return K3_ERR_HIP;
    }
    const int n = b * d_out;
    k_combine<<<(n + kBlock - 1) / kBlock, kBlock, 0, s>>>(part, d_out, slot_pos, topk_ids, E,
                                                            topk_w, b, k, y_add, y);
    const int st = launch_status();
    if (st == K3_OK)
        record_dispatch(K3_OP_MOE_EXPERTS, K3_VARIANT_GROUPED);
    return st;
}

namespace {
struct OutDense {  // y_s[t][r] = s (positions are tokens for the dense list)
    float *y;
    int d;
    __device__ void operator()(int p, int r, float s) const { y[(int64_t)p * d + r] = s; }
};
}  // namespace

extern "C" int k3_shared_expert(const uint16_t *x, int64_t ldx, int b, int d, const uint16_t *w13,
                                const uint16_t *w2, int I, float *y_s, int cu_budget,
                                void *workspace, size_t ws_bytes, void *stream) {
    if (!x || !w13 || !w2 || !y_s)
        return K3_ERR_INVALID_ARG;
    if (b <= 0 || d <= 0 || I <= 0 || ldx < d || cu_budget < 0)
        return K3_ERR_INVALID_ARG;
    if (b > K3_MAX_BATCH || I % 128 || d % 128 || d > 8192 || I > 8192 || ldx % 8 ||
        !aligned16(x) || !aligned16(w13) || !aligned16(w2))
        return K3_ERR_UNSUPPORTED;
    int variant = forced_variant(K3_OP_SHARED_EXPERT);
    if (variant == K3_VARIANT_NONE)
        variant = b <= kDot2MaxTokens ? K3_VARIANT_DOT2 : K3_VARIANT_MFMA;
    if ((variant != K3_VARIANT_DOT2 && variant != K3_VARIANT_MFMA) ||
        (variant == K3_VARIANT_DOT2 && b > kDot2MaxTokens))
        return K3_ERR_UNSUPPORTED;
    if (!workspace || ws_bytes < k3_shared_expert_workspace_size(b, d, I) || !aligned16(workspace))
        return K3_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    uint16_t *hbuf = (uint16_t *)workspace;
    const DenseList dl{b};
    const OutDense out{y_s, d};
    trace_begin(K3_OP_SHARED_EXPERT, s);
    if (variant == K3_VARIANT_DOT2) {
        const int tm = b == 1 ? 1 : kDot2MaxTokens;
        launch_gateup_dot2(tm, x, ldx, d, w13, I, dl, hbuf, cu_budget, s);
        trace_end(K3_OP_SHARED_EXPERT, s);
        launch_down_dot2(tm, hbuf, I, w2, d, dl, out, cu_budget, s);
    } else {
        const int g1 = budget_grid(I / 16, cu_budget, 4);
        k_gateup_mfma<8, DenseList><<<g1, kBlock, 0, s>>>(x, ldx, d, w13, I, dl, hbuf);
        trace_end(K3_OP_SHARED_EXPERT, s);
        const int g2 = budget_grid(d / 16, cu_budget, 4);
        k_down_mfma<16, DenseList, OutDense><<<g2, kBlock, 0, s>>>(hbuf, I, w2, d, dl, out);
    }
    const int st = launch_status();
    if (st == K3_OK)
        record_dispatch(K3_OP_SHARED_EXPERT, variant);
    return st;
}
