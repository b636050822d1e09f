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
#include "k3_gemv.h"
#include "k3_internal.h"
#include "k3_skinny.h"

namespace k3 {

constexpr int kDot2MaxTokens = 4;
constexpr int kAllMfmaMin = 5;  // batches from which light experts join the MFMA launches

// ------------------------------------------------------------------ expert lists
struct ExpertList {  // a compacted list written by the permutation kernel
    const int *n;
    const int *expert, *start, *ntok;
    const int *sorted_token;
    // a is the same in every lane: the entries come through the scalar cache
    __device__ int count() const { return ld_scalar(n); }
    __device__ void get(int a, int &e, int &p0, int &na) const {
        e = ld_scalar(expert + a);
        p0 = ld_scalar(start + a);
        na = ld_scalar(ntok + a);
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
// Where the permutation writes: the two compacted expert lists (light: at
// most kDot2MaxTokens tokens, heavy: more), the tokens sorted by expert and
// every (token, slot)'s position.
struct PermuteOut {
    int *n_light, *light_expert, *light_start, *light_ntok;
    int *n_heavy, *heavy_expert, *heavy_start, *heavy_ntok;
    int *sorted_token, *slot_pos;
};

// One workgroup. Token t's choice of expert e sets bit t of mask[e]; an
// expert's token count is the popcount, so every (expert, token) pair gets
// exactly one position and all positions [0, total) are written. Ids outside
// [0, E) are dropped (slot_pos = -1). Exclusive scans over the experts give
// the positions and the two compacted lists.
__device__ __forceinline__ void moe_permute_block(const int32_t *__restrict__ ids, int b, int k,
                                                  int E, const PermuteOut &o) {
    int *n_light = o.n_light, *light_expert = o.light_expert, *light_start = o.light_start;
    int *light_ntok = o.light_ntok, *n_heavy = o.n_heavy, *heavy_expert = o.heavy_expert;
    int *heavy_start = o.heavy_start, *heavy_ntok = o.heavy_ntok;
    int *sorted_token = o.sorted_token, *slot_pos = o.slot_pos;
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

__global__ void __launch_bounds__(kBlock)
k_moe_permute(const int32_t *__restrict__ ids, int b, int k, int E, PermuteOut o) {
    moe_permute_block(ids, b, k, E, o);
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
    const int wq = wave_in_block();
    const int total = L.count() * I;
    int g0, g1;
    split_range(total, gridDim.x, blockIdx.x, g0, g1);
    for (int s0 = g0; s0 < g1;) {
        const int a = s0 / I;
        const int s1 = min(g1, (a + 1) * I);
        int e, p0, na;
        L.get(a, e, p0, na);
        if (na > 0) {
            __syncthreads();  // the previous segment's readers of xs are done
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
                },
                [&]() {
                    stage_rows(xs, nv, na, nv,
                               [&](int t) { return z + (int64_t)L.token(p0 + t) * ldz; });
                    __syncthreads();
                });
        }
        s0 = s1;
    }
}

// ------------------------------------------------------------------ 8-row gate/up
// Routed gate/up at 2-4 tokens on the 8-row engine (k3_gemv.h): every active
// expert is on the light list, holding at most NT = b tokens. All b token
// rows are staged in LDS; as at batch 1 a group is (list entry a, columns
// 4c .. 4c + 3) -- gate rows 4c .. 4c + 3 and up rows I + 4c .. I + 4c + 3 of
// w13[e_a] -- and workgroup w takes the same column blocks (an even share of
// the I / 4) of every entry, so its stream runs on across the experts. A
// group's sums are taken for its entry's tokens only (the entry's count is
// wave-uniform). h of position p = start_a + t, column j goes to hbuf[p][j].
template <int U, int NT>
__global__ void __launch_bounds__(kBlock)
k_gateup_rows8(const uint16_t *__restrict__ z, int64_t ldz, int d,
               const uint16_t *__restrict__ w13, int I, ExpertList L,
               uint16_t *__restrict__ hbuf, int ps_stride) {
    extern __shared__ u32x4 zs[];  // NT token rows (d / 8 vectors each), then ps[4][NT][ps_stride]
    const int nv = d >> 3;
    float *ps = reinterpret_cast<float *>(zs + NT * nv);
    int c0, c1;
    split_range(I >> 2, gridDim.x, blockIdx.x, c0, c1);
    const int cps = c1 - c0;  // this workgroup's column blocks per entry
    const int n = L.count();
    struct Slot {
        int nt;
        int off[NT];  // the entry's token rows in zs (vectors), unused ones repeat the last
    };
    GvStage<4> st[NT];  // d <= 8192
    gemv8_stream_slots<U, NT>(
        n * cps, d,
        [&](int g, const uint16_t *&base, int &nr, int &skip) {
            const int a = g / cps, c = c0 + (g - a * cps);
            int e, p0, na;
            L.get(a, e, p0, na);
            base = w13 + ((int64_t)e * 2 * I + 4 * c) * d;
            nr = 8;
            skip = I - 4;
        },
        [&](int g) {
            Slot cx;
            int e, p0, na;
            L.get(g / cps, e, p0, na);
            cx.nt = na;
#pragma unroll
            for (int t = 0; t < NT; ++t)
                cx.off[t] = ld_scalar(L.sorted_token + p0 + min(t, na - 1)) * nv;
            return cx;
        },
        [&](const Slot &cx, int kv, int t) { return zs[cx.off[t] + kv]; }, ps, ps_stride,
        [&]() {
#pragma unroll
            for (int t = 0; t < NT; ++t)
                st[t].load(z + (int64_t)t * ldz, nv);
        },
        [&]() {
#pragma unroll
            for (int t = 0; t < NT; ++t)
                st[t].store(zs + t * nv, nv);
            __syncthreads();
        });
    const int nrow = 8 * n * cps;
    for (int q = threadIdx.x; q < NT * nrow; q += kBlock) {
        const int t = q / nrow, i = q - t * nrow, r = i & 7;
        const int g = i >> 3, a = g / cps;
        if (r < 4 && t < L.ntok[a])
            hbuf[(int64_t)(L.start[a] + t) * I + 4 * (c0 + g - a * cps) + r] =
                f32_to_bf16(silu(gv_total(ps, ps_stride, i, NT, t)) *
                            gv_total(ps, ps_stride, i + 4, NT, t));
    }
}

// ------------------------------------------------------------------ 8-row down + combine
// Routed down projection at 2-4 tokens on the 8-row engine, with the
// weighted combine in its epilogue: y[t][r] = bf16(y_add[t][r] + sum_j
// w[t][j] o[slot_pos[t][j]][r]), slots in order j = 0..k-1 (as k_combine
// adds them). Workgroup w owns rows [rb0, rb1) of the output (at most 8 GPS)
// for every entry of the light list; its units are (entry a, 8-row group
// rg), entry-major, one unit per group: wave wq streams K-quarter wq (U
// pieces of 64, I = 256 U) of the group's rows of w2[e_a]. A wave needs only
// its own quarter of the entry's h rows, so it stages them itself into a
// two-slot ring in LDS: at the start of entry a it stores entry a + 1's
// quarter rows (loaded one entry earlier, so the weight loads issued since
// then keep streaming) and issues the loads of entry a + 2's. With GPS
// groups per entry the staging falls on fixed steps of the unit pairs, so
// every load is issued on every path.
template <int NT, int GPS>
__global__ void __launch_bounds__(kBlock)
k_down_rows8(const uint16_t *__restrict__ hbuf, int I, const uint16_t *__restrict__ w2, int d_out,
             ExpertList L, const int *__restrict__ slot_pos, const float *__restrict__ topk_w,
             int k, const float *__restrict__ y_add, uint16_t *__restrict__ y, int ps_stride) {
    constexpr int U = 8;            // pieces per wave quarter: I = 256 U = 2048
    constexpr int QV = U * 8;       // 16-byte vectors in a quarter row (one per lane)
    __shared__ u32x4 hq[4][2][NT][QV];  // [wave][ring slot][token][vector]
    __shared__ int s_entry[NT * K3_MAX_TOPK], s_pos[NT * K3_MAX_TOPK];
    __shared__ float s_w[NT * K3_MAX_TOPK], s_ya[NT * 8 * GPS];
    extern __shared__ float ps[];   // [4][NT][ps_stride]
    const int lane = threadIdx.x & (kWave - 1), wq = wave_in_block();
    int rb0, rb1;
    split_range(d_out, gridDim.x, blockIdx.x, rb0, rb1);
    const int rows = rb1 - rb0;
    const int n = L.count();
    const int nunits = n * GPS;
    const int P = NT * k;  // (token, slot) pairs; NT is the batch
    // h quarter rows of entry a into registers: token t's vector `lane`
    // (tokens past the entry's count, and entries past the list, read zeros)
    auto hload = [&](u32x4 (&hr)[NT], int a) {
        const int ac = min(a, n - 1);
        int e, p0, na;
        L.get(ac < 0 ? 0 : ac, e, p0, na);
        na = a < n ? na : 0;
        const rsrc_t r = act_range(hbuf);
#pragma unroll
        for (int t = 0; t < NT; ++t)
            hr[t] = ld_act16(r, t < na ? ((uint32_t)(p0 + t) * (uint32_t)I +
                                          (uint32_t)(wq * QV + lane) * 8u) * 2u
                                       : kOffNone);
    };
    auto hstore = [&](const u32x4 (&hr)[NT], int slot) {
#pragma unroll
        for (int t = 0; t < NT; ++t)
            hq[wq][slot][t][lane] = hr[t];
    };
    const int rl = lane >> 3, el = (lane & 7) * 8;
    auto load = [&](u32x4 (&b)[U], int u) {
        const int a = u / GPS, rg = u - a * GPS;
        int e, p0, na;
        L.get(u < nunits ? a : 0, e, p0, na);
        const int nr = max(0, min(8, rows - 8 * rg));
        const uint32_t bytes = u < nunits ? (uint32_t)nr * (uint32_t)I * 2u : 0u;
        const rsrc_t r = weight_range(
            uniform_ptr(w2 + (int64_t)e * d_out * I + (int64_t)(rb0 + 8 * rg) * I), bytes);
#pragma unroll
        for (int i = 0; i < U; ++i)
            b[i] = ld_weight16(r, ((uint32_t)(rl * I + (wq * U + i) * 64 + el)) * 2u);
    };
    float acc[NT];
    auto fin = [&](const u32x4 (&b)[U], int u) {
        const int a = u / GPS, rg = u - a * GPS;
        int e, p0, na;
        L.get(u < nunits ? a : 0, e, p0, na);
        const int slot = a & 1;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            acc[t] = 0.0f;
            if (t < na) {
#pragma unroll
                for (int i = 0; i < U; ++i)
                    acc[t] = dot8(b[i], hq[wq][slot][t][i * 8 + (lane & 7)], acc[t]);
            }
        }
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            const float sum = gv_red8(acc[t]);
            if (u < nunits && (lane & 7) == 0)
                ps[(wq * NT + t) * ps_stride + 8 * (a * GPS + rg) + rl] = sum;
        }
    };
    // the combine's inputs and the list's entries, loaded before any weights
    const int q = threadIdx.x;
    const int pq = min(q, P - 1), yq = min(q, NT * rows - 1);
    const int sp = slot_pos[pq];
    const float sw = topk_w[pq];
    const float ya = y_add ? y_add[(int64_t)(yq / rows) * d_out + rb0 + yq % rows] : 0.0f;
    const int qa = min(q, max(n - 1, 0));
    const int q_start = L.start[qa], q_ntok = q < n ? L.ntok[qa] : 0;
    u32x4 h0[NT], hr[NT];
    hload(h0, 0);
    hload(hr, 1);
    u32x4 A[U], B[U];
    load(A, 0);
    hstore(h0, 0);
    if (q < P) {
        s_pos[q] = sp;
        s_w[q] = sw;
    }
    if (q < NT * rows)
        s_ya[q] = ya;
    for (int t = 0; t < q_ntok; ++t)
        s_entry[q_start + t] = q;
    __syncthreads();
    // entry a starts at unit GPS a: store entry a + 1's quarter rows (slot
    // (a + 1) & 1, which entry a - 1 used), then issue entry a + 2's. Units
    // run in pairs, so with GPS = 2 every pair starts one entry and with
    // GPS = 1 each unit does.
    auto stage = [&](int a) {
        hstore(hr, (a + 1) & 1);
        hload(hr, a + 2);
    };
    static_assert(GPS == 1 || GPS == 2, "one or two row groups per entry");
    for (int u = 0; u < nunits; u += 2) {
        load(B, u + 1);
        stage(u / GPS);
        __builtin_amdgcn_sched_barrier(0);
        fin(A, u);
        load(A, u + 2);
        if constexpr (GPS == 1)
            stage(u + 1);
        __builtin_amdgcn_sched_barrier(0);
        fin(B, u + 1);
    }
    __syncthreads();
    for (int i = threadIdx.x; i < NT * rows; i += kBlock) {
        const int t = i / rows, rr = i - t * rows;
        float sum = s_ya[i];
        for (int j = 0; j < k; ++j) {
            const int pos = s_pos[t * k + j];
            if (pos >= 0) {
                const int a = s_entry[pos];
                const int tt = pos - L.start[a];
                sum += s_w[t * k + j] *
                       gv_total(ps, ps_stride, 8 * (a * GPS + (rr >> 3)) + (rr & 7), NT, tt);
            }
        }
        y[(int64_t)t * d_out + rb0 + rr] = f32_to_bf16(sum);
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
    const int wq = wave_in_block();
    const int total = L.count() * d_out;
    int g0, g1;
    split_range(total, gridDim.x, blockIdx.x, g0, g1);
    for (int s0 = g0; s0 < g1;) {
        const int a = s0 / d_out;
        const int s1 = min(g1, (a + 1) * d_out);
        int e, p0, na;
        L.get(a, e, p0, na);
        if (na > 0) {
            __syncthreads();  // the previous segment's readers of xs are done
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
                },
                [&]() {
                    stage_rows(xs, nv, na, nv, [&](int t) { return hbuf + (int64_t)(p0 + t) * I; });
                    __syncthreads();
                });
        }
        s0 = s1;
    }
}

// ------------------------------------------------------------------ heavy experts (MFMA)
// Experts with more than kDot2MaxTokens tokens run on the split-K MFMA
// engine of k3_skinny.h with one K range per tile, so the epilogue finishes
// the outputs itself. Gate/up (pair == true): a tile is 32 columns j of h;
// waves 0-1 stream gate rows j, waves 2-3 the matching up rows I + j, the up
// sums cross to the gate waves through LDS and h = silu(g) * u is written
// for the expert's positions. Down (pair == false): a tile is 64 output
// rows; the sums go to part[p][n]. A down launch may carry one extra dense
// job after the list: the shared expert's down projection into y_s.
struct SkExperts {
    int tpw = 1;  // 16-row tiles per wave of the launch (a wave streams 16 tpw rows)
    int sa = 0, sp = 0;  // slot shares of the stream kernel (0: none)
    ExpertList L;
    ExpertList L2;  // a second list after L (its n may be null: none)
    const uint16_t *w;  // expert e: w + e * w_stride, [rows][K] (gate/up: [2I][K])
    int64_t w_stride;
    int K;
    bool pair;
    int I;     // gate/up: columns of h
    int rows;  // down: output rows
    const uint16_t *x;  // gate/up: z rows by token; down: h rows by position
    int64_t ldx;
    bool gather;
    uint16_t *h;  // gate/up output [P][I]
    float *out;   // down output [P][rows]
    const uint16_t *w_x;  // extra job: weights [rows][K], or null
    const uint16_t *x_x;
    int64_t ldx_x;
    int xT;
    float *out_x;  // [xT][rows]

    struct Job {
        int T;
        int e;       // expert id (list jobs)
        int p0;      // first position (list jobs)
        bool extra;  // the extra dense job
    };
    // List entries are read once per workgroup and taken from lane 0, so the
    // compiler keeps the item state (and the ranges built from it) in scalar
    // registers.
    __device__ int n1() const { return __builtin_amdgcn_readfirstlane(L.count()); }
    __device__ int nlist() const {
        return n1() + (L2.n ? __builtin_amdgcn_readfirstlane(L2.count()) : 0);
    }
    __device__ int count() const { return nlist() + (w_x ? 1 : 0); }
    // Down launches group each XCD's items; gate/up launches keep the plain
    // interleave, which was faster for them at 8-64 tokens. Measured on the
    // whole MoE block, grouped against plain down launches in one process
    // (medians of six graph replays of 30 blocks): 821.5 against 829.4 us at
    // 8 tokens, 1525.5 against 1534.5 us at 16, 2595 against 2601 us at 32,
    // equal (859.3 us) at 64 with the Zipf bias.
    __device__ bool xcd_grouped() const { return !pair; }
    __device__ int share_p() const { return sp; }
    __device__ int share_a() const { return sa; }
    __device__ int tiles() const {
        return pair ? I / (32 * tpw) : (rows + 64 * tpw - 1) / (64 * tpw);
    }
    __device__ Job job(int a) const {
        if (w_x && a == nlist())
            return Job{xT, 0, 0, true};
        int e, p0, na;
        const int m = n1();
        if (a < m)
            L.get(a, e, p0, na);
        else
            L2.get(a - m, e, p0, na);
        return Job{__builtin_amdgcn_readfirstlane(na), __builtin_amdgcn_readfirstlane(e),
                   __builtin_amdgcn_readfirstlane(p0), false};
    }
    __device__ void wave_rows(const Job &jb, int tile, int wq, const uint16_t *&wr,
                              int &n) const {
        const int wr_rows = 16 * tpw;  // the wave's rows (tpw tiles of 16)
        if (jb.extra) {
            const int r0 = tile * 4 * wr_rows + wq * wr_rows;
            n = max(0, min(wr_rows, rows - r0));
            wr = w_x + (int64_t)(n > 0 ? r0 : 0) * K;
            return;
        }
        const uint16_t *base = w + (int64_t)jb.e * w_stride;
        if (pair) {
            // waves 0-1 stream gate rows j, waves 2-3 the matching up rows I + j
            const int j0 = 2 * wr_rows * tile;
            const int r = wq < 2 ? j0 + wr_rows * wq : I + j0 + wr_rows * (wq - 2);
            n = wr_rows;
            wr = base + (int64_t)r * K;
        } else {
            const int r0 = tile * 4 * wr_rows + wq * wr_rows;
            n = max(0, min(wr_rows, rows - r0));
            wr = base + (int64_t)(n > 0 ? r0 : 0) * K;
        }
    }
    __device__ const uint16_t *xbase(const Job &jb) const { return jb.extra ? x_x : x; }
    // The choice is uniform; on the gathering path the looked-up row is the
    // result itself, so nothing waits for the lookup until the row is used.
    __device__ int xrow(const Job &jb, int t) const {
        if (jb.extra)
            return t;
        if (!gather)
            return jb.p0 + t;
        return L.token(jb.p0 + t);
    }
    __device__ int xld(const Job &jb) const { return (int)(jb.extra ? ldx_x : ldx); }
    // Epilogue of tile tt of the wave's tpw tiles.
    template <int MT>
    __device__ __forceinline__ void store(const Job &jb, int tile, int, int wq, int tt,
                                          const f32x4 (&acc)[MT],
                                          float (*xch)[MT][4][kWave]) const {
        const int lane = threadIdx.x & (kWave - 1);
        const int g = lane >> 4, rl = lane & 15;
        const int T = jb.T;
        const int wr_rows = 16 * tpw;
        if (pair) {
            if (wq >= 2)
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        xch[wq - 2][mt][i][lane] = acc[mt][i];
            __syncthreads();
            if (wq < 2) {
                const int j = 2 * wr_rows * tile + wr_rows * wq + 16 * tt + rl;
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        const int t = mt * 16 + 4 * g + i;
                        if (t < T)
                            h[(int64_t)(jb.p0 + t) * I + j] =
                                f32_to_bf16(silu(acc[mt][i]) * xch[wq][mt][i][lane]);
                    }
            }
            __syncthreads();  // xch is read before the next tile's exchange
            return;
        }
        const int n = tile * 4 * wr_rows + wq * wr_rows + 16 * tt + rl;
        if (n >= rows)
            return;
        float *o = jb.extra ? out_x : out + (int64_t)jb.p0 * rows;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int t = mt * 16 + 4 * g + i;
                if (t < T)
                    o[(int64_t)t * rows + n] = acc[mt][i];
            }
    }
};

// ------------------------------------------------------------------ combine
// y[t][r] = bf16(y_add[t][r] + sum_j w[t][j] * part[slot_pos[t][j]][r]),
// slots added in order j = 0..k-1; eight slots' loads go out together.
__global__ void __launch_bounds__(kBlock)
k_combine(const float *__restrict__ part, int d_out, const int *__restrict__ slot_pos,
          const float *__restrict__ topk_w, int b, int k, const float *__restrict__ y_add,
          uint16_t *__restrict__ y) {
    const int i = blockIdx.x * kBlock + threadIdx.x;
    if (i >= b * d_out)
        return;
    const int t = i / d_out, r = i - t * d_out;
    float s = y_add ? y_add[i] : 0.0f;
    for (int j0 = 0; j0 < k; j0 += 8) {
        float pv[8], wv[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int j = j0 + u;
            const int pos = j < k ? slot_pos[t * k + j] : -1;
            wv[u] = pos >= 0 ? topk_w[t * k + j] : 0.0f;
            pv[u] = pos >= 0 ? part[(int64_t)pos * d_out + r] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (j0 + u < k && slot_pos[t * k + j0 + u] >= 0)
                s += wv[u] * pv[u];
    }
    y[i] = f32_to_bf16(s);
}

// slot_pos for batch 1 without a permutation: slot j sits at position j when
// its id is valid.
__global__ void k_slot_identity(const int32_t *__restrict__ ids, int k, int E, int *slot_pos) {
    const int j = threadIdx.x;
    if (j < k)
        slot_pos[j] = (ids[j] >= 0 && ids[j] < E) ? j : -1;
}

// ------------------------------------------------------------------ top-k + shared down
// Second kernel of the fused MoE block: workgroup 0 picks every token's
// experts from the logits the first kernel wrote (one wave per token) and,
// with `permute`, sorts the (token, slot) pairs by expert right after (the
// permutation kernel's work, one launch fewer); the other workgroups stream
// the shared expert's down projection meanwhile, so the selection's latency
// hides under useful weight reads.
template <int TM, int CB>
__global__ void __launch_bounds__(kBlock)
k_topk_shared_down(const float *__restrict__ logits, int E, int k, int b,
                   int32_t *__restrict__ ids, float *__restrict__ wts,
                   const uint16_t *__restrict__ hs, int Is, const uint16_t *__restrict__ W2s,
                   int d, float *__restrict__ y_s, bool permute, PermuteOut po) {
    const int wq = wave_in_block();
    if (blockIdx.x == 0) {
        for (int t = wq; t < b; t += kBlock / kWave)
            topk_wave(logits + (int64_t)t * E, E, k, ids + (int64_t)t * k, wts + (int64_t)t * k);
        if (permute) {
            __syncthreads();  // every token's ids are written (and visible to the block)
            moe_permute_block(ids, b, k, E, po);
        }
        return;
    }
    extern __shared__ u32x4 xs[];
    const int nv = Is >> 3;
    const int lane = threadIdx.x & (kWave - 1);
    const int waves = (gridDim.x - 1) * (kBlock / kWave);
    const int wave = (blockIdx.x - 1) * (kBlock / kWave) + wq;
    int r0, r1;
    split_range(d, waves, wave, r0, r1);
    stream_rows<TM, 16 / CB, CB>(
        r0, r1, nv, xs, nv, b, [&](int r) { return W2s + (int64_t)r * Is; },
        [&](int r, int t, float s) {
            if (lane == 0)
                y_s[(int64_t)t * d + r] = s;
        },
        [&]() {
            stage_rows(xs, nv, b, nv, [&](int t) { return hs + (int64_t)t * Is; });
            __syncthreads();
        });
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

namespace {
// Fused-block workspace: router logits, shared-expert h, then the routed
// experts' workspace.
struct BlockWorkspace {
    size_t logits, hs, moe, part, total;
};
BlockWorkspace block_workspace_layout(int b, int E, int k, int I, int d, int d_lat, int I_s) {
    BlockWorkspace w;
    w.logits = 256;
    w.hs = w.logits + align_up((size_t)b * E * sizeof(float), 256);
    w.moe = w.hs + align_up((size_t)b * I_s * sizeof(uint16_t), 256);
    w.part = w.moe + moe_workspace_layout(b, E, k, I, d).total;
    // the partials of the router + latent + shared gate/up pass (K = d)
    w.total = w.part + sk_partial_bytes(b, E + d_lat + 2 * I_s, d);
    return w;
}
}  // namespace

extern "C" size_t k3_moe_experts_workspace_size(int b, int d_in, int E, int k, int I, int d_out) {
    (void)d_in;
    if (b <= 0 || E <= 0 || k <= 0 || I <= 0 || d_out <= 0)
        return 0;
    return moe_workspace_layout(b, E, k, I, d_out).total;
}

namespace {
size_t shared_part_offset(int b, int I) { return align_up((size_t)b * I * sizeof(uint16_t), 256); }
}  // namespace

extern "C" size_t k3_shared_expert_workspace_size(int b, int d, int I) {
    if (b <= 0 || I <= 0 || d <= 0)
        return 0;
    // gate/up: 2I rows over K = d; down: d rows over K = I
    const size_t g = sk_partial_bytes(b, 2 * I, d), dn = sk_partial_bytes(b, d, I);
    return shared_part_offset(b, I) + (g > dn ? g : dn);
}

extern "C" size_t k3_moe_block_workspace_size(int b, int d, int E, int k, int d_lat, int I,
                                              int I_s) {
    if (b <= 0 || d <= 0 || E <= 0 || k <= 0 || I <= 0 || I_s <= 0 || d_lat <= 0)
        return 0;
    return block_workspace_layout(b, E, k, I, d, d_lat, I_s).total;
}

// ------------------------------------------------------------------ launchers
namespace {

int dot2_grid(int cu_budget) { return budget_grid(1 << 30, cu_budget, 2); }

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

// The 8-row gate/up at 2 <= b <= 4: one workgroup per column block of I / 4
// at most, two per compute unit; LDS holds the b token rows and the partial
// sums of every entry of the share.
int rows8_grid(int I, int cu_budget) { return budget_grid(I / 4, cu_budget, 2); }

size_t rows8_lds(int b, int d, int k, int E, int I, int grid, int &ps_stride) {
    const int entries = b * k < E ? b * k : E;
    ps_stride = 8 * entries * ((I / 4 + grid - 1) / grid);
    return (size_t)b * d * sizeof(uint16_t) + (size_t)4 * b * ps_stride * sizeof(float);
}

bool rows8_fits(int b, int d, int k, int E, int I, int cu_budget) {
    int ps_stride;
    const size_t cap = device_max_lds() < 81920 ? device_max_lds() : 81920;
    return b >= 2 && b <= kDot2MaxTokens && d % 64 == 0 && d <= 8192 && I % 4 == 0 &&
           rows8_lds(b, d, k, E, I, rows8_grid(I, cu_budget), ps_stride) <= cap;
}

void launch_gateup_rows8(int b, const uint16_t *z, int64_t ldz, int d, const uint16_t *w13, int I,
                         int k, int E, ExpertList L, uint16_t *hbuf, int cu_budget,
                         hipStream_t s) {
    const int grid = rows8_grid(I, cu_budget);
    int ps_stride;
    const size_t lds = rows8_lds(b, d, k, E, I, grid, ps_stride);
#define K3_R8(U_, T_) \
    k_gateup_rows8<U_, T_><<<grid, kBlock, lds, s>>>(z, ldz, d, w13, I, L, hbuf, ps_stride)
    const bool u7 = gv_unit_pieces(d) == 7;
    if (b == 2) {
        if (u7)
            K3_R8(7, 2);
        else
            K3_R8(8, 2);
    } else if (b == 3) {
        if (u7)
            K3_R8(7, 3);
        else
            K3_R8(8, 3);
    } else {
        if (u7)
            K3_R8(7, 4);
        else
            K3_R8(8, 4);
    }
#undef K3_R8
}

// The 8-row down + combine at 2 <= b <= 4: two workgroups per compute unit,
// each owning at most 16 output rows (one or two 8-row groups per entry).
int down_rows8_grid(int d_out, int cu_budget) { return budget_grid(d_out, cu_budget, 2); }

bool down_rows8_fits(int b, int I, int d_out, int k, int E, int cu_budget, int &ps_stride,
                     size_t &lds) {
    if (b < 2 || b > kDot2MaxTokens || I != 2048 || k > K3_MAX_TOPK)
        return false;
    const int grid = down_rows8_grid(d_out, cu_budget);
    const int rows = (d_out + grid - 1) / grid;
    const int gps = (rows + 7) / 8;
    const int entries = b * k < E ? b * k : E;
    ps_stride = 8 * entries * gps;
    lds = (size_t)4 * b * ps_stride * sizeof(float);
    // static LDS: the h ring (8 KB per token) and the combine's tables
    const size_t fixed = (size_t)b * 8192 + 4096;
    const size_t cap = device_max_lds() < 81920 ? device_max_lds() : 81920;
    return gps <= 2 && lds + fixed <= cap;
}

void launch_down_rows8(int b, const uint16_t *hbuf, int I, const uint16_t *w2, int d_out,
                       ExpertList L, const int *slot_pos, const float *topk_w, int k,
                       const float *y_add, uint16_t *y, int cu_budget, int ps_stride, size_t lds,
                       hipStream_t s) {
    const int grid = down_rows8_grid(d_out, cu_budget);
    const int gps = ((d_out + grid - 1) / grid + 7) / 8;
#define K3_D8(T_, G_)                                                                       \
    k_down_rows8<T_, G_><<<grid, kBlock, lds, s>>>(hbuf, I, w2, d_out, L, slot_pos, topk_w, \
                                                   k, y_add, y, ps_stride)
    if (b == 2) {
        if (gps == 1)
            K3_D8(2, 1);
        else
            K3_D8(2, 2);
    } else if (b == 3) {
        if (gps == 1)
            K3_D8(3, 1);
        else
            K3_D8(3, 2);
    } else {
        if (gps == 1)
            K3_D8(4, 1);
        else
            K3_D8(4, 2);
    }
#undef K3_D8
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

struct OutDense {  // y_s[t][r] = s (positions are tokens for the dense list)
    float *y;
    int d;
    __device__ void operator()(int p, int r, float s) const { y[(int64_t)p * d + r] = s; }
};

// Expert launch over at most max_jobs jobs. At 64 tokens a wave streams two
// 16-row tiles per chunk (half the token staging and token reads per weight
// byte); below, one.
void launch_sk_experts(SkExperts J, int b, int max_jobs, int cu_budget, hipStream_t s) {
    const int mt = sk_mt(b);
    J.tpw = mt == 4 ? 2 : 1;
    const int tiles = J.pair ? J.I / (32 * J.tpw) : (J.rows + 64 * J.tpw - 1) / (64 * J.tpw);
    const int items = max_jobs * tiles;
    // two workgroups per compute unit, each streaming its items back to back
    const int grid = budget_grid(items < 1 ? 1 : items, cu_budget, 2);
    // Slot shares: the first workgroup of each compute unit takes 4 of every
    // 7 rounds at 33-64 tokens, 7 of every 12 at 17-32. Measured on the MoE
    // block in one process, uniform routing: 33 tokens 2640 -> 2619 us, 40
    // 2941 -> 2898, 48 3276 -> 3227, 56 3562 -> 3518, 64 3791 -> 3729 (64
    // with the Zipf bias unchanged, 826 -> 827; 7:12 and 5:9 gained less at
    // 64); 17 tokens 1562 -> 1560, 24 2056 -> 2039, 32 2522 -> 2510 (4:7
    // gained less there). At 5-16 tokens no ratio paid (16 tokens +0.3%).
    if (mt >= 2 && cu_budget == 0 && grid == 2 * device_cu_count()) {
        J.sa = mt == 4 ? 4 : 7;
        J.sp = mt == 4 ? 7 : 12;
    }
    switch (mt) {
    case 1:
        k_sk_gemm_stream<1, SkExperts, 1><<<grid, kBlock, 0, s>>>(J, J.K, 1);
        break;
    case 2:
        k_sk_gemm_stream<2, SkExperts, 1><<<grid, kBlock, 0, s>>>(J, J.K, 1);
        break;
    default:
        k_sk_gemm_stream<4, SkExperts, 2><<<grid, kBlock, 0, s>>>(J, J.K, 1);
        break;
    }
}

// The routed experts after validation: batch 1 reads the ids directly; larger
// batches permute, then run light experts on dot2 rows and heavy ones on MFMA
// tiles; y = y_add + the weighted expert outputs.
// A dense job the heavy down launch can carry: y_x[t][n] = w_x[n] . x_x[t]
// (fp32), t < xT, n < d_out, K = I (the shared expert's down projection).
struct DownExtra {
    const uint16_t *w_x;
    const uint16_t *x_x;
    int64_t ldx_x;
    int xT;
    float *out_x;
};

// The permutation's outputs in a routed-experts workspace.
PermuteOut permute_out(const MoeWorkspace &L, char *ws) {
    return PermuteOut{(int *)(ws + L.n_light),      (int *)(ws + L.light_expert),
                      (int *)(ws + L.light_start),  (int *)(ws + L.light_ntok),
                      (int *)(ws + L.n_heavy),      (int *)(ws + L.heavy_expert),
                      (int *)(ws + L.heavy_start),  (int *)(ws + L.heavy_ntok),
                      (int *)(ws + L.sorted_token), (int *)(ws + L.slot_pos)};
}

// The engine of the expert products of a b-token call: dot2 rows while every
// expert holds at most kDot2MaxTokens tokens (b < kAllMfmaMin), MFMA tiles
// above; a forced K3_OP_EXPERT_ENGINE variant overrides it. 0 when the
// forced engine cannot run b tokens (MFMA needs b >= 2: batch 1 has no
// permutation; dot2 holds at most kDot2MaxTokens tokens per expert).
int expert_engine(int b) {
    const int fv = forced_variant(K3_OP_EXPERT_ENGINE);
    if (fv == K3_VARIANT_NONE)
        return b >= kAllMfmaMin ? K3_VARIANT_MFMA : K3_VARIANT_DOT2;
    if (fv == K3_VARIANT_MFMA)
        return b >= 2 ? fv : 0;
    if (fv == K3_VARIANT_DOT2)
        return b < kAllMfmaMin ? fv : 0;
    return 0;
}

void run_moe_experts(const uint16_t *z, int64_t ldz, int b, int d_in, const int32_t *topk_ids,
                     const float *topk_w, int k, const uint16_t *w13, const uint16_t *w2, int E,
                     int I, int d_out, const float *y_add, hipEvent_t y_add_ready, uint16_t *y,
                     int cu_budget, char *ws, int trace_op, hipStream_t s, int engine,
                     const DownExtra *extra = nullptr, bool permuted = false) {
    const MoeWorkspace L = moe_workspace_layout(b, E, k, I, d_out);
    uint16_t *hbuf = (uint16_t *)(ws + L.hbuf);
    float *part = (float *)(ws + L.part);
    const OutPart out{part, d_out};
    int *slot_pos = (int *)(ws + L.slot_pos);
    trace_begin(trace_op, s);
    if (b == 1) {
        const SlotList sl{topk_ids, k, E};
        // the batch-1 pair shares its own h layout: both kernels or neither
        const bool b1 = up_b1_fits(d_in, k, I, cu_budget) &&
                        down_b1_fits(k, I, d_out, false, cu_budget);
        if (b1)
            launch_up_b1(false, z, d_in, w13, I, E, k, topk_ids, nullptr, nullptr, nullptr, hbuf,
                         cu_budget, s);
        else
            launch_gateup_dot2(1, z, ldz, d_in, w13, I, sl, hbuf, cu_budget, s);
        trace_end(trace_op, s);
        if (y_add_ready)
            (void)hipStreamWaitEvent(s, y_add_ready, 0);
        if (b1) {
            launch_down_b1(hbuf, I, w2, d_out, topk_ids, topk_w, k, E, y_add, nullptr, nullptr,
                           nullptr, y, cu_budget, s);
            return;
        }
        launch_down_dot2(1, hbuf, I, w2, d_out, sl, out, cu_budget, s);
        k_slot_identity<<<1, kBlock, 0, s>>>(topk_ids, k, E, slot_pos);
    } else {
        int *n_light = (int *)(ws + L.n_light), *n_heavy = (int *)(ws + L.n_heavy);
        const ExpertList light{n_light, (int *)(ws + L.light_expert), (int *)(ws + L.light_start),
                               (int *)(ws + L.light_ntok), (int *)(ws + L.sorted_token)};
        const ExpertList heavy{n_heavy, (int *)(ws + L.heavy_expert), (int *)(ws + L.heavy_start),
                               (int *)(ws + L.heavy_ntok), (int *)(ws + L.sorted_token)};
        // the lists come from the permutation kernel, or were written by the
        // selection kernel before this call (permuted)
        if (!permuted)
            k_moe_permute<<<1, kBlock, 0, s>>>(topk_ids, b, k, E, permute_out(L, ws));
        // On the MFMA engine every expert runs in the MFMA launches (heavy
        // list first, then the light one); on the dot2 engine every expert is
        // light (at most kDot2MaxTokens tokens) and runs on dot2 rows.
        const bool all_mfma = engine == K3_VARIANT_MFMA;
        if (!all_mfma && rows8_fits(b, d_in, k, E, I, cu_budget))
            launch_gateup_rows8(b, z, ldz, d_in, w13, I, k, E, light, hbuf, cu_budget, s);
        else if (!all_mfma)
            launch_gateup_dot2(kDot2MaxTokens, z, ldz, d_in, w13, I, light, hbuf, cu_budget, s);
        const int max_jobs = b * k < E ? b * k : E;
        if (all_mfma) {
            SkExperts J{};
            J.L = heavy;
            J.L2 = light;
            J.w = w13;
            J.w_stride = (int64_t)2 * I * d_in;
            J.K = d_in;
            J.pair = true;
            J.I = I;
            J.x = z;
            J.ldx = ldz;
            J.gather = true;
            J.h = hbuf;
            launch_sk_experts(J, b, max_jobs, cu_budget, s);
        }
        trace_end(trace_op, s);
        int ps_stride = 0;
        size_t lds = 0;
        if (!all_mfma && !extra &&
            down_rows8_fits(b, I, d_out, k, E, cu_budget, ps_stride, lds)) {
            // down projection and combine in one kernel, which reads y_add
            if (y_add_ready)
                (void)hipStreamWaitEvent(s, y_add_ready, 0);
            launch_down_rows8(b, hbuf, I, w2, d_out, light, slot_pos, topk_w, k, y_add, y,
                              cu_budget, ps_stride, lds, s);
            return;
        }
        if (!all_mfma)
            launch_down_dot2(kDot2MaxTokens, hbuf, I, w2, d_out, light, out, cu_budget, s);
        if (all_mfma || extra) {
            const ExpertList none{nullptr, nullptr, nullptr, nullptr, nullptr};
            SkExperts J{};
            J.L = heavy;  // empty on the dot2 engine (every expert is light)
            J.L2 = all_mfma ? light : none;
            J.w = w2;
            J.w_stride = (int64_t)d_out * I;
            J.K = I;
            J.rows = d_out;
            J.x = hbuf;
            J.ldx = I;
            J.out = part;
            if (extra) {
                J.w_x = extra->w_x;
                J.x_x = extra->x_x;
                J.ldx_x = extra->ldx_x;
                J.xT = extra->xT;
                J.out_x = extra->out_x;
            }
            const int jobs = (all_mfma ? max_jobs : 0) + (extra ? 1 : 0);
            launch_sk_experts(J, b, jobs, cu_budget, s);
        }
        if (y_add_ready)
            (void)hipStreamWaitEvent(s, y_add_ready, 0);
    }
    const int n = b * d_out;
    k_combine<<<(n + kBlock - 1) / kBlock, kBlock, 0, s>>>(part, d_out, slot_pos, topk_w, b, k,
                                                            y_add, y);
}

// The shared expert; the MFMA variant keeps the partial sums of its K
// ranges in `part` (the larger of sk_partial_bytes(b, 2I, d) and
// sk_partial_bytes(b, d, I) bytes).
void run_shared_expert(int variant, const uint16_t *x, int64_t ldx, int b, int d,
                       const uint16_t *w13, const uint16_t *w2, int I, float *y_s, int cu_budget,
                       uint16_t *hbuf, float *part, int trace_op, hipStream_t s) {
    const DenseList dl{b};
    const OutDense out{y_s, d};
    trace_begin(trace_op, s);
    if (variant == K3_VARIANT_DOT2 && rls_fits(b, d, 0) && rls_gemv_fits(b, d, 0, 0, I) &&
        (b > 1 || gemv1_f32_fits(d, I))) {
        // gate/up on the 8-row engine, summing in the same order as the
        // fused block's router+latent+shared pass; the down rows as the
        // block sums them (one token: in the routed down kernel's order)
        launch_rls(x, ldx, b, d, nullptr, nullptr, 0, nullptr, nullptr, 0, nullptr, 0, w13, I, hbuf,
                   s, cu_budget);
        trace_end(trace_op, s);
        if (b == 1)
            launch_gemv1_f32(hbuf, w2, d, I, y_s, cu_budget, s);
        else
            launch_down_dot2(kDot2MaxTokens, hbuf, I, w2, d, dl, out, cu_budget, s);
    } else if (variant == K3_VARIANT_DOT2) {
        const int tm = b == 1 ? 1 : kDot2MaxTokens;
        launch_gateup_dot2(tm, x, ldx, d, w13, I, dl, hbuf, cu_budget, s);
        trace_end(trace_op, s);
        launch_down_dot2(tm, hbuf, I, w2, d, dl, out, cu_budget, s);
    } else {
        sk_swiglu(x, ldx, b, d, w13, I, hbuf, part, cu_budget, s);
        trace_end(trace_op, s);
        sk_proj_f32_direct(hbuf, I, b, w2, d, I, y_s, d, cu_budget, s);
    }
}

int check_moe_shapes(int b, int d_in, int k, int E, int I, int d_out, int64_t ldz) {
    if (b <= 0 || d_in <= 0 || k <= 0 || E <= 0 || I <= 0 || d_out <= 0 || ldz < d_in)
        return K3_ERR_INVALID_ARG;
    if (b > K3_MAX_BATCH || k > K3_MAX_TOPK || k > E || E > K3_MAX_EXPERTS || I % 128 ||
        d_in % 128 || d_in > 8192 || I > 8192 || d_out % 16 || ldz % 8)
        return K3_ERR_UNSUPPORTED;
    return K3_OK;
}

}  // namespace

// ------------------------------------------------------------------ entry points
extern "C" int k3_moe_experts(const uint16_t *z, int64_t ldz, int b, int d_in,
                              const int32_t *topk_ids, const float *topk_w, int k,
                              const uint16_t *w13, const uint16_t *w2, int E, int I, int d_out,
                              const float *y_add, void *y_add_ready, uint16_t *y, int cu_budget,
                              void *workspace, size_t ws_bytes, void *stream) {
    if (!z || !topk_ids || !topk_w || !w13 || !w2 || !y || cu_budget < 0)
        return K3_ERR_INVALID_ARG;
    const int chk = check_moe_shapes(b, d_in, k, E, I, d_out, ldz);
    if (chk != K3_OK)
        return chk;
    if (!aligned16(z) || !aligned16(w13) || !aligned16(w2))
        return K3_ERR_UNSUPPORTED;
    const int fv = forced_variant(K3_OP_MOE_EXPERTS);
    if (fv != K3_VARIANT_NONE && fv != K3_VARIANT_GROUPED)
        return K3_ERR_UNSUPPORTED;
    const int engine = expert_engine(b);
    if (!engine)
        return K3_ERR_UNSUPPORTED;
    if (!workspace || ws_bytes < moe_workspace_layout(b, E, k, I, d_out).total ||
        !aligned16(workspace))
        return K3_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    run_moe_experts(z, ldz, b, d_in, topk_ids, topk_w, k, w13, w2, E, I, d_out, y_add,
                    (hipEvent_t)y_add_ready, y, cu_budget, (char *)workspace, K3_OP_MOE_EXPERTS,
                    s, engine);
    const int st = launch_status();
    if (st == K3_OK) {
        record_dispatch(K3_OP_MOE_EXPERTS, K3_VARIANT_GROUPED);
        record_dispatch(K3_OP_EXPERT_ENGINE, engine);
    }
    return st;
}

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
    run_shared_expert(variant, x, ldx, b, d, w13, w2, I, y_s, cu_budget, (uint16_t *)workspace,
                      (float *)((char *)workspace + shared_part_offset(b, I)),
                      K3_OP_SHARED_EXPERT, (hipStream_t)stream);
    const int st = launch_status();
    if (st == K3_OK)
        record_dispatch(K3_OP_SHARED_EXPERT, variant);
    return st;
}

// The block on x, or, with nin, on x = RMSNorm(nin->h32) * gamma (x is then
// nin->x_out when that is not null, else xbuf in the workspace).
static int moe_block_run(const uint16_t *x, int64_t ldx, const NormIn *nin, int b, int d,
                         const uint16_t *w_router, const float *bias, int E, int k,
                         const uint16_t *w_lat, int d_lat, const uint16_t *w13,
                         const uint16_t *w2, int I, const uint16_t *w13_s, const uint16_t *w2_s,
                         int I_s, int32_t *topk_ids, float *topk_w, uint16_t *z, int64_t ldz,
                         float *y_s, uint16_t *y, void *workspace, size_t ws_bytes,
                         void *stream) {
    if ((!x && !nin) || !w_router || !w_lat || !w13 || !w2 || !w13_s || !w2_s || !topk_ids ||
        !topk_w || !z || !y_s || !y)
        return K3_ERR_INVALID_ARG;
    if (nin && (!nin->h32 || !nin->gamma || !(nin->eps >= 0.0f)))
        return K3_ERR_INVALID_ARG;
    if (nin)
        ldx = d;
    if (b <= 0 || d <= 0 || E <= 0 || k <= 0 || d_lat <= 0 || I <= 0 || I_s <= 0 || ldx < d ||
        ldz < d_lat)
        return K3_ERR_INVALID_ARG;
    const int chk = check_moe_shapes(b, d_lat, k, E, I, d, ldz);
    if (chk != K3_OK)
        return chk;
    if (d % 128 || d > 8192 || I_s % 128 || I_s > 8192 || ldx % 8 || (x && !aligned16(x)) ||
        !aligned16(w_router) || !aligned16(w_lat) || !aligned16(w13) || !aligned16(w2) ||
        !aligned16(w13_s) || !aligned16(w2_s) || !aligned16(z) ||
        (nin && (!aligned16(nin->h32) || (nin->x_out && !aligned16(nin->x_out)))))
        return K3_ERR_UNSUPPORTED;
    const BlockWorkspace L = block_workspace_layout(b, E, k, I, d, d_lat, I_s);
    const size_t need = L.total + (nin ? align_up((size_t)b * d * sizeof(uint16_t), 256) : 0);
    if (!workspace || ws_bytes < need || !aligned16(workspace))
        return K3_ERR_WORKSPACE;
    const int engine = expert_engine(b);
    if (!engine)
        return K3_ERR_UNSUPPORTED;
    int variant = forced_variant(K3_OP_MOE_BLOCK);
    const bool fits = b <= kDot2MaxTokens && rls_fits(b, d, E) &&
                      (size_t)b * I_s * 2 <= 65536;
    if (variant == K3_VARIANT_NONE)
        variant = fits ? K3_VARIANT_DOT2 : K3_VARIANT_MFMA;
    if ((variant != K3_VARIANT_DOT2 && variant != K3_VARIANT_MFMA) ||
        (variant == K3_VARIANT_DOT2 && !fits))
        return K3_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    char *ws = (char *)workspace;
    float *logits = (float *)(ws + L.logits);
    uint16_t *hs = (uint16_t *)(ws + L.hs);
    const bool fast = variant == K3_VARIANT_DOT2 && b == 1 && I_s == I &&
                      up_b1_fits(d_lat, k, I, 0) && down_b1_fits(k, I, d, true, 0);
    // the shared gate/up rows ride at the head of the routed gate/up kernel
    // (they stream while its selection waits for the logits) where x and z
    // are equally wide; else in the router pass
    const bool sh_up = fast && d_lat == d && up_b1_fits(d_lat, k, I, 0, true);
    const bool norm_in_pass =
        nin && fast && rls_gemv_fits(1, d, E, d_lat, sh_up ? 0 : I_s);
    if (nin && !norm_in_pass) {
        // the norm as its own kernel, into x_out or the workspace
        uint16_t *xb = nin->x_out ? nin->x_out : (uint16_t *)(ws + L.total);
        launch_rmsnorm(nin->h32, b, d, nin->gamma, nin->eps, xb, s);
        x = xb;
    }
    trace_begin(K3_OP_MOE_BLOCK, s);
    if (fast) {
        // 1. router and latent rows (and the shared gate/up rows unless step
        //    2 takes them) in one pass over x, with the norm of its input
        //    folded in when it comes as h32 (the pass then publishes x);
        // 2. [shared gate/up,] expert selection and routed gate/up;
        // 3. routed and shared down rows with the combine
        NormIn nin2{};
        const uint16_t *xs = x;
        if (norm_in_pass) {
            nin2 = *nin;
            if (sh_up && !nin2.x_out)
                nin2.x_out = (uint16_t *)(ws + L.total);
            xs = nin2.x_out;
        }
        launch_rls(x, ldx, b, d, w_router, bias, E, logits, w_lat, d_lat, z, ldz,
                   sh_up ? nullptr : w13_s, sh_up ? 0 : I_s, sh_up ? nullptr : hs, s, 0,
                   norm_in_pass ? &nin2 : nullptr);
        trace_end(K3_OP_MOE_BLOCK, s);
        uint16_t *hbuf = (uint16_t *)(ws + L.moe + moe_workspace_layout(b, E, k, I, d).hbuf);
        trace_begin(K3_OP_MOE_EXPERTS, s);
        launch_up_b1(true, z, d_lat, w13, I, E, k, nullptr, logits, topk_ids, topk_w, hbuf, 0, s,
                     sh_up ? xs : nullptr, sh_up ? w13_s : nullptr, sh_up ? hs : nullptr);
        trace_end(K3_OP_MOE_EXPERTS, s);
        launch_down_b1(hbuf, I, w2, d, topk_ids, topk_w, k, E, nullptr, hs, w2_s, y_s, y, 0, s);
        const int st = launch_status();
        if (st == K3_OK) {
            record_dispatch(K3_OP_MOE_BLOCK, variant);
            record_dispatch(K3_OP_EXPERT_ENGINE, engine);
        }
        return st;
    }
    bool permuted = false;  // the selection kernel wrote the expert lists too
    if (variant == K3_VARIANT_DOT2) {
        // 1. router, latent and shared gate/up rows in one pass over x
        launch_rls(x, ldx, b, d, w_router, bias, E, logits, w_lat, d_lat, z, ldz, w13_s, I_s, hs,
                   s);
        trace_end(K3_OP_MOE_BLOCK, s);
        // 2. top-k (and, above one token, the permutation) in workgroup 0,
        //    the shared down projection in the others
        const int grid = dot2_grid(0);
        const size_t lds = (size_t)b * I_s * sizeof(uint16_t);
        const int cb = I_s > 2048 ? 16 : (I_s > 512 ? 4 : 1);
        permuted = b > 1;
        const PermuteOut po = permute_out(moe_workspace_layout(b, E, k, I, d), ws + L.moe);
#define K3_TSD(TM_, CB_)                                                                       \
    k_topk_shared_down<TM_, CB_><<<grid, kBlock, lds, s>>>(logits, E, k, b, topk_ids, topk_w, \
                                                           hs, I_s, w2_s, d, y_s, permuted, po)
        if (b == 1 && cb == 16)
            K3_TSD(1, 16);
        else if (b == 1 && cb == 4)
            K3_TSD(1, 4);
        else if (b == 1)
            K3_TSD(1, 1);
        else if (cb == 16)
            K3_TSD(kDot2MaxTokens, 16);
        else if (cb == 4)
            K3_TSD(kDot2MaxTokens, 4);
        else
            K3_TSD(kDot2MaxTokens, 1);
#undef K3_TSD
    } else {
        // router, latent and shared gate/up rows in one split-K pass over x;
        // the shared down projection follows the selection
        float *part = (float *)(ws + L.part);
        sk_router_latent_shared(x, ldx, b, d, w_router, E, bias, k, logits, topk_ids, topk_w,
                                w_lat, d_lat, z, ldz, w13_s, I_s, hs, part, s);
        trace_end(K3_OP_MOE_BLOCK, s);
        // the shared down projection rides in the routed down launch of the
        // heavy experts when it has their shape; else it runs on its own
        if (b > kDot2MaxTokens && I_s == I) {
            const DownExtra ex{w2_s, hs, I_s, b, y_s};
            run_moe_experts(z, ldz, b, d_lat, topk_ids, topk_w, k, w13, w2, E, I, d, y_s, nullptr,
                            y, 0, ws + L.moe, K3_OP_MOE_EXPERTS, s, engine, &ex);
            const int st = launch_status();
            if (st == K3_OK) {
                record_dispatch(K3_OP_MOE_BLOCK, variant);
                record_dispatch(K3_OP_EXPERT_ENGINE, engine);
            }
            return st;
        }
        sk_proj_f32_direct(hs, I_s, b, w2_s, d, I_s, y_s, d, 0, s);
    }
    // 3-4. routed gate/up, down and combine with the shared output added
    run_moe_experts(z, ldz, b, d_lat, topk_ids, topk_w, k, w13, w2, E, I, d, y_s, nullptr, y, 0,
                    ws + L.moe, K3_OP_MOE_EXPERTS, s, engine, nullptr, permuted);
    const int st = launch_status();
    if (st == K3_OK) {
        record_dispatch(K3_OP_MOE_BLOCK, variant);
        record_dispatch(K3_OP_EXPERT_ENGINE, engine);
    }
    return st;
}

extern "C" int k3_moe_block(const uint16_t *x, int64_t ldx, int b, int d,
                            const uint16_t *w_router, const float *bias, int E, int k,
                            const uint16_t *w_lat, int d_lat, const uint16_t *w13,
                            const uint16_t *w2, int I, const uint16_t *w13_s,
                            const uint16_t *w2_s, int I_s, int32_t *topk_ids, float *topk_w,
                            uint16_t *z, int64_t ldz, float *y_s, uint16_t *y, void *workspace,
                            size_t ws_bytes, void *stream) {
    if (!x)
        return K3_ERR_INVALID_ARG;
    return moe_block_run(x, ldx, nullptr, b, d, w_router, bias, E, k, w_lat, d_lat, w13, w2, I,
                         w13_s, w2_s, I_s, topk_ids, topk_w, z, ldz, y_s, y, workspace, ws_bytes,
                         stream);
}

extern "C" size_t k3_moe_block_rmsnorm_workspace_size(int b, int d, int E, int k, int d_lat,
                                                      int I, int I_s) {
    const size_t w = k3_moe_block_workspace_size(b, d, E, k, d_lat, I, I_s);
    return w ? w + align_up((size_t)b * d * sizeof(uint16_t), 256) : 0;
}

extern "C" int k3_moe_block_rmsnorm(const float *h32, int b, int d, const uint16_t *gamma,
                                    float eps, uint16_t *x_out, const uint16_t *w_router,
                                    const float *bias, int E, int k, const uint16_t *w_lat,
                                    int d_lat, const uint16_t *w13, const uint16_t *w2, int I,
                                    const uint16_t *w13_s, const uint16_t *w2_s, int I_s,
                                    int32_t *topk_ids, float *topk_w, uint16_t *z, int64_t ldz,
                                    float *y_s, uint16_t *y, void *workspace, size_t ws_bytes,
                                    void *stream) {
    const NormIn nin{h32, gamma, eps, x_out};
    return moe_block_run(nullptr, d, &nin, b, d, w_router, bias, E, k, w_lat, d_lat, w13, w2, I,
                         w13_s, w2_s, I_s, topk_ids, topk_w, z, ldz, y_s, y, workspace, ws_bytes,
                         stream);
}
