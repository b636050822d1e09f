// moe_b1.hip -- the routed experts at batch 1, where the slots are the
// experts (k distinct ids) and no permutation is needed.
//
// "Hyper Optimizing Kimi K3 in vLLM", Part 1 section 3 ("Improve MoE
// scheduling and overlap"): the routed experts follow the router and the
// latent projection; the shared expert's work fills the gap the routing
// leaves. Here that gap is the expert selection itself: every workgroup of
// the gate/up kernel selects the experts while its first units -- rows of
// the shared expert's down projection -- are in flight.
#include <math.h>

#include "k3_device.h"
#include "k3_gemv.h"
#include "k3_internal.h"

namespace k3 {

// ------------------------------------------------------------------ batch-1 kernels
// Both kernels run on the 8-row engine of k3_gemv.h. At batch 1 the slots are
// the experts (k distinct ids).

// Routed gate/up at batch 1, optionally with the expert selection folded in.
// The groups are (slot a, columns j0 .. j0 + 3): the gate rows j0 .. j0 + 3
// and the up rows I + j0 .. I + j0 + 3 of w13[ids[a]], so one group holds
// both halves of its four outputs: hbuf[a][j] = bf16(silu(gate . z) *
// (up . z)). With TOPK, wave 0 of every workgroup selects the experts from
// the router logits while all threads stage z (workgroup 0 publishes ids and
// weights); without it the ids come from ids_in and slots outside [0, E)
// are skipped.
template <bool TOPK, int U>
__global__ void __launch_bounds__(kBlock)
k_moe_up_b1(const uint16_t *__restrict__ z, int d, const uint16_t *__restrict__ w13, int I,
            int E, int k, const int32_t *__restrict__ ids_in, const float *__restrict__ logits,
            int32_t *__restrict__ ids_out, float *__restrict__ w_out,
            uint16_t *__restrict__ hbuf, int ps_stride) {
    extern __shared__ u32x4 zs[];  // z (d / 8 vectors), then ps[4][ps_stride]
    __shared__ int sid[K3_MAX_TOPK];
    __shared__ float swt[K3_MAX_TOPK];
    const int nv = d >> 3;
    float *ps = reinterpret_cast<float *>(zs + nv);
    const int lane = threadIdx.x & (kWave - 1), wq = wave_in_block();
    // wave 0 issues the logit loads, then every wave its z loads; the
    // selection waits for the logits only and z arrives meanwhile
    float lv[kTopkPer];
    if (TOPK && wq == 0)
        topk_load(logits, E, lv);
    GvStage<4> zst;  // d <= 8192
    zst.load(z, nv);
    if (TOPK) {
        if (wq == 0) {
            uint32_t key[kTopkPer];
            topk_keys(lv, E, key);
            topk_select(key, k, sid, swt, E);
            if (blockIdx.x == 0 && lane < k) {
                ids_out[lane] = sid[lane];
                w_out[lane] = swt[lane];
            }
        }
    } else if (threadIdx.x < k) {
        const int e = ids_in[threadIdx.x];
        sid[threadIdx.x] = (e >= 0 && e < E) ? e : -1;
    }
    zst.store(zs, nv);
    __syncthreads();
    const int gpe = I >> 2;  // groups per expert
    int g0, g1;
    split_range(k * gpe, gridDim.x, blockIdx.x, g0, g1);
    gemv8_stream<U>(
        g1 - g0, d,
        [&](int g, const uint16_t *&base, int &nr, int &skip) {
            const int vg = g0 + g, a = vg / gpe, j0 = 4 * (vg - a * gpe);
            const int e = __builtin_amdgcn_readfirstlane(sid[a]);
            base = w13 + ((int64_t)(e < 0 ? 0 : e) * 2 * I + j0) * d;
            nr = e >= 0 ? 8 : 0;
            skip = I - 4;
        },
        [&](int, int kv, int) { return zs[kv]; }, ps, ps_stride, [&]() {}, [&]() {});
    for (int i = threadIdx.x; i < 8 * (g1 - g0); i += kBlock) {
        const int r = i & 7, vg = g0 + (i >> 3), a = vg / gpe, j = 4 * (vg - a * gpe) + r;
        if (r < 4 && sid[a] >= 0)
            hbuf[(int64_t)a * I + j] =
                f32_to_bf16(silu(gv_total(ps, ps_stride, i)) * gv_total(ps, ps_stride, i + 4));
    }
}

// Down projection at batch 1 with the weighted combine folded in. Workgroup
// g owns an even share of the output rows; its groups are (slot j, 8
// consecutive rows of w2[ids[j]]), slot-major, and every wave streams its
// K-quarter of each. With w2s the shared expert's down rows are one more
// slot (its h row hs): y_s[r] = its sum. Once all partial sums are in LDS,
// y[r] = bf16(base[r] + sum_j w_j o_j[r]) in slot order, base = y_s[r] with
// the shared slot, else y_add[r] (or 0). The h rows sit in LDS. Slots with an
// id outside [0, E) read no weights and are skipped in the sum.
template <int U>
__global__ void __launch_bounds__(kBlock)
k_down_b1(const uint16_t *__restrict__ hbuf, int I, const uint16_t *__restrict__ w2, int d_out,
          const int32_t *__restrict__ ids, const float *__restrict__ topk_w, int k, int E,
          const float *__restrict__ y_add, const uint16_t *__restrict__ hs,
          const uint16_t *__restrict__ w2s, float *__restrict__ y_s, uint16_t *__restrict__ y,
          int ps_stride) {
    extern __shared__ u32x4 hl[];  // the slots' h rows, then ps[4][ps_stride], then y_add
    __shared__ float sw[K3_MAX_TOPK];
    __shared__ int sv[K3_MAX_TOPK];
    const int nv = I >> 3;
    const int ns = k + (w2s ? 1 : 0);  // slots
    float *ps = reinterpret_cast<float *>(hl + ns * nv);
    float *ya = ps + 4 * ps_stride;
    int rb0, rb1;
    split_range(d_out, gridDim.x, blockIdx.x, rb0, rb1);
    const int rows = rb1 - rb0, gps = (rows + 7) >> 3;
    // the slots' h rows: the k routed rows are contiguous in hbuf (staged in
    // registers before the first weight loads when they fit), the shared one
    // is hs
    const bool early = k * nv <= 8 * kBlock && nv <= kBlock;
    GvStage<8> sr;
    GvStage<1> ss;
    float yv = 0.0f;
    gemv8_stream<U>(
        ns * gps, I,
        [&](int g, const uint16_t *&base, int &nr, int &skip) {
            const int j = g / gps, gg = g - j * gps;
            skip = 0;
            if (j < k) {
                const int e = ld_scalar(ids + j);  // the same in every lane
                const bool ok = e >= 0 && e < E;
                base = w2 + (ok ? (int64_t)e * d_out * I : 0) + (int64_t)(rb0 + 8 * gg) * I;
                nr = ok ? min(8, rows - 8 * gg) : 0;
            } else {
                base = w2s + (int64_t)(rb0 + 8 * gg) * I;
                nr = min(8, rows - 8 * gg);
            }
        },
        [&](int g, int kv, int) { return hl[min(g / gps, ns - 1) * nv + kv]; }, ps, ps_stride,
        [&]() {
            if (early) {
                sr.load(hbuf, k * nv);
                if (w2s)
                    ss.load(hs, nv);
            }
            if (y_add && rows <= kBlock)
                yv = y_add[rb0 + min((int)threadIdx.x, rows - 1)];
        },
        [&]() {
            if (early) {
                sr.store(hl, k * nv);
                if (w2s)
                    ss.store(hl + k * nv, nv);
            } else {
                stage_rows(hl, nv, ns, nv,
                           [&](int j) { return j < k ? hbuf + (int64_t)j * I : hs; });
            }
            if (rows <= kBlock) {
                if ((int)threadIdx.x < rows)
                    ya[threadIdx.x] = yv;
            } else {
                for (int i = threadIdx.x; i < rows; i += kBlock)
                    ya[i] = y_add ? y_add[rb0 + i] : 0.0f;
            }
            if (threadIdx.x < k) {
                const int e = ids[threadIdx.x];
                sv[threadIdx.x] = e >= 0 && e < E;
                sw[threadIdx.x] = topk_w[threadIdx.x];
            }
            __syncthreads();
        });
    for (int i = threadIdx.x; i < rows; i += kBlock) {
        float acc = ya[i];
        if (w2s) {
            acc = gv_total(ps, ps_stride, 8 * k * gps + i);
            y_s[rb0 + i] = acc;
        }
        for (int j = 0; j < k; ++j)
            if (sv[j])
                acc += sw[j] * gv_total(ps, ps_stride, 8 * j * gps + i);
        y[rb0 + i] = f32_to_bf16(acc);
    }
}

// ------------------------------------------------------------------ launchers
static int down_b1_grid(int d_out, int cu_budget) { return budget_grid(d_out, cu_budget, 2); }

// LDS of the down kernel: the slots' h rows, the partial sums, y_add of the
// share.
static size_t down_b1_lds(int ns, int I, int d_out, int grid, int &ps_stride) {
    const int rows = (d_out + grid - 1) / grid;
    ps_stride = 8 * ns * ((rows + 7) / 8);
    return (size_t)ns * I * sizeof(uint16_t) + ((size_t)4 * ps_stride + rows) * sizeof(float);
}

bool down_b1_fits(int k, int I, int d_out, bool shared, int cu_budget) {
    int ps_stride;
    return I <= 2048 && I % 64 == 0 &&
           down_b1_lds(k + (shared ? 1 : 0), I, d_out, down_b1_grid(d_out, cu_budget),
                       ps_stride) <= 65536;
}

void launch_down_b1(const uint16_t *hbuf, int I, const uint16_t *w2, int d_out,
                    const int32_t *ids, const float *wts, int k, int E, const float *y_add,
                    const uint16_t *hs, const uint16_t *w2s, float *y_s, uint16_t *y,
                    int cu_budget, hipStream_t s) {
    const int grid = down_b1_grid(d_out, cu_budget);
    int ps_stride;
    const size_t lds = down_b1_lds(k + (w2s ? 1 : 0), I, d_out, grid, ps_stride);
    if (gv_unit_pieces(I) == 7)
        k_down_b1<7><<<grid, kBlock, lds, s>>>(hbuf, I, w2, d_out, ids, wts, k, E, y_add, hs, w2s,
                                              y_s, y, ps_stride);
    else
        k_down_b1<8><<<grid, kBlock, lds, s>>>(hbuf, I, w2, d_out, ids, wts, k, E, y_add, hs, w2s,
                                              y_s, y, ps_stride);
}

// LDS of the gate/up kernel: z, then the partial sums of the share.
static size_t up_b1_lds(int d, int k, int I, int grid, int &ps_stride) {
    const int groups = k * (I / 4);
    ps_stride = 8 * ((groups + grid - 1) / grid);
    return (size_t)d * sizeof(uint16_t) + (size_t)4 * ps_stride * sizeof(float);
}

bool up_b1_fits(int d, int k, int I, int cu_budget) {
    int ps_stride;
    const int grid = budget_grid(k * (I / 4), cu_budget, 2);
    return d % 64 == 0 && d <= 8192 && I % 4 == 0 &&
           up_b1_lds(d, k, I, grid, ps_stride) <= 65536;
}

void launch_up_b1(bool topk, const uint16_t *z, int d, const uint16_t *w13, int I, int E, int k,
                  const int32_t *ids_in, const float *logits, int32_t *ids_out, float *w_out,
                  uint16_t *hbuf, int cu_budget, hipStream_t s) {
    const int grid = budget_grid(k * (I / 4), cu_budget, 2);
    int ps_stride;
    const size_t lds = up_b1_lds(d, k, I, grid, ps_stride);
#define K3_UP(T_, U_)                                                                          \
    k_moe_up_b1<T_, U_><<<grid, kBlock, lds, s>>>(z, d, w13, I, E, k, ids_in, logits, ids_out, \
                                                 w_out, hbuf, ps_stride)
    if (topk && gv_unit_pieces(d) == 7)
        K3_UP(true, 7);
    else if (topk)
        K3_UP(true, 8);
    else if (gv_unit_pieces(d) == 7)
        K3_UP(false, 7);
    else
        K3_UP(false, 8);
#undef K3_UP
}

}  // namespace k3
