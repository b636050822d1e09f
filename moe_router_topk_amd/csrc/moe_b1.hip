// moe_b1.hip -- the routed experts at batch 1, where the slots are the
// experts (k distinct ids) and no permutation is needed.
//
// "Hyper Optimizing Kimi K3 in vLLM", Part 1 section 3 ("Improve MoE
// scheduling and overlap"): the routed experts follow the router and the
// latent projection; the shared expert's work fills the gap the routing
// leaves. Here the shared expert's rows ride in the passes of the routed
// ones (its gate/up rows at the head of the routed gate/up kernel, streaming
// while the selection waits for the router's logits; its down rows as one
// more slot of the routed down kernel), and the expert selection itself
// runs while the routed weights stream: each pick is made just before its
// expert's rows are needed.
#include <math.h>

#include "k3_device.h"
#include "k3_gemv.h"
#include "k3_internal.h"

namespace k3 {

// ------------------------------------------------------------------ batch-1 kernels
// Both kernels run on the 8-row engine of k3_gemv.h. At batch 1 the slots are
// the experts (k distinct ids).

// The batch-1 routed h: h[a][j] (slot a, column j) sits at hbuf[((j / 4) k
// + a) 4 + j % 4], i.e. [column block][slot][4]. The gate/up kernel's
// workgroups own column blocks of every slot, so each writes one contiguous
// piece; the down kernel gathers the 8-byte pieces into its LDS rows.
__device__ __forceinline__ int64_t hb1_index(int a, int j, int k) {
    return ((int64_t)(j >> 2) * k + a) * 4 + (j & 3);
}

// Routed gate/up at batch 1, optionally with the expert selection folded in.
// A group is (slot a, columns 4c .. 4c + 3): the gate rows 4c .. 4c + 3 and
// the up rows I + 4c .. I + 4c + 3 of w13[ids[a]], so one group holds both
// halves of its four outputs: h[a][j] = bf16(silu(gate . z) * (up . z)).
// Workgroup w takes the same column blocks (an even share of the I / 4) of
// every slot, slot 0 first. With TOPK every wave picks the experts itself
// from the router logits, one pick just before it first needs that slot's
// expert: the first weight loads wait for one pick only, and the later picks
// run while earlier loads are in flight (workgroup 0 publishes ids and
// weights). Without TOPK the ids come from ids_in and slots outside [0, E)
// are skipped. With w13s the shared expert's gate/up rows (input xs, the
// block's x, d wide like z) come first as one more slot: its rows stream
// while the selection waits for the logits, and hs[j] = bf16(silu(gate) *
// up) in the router pass's order and rounding.
template <bool TOPK, int U>
__global__ void __launch_bounds__(kBlock)
k_moe_up_b1(const uint16_t *__restrict__ z, int d, const uint16_t *__restrict__ w13, int I,
            int E, int k, const int32_t *__restrict__ ids_in, const float *__restrict__ logits,
            int32_t *__restrict__ ids_out, float *__restrict__ w_out,
            uint16_t *__restrict__ hbuf, int ps_stride, const uint16_t *__restrict__ xs,
            const uint16_t *__restrict__ w13s, uint16_t *__restrict__ hs) {
    extern __shared__ u32x4 zs[];  // z (d / 8 vectors), x with w13s, then ps[4][ps_stride]
    const int nv = d >> 3;
    const int sh = w13s ? 1 : 0;  // the shared slot comes first
    float *ps = reinterpret_cast<float *>(zs + (1 + sh) * nv);
    const int gpe = I >> 2;  // column blocks (groups) per slot
    int c0, c1;
    split_range(gpe, gridDim.x, blockIdx.x, c0, c1);
    const int cps = c1 - c0;  // this workgroup's groups per slot
    const int gsh = sh * cps;  // the shared slot's groups
    // the expert of the slot the stream is on (slots come in order)
    TopkPicker pk;
    float lv[kTopkPer];
    int cur_a = -1, cur_e = -1;
    auto slot_expert = [&](int a) {
        while (cur_a < a) {
            ++cur_a;
            if (TOPK) {
                cur_e = pk.next();
            } else {
                const int e = ld_scalar(ids_in + cur_a);
                cur_e = (e >= 0 && e < E) ? e : -1;
            }
        }
        return cur_e;
    };
    GvStage<4> zst, xst;  // d <= 8192
    gemv8_stream<U>(
        gsh + k * cps, d,
        [&](int g, const uint16_t *&base, int &nr, int &skip) {
            skip = I - 4;
            if (g < gsh) {
                base = w13s + (int64_t)(4 * (c0 + g)) * d;
                nr = 8;
                return;
            }
            const int gr = g - gsh, a = gr / cps, c = c0 + (gr - a * cps);
            const int e = slot_expert(a);
            base = w13 + ((int64_t)(e < 0 ? 0 : e) * 2 * I + 4 * c) * d;
            nr = e >= 0 ? 8 : 0;
        },
        [&](int g, int kv, int) { return zs[(g < gsh ? nv : 0) + kv]; }, ps, ps_stride,
        [&]() {
            // the logits first: the first pick waits for them, not for z
            if (TOPK) {
                topk_load(logits, E, lv);
                pk.init(E);
            }
            zst.load(z, nv);
            if (sh) {
                xst.load(xs, nv);
            } else if (TOPK) {
                topk_keys(lv, E, pk.key);
            }
        },
        [&]() {
            // with the shared slot first the first weight loads are out
            // before the selection waits for the logits
            if (TOPK && sh)
                topk_keys(lv, E, pk.key);
            zst.store(zs, nv);
            if (sh)
                xst.store(zs + nv, nv);
            __syncthreads();
        });
    for (int i = threadIdx.x; i < 8 * gsh; i += kBlock) {
        const int r = i & 7, j = 4 * (c0 + (i >> 3)) + r;
        if (r < 4)
            hs[j] = f32_to_bf16(silu(gv_total(ps, ps_stride, i)) * gv_total(ps, ps_stride, i + 4));
    }
    for (int q = threadIdx.x; q < 8 * k * cps; q += kBlock) {
        const int i = 8 * gsh + q;
        const int r = q & 7, g = q >> 3, a = g / cps, j = 4 * (c0 + g - a * cps) + r;
        bool ok = true;
        if (!TOPK) {
            const int e = ids_in[a];
            ok = e >= 0 && e < E;
        }
        if (r < 4 && ok)
            hbuf[hb1_index(a, j, k)] =
                f32_to_bf16(silu(gv_total(ps, ps_stride, i)) * gv_total(ps, ps_stride, i + 4));
    }
    if (TOPK && blockIdx.x == 0 && threadIdx.x < kWave) {
        while (pk.n < k)
            pk.next();
        pk.finish(k, ids_out, w_out);
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
    // the slots' h rows: the k routed rows are gathered from hbuf's 8-byte
    // pieces (loaded before the first weight loads when they fit), the shared
    // one is hs
    const int npc = 2 * k * nv;  // 8-byte pieces of the routed rows
    const bool early = npc <= 16 * kBlock && nv <= kBlock;
    uint2 hp[16];
    GvStage<1> ss;
    int e_ld = 0;
    float w_ld = 0.0f;
    uint2 *hl8 = reinterpret_cast<uint2 *>(hl);
    // piece p = (column block c, slot a) goes to half c % 2 of LDS vector (a, c / 2)
    auto put = [&](int p, uint2 v) {
        const int c = p / k, a = p - c * k;
        hl8[(a * nv + (c >> 1)) * 2 + (c & 1)] = v;
    };
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
                const rsrc_t r = act_range(uniform_ptr(hbuf));
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int p = threadIdx.x + q * kBlock;
                    // past npc: the sign bit of npc - 1 - p (arithmetic, no branch)
                    hp[q] = ld_act8(r, ((uint32_t)p * 8u) | ((uint32_t)(npc - 1 - p) & 0x80000000u));
                }
                if (w2s)
                    ss.load(hs, nv);
            }
            if (y_add && rows <= kBlock)
                yv = y_add[rb0 + min((int)threadIdx.x, rows - 1)];
            // the slots' ids and weights too (clamped, unconditional loads)
            const int ti = min((int)threadIdx.x, k - 1);
            e_ld = ids[ti];
            w_ld = topk_w[ti];
        },
        [&]() {
            if (early) {
#pragma unroll
                for (int q = 0; q < 16; ++q) {
                    const int p = threadIdx.x + q * kBlock;
                    if (p < npc)
                        put(p, hp[q]);
                }
                if (w2s)
                    ss.store(hl + k * nv, nv);
            } else {
                const uint2 *h8 = reinterpret_cast<const uint2 *>(hbuf);
                for (int p = threadIdx.x; p < npc; p += kBlock)
                    put(p, h8[p]);
                if (w2s)
                    for (int i = threadIdx.x; i < nv; i += kBlock)
                        hl[k * nv + i] = ld_act16(hs + 8 * i);
            }
            if (rows <= kBlock) {
                if ((int)threadIdx.x < rows)
                    ya[threadIdx.x] = yv;
            } else {
                for (int i = threadIdx.x; i < rows; i += kBlock)
                    ya[i] = y_add ? y_add[rb0 + i] : 0.0f;
            }
            if (threadIdx.x < k) {
                sv[threadIdx.x] = e_ld >= 0 && e_ld < E;
                sw[threadIdx.x] = w_ld;
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

// LDS of the gate/up kernel: z (and x with the shared slot), then the
// partial sums of the share (the slots x the workgroup's column blocks).
static size_t up_b1_lds(int d, int k, int I, int grid, int &ps_stride, bool shared) {
    const int ns = k + (shared ? 1 : 0);
    ps_stride = 8 * ns * ((I / 4 + grid - 1) / grid);
    return (size_t)(shared ? 2 : 1) * d * sizeof(uint16_t) + (size_t)4 * ps_stride * sizeof(float);
}

// One workgroup per column block of I / 4 at most, two per compute unit.
static int up_b1_grid(int I, int cu_budget) { return budget_grid(I / 4, cu_budget, 2); }

bool up_b1_fits(int d, int k, int I, int cu_budget, bool shared) {
    int ps_stride;
    return d % 64 == 0 && d <= 8192 && I % 4 == 0 && I >= 4 &&
           up_b1_lds(d, k, I, up_b1_grid(I, cu_budget), ps_stride, shared) <= 65536;
}

void launch_up_b1(bool topk, const uint16_t *z, int d, const uint16_t *w13, int I, int E, int k,
                  const int32_t *ids_in, const float *logits, int32_t *ids_out, float *w_out,
                  uint16_t *hbuf, int cu_budget, hipStream_t s, const uint16_t *xs,
                  const uint16_t *w13s, uint16_t *hs) {
    const int grid = up_b1_grid(I, cu_budget);
    int ps_stride;
    const size_t lds = up_b1_lds(d, k, I, grid, ps_stride, w13s != nullptr);
#define K3_UP(T_, U_)                                                                          \
    k_moe_up_b1<T_, U_><<<grid, kBlock, lds, s>>>(z, d, w13, I, E, k, ids_in, logits, ids_out, \
                                                 w_out, hbuf, ps_stride, xs, w13s, hs)
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
