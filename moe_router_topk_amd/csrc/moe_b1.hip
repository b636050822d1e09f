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
// At batch 1 the slots are the experts (k distinct ids). A unit of work is 28
// 16-byte vectors per lane (28 KB per wave); with two unit buffers in each of
// four waves, about 224 KB of weights are in flight per compute unit, which
// is what HBM3E needs to approach its streaming rate.
constexpr int kUpRow = 14;                   // vectors per lane of a gate/up row
constexpr int kSdRow = 4;                    // vectors per lane of a shared down row
constexpr int kSdRows = 2 * kUpRow / kSdRow; // shared down rows per unit
constexpr int kUpNB = 2 * kUpRow;
constexpr int kUpMaxD = kUpRow * kWave * 8;  // 7168
constexpr int kSdMaxI = kSdRow * kWave * 8;  // 2048

// Copy n 16-byte vectors into LDS, vector i from src(i); eight loads per
// thread go out before their stores.
template <class Src>
__device__ __forceinline__ void stage_flat(u32x4 *dst, int n, Src src) {
    for (int i0 = threadIdx.x; i0 < n; i0 += 8 * kBlock) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * kBlock;
            if (i < n)
                v[u] = ld_act16(src(i));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * kBlock;
            if (i < n)
                dst[i] = v[u];
        }
    }
}

// Routed gate/up at batch 1, optionally with the expert selection and the
// shared expert's down projection folded in. Every wave walks its even share
// of the shared down rows (chunks of kSdRows rows of w2s, y_s[r] = w2s[r] . hs)
// and then its even share of the (slot, column) pairs: pair (a, j) streams
// gate row j and up row I + j of w13[ids[a]] as one unit and writes
// hbuf[a][j] = bf16(silu(gate . z) * (up . z)). With TOPK, wave 0 of every
// workgroup selects the experts from the router logits while its first
// (shared) unit is in flight; workgroup 0 publishes ids and weights. Without
// TOPK the ids come from ids_in and slots outside [0, E) are skipped.
template <bool TOPK>
__global__ void __launch_bounds__(kBlock)
k_moe_up_b1(const uint16_t *__restrict__ z, int d, const uint16_t *__restrict__ w13, int I,
            int E, int k, const int32_t *__restrict__ ids_in, const float *__restrict__ logits,
            int32_t *__restrict__ ids_out, float *__restrict__ w_out,
            const uint16_t *__restrict__ hs, int Is, const uint16_t *__restrict__ w2s, int d_s,
            float *__restrict__ y_s, uint16_t *__restrict__ hbuf) {
    extern __shared__ u32x4 lds[];  // z (nv vectors), then hs (nvs vectors)
    __shared__ int sid[K3_MAX_TOPK];
    __shared__ float swt[K3_MAX_TOPK];
    const int nv = d >> 3, nvs = w2s ? Is >> 3 : 0;
    const u32x4 *zs = lds, *hss = lds + nv;
    const int lane = threadIdx.x & (kWave - 1), wq = wave_in_block();
    const int waves = gridDim.x * (kBlock / kWave);
    const int wave = blockIdx.x * (kBlock / kWave) + wq;
    const int n_sc = w2s ? (d_s + kSdRows - 1) / kSdRows : 0;
    int c0, c1, p0, p1;
    split_range(n_sc, waves, wave, c0, c1);
    split_range(k * I, waves, wave, p0, p1);
    const int ns = c1 - c0;  // units [0, ns) are shared chunks, then pairs p0, p0 + 1, ...
    float lv[kTopkPer];
    if (TOPK) {
        if (wq == 0)
            topk_load(logits, E, lv);  // issued ahead of the first weight loads
    } else {
        if (threadIdx.x < k) {
            const int e = ids_in[threadIdx.x];
            sid[threadIdx.x] = (e >= 0 && e < E) ? e : -1;
        }
        __syncthreads();
    }
    stream_units<kUpNB>(
        0, ns + p1 - p0,
        [&](u32x4 (&buf)[kUpNB], int u) {
            if (u < ns) {
                // rows r0 .. r0 + kSdRows - 1 of w2s as one range
                const int r0 = (c0 + u) * kSdRows;
                const int nr = min(kSdRows, d_s - r0);
                const rsrc_t rs = weight_range(w2s + (int64_t)r0 * Is, (uint32_t)nr * Is * 2);
#pragma unroll
                for (int i = 0; i < kSdRows; ++i)
#pragma unroll
                    for (int c = 0; c < kSdRow; ++c) {
                        const int v = c * kWave + lane;
                        buf[i * kSdRow + c] = ld_weight16(
                            rs, v < nvs ? (uint32_t)(i * Is + v * 8) * 2 : kOffNone);
                    }
            } else {
                const int p = p0 + u - ns, a = p / I, j = p - a * I;
                const int e = __builtin_amdgcn_readfirstlane(sid[a]);
                const uint32_t bytes = e >= 0 ? (uint32_t)d * 2 : 0u;
                const uint16_t *g = w13 + ((int64_t)(e < 0 ? 0 : e) * 2 * I + j) * d;
                const rsrc_t rg = weight_range(g, bytes);
                const rsrc_t ru = weight_range(g + (int64_t)I * d, bytes);
#pragma unroll
                for (int c = 0; c < kUpRow; ++c) {
                    const uint32_t off = (uint32_t)(c * kWave + lane) * 16;
                    buf[c] = ld_weight16(rg, off);
                    buf[kUpRow + c] = ld_weight16(ru, off);
                }
            }
        },
        [&](u32x4 (&buf)[kUpNB], int u) {
            if (u < ns) {
                const int r0 = (c0 + u) * kSdRows;
                float acc[kSdRows];
#pragma unroll
                for (int i = 0; i < kSdRows; ++i) {
                    acc[i] = 0.0f;
#pragma unroll
                    for (int c = 0; c < kSdRow; ++c) {
                        const int v = c * kWave + lane;
                        if (v < nvs)
                            acc[i] = dot8(buf[i * kSdRow + c], hss[v], acc[i]);
                    }
                }
#pragma unroll
                for (int i = 0; i < kSdRows; ++i) {
                    const float sum = wave_sum(acc[i]);
                    if (lane == 0 && r0 + i < d_s)
                        y_s[r0 + i] = sum;
                }
            } else {
                const int p = p0 + u - ns, a = p / I, j = p - a * I;
                float g = 0.0f, v_up = 0.0f;
#pragma unroll
                for (int c = 0; c < kUpRow; ++c) {
                    const int v = c * kWave + lane;
                    if (v < nv) {
                        const u32x4 x = zs[v];
                        g = dot8(buf[c], x, g);
                        v_up = dot8(buf[kUpRow + c], x, v_up);
                    }
                }
                g = wave_sum(g);
                v_up = wave_sum(v_up);
                if (lane == 0 && sid[a] >= 0)
                    hbuf[(int64_t)a * I + j] = f32_to_bf16(silu(g) * v_up);
            }
        },
        [&]() {
            // wave 0 selects first: it waits for the logits only, not for
            // the weight and staging loads issued after them
            if (TOPK && wq == 0) {
                uint32_t key[kTopkPer];
                topk_keys(lv, E, key);
                topk_select(key, k, sid, swt);
                if (blockIdx.x == 0 && lane < k) {
                    ids_out[lane] = sid[lane];
                    w_out[lane] = swt[lane];
                }
            }
            stage_flat(lds, nv + nvs, [&](int i) {
                return i < nv ? z + (int64_t)i * 8 : hs + (int64_t)(i - nv) * 8;
            });
            __syncthreads();
        },
        !TOPK || ns > 0);
}

// Down projection at batch 1 with the weighted combine folded in, on the
// 8-row engine (k3_gemv.h). Workgroup g owns an even share of the output
// rows; its groups are (slot j, 8 consecutive rows of w2[ids[j]]), slot-major,
// and every wave streams its K-quarter of each. Once all partial sums are in
// LDS, y[r] = bf16(y_add[r] + sum_j w_j o_j[r]) in slot order. The h rows of
// all k slots sit in LDS. Slots with an id outside [0, E) read no weights and
// are skipped in the sum.
template <int U>
__global__ void __launch_bounds__(kBlock)
k_down_b1(const uint16_t *__restrict__ hbuf, int I, const uint16_t *__restrict__ w2, int d_out,
          const int32_t *__restrict__ ids, const float *__restrict__ topk_w, int k, int E,
          const float *__restrict__ y_add, uint16_t *__restrict__ y, int ps_stride) {
    extern __shared__ u32x4 hs[];  // k rows of h, then ps[4][ps_stride], then y_add[rows]
    __shared__ float sw[K3_MAX_TOPK];
    __shared__ int sv[K3_MAX_TOPK];
    const int nv = I >> 3;
    float *ps = reinterpret_cast<float *>(hs + k * nv);
    float *ya = ps + 4 * ps_stride;
    int rb0, rb1;
    split_range(d_out, gridDim.x, blockIdx.x, rb0, rb1);
    const int rows = rb1 - rb0, gps = (rows + 7) >> 3;
    gemv8_stream<U>(
        k * gps, I,
        [&](int g, const uint16_t *&base, int &nr, int &skip) {
            const int j = g / gps, gg = g - j * gps;
            const int e = ld_scalar(ids + j);  // the same in every lane
            const bool ok = e >= 0 && e < E;
            base = w2 + (ok ? (int64_t)e * d_out * I : 0) + (int64_t)(rb0 + 8 * gg) * I;
            nr = ok ? min(8, rows - 8 * gg) : 0;
            skip = 0;
        },
        [&](int g, int kv) { return hs[min(g / gps, k - 1) * nv + kv]; }, ps, ps_stride,
        [&]() {
            stage_rows(hs, nv, k, nv, [&](int j) { return hbuf + (int64_t)j * I; });
            for (int i = threadIdx.x; i < rows; i += kBlock)
                ya[i] = y_add ? y_add[rb0 + i] : 0.0f;
            if (threadIdx.x < k) {
                const int e = ids[threadIdx.x];
                sv[threadIdx.x] = e >= 0 && e < E;
                sw[threadIdx.x] = topk_w[threadIdx.x];
            }
            __syncthreads();
        });
    for (int i = threadIdx.x; i < rows; i += kBlock) {
        float acc = ya[i];
        for (int j = 0; j < k; ++j)
            if (sv[j])
                acc += sw[j] * gv_total(ps, ps_stride, 8 * j * gps + i);
        y[rb0 + i] = f32_to_bf16(acc);
    }
}

// ------------------------------------------------------------------ launchers
static int down_b1_grid(int d_out, int cu_budget) { return budget_grid(d_out, cu_budget, 2); }

// LDS of the down kernel: k rows of h, the partial sums, y_add of the share.
static size_t down_b1_lds(int k, int I, int d_out, int grid, int &ps_stride) {
    const int rows = (d_out + grid - 1) / grid;
    ps_stride = 8 * k * ((rows + 7) / 8);
    return (size_t)k * I * sizeof(uint16_t) + ((size_t)4 * ps_stride + rows) * sizeof(float);
}

bool down_b1_fits(int k, int I, int d_out, int cu_budget) {
    int ps_stride;
    return I <= 2048 && I % 64 == 0 &&
           down_b1_lds(k, I, d_out, down_b1_grid(d_out, cu_budget), ps_stride) <= 65536;
}

void launch_down_b1(const uint16_t *hbuf, int I, const uint16_t *w2, int d_out,
                    const int32_t *ids, const float *wts, int k, int E, const float *y_add,
                    uint16_t *y, int cu_budget, hipStream_t s) {
    const int grid = down_b1_grid(d_out, cu_budget);
    int ps_stride;
    const size_t lds = down_b1_lds(k, I, d_out, grid, ps_stride);
    if (gv_unit_pieces(I) == 7)
        k_down_b1<7><<<grid, kBlock, lds, s>>>(hbuf, I, w2, d_out, ids, wts, k, E, y_add, y,
                                              ps_stride);
    else
        k_down_b1<8><<<grid, kBlock, lds, s>>>(hbuf, I, w2, d_out, ids, wts, k, E, y_add, y,
                                              ps_stride);
}

// The fused batch-1 gate/up kernel: d <= 7168 and, with the shared down
// projection folded in, I_s <= 2048; one workgroup per compute unit (its two
// 28-vector buffers leave no room for a second).
bool up_b1_fits(int d, int Is) { return d <= kUpMaxD && Is <= kSdMaxI; }

void launch_up_b1(bool topk, const uint16_t *z, int d, const uint16_t *w13, int I, int E, int k,
                  const int32_t *ids_in, const float *logits, int32_t *ids_out, float *w_out,
                  const uint16_t *hs, int Is, const uint16_t *w2s, int d_s, float *y_s,
                  uint16_t *hbuf, int cu_budget, hipStream_t s) {
    const int grid = budget_grid(1 << 30, cu_budget, 1);
    const size_t lds = ((size_t)d + (w2s ? (size_t)Is : 0)) * sizeof(uint16_t);
    if (topk)
        k_moe_up_b1<true><<<grid, kBlock, lds, s>>>(z, d, w13, I, E, k, nullptr, logits, ids_out,
                                                    w_out, hs, Is, w2s, d_s, y_s, hbuf);
    else
        k_moe_up_b1<false><<<grid, kBlock, lds, s>>>(z, d, w13, I, E, k, ids_in, nullptr,
                                                     nullptr, nullptr, hs, Is, w2s, d_s, y_s,
                                                     hbuf);
}


}  // namespace k3
