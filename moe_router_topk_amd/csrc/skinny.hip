// skinny.hip -- launchers of the MFMA engine (k3_skinny.h) for dense
// projections above batch 4, and the kernels that finish their outputs from
// the fp32 partial sums of the K ranges (always summed in range order).
#include <math.h>

#include "k3_device.h"
#include "k3_internal.h"
#include "k3_skinny.h"

namespace k3 {

// ------------------------------------------------------------------ finishing kernels
// Output column c of the reduce runs over the segments' outputs in order;
// segment s contributes cols[s] columns read from partial rows starting at
// rows_before[s]. SkOut modes:
//   BF16:   y[t][j]  = bf16(sum)                       (ldy)
//   F32:    y[t][j]  = sum (+ bias[j])                 (ldy), fp32
//   SWIGLU: h[t][j]  = bf16(silu(sum_gate j) * sum_up j), gate row j and up
//           row I + j of the segment (cols = I)
//   RESID:  v = r[t][j] + sum; r[t][j] = bf16(v) in place (y = r), h32[t][j] = v
struct SkOutSeg {
    int mode;  // 0 BF16, 1 F32, 2 SWIGLU, 3 RESID
    int cols;
    int rows_before;
    void *y;
    int64_t ldy;
    const float *bias;
    float *h32;
};
struct SkOuts {
    SkOutSeg s[3];
    int nseg;
    int cols_total;
};

// The K ranges' partials of element i, added in range order. Every range's
// load is issued up front (ranges past ks re-read range 0 and are not
// added), so the sum waits for one memory latency, not ks of them.
__device__ __forceinline__ float sk_sum(const float *part, int ks, int64_t stride, int64_t i) {
    float p[kSkMaxSplit];
#pragma unroll
    for (int r = 0; r < kSkMaxSplit; ++r)
        p[r] = part[i + (r < ks ? r : 0) * stride];
    float v = p[0];
#pragma unroll
    for (int r = 1; r < kSkMaxSplit; ++r)
        if (r < ks)
            v += p[r];
    return v;
}

// Segment s's descriptor, s differing between lanes. Each field is chosen
// among the three segments' copies, which are uniform (scalar loads of the
// kernel arguments): indexing O.s[s] directly made the compiler read the
// descriptor with vector loads from the argument buffer, one dependent
// memory round trip per field, before the partials' loads could go out.
__device__ __forceinline__ SkOutSeg sk_seg(const SkOuts &O, int s) {
    // readfirstlane keeps each copy a scalar value, so the compiler cannot
    // fold the choice back into a per-lane index into the arguments
    auto u32 = [](int v) { return __builtin_amdgcn_readfirstlane(v); };
    auto u64 = [](int64_t v) {
        const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
        const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
        return (int64_t)(((uint64_t)hi << 32) | lo);
    };
    SkOutSeg q;
    q.mode = s == 0 ? u32(O.s[0].mode) : (s == 1 ? u32(O.s[1].mode) : u32(O.s[2].mode));
    q.cols = s == 0 ? u32(O.s[0].cols) : (s == 1 ? u32(O.s[1].cols) : u32(O.s[2].cols));
    q.rows_before = s == 0 ? u32(O.s[0].rows_before)
                           : (s == 1 ? u32(O.s[1].rows_before) : u32(O.s[2].rows_before));
    q.y = s == 0 ? uniform_ptr(O.s[0].y) : (s == 1 ? uniform_ptr(O.s[1].y) : uniform_ptr(O.s[2].y));
    q.ldy = s == 0 ? u64(O.s[0].ldy) : (s == 1 ? u64(O.s[1].ldy) : u64(O.s[2].ldy));
    q.bias = s == 0 ? uniform_ptr(O.s[0].bias)
                    : (s == 1 ? uniform_ptr(O.s[1].bias) : uniform_ptr(O.s[2].bias));
    q.h32 = s == 0 ? uniform_ptr(O.s[0].h32)
                   : (s == 1 ? uniform_ptr(O.s[1].h32) : uniform_ptr(O.s[2].h32));
    return q;
}

__device__ __forceinline__ void sk_finish_one(const float *__restrict__ part, int ks, int T,
                                              int64_t ldp, const SkOuts &O, int64_t i) {
    const int t = (int)(i / O.cols_total);
    int c = (int)(i - (int64_t)t * O.cols_total);
    const int c0 = O.s[0].cols, c1 = O.s[1].cols;
    const int s = (O.nseg > 1 && c >= c0) ? ((O.nseg > 2 && c >= c0 + c1) ? 2 : 1) : 0;
    c -= (s >= 1 ? c0 : 0) + (s >= 2 ? c1 : 0);
    const SkOutSeg q = sk_seg(O, s);
    const int64_t stride = (int64_t)T * ldp;
    const int64_t base = (int64_t)t * ldp + q.rows_before;
    if (q.mode == 2) {
        const float g = sk_sum(part, ks, stride, base + c);
        const float u = sk_sum(part, ks, stride, base + q.cols + c);
        ((uint16_t *)q.y)[(int64_t)t * q.ldy + c] = f32_to_bf16(silu(g) * u);
    } else {
        const float v = sk_sum(part, ks, stride, base + c);
        const int64_t o = (int64_t)t * q.ldy + c;
        if (q.mode == 0) {
            ((uint16_t *)q.y)[o] = f32_to_bf16(v);
        } else if (q.mode == 1) {
            ((float *)q.y)[o] = q.bias ? v + q.bias[c] : v;
        } else {
            uint16_t *r = (uint16_t *)q.y;
            const float h = bf16_to_f32(r[o]) + v;
            r[o] = f32_to_bf16(h);
            q.h32[o] = h;
        }
    }
}

__global__ void __launch_bounds__(kBlock)
k_sk_finish(const float *__restrict__ part, int ks, int T, int64_t ldp, SkOuts O) {
    const int64_t n = (int64_t)T * O.cols_total;
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * kBlock)
        sk_finish_one(part, ks, T, ldp, O, i);
}

// The finish of a pass whose first segment is the router (fp32 logits, +
// bias) fused with the expert selection: workgroup t < T sums token t's
// logits (exactly as k_sk_finish does), writes them out, keeps them in LDS,
// and its first wave picks the token's experts from there (as the top-k
// kernel would from memory); the other workgroups finish every other column
// of every token. One launch instead of two.
__global__ void __launch_bounds__(kBlock)
k_sk_finish_topk(const float *__restrict__ part, int ks, int T, int64_t ldp, SkOuts O, int k,
                 int32_t *__restrict__ ids, float *__restrict__ wts) {
    const SkOutSeg &r = O.s[0];
    const int E = r.cols;
    if ((int)blockIdx.x < T) {
        __shared__ float lg[K3_MAX_EXPERTS];
        const int t = blockIdx.x;
        const int64_t stride = (int64_t)T * ldp;
        // every load of the token's logits (partials and bias) goes out
        // before the first sum, so the row waits for one memory latency
        constexpr int PER = K3_MAX_EXPERTS / kBlock;
        float v[PER], bv[PER];
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int c = threadIdx.x + j * kBlock;
            const int cc = c < E ? c : 0;
            v[j] = sk_sum(part, ks, stride, (int64_t)t * ldp + cc);
            bv[j] = r.bias ? r.bias[cc] : 0.0f;
        }
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int c = threadIdx.x + j * kBlock;
            if (c < E) {
                const float l = r.bias ? v[j] + bv[j] : v[j];
                ((float *)r.y)[(int64_t)t * r.ldy + c] = l;
                lg[c] = l;
            }
        }
        __syncthreads();
        if (threadIdx.x < kWave)
            topk_wave(lg, E, k, ids + (int64_t)t * k, wts + (int64_t)t * k);
        return;
    }
    const int rest = O.cols_total - E;
    const int64_t n = (int64_t)T * rest;
    for (int64_t i = (int64_t)(blockIdx.x - T) * kBlock + threadIdx.x; i < n;
         i += (int64_t)(gridDim.x - T) * kBlock) {
        const int t = (int)(i / rest);
        sk_finish_one(part, ks, T, ldp, O, (int64_t)t * O.cols_total + E + (i - (int64_t)t * rest));
    }
}

// ------------------------------------------------------------------ launchers
int sk_mt(int T) { return T <= 16 ? 1 : (T <= 32 ? 2 : 4); }

// The split-K dense passes at 5-32 tokens run token-resident (k_sk_res); at
// 33-64 tokens, whose range tokens would fill the LDS, the per-chunk staging
// kernel (k_sk_gemm). Measured on the chain (in-process A/B): the resident
// pass 2-5% faster at 8-32 tokens, 1% slower at 64. (Single projections at
// 5-32 tokens take the whole-K pass first: sk_kw_launch.)
static bool sk_resident(int T) { return sk_mt(T) <= 2; }

// K ranges of a K-wide dense pass over T tokens: a function of K and T alone,
// so every call that streams the same rows against the same tokens sums them
// in the same order, whichever other rows share its launch. Token-resident:
// kSkMaxSplit ranges of K / kSkMaxSplit (ranges of 128 when K is narrower);
// K % 128 == 0 and K <= 8192, so a range is a multiple of 16 and at most
// kResMaxRange wide. Per-chunk staging: about four 256-wide chunks per range,
// at most four ranges, except eight for K = 8192 (the o-projection): its
// 7168 rows then make exactly one 224-row tile per compute unit (below), which
// streams faster than four ranges of 112-row tiles (26.7 against 28.7 us at
// 64 tokens) by more than the finish + norm costs over the fused one-pass
// finish (9.4 against 7.2 us).
int sk_ksplit(int K, int T) {
    if (sk_resident(T)) {
        const int ks = K / 128;
        return ks < 1 ? 1 : (ks > kSkMaxSplit ? kSkMaxSplit : ks);
    }
    if (K >= 8192)
        return kSkMaxSplit;
    const int ks = ((K + kSkKc - 1) / kSkKc) / 4;
    return ks < 1 ? 1 : (ks > 4 ? 4 : ks);
}

size_t sk_partial_bytes(int T, int rows, int K) {
    const size_t ks = K > 0 ? sk_ksplit(K, T) : kSkMaxSplit;
    return align_up(ks * T * rows * sizeof(float), 256);
}

// Tile shape of a per-chunk dense pass at 33-64 tokens. With four waves per
// workgroup and 128-row tiles the launches do not divide over the compute
// units: 384 items for the 12288-row input projection (some compute units
// run two workgroups, some one) and 224 for the o-projection (32 idle). A
// workgroup of WPB waves with one tile of 16 TPW WPB rows per compute unit
// balances them: where some shape gives between 15/16 of the compute units
// and all of them items, one workgroup runs per compute unit. Measured on the
// chain of projections at 64 tokens (in-process A/B): input projection 41.6
// -> 33.2 us with six waves of two tiles (192 rows), chain 83.7 -> 72.4 us
// with the o-projection at seven waves of one tile; twelve waves of one tile
// (three waves per SIMD) ran the input projection at 39.5 us.
namespace {
struct SkShape {
    int wpb, tpw;
};
SkShape sk_dense_shape(const int *N, int nseg, int ks, int cu_budget) {
    int cus = device_cu_count();
    if (cu_budget > 0 && cu_budget < cus)
        cus = cu_budget;
    const SkShape cand[] = {{6, 2}, {7, 2}, {7, 1}};
    for (const SkShape &c : cand) {
        const int rows = 16 * c.wpb * c.tpw;
        int tiles = 0;
        for (int i = 0; i < nseg; ++i)
            tiles += (N[i] + rows - 1) / rows;
        const int items = tiles * ks;
        if (items <= cus && 16 * items >= 15 * cus)
            return c;
    }
    return SkShape{4, 2};
}
}  // namespace

// Partial sums of up to three row segments against the same tokens:
// part[(ks * T + t) * rows_total + n]. Returns the number of K ranges used.
// ks_force > 0 fixes the number of K ranges (1: part is the output itself,
// row stride ldp_force).
int sk_dense_partials(const uint16_t *const *W, const int *N, int nseg, int K, const uint16_t *x,
                      int64_t ldx, int T, float *part, int cu_budget, hipStream_t s,
                      int ks_force = 0, int64_t ldp_force = 0) {
    SkDense J{};
    // at 33-64 tokens each wave streams two 16-row tiles (half the token
    // staging per weight byte); below, one
    const int mt = sk_mt(T);
    J.tpw = mt == 4 ? 2 : 1;
    J.wpb = 4;
    if (mt == 4 && ks_force <= 0) {
        const SkShape sh = sk_dense_shape(N, nseg, sk_ksplit(K, T), cu_budget);
        J.wpb = sh.wpb;
        J.tpw = sh.tpw;
    }
    const int tile_rows = 16 * J.wpb * J.tpw;
    int tiles = 0, rows = 0;
    for (int i = 0; i < 3; ++i) {
        J.W[i] = i < nseg ? W[i] : W[0];
        J.N[i] = i < nseg ? N[i] : 0;
        J.tiles_before[i] = tiles;
        J.rows_before[i] = rows;
        if (i < nseg) {
            tiles += (N[i] + tile_rows - 1) / tile_rows;
            rows += N[i];
        }
    }
    J.tiles_before[3] = tiles;
    J.K = K;
    J.x = x;
    J.ldx = ldx;
    J.T = T;
    J.part = part;
    J.ldp = ldp_force > 0 ? ldp_force : rows;
    if (ks_force <= 0 && sk_resident(T)) {
        // the token-resident pass: each workgroup stages its K range's tokens
        // once (at most 66 KB), then its waves stream 16-row tiles. Four
        // waves per workgroup and two workgroups per compute unit, or seven
        // waves and one where that gives every wave the same number of tiles
        // and four waves do not (the 7168-row o-projection: 448 tiles per
        // range, 1.75 per wave against 2)
        const int ks = sk_ksplit(K, T), kr = K / ks;
        int tiles16 = 0;
        for (int i = 0; i < nseg; ++i)
            tiles16 += (N[i] + 15) / 16;
        auto waves_per_range = [&](int wpb, int per_cu) {
            int g = budget_grid(1 << 30, cu_budget, per_cu);
            g = g < ks ? ks : g / ks * ks;
            return g / ks * wpb;
        };
        const int w4 = waves_per_range(4, 2), w7 = waves_per_range(7, 1);
        const bool seven = tiles16 % w4 != 0 && tiles16 % w7 == 0;
        int grid = budget_grid(1 << 30, cu_budget, seven ? 1 : 2);
        grid = grid < ks ? ks : grid / ks * ks;
        const int kq = (kr + kResKc - 1) / kResKc * (kResKc / 8);
        const size_t lds = (size_t)mt * 16 * (kq + 1) * sizeof(u32x4);
        if (seven && mt == 1)
            k_sk_res<1, 7><<<grid, 7 * kWave, lds, s>>>(J, K, ks, kr);
        else if (seven)
            k_sk_res<2, 7><<<grid, 7 * kWave, lds, s>>>(J, K, ks, kr);
        else if (mt == 1)
            k_sk_res<1, 4><<<grid, kBlock, lds, s>>>(J, K, ks, kr);
        else
            k_sk_res<2, 4><<<grid, kBlock, lds, s>>>(J, K, ks, kr);
        record_dispatch(K3_OP_DENSE_PASS, K3_VARIANT_RESIDENT);
        return ks;
    }
    const int ks = ks_force > 0 ? ks_force : sk_ksplit(K, T);
    const int grid = budget_grid(tiles * ks, cu_budget, J.wpb == 4 ? 2 : 1);
    // dynamic LDS: two token buffers of 16 MT rows x (kSkKc / TPW / 8 + 1) vectors
    auto lds = [](int m, int tpw) {
        return (size_t)2 * 16 * m * (kSkKc / tpw / 8 + 1) * sizeof(u32x4);
    };
    switch (mt) {
    case 1:
        k_sk_gemm<1, SkDense, 1><<<grid, kBlock, lds(1, 1), s>>>(J, K, ks);
        break;
    case 2:
        k_sk_gemm<2, SkDense, 1><<<grid, kBlock, lds(2, 1), s>>>(J, K, ks);
        break;
    default:
        if (J.wpb == 6)
            k_sk_gemm<4, SkDense, 2, 6><<<grid, 6 * kWave, lds(4, 2), s>>>(J, K, ks);
        else if (J.wpb == 7 && J.tpw == 2)
            k_sk_gemm<4, SkDense, 2, 7><<<grid, 7 * kWave, lds(4, 2), s>>>(J, K, ks);
        else if (J.wpb == 7)
            k_sk_gemm<4, SkDense, 1, 7><<<grid, 7 * kWave, lds(4, 1), s>>>(J, K, ks);
        else
            k_sk_gemm<4, SkDense, 2><<<grid, kBlock, lds(4, 2), s>>>(J, K, ks);
        break;
    }
    record_dispatch(K3_OP_DENSE_PASS, K3_VARIANT_SPLITK);
    return ks;
}

void sk_finish(const float *part, int ks, int T, int64_t ldp, const SkOuts &O, int cu_budget,
               hipStream_t s) {
    const int64_t n = (int64_t)T * O.cols_total;
    const int want = (int)((n + kBlock - 1) / kBlock);
    k_sk_finish<<<budget_grid(want < 1 ? 1 : want, cu_budget, 8), kBlock, 0, s>>>(part, ks, T,
                                                                                  ldp, O);
}

// The finish of a pass whose segment 0 is the router, with the selection
// (k_sk_finish_topk): T workgroups for the tokens' logits and picks, then
// enough for the other columns.
void sk_finish_topk(const float *part, int ks, int T, int64_t ldp, const SkOuts &O, int k,
                    int32_t *ids, float *wts, hipStream_t s) {
    const int64_t n = (int64_t)T * (O.cols_total - O.s[0].cols);
    const int want = (int)((n + kBlock - 1) / kBlock);
    const int grid = T + (want > 0 ? budget_grid(want, 0, 8) : 0);
    k_sk_finish_topk<<<grid, kBlock, 0, s>>>(part, ks, T, ldp, O, k, ids, wts);
}

SkOuts sk_outs1(int mode, int cols, void *y, int64_t ldy, const float *bias) {
    SkOuts O{};
    O.s[0] = SkOutSeg{mode, cols, 0, y, ldy, bias, nullptr};
    O.nseg = 1;
    O.cols_total = cols;
    return O;
}

// The whole-K pass (k_sk_kw) for 5..kKwMaxTokens tokens: K a multiple of
// kKwSlice with seven or eight slices (one wave each), two to four 16-row
// tiles per workgroup on one workgroup per compute unit; token slices staged
// whole up to 8 tokens, in halves up to 16, in quarters (two token blocks)
// up to 32. Returns false (and launches nothing) for other shapes.
static bool sk_kw_launch(KwJob J, hipStream_t s) {
    if (J.T < 5 || J.T > kKwMaxTokens || J.K % kKwSlice)
        return false;
    const int nw = J.K / kKwSlice;
    if (nw != 7 && nw != 8)
        return false;
    const int cus = device_cu_count();
    J.R = (J.N + cus - 1) / cus;
    const int nt = (J.R + 15) / 16;
    if (nt < 2 || nt > 4)
        return false;
    const int grid = (J.N + J.R - 1) / J.R;
    const int ph = J.T <= 8 ? 1 : J.T <= 16 ? 2 : 4;
#define K3_KW(NW_, NT_, PH_, TB_)                                                        \
    k_sk_kw<NW_, NT_, PH_, TB_>                                                          \
        <<<grid, NW_ * kWave, kw_lds_bytes(NW_, NT_, PH_, TB_), s>>>(J)
#define K3_KW_NT(NW_, PH_, TB_)                                                          \
    (nt == 2 ? K3_KW(NW_, 2, PH_, TB_)                                                   \
             : nt == 3 ? K3_KW(NW_, 3, PH_, TB_) : K3_KW(NW_, 4, PH_, TB_))
#define K3_KW_PH(NW_)                                                                    \
    (ph == 1 ? K3_KW_NT(NW_, 1, 1) : ph == 2 ? K3_KW_NT(NW_, 2, 1) : K3_KW_NT(NW_, 4, 2))
    if (nw == 7)
        K3_KW_PH(7);
    else
        K3_KW_PH(8);
#undef K3_KW_PH
#undef K3_KW_NT
#undef K3_KW
    record_dispatch(K3_OP_DENSE_PASS, K3_VARIANT_WHOLEK);
    return true;
}

// y[t][n] = bf16(x . W^T): whole-K pass where it applies, else partials and
// the finishing kernel.
void sk_proj_bf16(const uint16_t *x, int64_t ldx, int T, const uint16_t *W, int N, int K,
                  uint16_t *y, int64_t ldy, float *part, hipStream_t s) {
    if (sk_kw_launch(KwJob{W, N, K, x, ldx, T, 0, 0, y, ldy, nullptr}, s))
        return;
    const int ks = sk_dense_partials(&W, &N, 1, K, x, ldx, T, part, 0, s);
    sk_finish(part, ks, T, N, sk_outs1(0, N, y, ldy, nullptr), 0, s);
}

// y[t][n] = x . W^T in fp32 (the shared expert's down projection).
void sk_proj_f32(const uint16_t *x, int64_t ldx, int T, const uint16_t *W, int N, int K,
                 float *y, int64_t ldy, float *part, int cu_budget, hipStream_t s) {
    const int ks = sk_dense_partials(&W, &N, 1, K, x, ldx, T, part, cu_budget, s);
    sk_finish(part, ks, T, N, sk_outs1(1, N, y, ldy, nullptr), cu_budget, s);
}

// y[t][n] = x . W^T in fp32 with one K range: the engine's epilogue writes
// the outputs directly (no partials, no finishing kernel).
void sk_proj_f32_direct(const uint16_t *x, int64_t ldx, int T, const uint16_t *W, int N, int K,
                        float *y, int64_t ldy, int cu_budget, hipStream_t s) {
    sk_dense_partials(&W, &N, 1, K, x, ldx, T, y, cu_budget, s, 1, ldy);
}

// Router scores and top-k: logits (fp32, + bias) from the router rows'
// partials, finished together with the selection.
void sk_router_topk(const uint16_t *x, int64_t ldx, int T, const uint16_t *W, int E, int K,
                    const float *bias, int k, float *logits, int32_t *ids, float *wts,
                    float *part, hipStream_t s) {
    const int ks = sk_dense_partials(&W, &E, 1, K, x, ldx, T, part, 0, s);
    sk_finish_topk(part, ks, T, E, sk_outs1(1, E, logits, E, bias), k, ids, wts, s);
}

// Router top-k and latent projection in one pass over x.
void sk_router_topk_latent(const uint16_t *x, int64_t ldx, int T, int K, const uint16_t *W_r,
                           int E, const float *bias, int k, float *logits, int32_t *ids,
                           float *wts, const uint16_t *W_lat, int d_lat, uint16_t *z,
                           int64_t ldz, float *part, hipStream_t s) {
    const uint16_t *W[2] = {W_r, W_lat};
    const int N[2] = {E, d_lat};
    const int ks = sk_dense_partials(W, N, 2, K, x, ldx, T, part, 0, s);
    SkOuts O{};
    O.s[0] = SkOutSeg{1, E, 0, logits, E, bias, nullptr};
    O.s[1] = SkOutSeg{0, d_lat, E, z, ldz, nullptr, nullptr};
    O.nseg = 2;
    O.cols_total = E + d_lat;
    sk_finish_topk(part, ks, T, E + d_lat, O, k, ids, wts, s);
}

// Router top-k, latent projection and the shared expert's gate/up + SwiGLU
// in one pass over x.
void sk_router_latent_shared(const uint16_t *x, int64_t ldx, int T, int K, const uint16_t *W_r,
                             int E, const float *bias, int k, float *logits, int32_t *ids,
                             float *wts, const uint16_t *W_lat, int d_lat, uint16_t *z,
                             int64_t ldz, const uint16_t *W13_s, int I_s, uint16_t *hs,
                             float *part, hipStream_t s) {
    const uint16_t *W[3] = {W_r, W_lat, W13_s};
    const int N[3] = {E, d_lat, 2 * I_s};
    const int ks = sk_dense_partials(W, N, 3, K, x, ldx, T, part, 0, s);
    SkOuts O{};
    O.s[0] = SkOutSeg{1, E, 0, logits, E, bias, nullptr};
    O.s[1] = SkOutSeg{0, d_lat, E, z, ldz, nullptr, nullptr};
    O.s[2] = SkOutSeg{2, I_s, E + d_lat, hs, I_s, nullptr, nullptr};
    O.nseg = 3;
    O.cols_total = E + d_lat + I_s;
    sk_finish_topk(part, ks, T, E + d_lat + 2 * I_s, O, k, ids, wts, s);
}

// Shared expert's gate/up + SwiGLU: hs[t][j] (bf16, row stride I).
void sk_swiglu(const uint16_t *x, int64_t ldx, int T, int K, const uint16_t *W13, int I,
               uint16_t *hs, float *part, int cu_budget, hipStream_t s) {
    const int N = 2 * I;
    const int ks = sk_dense_partials(&W13, &N, 1, K, x, ldx, T, part, cu_budget, s);
    sk_finish(part, ks, T, N, sk_outs1(2, I, hs, I, nullptr), cu_budget, s);
}

// Output projection + residual: residual <- bf16(residual + a . W_o^T) in
// place and h32 = the fp32 sum (the RMSNorm kernel reads it).
// The o-projection's partial sums alone; returns the number of K ranges.
int sk_oproj_partials(const uint16_t *a, int64_t lda, int T, int K, const uint16_t *W_o, int d,
                      float *part, hipStream_t s) {
    return sk_dense_partials(&W_o, &d, 1, K, a, lda, T, part, 0, s);
}

void sk_oproj_residual(const uint16_t *a, int64_t lda, int T, int K, const uint16_t *W_o, int d,
                       uint16_t *residual, float *h32, float *part, hipStream_t s) {
    if (sk_kw_launch(KwJob{W_o, d, K, a, lda, T, 0, 1, residual, d, h32}, s))
        return;
    const int ks = sk_dense_partials(&W_o, &d, 1, K, a, lda, T, part, 0, s);
    SkOuts O{};
    O.s[0] = SkOutSeg{3, d, 0, residual, d, nullptr, h32};
    O.nseg = 1;
    O.cols_total = d;
    sk_finish(part, ks, T, d, O, 0, s);
}

}  // namespace k3
