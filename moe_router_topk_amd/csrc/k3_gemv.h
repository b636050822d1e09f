// k3_gemv.h -- the batch-1 streaming engine: out[r] = sum_k W[r][k] x[k].
//
// One load instruction covers 8 weight rows x 128 bytes (lane l: row l / 8,
// bytes 16 (l % 8) of the row's 128-byte piece). Measured on gfx950, that
// pattern streams 7-10% faster than walking one row at a time in 1 KB
// steps, because more DRAM rows are open at once.
//
// A workgroup owns an even share of the rows, taken as groups of 8 (the
// last one may be partial); wave w of the four streams K-quarter w of every
// group, U 128-byte pieces per register buffer, two buffers in flight, and
// the pipeline runs on across groups. Each group's 8-lane partial sums are
// reduced with DPP and parked in LDS; after a barrier the four quarters of a
// row are added in wave order, so every output has one fixed summation order.
#pragma once
#include "k3_device.h"

namespace k3 {

// Sum over the 8 lanes (l & ~7) .. (l & ~7) + 7; every one of them gets it.
__device__ __forceinline__ float gv_red8(float v) {
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xf, 0xf, false));
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xf, 0xf, false));
    return v;
}

// Pieces per register buffer for a K-wide row: a K-quarter holds K / 256
// pieces (K % 256 == 0); 7 or 8 divide the common widths exactly.
constexpr int gv_unit_pieces(int K) { return (K / 256) % 8 == 0 ? 8 : ((K / 256) % 7 == 0 ? 7 : 8); }

// Two-phase staging of n 16-byte vectors of one buffer into LDS: load()
// issues all the loads at once (vectors past n read nothing: their offsets
// leave the range), store() writes them. A kernel issues the loads before
// its first weight loads and stores them after: vector loads retire in
// order, so waiting for these then never waits for the weights.
template <int M>
struct GvStage {
    u32x4 v[M];
    __device__ __forceinline__ void load(const uint16_t *base, int n) {
        const rsrc_t r = act_range(uniform_ptr(base));
#pragma unroll
        for (int j = 0; j < M; ++j) {
            const int i = threadIdx.x + j * kBlock;
            // past n: the sign bit of n - 1 - i (arithmetic, so no branch)
            v[j] = ld_act16(r, ((uint32_t)i * 16u) | ((uint32_t)(n - 1 - i) & 0x80000000u));
        }
    }
    __device__ __forceinline__ void store(u32x4 *dst, int n) const {
#pragma unroll
        for (int j = 0; j < M; ++j) {
            const int i = threadIdx.x + j * kBlock;
            if (i < n)
                dst[i] = v[j];
        }
    }
};

// Streams the workgroup's groups. grp(g, base, nrows, skip): the 8-row
// group g starts at base, rows K elements apart, and has nrows valid rows
// (<= 8); rows 4..7 sit skip rows further on (a gate/up pair group: four
// gate rows, then the four matching up rows of the same columns).
// xv(g, kv): the activation vector kv (8 elements) group g multiplies.
// ps[w * ps_stride + 8 g + r]: wave w's partial sum of row r of group g.
// first(): runs before the first weight loads are issued (issue the
// activation loads there, GvStage::load); pre(): runs right after them (store
// the activations to LDS) and must end with __syncthreads().
// NT tokens (1..4): xv(g, kv, t) is token t's vector; the partial sums of
// token t sit at ps[(w * NT + t) * ps_stride + 8 g + r].
template <int U, int NT = 1, class Grp, class XV, class First, class Pre>
__device__ __forceinline__ void gemv8_stream(int ngroups, int K, Grp grp, XV xv, float *ps,
                                             int ps_stride, First first, Pre pre) {
    const int lane = threadIdx.x & (kWave - 1), wq = wave_in_block();
    int p0, p1;
    split_range(K >> 6, kBlock / kWave, wq, p0, p1);
    // units per group; a wave whose quarter is empty (K < 256) still runs
    // one masked unit per group, so its partial sums are written as zeros
    const int upg = max(1, (p1 - p0 + U - 1) / U);
    const int nunits = ngroups * upg;
    const int rl = lane >> 3, el = (lane & 7) * 8;
    auto load = [&](u32x4 (&b)[U], int u) {
        const int g = u / upg, c = u - g * upg;
        const uint16_t *base;
        int nr, skip;
        grp(g < ngroups ? g : 0, base, nr, skip);
        skip = __builtin_amdgcn_readfirstlane(skip);
        const uint32_t bytes =
            u < nunits ? (uint32_t)__builtin_amdgcn_readfirstlane(nr + (nr > 4 ? skip : 0)) *
                             (uint32_t)K * 2u
                       : 0u;
        const rsrc_t r = weight_range(uniform_ptr(base), bytes);
        const int row = rl + (rl >= 4 ? skip : 0);
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int p = p0 + c * U + i;
            // pieces past the quarter: the sign bit of p1 - 1 - p moves the
            // offset out of the range (arithmetic, so no branch)
            const uint32_t past = (uint32_t)(p1 - 1 - p) & 0x80000000u;
            b[i] = ld_weight16(r, ((uint32_t)(row * K + p * 64 + el) * 2u) | past);
        }
    };
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
        acc[t] = 0.0f;
    // When the quarter is a non-empty whole number of units every piece of a
    // unit lies inside it and needs no mask; the sums of the empty units at
    // the end belong to groups past the last and are never stored. (An empty
    // quarter, K < 256, takes the masked path: its one unit per group must
    // add nothing.)
    const bool exact = p1 > p0 && (p1 - p0) % U == 0;
    auto fin = [&](u32x4 (&b)[U], int u) {
        const int g = u / upg, c = u - g * upg;
        if (exact) {
#pragma unroll
            for (int i = 0; i < U; ++i) {
                const int kv = (p0 + c * U + i) * 8 + (lane & 7);
#pragma unroll
                for (int t = 0; t < NT; ++t)
                    acc[t] = dot8(b[i], xv(g, kv, t), acc[t]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < U; ++i) {
                // a piece past the quarter has zero weights; its activations
                // are masked to zero too (a mask, not a branch around loads)
                const int p = p0 + c * U + i;
                const uint32_t m = (p < p1 && u < nunits) ? 0xffffffffu : 0u;
                const int kv = min(p, p1 - 1) * 8 + (lane & 7);
#pragma unroll
                for (int t = 0; t < NT; ++t) {
                    const u32x4 xa = xv(g, kv, t);
                    acc[t] = dot8(b[i], u32x4{xa.x & m, xa.y & m, xa.z & m, xa.w & m}, acc[t]);
                }
            }
        }
        if (c == upg - 1) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const float s = gv_red8(acc[t]);
                acc[t] = 0.0f;
                if (g < ngroups && (lane & 7) == 0)
                    ps[(wq * NT + t) * ps_stride + 8 * g + rl] = s;
            }
        }
    };
    // Units run in pairs; an odd count ends with an empty unit (no weights,
    // masked activations), so the loop has a single exit and every load is
    // issued on every path: the waits then count exactly the loads behind.
    u32x4 A[U], B[U];
    first();
    load(A, 0);
    pre();
    for (int u = 0; u < nunits; u += 2) {
        load(B, u + 1);
        __builtin_amdgcn_sched_barrier(0);  // keep the prefetch ahead of the math
        fin(A, u);
        load(A, u + 2);
        __builtin_amdgcn_sched_barrier(0);
        fin(B, u + 1);
    }
    __syncthreads();  // every quarter's partials are in ps
}

// gemv8_stream for groups that each serve their own tokens (the routed
// experts at batches 2-4: a group belongs to one expert, whose few tokens are
// some of the NT token rows in LDS). slot(g) returns the group's context, with
// a member nt (<= NT, the same in every lane): tokens t < nt are multiplied,
// the others skipped (their partial sums are written as zeros). xv(cx, kv, t)
// gives token t's activation vector kv for that context. Every other argument
// is gemv8_stream's, and so is every summation order.
template <int U, int NT, class Grp, class Slot, class XV, class First, class Pre>
__device__ __forceinline__ void gemv8_stream_slots(int ngroups, int K, Grp grp, Slot slot, XV xv,
                                                   float *ps, int ps_stride, First first,
                                                   Pre pre) {
    const int lane = threadIdx.x & (kWave - 1), wq = wave_in_block();
    int p0, p1;
    split_range(K >> 6, kBlock / kWave, wq, p0, p1);
    const int upg = max(1, (p1 - p0 + U - 1) / U);
    const int nunits = ngroups * upg;
    const int rl = lane >> 3, el = (lane & 7) * 8;
    auto load = [&](u32x4 (&b)[U], int u) {
        const int g = u / upg, c = u - g * upg;
        const uint16_t *base;
        int nr, skip;
        grp(g < ngroups ? g : 0, base, nr, skip);
        skip = __builtin_amdgcn_readfirstlane(skip);
        const uint32_t bytes =
            u < nunits ? (uint32_t)__builtin_amdgcn_readfirstlane(nr + (nr > 4 ? skip : 0)) *
                             (uint32_t)K * 2u
                       : 0u;
        const rsrc_t r = weight_range(uniform_ptr(base), bytes);
        const int row = rl + (rl >= 4 ? skip : 0);
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int p = p0 + c * U + i;
            const uint32_t past = (uint32_t)(p1 - 1 - p) & 0x80000000u;
            b[i] = ld_weight16(r, ((uint32_t)(row * K + p * 64 + el) * 2u) | past);
        }
    };
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t)
        acc[t] = 0.0f;
    const bool exact = p1 > p0 && (p1 - p0) % U == 0;
    auto fin = [&](u32x4 (&b)[U], int u) {
        const int g = u / upg, c = u - g * upg;
        const auto cx = slot(g < ngroups ? g : 0);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
            if (t < cx.nt) {
                if (exact) {
#pragma unroll
                    for (int i = 0; i < U; ++i) {
                        const int kv = (p0 + c * U + i) * 8 + (lane & 7);
                        acc[t] = dot8(b[i], xv(cx, kv, t), acc[t]);
                    }
                } else {
#pragma unroll
                    for (int i = 0; i < U; ++i) {
                        const int p = p0 + c * U + i;
                        const uint32_t m = (p < p1 && u < nunits) ? 0xffffffffu : 0u;
                        const int kv = min(p, p1 - 1) * 8 + (lane & 7);
                        const u32x4 xa = xv(cx, kv, t);
                        acc[t] = dot8(b[i], u32x4{xa.x & m, xa.y & m, xa.z & m, xa.w & m}, acc[t]);
                    }
                }
            }
        }
        if (c == upg - 1) {
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const float s = gv_red8(acc[t]);
                acc[t] = 0.0f;
                if (g < ngroups && (lane & 7) == 0)
                    ps[(wq * NT + t) * ps_stride + 8 * g + rl] = s;
            }
        }
    };
    u32x4 A[U], B[U];
    first();
    load(A, 0);
    pre();
    for (int u = 0; u < nunits; u += 2) {
        load(B, u + 1);
        __builtin_amdgcn_sched_barrier(0);
        fin(A, u);
        load(A, u + 2);
        __builtin_amdgcn_sched_barrier(0);
        fin(B, u + 1);
    }
    __syncthreads();
}

// The four quarter sums of row i of the share, in wave order (token t of NT).
__device__ __forceinline__ float gv_total(const float *ps, int ps_stride, int i, int NT = 1,
                                          int t = 0) {
    const float *q = ps + (int64_t)t * ps_stride + i;
    const int64_t w = (int64_t)NT * ps_stride;
    return ((q[0] + q[w]) + q[2 * w]) + q[3 * w];
}

}  // namespace k3
