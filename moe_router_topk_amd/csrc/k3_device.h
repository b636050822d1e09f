// k3_device.h -- device-side helpers shared by the libk3dec kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/k3dec.h"

namespace k3 {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kBlock = 256;  // 4 waves per workgroup everywhere

// Weights are static while a call runs: they stream through with
// non-temporal 128-bit loads (read once, no reuse worth caching).
__device__ __forceinline__ u32x4 ld_weight16(const uint16_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// Activations are produced by earlier kernels: ordinary cached loads.
__device__ __forceinline__ u32x4 ld_act16(const uint16_t *p) {
    return *reinterpret_cast<const u32x4 *>(p);
}

__device__ __forceinline__ u32x4 zero16() { return u32x4{0u, 0u, 0u, 0u}; }

// Two bf16 products accumulated in fp32 (v_dot2c_f32_bf16). The operands
// are taken by value: bit-casting a vector element in place miscompiles.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                           __builtin_bit_cast(bf16x2, b), c, false);
}

// Eight bf16 products (one 16-byte vector of each operand) into c.
__device__ __forceinline__ float dot8(u32x4 w, u32x4 x, float c) {
    c = dot2(w.x, x.x, c);
    c = dot2(w.y, x.y, c);
    c = dot2(w.z, x.z, c);
    c = dot2(w.w, x.w, c);
    return c;
}

// D += A . B on one 16x16x32 bf16 tile. Lane l supplies A[l%16][8(l/16)..+7]
// and B[8(l/16)..+7][l%16] (8 bf16 each) and receives D[4(l/16)+i][l%16],
// i = 0..3.
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float((uint32_t)h << 16);
}

// fp32 -> bf16, round to nearest even; NaN stays NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)((u >> 16) | 0x0040u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Sum over the 64 lanes of a wave; every lane receives the same bits
// (each butterfly step adds the same two operands on both partners).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1)
        v += __shfl_xor(v, m, kWave);
    return v;
}

__device__ __forceinline__ float silu(float g) {
    return g / (1.0f + expf(-g));
}

}  // namespace k3

namespace k3 {

// ------------------------------------------------------------------ row streaming
// The weight-streaming engine of the small-batch kernels. A wave walks a
// sequence of units; load(buf, u) issues unit u's 16-byte weight loads into a
// register buffer of NB vectors and finish(buf, u) consumes them. Two buffers
// alternate, so unit u+1's loads are in flight while unit u is multiplied.
// Weight rows are read with lane l taking vectors l, l + 64, ..., so one
// load instruction covers 1 KB of a row contiguously. Activations come from
// LDS only: a global activation load issued behind the weight loads would
// have to wait for all of them (vector loads retire in order).
//
// stream_rows: units of RB rows, each multiplied against the token vectors
// staged in LDS (xs[t * xstride + v], t < nt <= TM); after each row, every
// lane holds the wave-reduced sum per token and calls epi(row, t, sum).
struct NoPrologue {
    __device__ void operator()() const {}
};

// pre() runs once, after the first unit's loads are issued and before any
// unit is consumed, in every wave (also waves without units), so it may stage
// activations and hold a block barrier: its latency overlaps the first loads.
template <int NB, class Load, class Finish, class Pre = NoPrologue>
__device__ __forceinline__ void stream_units(int u_begin, int u_end, Load load, Finish finish,
                                             Pre pre = Pre()) {
    u32x4 A[NB], B[NB];
    if (u_begin < u_end)
        load(A, u_begin);
    pre();
    if (u_begin >= u_end)
        return;
    for (int u = u_begin; u < u_end; u += 2) {
        if (u + 1 < u_end)
            load(B, u + 1);
        finish(A, u);
        if (u + 1 >= u_end)
            break;
        if (u + 2 < u_end)
            load(A, u + 2);
        finish(B, u + 1);
    }
}

// Rows of a row set, RB rows per unit: row i is nv 16-byte vectors long,
// starting at rowptr(i); lane l owns vectors l, l + 64, ... (CB of them).
template <int TM, int RB, int CB, class RowPtr, class Epi, class Pre = NoPrologue>
__device__ __forceinline__ void stream_rows(int r_begin, int r_end, int nv, const u32x4 *xs,
                                            int xstride, int nt, RowPtr rowptr, Epi epi,
                                            Pre pre = Pre()) {
    const int lane = threadIdx.x & (kWave - 1);
    const int units = (r_end - r_begin + RB - 1) / RB;
    stream_units<RB * CB>(
        0, units,
        [&](u32x4 (&buf)[RB * CB], int u) {
            const int r = r_begin + u * RB;
#pragma unroll
            for (int i = 0; i < RB; ++i) {
                const bool rv = r + i < r_end;
                const uint16_t *p = rv ? rowptr(r + i) : nullptr;
#pragma unroll
                for (int c = 0; c < CB; ++c) {
                    const int v = c * kWave + lane;
                    buf[i * CB + c] = (rv && v < nv) ? ld_weight16(p + (int64_t)v * 8) : zero16();
                }
            }
        },
        [&](u32x4 (&buf)[RB * CB], int u) {
            const int r = r_begin + u * RB;
            float acc[RB][TM];
#pragma unroll
            for (int i = 0; i < RB; ++i)
#pragma unroll
                for (int t = 0; t < TM; ++t)
                    acc[i][t] = 0.0f;
#pragma unroll
            for (int c = 0; c < CB; ++c) {
                const int v = c * kWave + lane;
                if (v < nv) {
#pragma unroll
                    for (int t = 0; t < TM; ++t) {
                        if (t < nt) {
                            const u32x4 xv = xs[t * xstride + v];
#pragma unroll
                            for (int i = 0; i < RB; ++i)
                                acc[i][t] = dot8(buf[i * CB + c], xv, acc[i][t]);
                        }
                    }
                }
            }
#pragma unroll
            for (int i = 0; i < RB; ++i)
                if (r + i < r_end)
#pragma unroll
                    for (int t = 0; t < TM; ++t)
                        if (t < nt)
                            epi(r + i, t, wave_sum(acc[i][t]));
        },
        pre);
}

// Copy nrows activation rows (nv 16-byte vectors each, row t starting at
// src(t)) into LDS rows of xstride vectors; all threads of the block help.
// Loads go out eight at a time before their LDS stores, so staging costs
// about one memory latency per 8 vectors a thread moves, not one per vector.
template <class Src>
__device__ __forceinline__ void stage_rows(u32x4 *xs, int xstride, int nrows, int nv, Src src) {
    const int n = nrows * nv;
    for (int i0 = threadIdx.x; i0 < n; i0 += 8 * kBlock) {
        u32x4 v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * kBlock;
            if (i < n) {
                const int t = i / nv;
                v[u] = ld_act16(src(t) + (int64_t)(i - t * nv) * 8);
            }
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * kBlock;
            if (i < n) {
                const int t = i / nv;
                xs[t * xstride + (i - t * nv)] = v[u];
            }
        }
    }
}

// Even split of [0, n) over `parts`: the part-th range.
__device__ __forceinline__ void split_range(int n, int parts, int part, int &lo, int &hi) {
    const int base = n / parts, rem = n % parts;
    lo = part * base + min(part, rem);
    hi = lo + base + (part < rem ? 1 : 0);
}

// ------------------------------------------------------------------ top-k
// One wave picks token t's k experts: lane l holds logits l, l + 64, ...;
// k rounds of a wave-wide argmax under the order (logit desc, index asc);
// lane j keeps the j-th pick. The weights are the softmax over the k picked
// logits (the full softmax renormalised over the selection).
__device__ __forceinline__ void topk_wave(const float *logits, int E, int k, int32_t *ids,
                                          float *wts) {
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

}  // namespace k3
