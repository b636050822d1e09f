// k3_device.h -- device-side helpers shared by the libk3dec kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

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
// The weight-streaming engine of the small-batch kernels. One wave walks
// rows [r_begin, r_end) of a row set, RB rows at a time: row i is NV
// 16-byte vectors long, lane l owns vectors l, l + 64, ... (CB of them, so
// one load instruction reads 1 KB of a row contiguously). Two register
// buffers alternate, so the next RB rows' loads are in flight while the
// current ones are multiplied against the token vectors staged in LDS
// (xs[t * xstride + v], t < nt <= TM). Activations come from LDS only: a
// global activation load issued behind the weight loads would have to wait
// for all of them (vector loads retire in order). After each row, every lane
// holds the wave-reduced sum for each token and calls epi(row, t, sum).
template <int TM, int RB, int CB, class RowPtr, class Epi>
__device__ __forceinline__ void stream_rows(int r_begin, int r_end, int nv, const u32x4 *xs,
                                            int xstride, int nt, RowPtr rowptr, Epi epi) {
    const int lane = threadIdx.x & (kWave - 1);
    u32x4 A[RB][CB], B[RB][CB];
    auto load = [&](u32x4 (&buf)[RB][CB], int r) {
#pragma unroll
        for (int i = 0; i < RB; ++i) {
            const bool rv = r + i < r_end;
            const uint16_t *p = rv ? rowptr(r + i) : nullptr;
#pragma unroll
            for (int c = 0; c < CB; ++c) {
                const int v = c * kWave + lane;
                buf[i][c] = (rv && v < nv) ? ld_weight16(p + (int64_t)v * 8) : zero16();
            }
        }
    };
    auto finish = [&](u32x4 (&buf)[RB][CB], int r) {
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
                            acc[i][t] = dot8(buf[i][c], xv, acc[i][t]);
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
    };
    if (r_begin >= r_end)
        return;
    load(A, r_begin);
    for (int r = r_begin; r < r_end; r += 2 * RB) {
        if (r + RB < r_end)
            load(B, r + RB);
        finish(A, r);
        if (r + RB >= r_end)
            break;
        if (r + 2 * RB < r_end)
            load(A, r + 2 * RB);
        finish(B, r + RB);
    }
}

// Copy nrows activation rows (nv 16-byte vectors each, row t starting at
// src(t)) into LDS rows of xstride vectors; all threads of the block help.
template <class Src>
__device__ __forceinline__ void stage_rows(u32x4 *xs, int xstride, int nrows, int nv, Src src) {
    for (int i = threadIdx.x; i < nrows * nv; i += blockDim.x) {
        const int t = i / nv, v = i - t * nv;
        xs[t * xstride + v] = ld_act16(src(t) + (int64_t)v * 8);
    }
}

// Even split of [0, n) over `parts`: the part-th range.
__device__ __forceinline__ void split_range(int n, int parts, int part, int &lo, int &hi) {
    const int base = n / parts, rem = n % parts;
    lo = part * base + min(part, rem);
    hi = lo + base + (part < rem ? 1 : 0);
}

}  // namespace k3
