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

// Weight loads through a buffer resource: the hardware checks each lane's
// byte offset against the range and returns zeros past its end, with no
// memory access, so masked-off lanes (row tails, invalid rows) need no branch
// -- a branch around a load makes the compiler wait for it at the join. The
// range base must be wave-uniform (it lives in scalar registers).
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t weight_range(const uint16_t *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base), (short)0, (int)bytes,
                                             0x00020000);
}

// 16 bytes at byte offset off of the range (non-temporal).
__device__ __forceinline__ u32x4 ld_weight16(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
}

// An offset past every range: the load returns zeros.
constexpr uint32_t kOffNone = 0x80000000u;

// Activations (re-read by many workgroups, so cached normally) through a
// buffer resource: a masked lane passes kOffNone and reads zeros without a
// memory access or a branch.
__device__ __forceinline__ rsrc_t act_range(const uint16_t *base) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(base), (short)0,
                                             (int)(kOffNone - 16u), 0x00020000);
}

__device__ __forceinline__ u32x4 ld_act16(rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// 8 bytes at byte offset off of the range.
__device__ __forceinline__ uint2 ld_act8(rsrc_t r, uint32_t off) {
    const auto v = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
    return uint2{(uint32_t)v[0], (uint32_t)v[1]};
}

// Index of the calling wave in its workgroup, known uniform to the compiler.
__device__ __forceinline__ int wave_in_block() {
    return __builtin_amdgcn_readfirstlane((int)(threadIdx.x / kWave));
}

// A load through the scalar data cache (s_load): the address must be the
// same in every lane and the memory must not change while the kernel runs
// (e.g. lists an earlier kernel wrote). Scalar loads count separately from
// vector loads, so waiting for one never waits for the weight loads in
// flight (vector loads retire in order).
__device__ __forceinline__ int ld_scalar(const int *p) {
    return *(const __attribute__((address_space(4))) int *)p;
}

// A pointer every lane of the wave holds (e.g. read from LDS), made known
// uniform to the compiler so that a range built from it stays scalar.
template <class T>
__device__ __forceinline__ T *uniform_ptr(T *p) {
    const uint64_t v = (uint64_t)p;
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
    return (T *)(((uint64_t)hi << 32) | lo);
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

// ------------------------------------------------------------------ wave reductions
// Cross-lane steps use DPP (GFX9 data-parallel primitives): row_shr 1, 2, 4, 8
// leave each 16-lane row's total in its lane 15, row_bcast 15 and 31 carry
// those totals into lane 63, and v_readlane broadcasts it, so every lane
// receives the same bits. Lanes a step reads from outside the row, and rows
// the step's row mask leaves out, contribute the operation's identity (`id`).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v, uint32_t id) {
    return (uint32_t)__builtin_amdgcn_update_dpp((int)id, (int)v, CTRL, ROW_MASK, 0xf, false);
}

template <class Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, uint32_t id, Op op) {
    v = op(v, dpp_u32<0x111, 0xf>(v, id));  // row_shr:1
    v = op(v, dpp_u32<0x112, 0xf>(v, id));  // row_shr:2
    v = op(v, dpp_u32<0x114, 0xf>(v, id));  // row_shr:4
    v = op(v, dpp_u32<0x118, 0xf>(v, id));  // row_shr:8
    v = op(v, dpp_u32<0x142, 0xa>(v, id));  // row_bcast:15 into rows 1 and 3
    v = op(v, dpp_u32<0x143, 0xc>(v, id));  // row_bcast:31 into rows 2 and 3
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Sum over the 64 lanes of a wave, in a fixed order.
__device__ __forceinline__ float wave_sum(float v) {
    return __uint_as_float(wave_reduce_u32(__float_as_uint(v), 0u, [](uint32_t a, uint32_t b) {
        return __float_as_uint(__uint_as_float(a) + __uint_as_float(b));
    }));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    return wave_reduce_u32(v, 0u, [](uint32_t a, uint32_t b) { return a > b ? a : b; });
}

__device__ __forceinline__ uint32_t wave_min_u32(uint32_t v) {
    return wave_reduce_u32(v, 0xffffffffu, [](uint32_t a, uint32_t b) { return a < b ? a : b; });
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
// With early == false the first unit is loaded only after pre() (its address
// depends on what pre() produces).
template <int NB, class Load, class Finish, class Pre = NoPrologue>
__device__ __forceinline__ void stream_units(int u_begin, int u_end, Load load, Finish finish,
                                             Pre pre = Pre(), bool early = true) {
    u32x4 A[NB], B[NB];
    if (early && u_begin < u_end)
        load(A, u_begin);
    pre();
    if (u_begin >= u_end)
        return;
    if (!early)
        load(A, u_begin);
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
                const rsrc_t rr = weight_range(uniform_ptr(rowptr(rv ? r + i : r_begin)),
                                               rv ? (uint32_t)nv * 16 : 0u);
#pragma unroll
                for (int c = 0; c < CB; ++c)
                    buf[i * CB + c] = ld_weight16(rr, (uint32_t)(c * kWave + lane) * 16);
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
// Selection order: logit descending, expert index ascending on equal logits;
// a NaN logit ranks with -inf and -0 with +0. order_key maps a logit to a
// 32-bit key whose unsigned order is that order of values (key 0 is never
// produced and marks an empty or taken entry).
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        u = 0xff800000u;
    if (u == 0x80000000u)
        u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t key) {
    return __uint_as_float((key & 0x80000000u) ? (key ^ 0x80000000u) : ~key);
}

constexpr int kTopkPer = K3_MAX_EXPERTS / kWave;  // logits per lane

// Lane l loads logits l, l + 64, ... (entries past E are empty). The loads
// are unconditional (clamped index) so that all of them are in flight at
// once; the keys are formed later, by topk_keys.
__device__ __forceinline__ void topk_load(const float *logits, int E, float (&lv)[kTopkPer]) {
    const int lane = threadIdx.x & (kWave - 1);
#pragma unroll
    for (int i = 0; i < kTopkPer; ++i) {
        const int e = i * kWave + lane;
        lv[i] = logits[e < E ? e : E - 1];
    }
}

__device__ __forceinline__ void topk_keys(const float (&lv)[kTopkPer], int E,
                                          uint32_t (&key)[kTopkPer]) {
    const int lane = threadIdx.x & (kWave - 1);
    // masked rather than selected: a branch here lets the compiler sink a
    // logit load into it and wait there for every load issued after it
#pragma unroll
    for (int i = 0; i < kTopkPer; ++i)
        key[i] = order_key(lv[i]) & (i * kWave + lane < E ? 0xffffffffu : 0u);
}

// One wave picks experts from the keys topk_load gave it, one per next():
// the wave-wide maximum of the keys, then the smallest expert index holding
// it; lane j keeps the j-th pick. finish(k) turns the k picks into weights,
// the softmax over the k picked logits (the full softmax renormalised over
// the selection), written by lanes j < k to ids[j], wts[j]. Only the first
// ceil(E / 64) keys of a lane can be non-empty; the rest are skipped (a
// wave-uniform bound: E is the same in every lane). Each lane keeps its
// largest remaining key and that key's slot (the first such slot), so a
// pick costs the two wave reductions and a rescan of the winning lane's
// slots only (about 200 instructions per pick when every lane rescanned
// every slot, and most of the selection's time).
struct TopkPicker {
    uint32_t key[kTopkPer];
    int per;  // key slots that can hold logits
    int n;    // picks so far
    uint32_t sel_key, top_key;
    int sel_e;
    uint32_t hk;     // this lane's largest remaining key (0: none left)
    int hs;          // its slot
    uint32_t taken;  // this lane's slots already picked (bit i: slot i)
    __device__ __forceinline__ void init(int E) {
        per = __builtin_amdgcn_readfirstlane((E + kWave - 1) / kWave);
        n = 0;
        sel_key = top_key = 0u;
        sel_e = 0;
        hk = 0u;
        hs = 0;
        taken = 0u;
    }
    // hk, hs from this lane's slots not yet taken. Slots go in groups of
    // four behind a wave-uniform test against per (slots past E hold key 0,
    // so a group's tail needs no test). Each group is its own instantiation
    // and a taken slot is a bit of `taken`, not a cleared key, so every
    // index is a constant and the keys stay in registers.
    static_assert(kTopkPer == 16, "four groups of four key slots");
    template <int G>
    __device__ __forceinline__ void head_group(uint32_t &bk, int &bs) const {
        if (4 * G < per)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (!((taken >> (4 * G + j)) & 1u) && key[4 * G + j] > bk) {
                    bk = key[4 * G + j];
                    bs = 4 * G + j;
                }
    }
    __device__ __forceinline__ void head() {
        uint32_t bk = 0u;
        int bs = 0;
        head_group<0>(bk, bs);
        head_group<1>(bk, bs);
        head_group<2>(bk, bs);
        head_group<3>(bk, bs);
        hk = bk;
        hs = bs;
    }
    // The next pick's expert (the same in every lane).
    __device__ __forceinline__ int next() {
        const int lane = threadIdx.x & (kWave - 1);
        if (n == 0)
            head();  // the keys are complete by the first pick
        const uint32_t m = wave_max_u32(hk);
        const uint32_t w = wave_min_u32(hk == m ? (uint32_t)(hs * kWave + lane) : 0xffffffffu);
        if ((int)(w & (kWave - 1)) == lane) {
            // the winning lane gives up the slot (its head) and finds its
            // next head
            taken |= 1u << hs;
            head();
        }
        if (lane == n) {
            sel_key = m;
            sel_e = (int)w;
        }
        if (n == 0)
            top_key = m;
        ++n;
        return (int)w;
    }
    __device__ __forceinline__ void finish(int k, int32_t *ids, float *wts) const {
        const int lane = threadIdx.x & (kWave - 1);
        const float sel_v = key_value(sel_key), top = key_value(top_key);
        const float dl = (sel_v == top) ? 0.0f : sel_v - top;
        const float p = lane < k ? expf(dl) : 0.0f;
        const float sum = wave_sum(p);
        if (lane < k) {
            ids[lane] = sel_e;
            wts[lane] = p / sum;
        }
    }
};

// All k picks at once.
__device__ __forceinline__ void topk_select(uint32_t (&key)[kTopkPer], int k, int32_t *ids,
                                            float *wts, int E = K3_MAX_EXPERTS) {
    TopkPicker pk;
#pragma unroll
    for (int i = 0; i < kTopkPer; ++i)
        pk.key[i] = key[i];
    pk.init(E);
    for (int j = 0; j < k; ++j)
        pk.next();
    pk.finish(k, ids, wts);
}

__device__ __forceinline__ void topk_wave(const float *logits, int E, int k, int32_t *ids,
                                          float *wts) {
    float lv[kTopkPer];
    uint32_t key[kTopkPer];
    topk_load(logits, E, lv);
    topk_keys(lv, E, key);
    topk_select(key, k, ids, wts, E);
}

}  // namespace k3
