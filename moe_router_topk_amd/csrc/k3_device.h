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
