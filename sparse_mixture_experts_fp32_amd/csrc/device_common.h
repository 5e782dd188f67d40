// Small device helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));  // one MFMA A/B operand
typedef float f32x4 __attribute__((ext_vector_type(4)));    // one 16x16 MFMA accumulator
typedef uint32_t u32x4 __attribute__((ext_vector_type(4))); // 16 raw bytes (native vector: stays in registers)

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bfloat16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint16_t f32_to_bf16_bits(float f) {
    return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// D = A(16x32) * B(32x16) + C on the matrix cores.
// Lane l supplies A[l % 16][8 * (l / 16) + i] and B[8 * (l / 16) + i][l % 16], i = 0..7,
// and holds D[4 * (l / 16) + i][l % 16], i = 0..3.
__device__ __forceinline__ f32x4 mfma_16x16x32(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
        uint32_t lo = __shfl_xor(static_cast<uint32_t>(v), off, kWave);
        uint32_t hi = __shfl_xor(static_cast<uint32_t>(v >> 32), off, kWave);
        uint64_t o = (static_cast<uint64_t>(hi) << 32) | lo;
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, kWave));
    return v;
}

// Monotone map of a float to uint32 for selection keys: larger float, larger key;
// -0.0 and +0.0 map to one key; NaN maps to 0, below every number.
__device__ __forceinline__ uint32_t order_key(float v) {
    if (v != v) return 0u;     // NaN: below every number
    if (v == 0.0f) v = 0.0f;   // -0.0 ties +0.0
    const uint32_t b = __float_as_uint(v);
    return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

__device__ __forceinline__ float key_value(uint32_t k) {
    if (k == 0u) return __uint_as_float(0x7fc00000u);
    return __uint_as_float((k & 0x80000000u) ? (k ^ 0x80000000u) : ~k);
}

}  // namespace moe
