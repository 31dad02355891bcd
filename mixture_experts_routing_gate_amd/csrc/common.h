// Device-side helpers shared by the gfx950 kernels of libmoe (wave64 CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_DEV __device__ __forceinline__

namespace moe {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// fp32 -> bf16 bits, round to nearest even (lowers to v_cvt_pk_bf16_f32).
MOE_DEV uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
MOE_DEV float bf16_to_f32(uint16_t b) { return __uint_as_float(((uint32_t)b) << 16); }

// Pack two fp32 into one dword of two bf16 (lo in bits 0..15).
MOE_DEV uint32_t pack_bf16x2(float lo, float hi) {
    return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}

// Reductions over aligned groups of G consecutive lanes (G a power of two <= 64).
template <int G>
MOE_DEV float group_max(float x) {
#pragma unroll
    for (int s = 1; s < G; s <<= 1) x = fmaxf(x, __shfl_xor(x, s, kWave));
    return x;
}
template <int G>
MOE_DEV int group_min(int x) {
#pragma unroll
    for (int s = 1; s < G; s <<= 1) x = min(x, __shfl_xor(x, s, kWave));
    return x;
}
template <int G>
MOE_DEV float group_sum(float x) {
#pragma unroll
    for (int s = 1; s < G; s <<= 1) x += __shfl_xor(x, s, kWave);
    return x;
}

MOE_DEV int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

}  // namespace moe
