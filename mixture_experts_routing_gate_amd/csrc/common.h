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

// Pack two fp32 into one dword of two bf16 (lo in bits 0..15), rounded to
// nearest even as f32_to_bf16 rounds each.  Written as one two-lane conversion
// so that it becomes a single v_cvt_pk_bf16_f32 of both operands, not two
// conversions followed by a shift and an OR.
typedef float f32x2_cv __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_cv __attribute__((ext_vector_type(2)));
MOE_DEV uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_cv{lo, hi}, bf16x2_cv));
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

typedef __attribute__((address_space(3))) void lds_void;

// Raw buffer resource (4 scalar dwords): 48-bit base, stride 0, num_records
// (loads at byte offsets past it return zeros), and the gfx9 dword-3 format word.
typedef int32_t rsrc_t __attribute__((ext_vector_type(4)));

MOE_DEV rsrc_t make_rsrc(const void* base, uint32_t num_records = 0x7fffffffu) {
    const uint64_t a = (uint64_t)base;
    rsrc_t r;
    r[0] = uniform((int)(uint32_t)a);
    r[1] = uniform((int)(uint32_t)(a >> 32) & 0xffff);
    r[2] = uniform((int)num_records);
    r[3] = 0x00020000;
    return r;
}

// 16 bytes per lane from global memory straight into LDS at m0 + 16*lane
// (m0 is an LDS byte address).  Issued through inline assembly on purpose: the
// compiler cannot tell which LDS bytes an LDS-DMA writes, so for the builtin it
// waits for every outstanding load before the next LDS read -- which would
// drain the whole prefetch pipeline each K-step.  The kernel orders the DMA
// itself with explicit vmcnt waits and barriers.  The s_nop covers the wait
// state required between writing M0 and an LDS-DMA that reads it.
MOE_DEV void dma16(const rsrc_t& r, uint32_t m0, uint32_t voff, uint32_t soff) {
    __asm__ volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds"
        :
        : "s"(uniform((int)m0)), "v"(voff), "s"(r), "s"(uniform((int)soff))
        : "memory", "m0");
}


}  // namespace moe
