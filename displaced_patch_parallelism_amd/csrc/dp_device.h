// Device-side helpers shared by the kernel translation units (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// float -> bf16, round to nearest even (the hardware conversion).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// Two floats -> packed bf16 pair (low half = a), round to nearest even: one
// v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    typedef float f32x2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    const f32x2_t v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Make every word of a kernel's argument block live in SGPRs at this point.  Left to itself
// the compiler requests argument fields lazily, next to their first use, and may re-request
// them after register pressure has pushed other values out to scratch; an empty asm that takes
// every word as an SGPR operand puts all the requests ahead of one wait at kernel entry.
template <typename T>
__device__ __forceinline__ void args_in_sgprs(const T& a) {
    static_assert(sizeof(T) % 4 == 0, "argument block of whole dwords");
    const uint32_t* w = reinterpret_cast<const uint32_t*>(&a);
#pragma unroll
    for (int i = 0; i < (int)(sizeof(T) / 4); ++i) asm volatile("" ::"s"(w[i]));
}

// The same for kernels whose arguments are separate parameters.
template <typename T>
__device__ __forceinline__ void sgpr_operand(T v) {
    asm volatile("" ::"s"(v));
}
template <typename... T>
__device__ __forceinline__ void params_in_sgprs(T... v) {
    (sgpr_operand(v), ...);
}

// Unpack a 16-byte vector of 8 bf16 into floats.
__device__ __forceinline__ void unpack8(const uint4& v, float* f) {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        f[2 * j] = __uint_as_float(w[j] << 16);
        f[2 * j + 1] = __uint_as_float(w[j] & 0xffff0000u);
    }
}

__device__ __forceinline__ uint4 pack8(const float* f) {
    uint4 v;
    v.x = pack_bf16x2(f[0], f[1]);
    v.y = pack_bf16x2(f[2], f[3]);
    v.z = pack_bf16x2(f[4], f[5]);
    v.w = pack_bf16x2(f[6], f[7]);
    return v;
}

// SiLU y * sigmoid(y) as y * rcp(1 + 2^(-y log2 e)): v_exp_f32 and v_rcp_f32 (about 1 ulp
// each) instead of an IEEE division.  Saturates correctly: exp overflows to inf for y << 0
// (rcp gives 0, so the result is -0) and underflows to 0 for y >> 0 (result y).
__device__ __forceinline__ float silu(float y) {
    return y * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-y * 1.4426950408889634f));
}

}  // namespace dp
