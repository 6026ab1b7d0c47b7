// Internal helpers shared by the gfx950 KDA kernels (device side) and the host dispatch.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2;

constexpr float kLog2e = 1.4426950408889634f;

// exp(x) through the hardware exp2 (one v_exp_f32 after a multiply).
__device__ __forceinline__ float fexp(float x) { return __builtin_amdgcn_exp2f(x * kLog2e); }

__device__ __forceinline__ float bf16lo_to_f(uint32_t packed) { return __uint_as_float(packed << 16); }
__device__ __forceinline__ float bf16hi_to_f(uint32_t packed) { return __uint_as_float(packed & 0xffff0000u); }

// Two floats -> packed bf16 pair (round to nearest even), low half = a.
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}
// Two floats -> packed f16 pair (round to nearest even), low half = a.
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, f16x2));
}
// Split a pair into bf16 hi + bf16 lo with a ~= hi + lo to about 16 significant bits.
// The remainders a - hi_a and b - hi_b are exact in float32.  Each is one v_dot2c_f32_bf16 of the
// packed hi with (-1, 0) or (0, -1), accumulated onto a or b, which saves unpacking hi into two
// floats; the result is bit for bit that of the plain subtraction (denormals included) for every
// finite pair whose hi does not round to infinity.  The (-1, 0) pair (0x0000bf80) is kept in a
// scalar register: the compiler folds it into the inline constant -1.0, which this instruction
// applies as the float32 bit pattern 0xbf800000, i.e. as (0, -1).
// a - (low half of hi as a float), b - (high half of hi as a float)
__device__ __forceinline__ float remainder_lo(uint32_t hi, float a) {
    uint32_t m_lo;
    asm("s_mov_b32 %0, 0xbf80" : "=s"(m_lo));
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, hi), __builtin_bit_cast(bf16x2, m_lo), a, false);
}
__device__ __forceinline__ float remainder_hi(uint32_t hi, float b) {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, hi), __builtin_bit_cast(bf16x2, 0xbf800000u), b,
                                           false);
}
__device__ __forceinline__ void split_bf16(float a, float b, uint32_t& hi, uint32_t& lo) {
    hi = pack_bf16(a, b);
    lo = pack_bf16(remainder_lo(hi, a), remainder_hi(hi, b));
}

// Workgroup barrier that orders LDS only (in-flight global loads and stores are not waited for).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                   0, 0, 0);
}
// 16x16x16 bf16: lane group g holds contraction indices 4g..4g+3 (one 8-byte operand)
typedef __attribute__((ext_vector_type(4))) short s16x4;
__device__ __forceinline__ f32x4 mfma_bf16_k16(u32x2 a, u32x2 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b), c,
                                                     0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f16(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c,
                                                  0, 0, 0);
}

}  // namespace kda
