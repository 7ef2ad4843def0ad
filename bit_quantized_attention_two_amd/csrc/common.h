// Shared device-side types and helpers of libminikv (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace minikv {

typedef _Float16 half_t;
typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef float float16_t __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float h2f(uint16_t b) {
    return (float)__builtin_bit_cast(half_t, b);
}
__device__ __forceinline__ uint16_t f2h_bits(float x) {
    return __builtin_bit_cast(uint16_t, (half_t)x);   // v_cvt_f16_f32, RNE
}

// 32x32x16 fp16 MFMA: A lane l holds A[l%32][8(l/32)+j], B lane l holds
// B[8(l/32)+j][l%32], C lane l register i holds
// C[8(i/4) + 4(l/32) + i%4][l%32].
__device__ __forceinline__ float16_t mfma32(half8_t a, half8_t b,
                                            float16_t c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Cross-lane exchange with lane ^ mask (ds_bpermute / DPP chosen by the
// compiler).
__device__ __forceinline__ float shfl_xor(float v, int mask) {
    return __shfl_xor(v, mask, 64);
}

}  // namespace minikv
