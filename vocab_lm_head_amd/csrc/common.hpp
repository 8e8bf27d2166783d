// Device-side vector types and small helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace vp {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__host__ __device__ constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
__host__ __device__ constexpr int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Four fp32 -> four bf16 (round to nearest even, v_cvt_pk_bf16_f32), packed in 8 bytes.
__device__ __forceinline__ u32x2 pack_bf16x4(float a, float b, float c, float d) {
    bf16x4 v;
    v[0] = (__bf16)a;
    v[1] = (__bf16)b;
    v[2] = (__bf16)c;
    v[3] = (__bf16)d;
    return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ uint16_t bf16_bits(float a) {
    return __builtin_bit_cast(uint16_t, (__bf16)a);
}

}  // namespace vp
