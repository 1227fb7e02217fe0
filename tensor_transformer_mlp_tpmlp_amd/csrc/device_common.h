// Device-side types and helpers shared by the tpmlp HIP kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tpmlp {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// sqrt(2/pi) and the cubic coefficient of the GPT-2 tanh approximation of
// GeLU ("Tensor-Parallel MLP (Megatron)", section "GeLU").
constexpr float kGeluC = 0.7978845608028654f;
constexpr float kGeluA = 0.044715f;

// GeLU_tanh(x) = x/2 (1 + tanh u), u = sqrt(2/pi) (x + 0.044715 x^3).
// Evaluated as x * sigmoid(2u) = x / (1 + exp(-2u)), which is the same
// function since (1 + tanh u)/2 = 1/(1 + exp(-2u)).  With exp(-2u) =
// 2^(x (k0 + k1 x^2)), k0 = -2 sqrt(2/pi) log2(e) and k1 = 0.044715 k0, that
// is two multiplies, one fma, one v_exp_f32, one add, one v_rcp_f32 and one
// multiply.  2^(...) overflows to +inf for very negative x, giving -0; it
// underflows to 0 for large x, giving x.  NaN propagates.
constexpr double kLog2e = 1.4426950408889634;
constexpr float kGeluK0 = (float)(-2.0 * (double)kGeluC * kLog2e);
constexpr float kGeluK1 = (float)(-2.0 * (double)kGeluC * (double)kGeluA * kLog2e);
__device__ __forceinline__ float gelu_tanh(float x) {
    const float z = x * __builtin_fmaf(x * x, kGeluK1, kGeluK0);
    return x * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z));
}

// d/dx GeLU_tanh(x), for the backward pass.  With s = (1 + tanh u)/2 =
// 1/(1 + exp(-2u)) and 1 - tanh^2 u = 4 s (1 - s), the product and chain
// rules give s (1 + q (1 - s)), q = 2 sqrt(2/pi) x (1 + 3 * 0.044715 x^2).
// exp(-2u) overflows to +inf for very negative x; then s = 0 and the result
// is 0 (without the select, 0 * x^3 could become NaN for huge |x|).
__device__ __forceinline__ float gelu_tanh_grad(float x) {
    const float z = x * __builtin_fmaf(x * x, kGeluK1, kGeluK0);
    const float s = __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z));
    const float q = (2.0f * kGeluC) * x * __builtin_fmaf((3.0f * kGeluA) * x, x, 1.0f);
    const float r = s * __builtin_fmaf(q, 1.0f - s, 1.0f);
    return s == 0.0f ? 0.0f : r;
}

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return static_cast<float>(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return static_cast<bf16>(v); }

}  // namespace tpmlp
