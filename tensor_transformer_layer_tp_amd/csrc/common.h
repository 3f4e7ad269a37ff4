// Internal device helpers shared by the HIP kernels of the layer shard.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kernels.h"

namespace tpk {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// tanh-form GeLU and its derivative in fp32:
// gelu(x) = 0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3).
// With s = (1 + tanh(u)) / 2 = 1 / (1 + exp(-2u)) (the logistic function of
// 2u): gelu(x) = x s, and gelu'(x) = s + 2 x s (1 - s) u'(x),
// u'(x) = sqrt(2/pi) (1 + 3 * 0.044715 x^2). exp(-2u) is one hardware 2^w
// (w = -2u log2(e)) and 1 / (1 + exp(-2u)) one hardware reciprocal (both
// within a few ulp, far below the outputs' bf16 rounding; an IEEE division
// costs about ten instructions). Saturates correctly: 2^w overflows to inf
// for very negative x (s = 0) and underflows to 0 for large x (s = 1).
constexpr float kGeluK0 = 0.7978845608028654f;                    // sqrt(2/pi)
constexpr float kGeluW = -2.0f * 0.7978845608028654f * 1.4426950408889634f;  // -2 sqrt(2/pi) log2(e)
__device__ __forceinline__ float gelu_logistic(float x, float x2) {
  const float w = (kGeluW * x) * fmaf(0.044715f, x2, 1.0f);
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(w));
}
__device__ __forceinline__ float gelu_f(float x) { return x * gelu_logistic(x, x * x); }
__device__ __forceinline__ float gelu_grad_f(float x) {
  const float x2 = x * x;
  const float s = gelu_logistic(x, x2);
  const float du = fmaf(3.0f * 0.044715f * kGeluK0, x2, kGeluK0);
  return fmaf(2.0f * x * du, fmaf(-s, s, s), s);
}

template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16>(bf16 v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float v) { return (bf16)v; }

}  // namespace tpk
