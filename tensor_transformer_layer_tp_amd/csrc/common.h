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

// tanh-form GeLU and its derivative in fp32.
// gelu(x) = 0.5 x (1 + tanh(u)), u = sqrt(2/pi) (x + 0.044715 x^3).
// tanh(u) is evaluated as 1 - 2 / (exp(2u) + 1), which saturates correctly
// for large |u| (exp overflow to inf gives 1, underflow to 0 gives -1).
__device__ __forceinline__ float tanh_via_exp(float u) {
  float e = __expf(2.0f * u);
  return 1.0f - 2.0f / (e + 1.0f);
}
__device__ __forceinline__ float gelu_f(float x) {
  const float k0 = 0.7978845608028654f;
  float u = k0 * (x + 0.044715f * x * x * x);
  return 0.5f * x * (1.0f + tanh_via_exp(u));
}
__device__ __forceinline__ float gelu_grad_f(float x) {
  const float k0 = 0.7978845608028654f;
  float x2 = x * x;
  float u = k0 * (x + 0.044715f * x2 * x);
  float t = tanh_via_exp(u);
  float du = k0 * (1.0f + 3.0f * 0.044715f * x2);
  return 0.5f * (1.0f + t) + 0.5f * x * (1.0f - t * t) * du;
}

template <typename T> __device__ __forceinline__ float to_f(T v);
template <> __device__ __forceinline__ float to_f<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f<bf16>(bf16 v) { return (float)v; }
template <typename T> __device__ __forceinline__ T from_f(float v);
template <> __device__ __forceinline__ float from_f<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f<bf16>(float v) { return (bf16)v; }

}  // namespace tpk
