// Device helpers of the row-wise (HBM-bound) kernels: packed 8-element
// vectors, an LDS-only workgroup barrier and fixed-order workgroup sums.
#pragma once
#include "common.h"

namespace tpk {

// Eight consecutive elements in the storage type, kept packed.
template <typename T> struct V8;
template <> struct V8<bf16> {
  bf16x8 v;
  __device__ __forceinline__ void load(const bf16* p) { v = *(const bf16x8*)p; }
  __device__ __forceinline__ float operator[](int e) const { return (float)v[e]; }
  // Make the packed value opaque to the compiler here, so that widened copies
  // made before this point are not kept alive past it (they are recomputed).
  __device__ __forceinline__ void opaque() { asm volatile("" : "+v"(v)); }
};
template <> struct V8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *(const f32x4*)p;
    b = *(const f32x4*)(p + 4);
  }
  __device__ __forceinline__ float operator[](int e) const { return e < 4 ? a[e] : b[e - 4]; }
  __device__ __forceinline__ void opaque() {}
};

// Buffer access to one row: a resource based at the row (workgroup-uniform,
// in scalar registers; `bytes` bounds it) and a per-lane byte offset, so one
// offset register per column chunk serves every row and array instead of a
// 64-bit address per chunk, row and array.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t row_rsrc(const void* row, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(row), (short)0, (int)bytes, 0x00020000);
}
template <typename T> __device__ __forceinline__ void load8_buf(V8<T>& v, __amdgpu_buffer_rsrc_t rs, uint32_t off);
template <> __device__ __forceinline__ void load8_buf<bf16>(V8<bf16>& v, __amdgpu_buffer_rsrc_t rs, uint32_t off) {
  v.v = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0));
}
template <> __device__ __forceinline__ void load8_buf<float>(V8<float>& v, __amdgpu_buffer_rsrc_t rs, uint32_t off) {
  v.a = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off, 0, 0));
  v.b = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, (int)off + 16, 0, 0));
}
__device__ __forceinline__ void store8_buf(bf16, __amdgpu_buffer_rsrc_t rs, uint32_t off, const float (&x)[8]) {
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (bf16)x[e];
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rs, (int)off, 0, 0);
}
__device__ __forceinline__ void store8_buf(float, __amdgpu_buffer_rsrc_t rs, uint32_t off, const float (&x)[8]) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{x[0], x[1], x[2], x[3]}), rs, (int)off, 0, 0);
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{x[4], x[5], x[6], x[7]}), rs, (int)off + 16,
                                         0, 0);
}

template <typename T> __device__ __forceinline__ void load8(const T* p, float (&x)[8]) {
  V8<T> v;
  v.load(p);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] = v[e];
}
__device__ __forceinline__ void store8(bf16* p, const float (&x)[8]) {
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (bf16)x[e];
  *(bf16x8*)p = v;
}
__device__ __forceinline__ void store8(float* p, const float (&x)[8]) {
  *(f32x4*)p = f32x4{x[0], x[1], x[2], x[3]};
  *(f32x4*)(p + 4) = f32x4{x[4], x[5], x[6], x[7]};
}

// Workgroup barrier for LDS exchanges only: this thread's LDS accesses have
// completed, then s_barrier. Unlike __syncthreads it does not wait for
// outstanding global loads and stores.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Sum of K values over the workgroup (NT threads); every thread receives the
// totals, formed in one fixed order. `red` holds NT/64 * K floats.
template <int NT, int K>
__device__ __forceinline__ void block_sum(float (&x)[K], float* red) {
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x[k] += __shfl_xor(x[k], o);
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
#pragma unroll
    for (int k = 0; k < K; ++k) red[w * K + k] = x[k];
  }
  lds_barrier();
#pragma unroll
  for (int k = 0; k < K; ++k) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) s += red[i * K + k];
    x[k] = s;
  }
  lds_barrier();  // `red` may be written again after this
}

// Maximum of K values over the workgroup (same pattern as block_sum).
template <int NT, int K>
__device__ __forceinline__ void block_max(float (&x)[K], float* red) {
#pragma unroll
  for (int k = 0; k < K; ++k)
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x[k] = fmaxf(x[k], __shfl_xor(x[k], o));
  const int w = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
#pragma unroll
    for (int k = 0; k < K; ++k) red[w * K + k] = x[k];
  }
  lds_barrier();
#pragma unroll
  for (int k = 0; k < K; ++k) {
    float m = red[k];
#pragma unroll
    for (int i = 1; i < NT / 64; ++i) m = fmaxf(m, red[i * K + k]);
    x[k] = m;
  }
  lds_barrier();
}

}  // namespace tpk
