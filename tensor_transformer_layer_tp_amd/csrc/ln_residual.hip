// Residual add + LayerNorm after a tensor-parallel block, forward and backward.
//
// The layer wraps its attention and MLP blocks in residual connections and
// layer normalizations (Megatron-LM deep dive, Fig. 2); g completes each
// block's output before the residual add (same page, Fig. 4), and the
// Megatron-DeepSpeed blog (section 4.3) fuses the residual add into the
// LayerNorm kernel. Definitions (h = hidden, per token row t):
//
//   r    = resid_in + sum_k parts[k] + bias      stored in the storage type
//   mu   = mean_j r,  var = mean_j (r - mu)^2,   rstd = 1 / sqrt(var + eps)
//   y    = (r - mu) rstd gamma + beta
//
//   backward (dy = dL/dy, dr_in = gradient reaching r along the residual path):
//   xhat = (r - mu) rstd,  g = dy gamma
//   dr   = dr_in + rstd (g - mean_j g - xhat mean_j (g xhat))
//   dgamma = sum_t dy xhat,  dbeta = sum_t dy,  dbias = sum_t dr
//
// Both directions are HBM-bound (a few flops per element): each tensor is
// read or written once, in 16-byte vectors of 8 elements. The statistics are
// taken over the stored (rounded) r, so the backward pass, which rereads r,
// sees exactly the values the forward pass normalized.
//
// Forward: one workgroup of 1024 threads per row; the row stays in registers
// between the two reductions (mean, then variance about the mean).
// Backward: one workgroup of 512 threads per run of rows; each thread owns
// the same columns in every row of its run and keeps fp32 column partials of
// dy xhat, dy and dr in registers; a second kernel adds the runs' partials in
// a fixed order (no atomics: results do not depend on scheduling).
#include "common.h"
#include "kernels.h"

namespace tpk {
namespace {

constexpr int FWD_T = 1024;
constexpr int BWD_T = 512;
constexpr int BWD_RUNS = 256;  // target number of row runs (one per CU)

// Eight consecutive elements in the storage type, kept packed.
template <typename T> struct V8;
template <> struct V8<bf16> {
  bf16x8 v;
  __device__ __forceinline__ void load(const bf16* p) { v = *(const bf16x8*)p; }
  __device__ __forceinline__ float operator[](int e) const { return (float)v[e]; }
};
template <> struct V8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *(const f32x4*)p;
    b = *(const f32x4*)(p + 4);
  }
  __device__ __forceinline__ float operator[](int e) const { return e < 4 ? a[e] : b[e - 4]; }
};

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
  __syncthreads();
#pragma unroll
  for (int k = 0; k < K; ++k) {
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < NT / 64; ++i) s += red[i * K + k];
    x[k] = s;
  }
  __syncthreads();  // `red` may be written again after this
}

struct PartPtrs {
  const void* p[64];
};

template <typename T, int NV>
__global__ __launch_bounds__(FWD_T) void ln_residual_fwd_kernel(const T* __restrict__ resid_in, PartPtrs parts,
                                                                int n_parts, const T* __restrict__ bias,
                                                                const T* __restrict__ gamma,
                                                                const T* __restrict__ beta, float eps, int h,
                                                                T* __restrict__ resid_out, T* __restrict__ y,
                                                                float* __restrict__ mean, float* __restrict__ rstd) {
  __shared__ float red[FWD_T / 64];
  const long base = (long)blockIdx.x * h;
  const int nc = h >> 3;
  float v[NV][8];
  float s[1] = {0.f};
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = threadIdx.x + i * FWD_T;
    if (c >= nc) continue;
    load8(resid_in + base + 8 * c, v[i]);
    for (int k = 0; k < n_parts; ++k) {
      float p[8];
      load8((const T*)parts.p[k] + base + 8 * c, p);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] += p[e];
    }
    if (bias) {
      float b[8];
      load8(bias + 8 * c, b);
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] += b[e];
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) v[i][e] = to_f(from_f<T>(v[i][e]));  // the value stored
    store8(resid_out + base + 8 * c, v[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) s[0] += v[i][e];
  }
  block_sum<FWD_T, 1>(s, red);
  const float mu = s[0] / (float)h;
  float q[1] = {0.f};
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (threadIdx.x + i * FWD_T >= nc) continue;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = v[i][e] - mu;
      q[0] += d * d;
    }
  }
  block_sum<FWD_T, 1>(q, red);
  const float rs = 1.0f / sqrtf(q[0] / (float)h + eps);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = threadIdx.x + i * FWD_T;
    if (c >= nc) continue;
    float gm[8], bt[8], o[8];
    load8(gamma + 8 * c, gm);
    load8(beta + 8 * c, bt);
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (v[i][e] - mu) * rs * gm[e] + bt[e];
    store8(y + base + 8 * c, o);
  }
  if (threadIdx.x == 0) {
    mean[blockIdx.x] = mu;
    rstd[blockIdx.x] = rs;
  }
}

// Rows [run * rows_per, ...) of the backward pass; writes dr and this run's
// column partials part[(3 run + j) h + col], j = 0: dy xhat, 1: dy, 2: dr.
template <typename T, int NV>
__global__ __launch_bounds__(BWD_T) void ln_residual_bwd_kernel(const T* __restrict__ r, const float* __restrict__ mean,
                                                                const float* __restrict__ rstd,
                                                                const T* __restrict__ gamma, const T* __restrict__ dy,
                                                                const T* __restrict__ dr_in, int h, long rows,
                                                                int rows_per, T* __restrict__ dr,
                                                                float* __restrict__ part) {
  __shared__ float red[2 * BWD_T / 64];
  const int nc = h >> 3;
  const long r0 = (long)blockIdx.x * rows_per;
  const long r1 = r0 + rows_per < rows ? r0 + rows_per : rows;
  V8<T> gm[NV];
  float ag[NV][8], ab[NV][8], ar[NV][8];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = threadIdx.x + i * BWD_T;
    if (c < nc) gm[i].load(gamma + 8 * c);
#pragma unroll
    for (int e = 0; e < 8; ++e) ag[i][e] = ab[i][e] = ar[i][e] = 0.f;
  }
  for (long t = r0; t < r1; ++t) {
    const long base = t * h;
    const float mu = mean[t], rs = rstd[t];
    V8<T> dyv[NV], rv[NV];
    float s[2] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = threadIdx.x + i * BWD_T;
      if (c >= nc) continue;
      dyv[i].load(dy + base + 8 * c);
      rv[i].load(r + base + 8 * c);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float g = dyv[i][e] * gm[i][e];
        s[0] += g;
        s[1] += g * ((rv[i][e] - mu) * rs);
      }
    }
    block_sum<BWD_T, 2>(s, red);
    const float a = s[0] / (float)h, b = s[1] / (float)h;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int c = threadIdx.x + i * BWD_T;
      if (c >= nc) continue;
      float o[8];
      if (dr_in) load8(dr_in + base + 8 * c, o);
      else {
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float xh = (rv[i][e] - mu) * rs;
        o[e] += rs * (dyv[i][e] * gm[i][e] - a - xh * b);
        ag[i][e] += dyv[i][e] * xh;
        ab[i][e] += dyv[i][e];
        ar[i][e] += o[e];
      }
      store8(dr + base + 8 * c, o);
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = threadIdx.x + i * BWD_T;
    if (c >= nc) continue;
    float* p = part + (long)3 * blockIdx.x * h + 8 * c;
    store8(p, ag[i]);
    store8(p + h, ab[i]);
    store8(p + 2 * h, ar[i]);
  }
}

// out_j[col] = sum over runs of part[(3 run + j) h + col], runs in order;
// 4 column vectors x 64 threads per workgroup, 4 thread rows split the runs
// (interleaved) and are added in a fixed order.
template <typename T>
__global__ __launch_bounds__(256) void ln_residual_bwd_final_kernel(const float* __restrict__ part, int runs, int h,
                                                                    T* dgamma, T* dbeta, T* dbias) {
  __shared__ f32x4 red[3][64];
  const int j = blockIdx.y;
  T* out = j == 0 ? dgamma : (j == 1 ? dbeta : dbias);
  if (!out) return;  // uniform over the workgroup
  const int tc = threadIdx.x & 63, tr = threadIdx.x >> 6;
  const int col = 4 * (blockIdx.x * 64 + tc);
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  if (col < h) {
    for (int w = tr; w < runs; w += 4) s += *(const f32x4*)(part + ((long)3 * w + j) * h + col);
  }
  if (tr > 0) red[tr - 1][tc] = s;
  __syncthreads();
  if (tr == 0 && col < h) {
#pragma unroll
    for (int k = 0; k < 3; ++k) s += red[k][tc];
#pragma unroll
    for (int e = 0; e < 4; ++e) out[col + e] = from_f<T>(s[e]);
  }
}

int ln_runs(long long rows, int& rows_per) {
  rows_per = (int)((rows + BWD_RUNS - 1) / BWD_RUNS);
  if (rows_per < 1) rows_per = 1;
  return (int)((rows + rows_per - 1) / rows_per);
}

template <typename T, int NV>
void fwd_nv(const LnDesc& d, const PartPtrs& ps, hipStream_t st) {
  hipLaunchKernelGGL((ln_residual_fwd_kernel<T, NV>), dim3((unsigned)d.T), dim3(FWD_T), 0, st,
                     (const T*)d.resid_in, ps, d.n_parts, (const T*)d.bias, (const T*)d.gamma, (const T*)d.beta,
                     d.eps, d.h, (T*)d.resid_out, (T*)d.y, d.mean, d.rstd);
}

template <typename T>
hipError_t fwd_t(const LnDesc& d, hipStream_t st) {
  PartPtrs ps{};
  for (int k = 0; k < d.n_parts; ++k) ps.p[k] = d.parts[k];
  const int nv = (d.h / 8 + FWD_T - 1) / FWD_T;
  switch (nv) {
    case 1: fwd_nv<T, 1>(d, ps, st); break;
    case 2: fwd_nv<T, 2>(d, ps, st); break;
    case 3: fwd_nv<T, 3>(d, ps, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T, int NV>
void bwd_nv(const LnDesc& d, int runs, int rows_per, float* part, hipStream_t st) {
  hipLaunchKernelGGL((ln_residual_bwd_kernel<T, NV>), dim3(runs), dim3(BWD_T), 0, st, (const T*)d.resid_out,
                     (const float*)d.mean, (const float*)d.rstd, (const T*)d.gamma, (const T*)d.dy,
                     (const T*)d.dr_in, d.h, (long)d.T, rows_per, (T*)d.dr, part);
}

template <typename T>
hipError_t bwd_t(const LnDesc& d, float* part, hipStream_t st) {
  int rows_per = 1;
  const int runs = ln_runs(d.T, rows_per);
  const int nv = (d.h / 8 + BWD_T - 1) / BWD_T;
  switch (nv) {
    case 1: bwd_nv<T, 1>(d, runs, rows_per, part, st); break;
    case 2: bwd_nv<T, 2>(d, runs, rows_per, part, st); break;
    case 3: bwd_nv<T, 3>(d, runs, rows_per, part, st); break;
    case 4: bwd_nv<T, 4>(d, runs, rows_per, part, st); break;
    case 5: bwd_nv<T, 5>(d, runs, rows_per, part, st); break;
    case 6: bwd_nv<T, 6>(d, runs, rows_per, part, st); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid((unsigned)((d.h / 4 + 63) / 64), 3);
  hipLaunchKernelGGL(ln_residual_bwd_final_kernel<T>, grid, dim3(256), 0, st, (const float*)part, runs, d.h,
                     (T*)d.dgamma, (T*)d.dbeta, (T*)d.dbias);
  return hipGetLastError();
}

}  // namespace

size_t ln_bwd_workspace_bytes(long long rows, int h) {
  if (rows <= 0) return 0;
  int rows_per = 1;
  return (size_t)ln_runs(rows, rows_per) * 3 * (size_t)h * sizeof(float);
}

hipError_t ln_fwd_launch(int dtype, const LnDesc& d, hipStream_t stream) {
  if (d.T <= 0) return hipSuccess;
  return dtype == DT_BF16 ? fwd_t<bf16>(d, stream) : fwd_t<float>(d, stream);
}

hipError_t ln_bwd_launch(int dtype, const LnDesc& d, void* ws, hipStream_t stream) {
  if (d.T <= 0) {  // no rows: the column sums are zero
    hipError_t e = zero_launch(dtype, d.dgamma, 1, d.h, d.h, stream);
    if (e == hipSuccess) e = zero_launch(dtype, d.dbeta, 1, d.h, d.h, stream);
    if (e == hipSuccess && d.dbias) e = zero_launch(dtype, d.dbias, 1, d.h, d.h, stream);
    return e;
  }
  return dtype == DT_BF16 ? bwd_t<bf16>(d, (float*)ws, stream) : bwd_t<float>(d, (float*)ws, stream);
}

}  // namespace tpk
