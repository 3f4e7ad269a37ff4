// Vocabulary-parallel cross-entropy around the logits GEMMs of the output
// layer (Megatron-LM deep dive, vocabulary-parallel loss fusion section).
//
// Rank r holds the logits of its vocabulary slice [v0, v0 + n), n = V/p:
//   stats:   m_r = max_j logits, s_r = sum_j exp(logits - m_r), z_r = the
//            target's logit if the label is in the slice, else 0   (per token)
//   combine: the exchange of those aggregates, emulated over the ranks'
//            stats: m = max m_r, S = sum s_r exp(m_r - m), z = sum z_r,
//            lse = m + log S, loss = lse - z
//   dlogits: (exp(logits - lse) - onehot(label)) * dloss
// The products themselves (logits = X W^T, dX = dlogits W, dW = dlogits^T X)
// run on the matrix-core GEMM. All three kernels are HBM-bound.
#include "common.h"
#include "kernels.h"
#include "rowops.h"

namespace tpk {
namespace {

constexpr int CE_T = 256;

// One workgroup per token row of the slice; the row stays in registers
// between the max and the sum of exponentials. Loads use clamped chunks.
template <typename T, int NV>
__global__ __launch_bounds__(CE_T) void ce_stats_kernel(const T* __restrict__ logits, int n, int v0,
                                                        const int* __restrict__ labels, long rows,
                                                        float* __restrict__ stats) {
  __shared__ float red[CE_T / 64];
  const long t = blockIdx.x;
  const T* row = logits + t * n;
  const int nc = n >> 3;
  float v[NV][8];
  bool ok[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = threadIdx.x + i * CE_T;
    ok[i] = c < nc;
    load8(row + 8 * (ok[i] ? c : nc - 1), v[i]);
  }
  float m[1] = {-INFINITY};
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (ok[i]) {
#pragma unroll
      for (int e = 0; e < 8; ++e) m[0] = fmaxf(m[0], v[i][e]);
    }
  block_max<CE_T, 1>(m, red);
  float s[1] = {0.f};
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (ok[i]) {
#pragma unroll
      for (int e = 0; e < 8; ++e) s[0] += __expf(v[i][e] - m[0]);
    }
  block_sum<CE_T, 1>(s, red);
  if (threadIdx.x == 0) {
    const int lab = labels[t] - v0;
    stats[t] = m[0];
    stats[rows + t] = s[0];
    stats[2 * rows + t] = (lab >= 0 && lab < n) ? to_f(row[lab]) : 0.f;
  }
}

struct StatPtrs {
  const float* p[64];
};

__global__ __launch_bounds__(256) void ce_combine_kernel(StatPtrs parts, int n_parts, long rows, float* loss,
                                                         float* lse) {
  const long stride = (long)gridDim.x * 256;
  for (long t = (long)blockIdx.x * 256 + threadIdx.x; t < rows; t += stride) {
    float m = -INFINITY;
    for (int k = 0; k < n_parts; ++k) m = fmaxf(m, parts.p[k][t]);
    float S = 0.f, z = 0.f;
    for (int k = 0; k < n_parts; ++k) {
      S += parts.p[k][rows + t] * __expf(parts.p[k][t] - m);
      z += parts.p[k][2 * rows + t];
    }
    const float l = m + logf(S);
    lse[t] = l;
    loss[t] = l - z;
  }
}

// One thread per 8-element chunk of the [rows, n] slice.
template <typename T>
__global__ __launch_bounds__(256) void ce_dlogits_kernel(const T* __restrict__ logits, int n, int v0,
                                                         const int* __restrict__ labels,
                                                         const float* __restrict__ lse,
                                                         const float* __restrict__ dloss, long rows,
                                                         T* __restrict__ dl) {
  const int nc = n >> 3;
  const long total = rows * nc;
  const long stride = (long)gridDim.x * 256;
  for (long i = (long)blockIdx.x * 256 + threadIdx.x; i < total; i += stride) {
    const long t = i / nc;
    const int c = (int)(i - t * nc);
    float x[8];
    load8(logits + t * n + 8 * c, x);
    const float l = lse[t], g = dloss[t];
    const int lab = labels[t] - v0 - 8 * c;
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = (__expf(x[e] - l) - (e == lab ? 1.f : 0.f)) * g;
    store8(dl + t * n + 8 * c, x);
  }
}

unsigned grid_of(long long work) {
  long long g = (work + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (unsigned)g;
}

template <typename T>
hipError_t stats_t(const CeDesc& d, hipStream_t st) {
  const int nv = (d.n / 8 + CE_T - 1) / CE_T;
  const dim3 grid((unsigned)d.T), block(CE_T);
  const T* lg = (const T*)d.logits;
  if (nv <= 1) hipLaunchKernelGGL((ce_stats_kernel<T, 1>), grid, block, 0, st, lg, d.n, d.v0, d.labels, (long)d.T, d.stats);
  else if (nv <= 2) hipLaunchKernelGGL((ce_stats_kernel<T, 2>), grid, block, 0, st, lg, d.n, d.v0, d.labels, (long)d.T, d.stats);
  else if (nv <= 4) hipLaunchKernelGGL((ce_stats_kernel<T, 4>), grid, block, 0, st, lg, d.n, d.v0, d.labels, (long)d.T, d.stats);
  else if (nv <= 8) hipLaunchKernelGGL((ce_stats_kernel<T, 8>), grid, block, 0, st, lg, d.n, d.v0, d.labels, (long)d.T, d.stats);
  else if (nv <= 16) hipLaunchKernelGGL((ce_stats_kernel<T, 16>), grid, block, 0, st, lg, d.n, d.v0, d.labels, (long)d.T, d.stats);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace

hipError_t ce_stats_launch(int dtype, const CeDesc& d, hipStream_t stream) {
  if (d.T <= 0) return hipSuccess;
  return dtype == DT_BF16 ? stats_t<bf16>(d, stream) : stats_t<float>(d, stream);
}

hipError_t ce_combine_launch(const float* const* stats, int n_parts, long long rows, float* loss, float* lse,
                             hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  StatPtrs ps{};
  for (int k = 0; k < n_parts; ++k) ps.p[k] = stats[k];
  hipLaunchKernelGGL(ce_combine_kernel, dim3(grid_of(rows)), dim3(256), 0, stream, ps, n_parts, (long)rows, loss, lse);
  return hipGetLastError();
}

hipError_t ce_dlogits_launch(int dtype, const CeDesc& d, void* dl, hipStream_t stream) {
  if (d.T <= 0) return hipSuccess;
  const unsigned g = grid_of(d.T * (long long)(d.n / 8));
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(ce_dlogits_kernel<bf16>, dim3(g), dim3(256), 0, stream, (const bf16*)d.logits, d.n, d.v0,
                       d.labels, d.lse, d.dloss, (long)d.T, (bf16*)dl);
  else
    hipLaunchKernelGGL(ce_dlogits_kernel<float>, dim3(g), dim3(256), 0, stream, (const float*)d.logits, d.n, d.v0,
                       d.labels, d.lse, d.dloss, (long)d.T, (float*)dl);
  return hipGetLastError();
}

}  // namespace tpk
