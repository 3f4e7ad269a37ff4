// Per-head causal attention on the vector ALUs: the path for fp32 storage and
// for head widths the matrix-core kernels do not instantiate. One workgroup per
// (query or key row, local head, batch element); qkv is fp32, ctx / dctx /
// dqkv use the storage type T. Keys are visited 128 at a time
// with a running max / sum (online softmax), so memory stays O(d) per row.
// Also: delta = rowsum(dctx * ctx), the softmax-backward row term, for both paths.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace tpk {

hipError_t attn_mfma_fwd(const AttnDesc& a, hipStream_t stream);
hipError_t attn_mfma_bwd(const AttnDesc& a, hipStream_t stream);

namespace {

constexpr int NT = 128;

__device__ __forceinline__ float block_max(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return fmaxf(red[0], red[1]);
}
__device__ __forceinline__ float block_sum(float v, float* red) {
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int w = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[w] = v;
  __syncthreads();
  return red[0] + red[1];
}

struct SP {
  int batch, seq, n_local, d, h_l, head0, n_heads, alibi;
  const float* qkv; void* ctx; float* lse; const void* dctx; const float* delta; void* dqkv;
};

__device__ __forceinline__ float slope_of(const SP& p, int l) {
  // ALiBi slope of global head k = head0 + l + 1 (1-based): 2^(-8k/n_heads)
  return p.alibi ? exp2f(-8.0f * (float)(p.head0 + l + 1) / (float)p.n_heads) : 0.0f;
}

template <typename T>
__global__ __launch_bounds__(NT) void fwd_kernel(SP p) {
  __shared__ float sq[256];
  __shared__ float sp[NT];
  __shared__ float red[2];
  const int i = blockIdx.x, l = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int d = p.d;
  const long ld = 3L * p.h_l;
  const float* qkv = p.qkv;
  const long row0 = (long)b * p.seq;
  const float* q = qkv + (row0 + i) * ld + (long)l * d;
  const float* kb = qkv + row0 * ld + p.h_l + (long)l * d;
  const float* vb = qkv + row0 * ld + 2L * p.h_l + (long)l * d;
  const float scale = 1.0f / sqrtf((float)d), slope = slope_of(p, l);
  for (int dd = tid; dd < d; dd += NT) sq[dd] = to_f(q[dd]) * scale;
  __syncthreads();
  float m = -INFINITY, lsum = 0.f, acc0 = 0.f, acc1 = 0.f;
  for (int j0 = 0; j0 <= i; j0 += NT) {
    const int j = j0 + tid;
    float s = -INFINITY;
    if (j <= i) {
      const float* kj = kb + (long)j * ld;
      float dot = 0.f;
      for (int dd = 0; dd < d; ++dd) dot = fmaf(sq[dd], to_f(kj[dd]), dot);
      s = dot - slope * (float)(i - j);
    }
    const float mn = fmaxf(m, block_max(s, red));
    const float pj = (j <= i) ? expf(s - mn) : 0.f;
    const float corr = expf(m - mn);
    const float csum = block_sum(pj, red);
    sp[tid] = pj;
    __syncthreads();
    lsum = lsum * corr + csum;
    const int cnt = min(NT, i - j0 + 1);
    if (tid < d) {
      float a = acc0 * corr;
      for (int jj = 0; jj < cnt; ++jj) a = fmaf(sp[jj], to_f(vb[(long)(j0 + jj) * ld + tid]), a);
      acc0 = a;
    }
    if (tid + NT < d) {
      float a = acc1 * corr;
      for (int jj = 0; jj < cnt; ++jj) a = fmaf(sp[jj], to_f(vb[(long)(j0 + jj) * ld + tid + NT]), a);
      acc1 = a;
    }
    m = mn;
    __syncthreads();
  }
  T* ctx = (T*)p.ctx + (row0 + i) * p.h_l + (long)l * d;
  if (tid < d) ctx[tid] = from_f<T>(acc0 / lsum);
  if (tid + NT < d) ctx[tid + NT] = from_f<T>(acc1 / lsum);
  if (tid == 0) p.lse[((long)b * p.n_local + l) * p.seq + i] = m + logf(lsum);
}

// dQ for query row i: dq = scale * sum_{j<=i} P_ij (dP_ij - delta_i) k_j,
// P_ij = exp(s_ij - lse_i), dP_ij = dctx_i . v_j.
template <typename T>
__global__ __launch_bounds__(NT) void dq_kernel(SP p) {
  __shared__ float sq[256], sdc[256];
  __shared__ float sds[NT];
  const int i = blockIdx.x, l = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int d = p.d;
  const long ld = 3L * p.h_l;
  const float* qkv = p.qkv;
  const long row0 = (long)b * p.seq;
  const float scale = 1.0f / sqrtf((float)d), slope = slope_of(p, l);
  const float* q = qkv + (row0 + i) * ld + (long)l * d;
  const T* dc = (const T*)p.dctx + (row0 + i) * p.h_l + (long)l * d;
  const float* kb = qkv + row0 * ld + p.h_l + (long)l * d;
  const float* vb = qkv + row0 * ld + 2L * p.h_l + (long)l * d;
  for (int dd = tid; dd < d; dd += NT) { sq[dd] = to_f(q[dd]) * scale; sdc[dd] = to_f(dc[dd]); }
  __syncthreads();
  const long hr = ((long)b * p.n_local + l) * p.seq + i;
  const float lse = p.lse[hr], dl = p.delta[hr];
  float a0 = 0.f, a1 = 0.f;
  for (int j0 = 0; j0 <= i; j0 += NT) {
    const int j = j0 + tid;
    float ds = 0.f;
    if (j <= i) {
      const float* kj = kb + (long)j * ld;
      const float* vj = vb + (long)j * ld;
      float s = 0.f, dp = 0.f;
      for (int dd = 0; dd < d; ++dd) {
        s = fmaf(sq[dd], to_f(kj[dd]), s);
        dp = fmaf(sdc[dd], to_f(vj[dd]), dp);
      }
      const float pij = expf(s - slope * (float)(i - j) - lse);
      ds = pij * (dp - dl);
    }
    sds[tid] = ds;
    __syncthreads();
    const int cnt = min(NT, i - j0 + 1);
    if (tid < d)
      for (int jj = 0; jj < cnt; ++jj) a0 = fmaf(sds[jj], to_f(kb[(long)(j0 + jj) * ld + tid]), a0);
    if (tid + NT < d)
      for (int jj = 0; jj < cnt; ++jj) a1 = fmaf(sds[jj], to_f(kb[(long)(j0 + jj) * ld + tid + NT]), a1);
    __syncthreads();
  }
  T* dq = (T*)p.dqkv + (row0 + i) * ld + (long)l * d;
  if (tid < d) dq[tid] = from_f<T>(a0 * scale);
  if (tid + NT < d) dq[tid + NT] = from_f<T>(a1 * scale);
}

// dK, dV for key row j: dv = sum_{i>=j} P_ij dctx_i ; dk = scale * sum_{i>=j} dS_ij q_i.
template <typename T>
__global__ __launch_bounds__(NT) void dkdv_kernel(SP p) {
  __shared__ float sk[256], sv[256];
  __shared__ float spp[NT], sds[NT];
  const int j = blockIdx.x, l = blockIdx.y, b = blockIdx.z, tid = threadIdx.x;
  const int d = p.d;
  const long ld = 3L * p.h_l;
  const float* qkv = p.qkv;
  const long row0 = (long)b * p.seq;
  const float scale = 1.0f / sqrtf((float)d), slope = slope_of(p, l);
  const float* kj = qkv + (row0 + j) * ld + p.h_l + (long)l * d;
  const float* vj = qkv + (row0 + j) * ld + 2L * p.h_l + (long)l * d;
  const float* qb = qkv + row0 * ld + (long)l * d;
  const T* dcb = (const T*)p.dctx + row0 * p.h_l + (long)l * d;
  for (int dd = tid; dd < d; dd += NT) { sk[dd] = to_f(kj[dd]) * scale; sv[dd] = to_f(vj[dd]); }
  __syncthreads();
  const long hr0 = ((long)b * p.n_local + l) * p.seq;
  float v0 = 0.f, v1 = 0.f, k0 = 0.f, k1 = 0.f;
  for (int i0 = j; i0 < p.seq; i0 += NT) {
    const int i = i0 + tid;
    float pij = 0.f, ds = 0.f;
    if (i < p.seq) {
      const float* qi = qb + (long)i * ld;
      const T* dci = dcb + (long)i * p.h_l;
      float s = 0.f, dp = 0.f;
      for (int dd = 0; dd < d; ++dd) {
        s = fmaf(sk[dd], to_f(qi[dd]), s);
        dp = fmaf(sv[dd], to_f(dci[dd]), dp);
      }
      pij = expf(s - slope * (float)(i - j) - p.lse[hr0 + i]);
      ds = pij * (dp - p.delta[hr0 + i]);
    }
    spp[tid] = pij;
    sds[tid] = ds;
    __syncthreads();
    const int cnt = min(NT, p.seq - i0);
    for (int ii = 0; ii < cnt; ++ii) {
      const float pp = spp[ii], dd_ = sds[ii];
      const float* qi = qb + (long)(i0 + ii) * ld;
      const T* dci = dcb + (long)(i0 + ii) * p.h_l;
      if (tid < d) { v0 = fmaf(pp, to_f(dci[tid]), v0); k0 = fmaf(dd_, to_f(qi[tid]), k0); }
      if (tid + NT < d) { v1 = fmaf(pp, to_f(dci[tid + NT]), v1); k1 = fmaf(dd_, to_f(qi[tid + NT]), k1); }
    }
    __syncthreads();
  }
  T* dk = (T*)p.dqkv + (row0 + j) * ld + p.h_l + (long)l * d;
  T* dv = (T*)p.dqkv + (row0 + j) * ld + 2L * p.h_l + (long)l * d;
  if (tid < d) { dk[tid] = from_f<T>(k0 * scale); dv[tid] = from_f<T>(v0); }
  if (tid + NT < d) { dk[tid + NT] = from_f<T>(k1 * scale); dv[tid + NT] = from_f<T>(v1); }
}

// delta[b][l][i] = sum_d dctx[t][l*D + d] * ctx[t][l*D + d], t = b*seq + i.
// Row r = t*n_local + l is the run of D/8 16-byte chunks (8 elements each)
// starting at chunk r*D/8 of the flattened [T, h_l] arrays, so consecutive
// threads read consecutive chunks whatever D is. A workgroup takes DU groups
// of G = 256/(D/8) whole rows; thread c multiplies chunk c of every group
// (all loads issued first, clamped in range), the chunk sums go through LDS,
// and one thread per row adds its D/8 chunk sums in chunk order.
constexpr int DU = 4;
template <typename T>
__global__ __launch_bounds__(256) void delta_kernel(const T* dctx, const T* ctx, float* delta, int seq,
                                                    int n_local, int d, long rows) {
  __shared__ float part[DU][256];
  const int cpr = d >> 3, G = 256 / cpr, c = threadIdx.x;
  const long r0 = (long)blockIdx.x * DU * G, chunks = rows * cpr;
  float x[DU][8], y[DU][8];
#pragma unroll
  for (int u = 0; u < DU; ++u) {
    const long q = (r0 + (long)u * G) * cpr + c;
    const long qq = q < chunks ? q : chunks - 1;
    const T* a = dctx + 8 * qq;
    const T* b = ctx + 8 * qq;
    if constexpr (sizeof(T) == 2) {
      const bf16x8 va = *(const bf16x8*)a, vb = *(const bf16x8*)b;
#pragma unroll
      for (int e = 0; e < 8; ++e) { x[u][e] = (float)va[e]; y[u][e] = (float)vb[e]; }
    } else {
      const f32x4 a0 = *(const f32x4*)a, a1 = *(const f32x4*)(a + 4);
      const f32x4 b0 = *(const f32x4*)b, b1 = *(const f32x4*)(b + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        x[u][e] = a0[e]; x[u][4 + e] = a1[e];
        y[u][e] = b0[e]; y[u][4 + e] = b1[e];
      }
    }
  }
#pragma unroll
  for (int u = 0; u < DU; ++u) {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s = fmaf(x[u][e], y[u][e], s);
    part[u][c] = s;
  }
  __syncthreads();
  for (int k = c; k < DU * G; k += 256) {
    const int u = k / G, j = k - u * G;
    const long r = r0 + (long)u * G + j;
    if (r >= rows) continue;
    float s = 0.f;
    for (int m = 0; m < cpr; ++m) s += part[u][j * cpr + m];
    const long t = r / n_local;
    const int l = (int)(r - t * n_local);
    const long b = t / seq, i = t - b * seq;
    delta[(b * n_local + l) * seq + i] = s;
  }
}

SP make_sp(const AttnDesc& a) {
  SP p{};
  p.batch = a.batch; p.seq = a.seq; p.n_local = a.n_local; p.d = a.head_dim;
  p.h_l = a.n_local * a.head_dim; p.head0 = a.head0; p.n_heads = a.n_heads; p.alibi = a.alibi;
  p.qkv = (const float*)a.qkv; p.ctx = a.ctx; p.lse = a.lse; p.dctx = a.dctx; p.delta = a.delta; p.dqkv = a.dqkv;
  return p;
}

}  // namespace

hipError_t delta_launch(int dtype, const AttnDesc& a, hipStream_t stream) {
  const long total = (long)a.batch * a.seq * a.n_local;
  if (total == 0) return hipSuccess;
  if (a.head_dim % 8 || a.head_dim < 8 || a.head_dim > 256) return hipErrorInvalidValue;
  const long per_wg = (long)DU * (256 / (a.head_dim / 8));  // whole rows per workgroup
  dim3 grid((unsigned)((total + per_wg - 1) / per_wg));
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(delta_kernel<bf16>, grid, dim3(256), 0, stream, (const bf16*)a.dctx, (const bf16*)a.ctx,
                       a.delta, a.seq, a.n_local, a.head_dim, total);
  else
    hipLaunchKernelGGL(delta_kernel<float>, grid, dim3(256), 0, stream, (const float*)a.dctx, (const float*)a.ctx,
                       a.delta, a.seq, a.n_local, a.head_dim, total);
  return hipGetLastError();
}

hipError_t attn_fwd_launch(int dtype, const AttnDesc& a, hipStream_t stream) {
  if (a.batch == 0 || a.seq == 0 || a.n_local == 0) return hipSuccess;
  if (attn_mfma_supported(dtype, a.head_dim)) return attn_mfma_fwd(a, stream);
  if (a.mask) return hipErrorInvalidValue;  // dropout runs on the matrix-core path only
  SP p = make_sp(a);
  dim3 grid(a.seq, a.n_local, a.batch);
  if (dtype == DT_BF16) hipLaunchKernelGGL(fwd_kernel<bf16>, grid, dim3(NT), 0, stream, p);
  else hipLaunchKernelGGL(fwd_kernel<float>, grid, dim3(NT), 0, stream, p);
  return hipGetLastError();
}

hipError_t attn_bwd_launch(int dtype, const AttnDesc& a, hipStream_t stream) {
  if (a.batch == 0 || a.seq == 0 || a.n_local == 0) return hipSuccess;
  if (a.mask && !attn_mfma_supported(dtype, a.head_dim)) return hipErrorInvalidValue;
  hipError_t e = delta_launch(dtype, a, stream);
  if (e != hipSuccess) return e;
  if (attn_mfma_supported(dtype, a.head_dim)) return attn_mfma_bwd(a, stream);
  SP p = make_sp(a);
  dim3 grid(a.seq, a.n_local, a.batch);
  if (dtype == DT_BF16) {
    hipLaunchKernelGGL(dq_kernel<bf16>, grid, dim3(NT), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(dkdv_kernel<bf16>, grid, dim3(NT), 0, stream, p);
  } else {
    hipLaunchKernelGGL(dq_kernel<float>, grid, dim3(NT), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(dkdv_kernel<float>, grid, dim3(NT), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace tpk
