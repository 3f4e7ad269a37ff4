// fp32 GEMM on the vector ALUs (the fp32 storage type), and the GEMM
// dispatcher. 64x64 output tile per workgroup of 256 threads, 4x4 outputs per
// thread, K staged 16 at a time through LDS. Any layout, any size (bounds are
// checked element by element); the same epilogues as the matrix-core path.
#include "common.h"
#include "kernels.h"

namespace tpk {

size_t gemm_mfma_workspace_bytes(int M, int N, int K);
hipError_t gemm_mfma_launch(const GemmDesc& g, void* ws, size_t ws_bytes, hipStream_t stream);
const char* gemm_mfma_kernel_name(const GemmDesc& g);

namespace {

constexpr int TB = 64, TK = 16;

struct SParams {
  const float* A; const float* B;
  long lda, ldb;
  int M, N, K;
  int a_kmajor, b_kmajor, epi;
  float* C; long ldc;
  float* C2; long ldc2;
  const float* bias;
  const float* aux; long ldaux;
};

__global__ __launch_bounds__(256) void gemm_f32_kernel(SParams p) {
  __shared__ float sA[TK][TB + 1];
  __shared__ float sB[TK][TB + 1];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.y * TB, n0 = blockIdx.x * TB;
  const int tx = tid & 15, ty = tid >> 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < p.K; k0 += TK) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + 256 * e;
      int mm, kk;
      if (p.a_kmajor) { mm = idx / TK; kk = idx % TK; } else { kk = idx / TB; mm = idx % TB; }
      const int m = m0 + mm, k = k0 + kk;
      float v = 0.f;
      if (m < p.M && k < p.K) v = p.a_kmajor ? p.A[(long)m * p.lda + k] : p.A[(long)k * p.lda + m];
      sA[kk][mm] = v;
      int nn;
      if (p.b_kmajor) { nn = idx / TK; kk = idx % TK; } else { kk = idx / TB; nn = idx % TB; }
      const int n = n0 + nn, k2 = k0 + kk;
      float w = 0.f;
      if (n < p.N && k2 < p.K) w = p.b_kmajor ? p.B[(long)n * p.ldb + k2] : p.B[(long)k2 * p.ldb + n];
      sB[kk][nn] = w;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = sB[kk][tx * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tx * 4 + j;
      if (n >= p.N) continue;
      float v = acc[i][j];
      if (p.epi == EPI_BIAS || p.epi == EPI_BIAS_GELU || p.epi == EPI_BIAS_F32) v += p.bias[n];
      if (p.epi == EPI_DGELU) v *= gelu_grad_f(p.aux[(long)m * p.ldaux + n]);
      p.C[(long)m * p.ldc + n] = v;
      if (p.epi == EPI_BIAS_GELU) p.C2[(long)m * p.ldc2 + n] = gelu_f(v);
    }
  }
}

}  // namespace

size_t gemm_workspace_bytes(int dtype, int M, int N, int K) {
  return dtype == DT_BF16 ? gemm_mfma_workspace_bytes(M, N, K) : 0;
}

const char* gemm_kernel_name(int dtype, const GemmDesc& g) {
  if (g.M <= 0 || g.N <= 0 || g.K <= 0) return nullptr;
  return dtype == DT_BF16 ? gemm_mfma_kernel_name(g) : "gemm_f32_kernel";
}

hipError_t gemm_launch(int dtype, const GemmDesc& g, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (g.M <= 0 || g.N <= 0) return hipSuccess;
  if (g.K <= 0) {  // empty contraction: the product is zero (only plain stores reach here)
    if (g.epi != EPI_STORE) return hipErrorInvalidValue;
    return zero_launch(dtype, g.C, g.M, g.N, g.ldc, stream);
  }
  if (dtype == DT_BF16) return gemm_mfma_launch(g, ws, ws_bytes, stream);
  SParams p{};
  p.A = (const float*)g.A; p.B = (const float*)g.B;
  p.lda = g.lda; p.ldb = g.ldb;
  p.M = g.M; p.N = g.N; p.K = g.K;
  p.a_kmajor = g.a_kmajor; p.b_kmajor = g.b_kmajor; p.epi = g.epi;
  p.C = (float*)g.C; p.ldc = g.ldc;
  p.C2 = (float*)g.C2; p.ldc2 = g.ldc2;
  p.bias = (const float*)g.bias;
  p.aux = (const float*)g.aux; p.ldaux = g.ldaux;
  dim3 grid((g.N + TB - 1) / TB, (g.M + TB - 1) / TB);
  hipLaunchKernelGGL(gemm_f32_kernel, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace tpk
