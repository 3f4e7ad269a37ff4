// Bandwidth-bound helpers: column sums (bias gradients), transposed copies of
// the weight gradients' token-major operands, the emulated f / g sum over
// ranks' partials, and zero fill.
#include "common.h"
#include "kernels.h"

namespace tpk {
namespace {

constexpr int CB = 256;  // columns per workgroup (one per thread)

// part[y][n] = sum of X[r][n] over the y-th run of rows.
template <typename T>
__global__ __launch_bounds__(CB) void colsum_part_kernel(const T* X, int M, int N, long ld, int rows_per,
                                                         float* part) {
  const int n = blockIdx.x * CB + threadIdx.x;
  if (n >= N) return;
  const int r0 = blockIdx.y * rows_per;
  const int r1 = min(M, r0 + rows_per);
  float s = 0.f;
  for (int r = r0; r < r1; ++r) s += to_f(X[(long)r * ld + n]);
  part[(long)blockIdx.y * N + n] = s;
}

// Same partial sums, 8 adjacent columns per thread (one 16-byte bf16 load or
// two 16-byte fp32 loads per row): 64 threads span 512 columns and 4 row
// groups split the run; the row groups are added in a fixed order.
template <typename T>
__global__ __launch_bounds__(256) void colsum_part_vec_kernel(const T* X, int M, int N, long ld, int rows_per,
                                                              float* part) {
  __shared__ float red[3][512];
  const int tc = threadIdx.x & 63, rg = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 512 + 8 * tc;
  const int r0 = blockIdx.y * rows_per;
  const int r1 = min(M, r0 + rows_per);
  float s[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (n0 < N) {
    // rows r0 + rg, r0 + rg + 4, ... added in that order; eight rows' loads in
    // flight at a time (a row past the run loads row r1 - 1 again, unused, so
    // that no load sits behind a branch)
    for (int r = r0 + rg; r < r1; r += 32) {
      float x[8][8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int ru = min(r + 4 * u, r1 - 1);
        const T* src = X + (long)ru * ld + n0;
        if constexpr (sizeof(T) == 2) {
          const bf16x8 v = *(const bf16x8*)src;
#pragma unroll
          for (int e = 0; e < 8; ++e) x[u][e] = (float)v[e];
        } else {
          const f32x4 a = *(const f32x4*)src, b = *(const f32x4*)(src + 4);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            x[u][e] = a[e];
            x[u][4 + e] = b[e];
          }
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (r + 4 * u < r1) {
#pragma unroll
          for (int e = 0; e < 8; ++e) s[e] += x[u][e];
        }
    }
  }
  if (rg > 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red[rg - 1][8 * tc + e] = s[e];
  }
  __syncthreads();
  if (rg == 0 && n0 < N) {
#pragma unroll
    for (int gq = 0; gq < 3; ++gq)
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] += red[gq][8 * tc + e];
#pragma unroll
    for (int e = 0; e < 8; ++e) part[(long)blockIdx.y * N + n0 + e] = s[e];
  }
}

// out[n] = sum of the R partial rows part[r][n]. A workgroup takes 32 columns
// and 8 row groups; group q adds rows q, q + 8, q + 16, ... in that order
// with eight rows' loads in flight (rows past R load row R - 1 again,
// unused), and the 8 group sums are added in group order: a fixed order for
// any R, and R / 8 dependent steps per thread instead of R (thousands of
// partial rows at 16384 tokens).
constexpr int FC = 32, FG = 8;
template <typename T>
__global__ __launch_bounds__(FC * FG) void colsum_final_kernel(const float* part, int R, int N, T* out) {
  __shared__ float red[FG][FC];
  const int c = threadIdx.x % FC, q = threadIdx.x / FC;
  const int n = blockIdx.x * FC + c;
  const int nn = n < N ? n : N - 1;  // clamped: every thread loads in range
  float s = 0.f;
  for (int r = q; r < R; r += 8 * FG) {
    float x[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) x[u] = part[(long)min(r + u * FG, R - 1) * N + nn];
#pragma unroll
    for (int u = 0; u < 8; ++u)
      if (r + u * FG < R) s += x[u];
  }
  red[q][c] = s;
  __syncthreads();
  if (q == 0 && n < N) {
    float t = red[0][c];
#pragma unroll
    for (int k = 1; k < FG; ++k) t += red[k][c];
    out[n] = from_f<T>(t);
  }
}

void colsum_split(int M, int N, int& R, int& rows_per) {
  const int cblocks = (N + CB - 1) / CB;
  R = (1024 + cblocks - 1) / cblocks;  // aim for ~1024 workgroups
  const int rmax = (M + 31) / 32;      // at least 32 rows per run
  if (R > rmax) R = rmax;
  if (R < 1) R = 1;
  rows_per = (M + R - 1) / R;
  if (rows_per < 1) rows_per = 1;
  R = (M + rows_per - 1) / rows_per;
  if (R < 1) R = 1;
}

struct Parts {
  const void* p[64];
};

template <typename T>
__global__ __launch_bounds__(256) void sum_partials_kernel(Parts parts, int n_parts, const T* bias, T* out,
                                                           long long count, int cols) {
  const long long stride = (long long)gridDim.x * 256;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < count; i += stride) {
    float s = 0.f;
    for (int k = 0; k < n_parts; ++k) s += to_f(((const T*)parts.p[k])[i]);
    if (bias) s += to_f(bias[i % cols]);
    out[i] = from_f<T>(s);
  }
}

template <typename T>
__global__ __launch_bounds__(256) void zero_kernel(T* p, long long rows, long long cols, long long ld) {
  const long long count = rows * cols;
  const long long stride = (long long)gridDim.x * 256;
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < count; i += stride) {
    const long long r = i / cols, c = i - r * cols;
    p[r * ld + c] = from_f<T>(0.f);
  }
}

// Transposed copy of a [R, C] bf16 matrix for the weight gradients (their
// K = tokens; a k-contiguous operand lets the product read it with the
// non-transposing LDS fragment loads): XT[c][r] = X[r][c], and optionally
// part[b][c] = the sum of X[r][c] over rows TR*b .. TR*b+TR-1 (two runs of
// TR/2 rows added in a fixed order), which leaves only the final pass over
// the partials for a bias gradient. Workgroup = one TR x TC tile staged in
// LDS (rows padded by 16 bytes); loads are 16-byte vectors over 256-byte row
// segments, stores 16-byte vectors, 4 lanes per 64-byte output segment. The
// output's 8-row group that holds row R-1 is written whole, rows past R as
// zeros, so XT's row length (ldt) is a multiple of 8 that is >= R and every
// k-chunk a product reads there is finite. Needs C % 8 == 0, ldx % 8 == 0
// and 16-byte aligned X, XT. (32 x 128 measured 5-17% faster than 64 x 64 at
// 2048 tokens.)
constexpr int TR = 32, TC = 128;
__global__ __launch_bounds__(256) void transpose_colsum_kernel(const bf16* __restrict__ X, int R, int C, long ldx,
                                                               bf16* __restrict__ XT, long ldt,
                                                               float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) bf16 tile[TR][TC + 8];
  __shared__ float red[TC];
  constexpr int CPR = TC / 8, NLD = TR * CPR / 256, RCH = TR / 8, NST = TC * RCH / 256;
  const int c0 = blockIdx.x * TC, r0 = blockIdx.y * TR, tid = threadIdx.x;
  bf16x8 v[NLD];
#pragma unroll
  for (int u = 0; u < NLD; ++u) {
    const int q = tid + 256 * u, r = q / CPR, ch = q % CPR;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[u][e] = (bf16)0.f;
    if (r0 + r < R && c0 + 8 * ch < C) v[u] = *(const bf16x8*)(X + (long)(r0 + r) * ldx + c0 + 8 * ch);
  }
#pragma unroll
  for (int u = 0; u < NLD; ++u) {
    const int q = tid + 256 * u, r = q / CPR, ch = q % CPR;
    *(bf16x8*)&tile[r][8 * ch] = v[u];
  }
  __syncthreads();
  if (part) {  // uniform over the grid
    const int c = tid % TC, g = tid / TC;
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < TR / 2; ++r) s += (float)tile[(TR / 2) * g + r][c];
    if (g > 0) red[c] = s;
    __syncthreads();
    if (g == 0 && c0 + c < C) part[(long)blockIdx.y * C + c0 + c] = s + red[c];
  }
#pragma unroll
  for (int u = 0; u < NST; ++u) {
    const int q = tid + 256 * u, c = q / RCH, rc = q % RCH;
    bf16x8 o;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = tile[8 * rc + e][c];
    if (c0 + c < C && r0 + 8 * rc < R) *(bf16x8*)(XT + (long)(c0 + c) * ldt + r0 + 8 * rc) = o;
  }
}

unsigned grid_for(long long count) {
  long long g = (count + 255) / 256;
  if (g > 65536) g = 65536;
  if (g < 1) g = 1;
  return (unsigned)g;
}

}  // namespace

hipError_t colsum_final_launch(int dtype, const float* part, int R, int N, void* out, hipStream_t stream);

size_t colsum_workspace_bytes(int M, int N) {
  int R, rows_per;
  colsum_split(M, N, R, rows_per);
  return (size_t)R * N * sizeof(float);
}

hipError_t colsum_launch(int dtype, const void* X, int M, int N, long ld, void* out, float* ws,
                         hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  int R, rows_per;
  colsum_split(M, N, R, rows_per);
  const unsigned cblocks = (N + CB - 1) / CB;
  const bool vec = (N % 8 == 0) && (ld % 8 == 0) && ((uintptr_t)X % 16 == 0);
  if (M > 0 && vec) {
    const unsigned vblocks = (N + 511) / 512;
    if (dtype == DT_BF16)
      hipLaunchKernelGGL(colsum_part_vec_kernel<bf16>, dim3(vblocks, R), dim3(256), 0, stream, (const bf16*)X, M, N,
                         ld, rows_per, ws);
    else
      hipLaunchKernelGGL(colsum_part_vec_kernel<float>, dim3(vblocks, R), dim3(256), 0, stream, (const float*)X, M,
                         N, ld, rows_per, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else if (M > 0) {
    if (dtype == DT_BF16)
      hipLaunchKernelGGL(colsum_part_kernel<bf16>, dim3(cblocks, R), dim3(CB), 0, stream, (const bf16*)X, M, N, ld,
                         rows_per, ws);
    else
      hipLaunchKernelGGL(colsum_part_kernel<float>, dim3(cblocks, R), dim3(CB), 0, stream, (const float*)X, M, N, ld,
                         rows_per, ws);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  } else {
    R = 0;  // no rows: the sum is zero
  }
  return colsum_final_launch(dtype, ws, R, N, out, stream);
}

int transpose_part_rows(int R) { return R > 0 ? (R + TR - 1) / TR : 0; }

hipError_t transpose_colsum_launch(const void* X, int R, int C, long ldx, void* XT, long ldt, float* part,
                                   hipStream_t stream) {
  if (R <= 0 || C <= 0) return hipSuccess;
  if (C % 8 || ldx % 8 || ldt % 8 || ldt < R || ((uintptr_t)X & 15) || ((uintptr_t)XT & 15))
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(transpose_colsum_kernel, dim3((C + TC - 1) / TC, (R + TR - 1) / TR), dim3(256), 0, stream,
                     (const bf16*)X, R, C, ldx, (bf16*)XT, ldt, part);
  return hipGetLastError();
}

hipError_t colsum_final_launch(int dtype, const float* part, int R, int N, void* out, hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  const unsigned fblocks = (N + FC - 1) / FC;
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(colsum_final_kernel<bf16>, dim3(fblocks), dim3(FC * FG), 0, stream, part, R, N, (bf16*)out);
  else
    hipLaunchKernelGGL(colsum_final_kernel<float>, dim3(fblocks), dim3(FC * FG), 0, stream, part, R, N, (float*)out);
  return hipGetLastError();
}

hipError_t sum_partials_launch(int dtype, const void* const* parts, int n_parts, const void* bias, void* out,
                               long long count, int cols, hipStream_t stream) {
  if (count <= 0) return hipSuccess;
  Parts ps{};
  for (int k = 0; k < n_parts; ++k) ps.p[k] = parts[k];
  const unsigned g = grid_for(count);
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(sum_partials_kernel<bf16>, dim3(g), dim3(256), 0, stream, ps, n_parts, (const bf16*)bias,
                       (bf16*)out, count, cols);
  else
    hipLaunchKernelGGL(sum_partials_kernel<float>, dim3(g), dim3(256), 0, stream, ps, n_parts, (const float*)bias,
                       (float*)out, count, cols);
  return hipGetLastError();
}

hipError_t zero_launch(int dtype, void* p, long long rows, long long cols, long long ld, hipStream_t stream) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  const unsigned g = grid_for(rows * cols);
  if (dtype == DT_BF16) hipLaunchKernelGGL(zero_kernel<bf16>, dim3(g), dim3(256), 0, stream, (bf16*)p, rows, cols, ld);
  else hipLaunchKernelGGL(zero_kernel<float>, dim3(g), dim3(256), 0, stream, (float*)p, rows, cols, ld);
  return hipGetLastError();
}

}  // namespace tpk
