// Bandwidth-bound helpers: column sums (bias gradients), transposed copies of
// the weight gradients' token-major operands, the emulated f / g sum over
// ranks' partials, and zero fill.
#include <climits>

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

// Up to two column sums over the same rows, done by one launch of each pass:
// job q sums the [M, N_q] matrix X_q (leading dimension ld_q) into out_q via
// the partial rows part_q [R][N_q]; the partial pass gives job 1 the
// workgroups from blk0 on (x), the final pass those from fblk0 on.
struct ColJob {
  const void* X;
  long ld;
  int N;
  int blk0, fblk0;
  float* part;
  void* out;
};
struct ColJobs {
  ColJob j[2];
};

// Same partial sums, 8 adjacent columns per thread (one 16-byte bf16 load or
// two 16-byte fp32 loads per row): 64 threads span 512 columns and 4 row
// groups split the run; the row groups are added in a fixed order.
template <typename T>
__global__ __launch_bounds__(256) void colsum_part_vec_kernel(ColJobs jobs, int M, int rows_per) {
  __shared__ float red[3][512];
  const bool q = (int)blockIdx.x >= jobs.j[1].blk0;
  const T* X = (const T*)(q ? jobs.j[1].X : jobs.j[0].X);
  const long ld = q ? jobs.j[1].ld : jobs.j[0].ld;
  const int N = q ? jobs.j[1].N : jobs.j[0].N;
  float* part = q ? jobs.j[1].part : jobs.j[0].part;
  const int bx = (int)blockIdx.x - (q ? jobs.j[1].blk0 : 0);
  const int tc = threadIdx.x & 63, rg = threadIdx.x >> 6;
  const int n0 = bx * 512 + 8 * tc;
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
__global__ __launch_bounds__(FC * FG) void colsum_final_kernel(ColJobs jobs, int R) {
  __shared__ float red[FG][FC];
  const bool second = (int)blockIdx.x >= jobs.j[1].fblk0;
  const float* part = second ? jobs.j[1].part : jobs.j[0].part;
  const int N = second ? jobs.j[1].N : jobs.j[0].N;
  T* out = (T*)(second ? jobs.j[1].out : jobs.j[0].out);
  const int bx = (int)blockIdx.x - (second ? jobs.j[1].fblk0 : 0);
  const int c = threadIdx.x % FC, q = threadIdx.x / FC;
  const int n = bx * FC + c;
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

namespace {

bool colsum_vec_ok(const void* X, int N, long ld) { return N % 8 == 0 && ld % 8 == 0 && (uintptr_t)X % 16 == 0; }

ColJobs single_job(const void* X, long ld, int N, float* part, void* out) {
  ColJobs jobs{};
  jobs.j[0].X = X; jobs.j[0].ld = ld; jobs.j[0].N = N; jobs.j[0].part = part; jobs.j[0].out = out;
  jobs.j[1].blk0 = jobs.j[1].fblk0 = INT_MAX;  // no second job
  return jobs;
}

hipError_t final_pass(int dtype, const ColJobs& jobs, int R, unsigned fblocks, hipStream_t stream) {
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(colsum_final_kernel<bf16>, dim3(fblocks), dim3(FC * FG), 0, stream, jobs, R);
  else
    hipLaunchKernelGGL(colsum_final_kernel<float>, dim3(fblocks), dim3(FC * FG), 0, stream, jobs, R);
  return hipGetLastError();
}

hipError_t vec_pass(int dtype, const ColJobs& jobs, unsigned vblocks, int R, int M, int rows_per,
                    hipStream_t stream) {
  if (dtype == DT_BF16)
    hipLaunchKernelGGL(colsum_part_vec_kernel<bf16>, dim3(vblocks, R), dim3(256), 0, stream, jobs, M, rows_per);
  else
    hipLaunchKernelGGL(colsum_part_vec_kernel<float>, dim3(vblocks, R), dim3(256), 0, stream, jobs, M, rows_per);
  return hipGetLastError();
}

}  // namespace

size_t colsum_workspace_bytes(int M, int N) {
  int R, rows_per;
  colsum_split(M, N, R, rows_per);
  return (size_t)R * N * sizeof(float);
}

size_t colsum_pair_workspace_bytes(int M, int N1, int N2) {
  size_t b = colsum_workspace_bytes(M, N1);
  const size_t b2 = colsum_workspace_bytes(M, N2);
  b = b2 > b ? b2 : b;
  int R, rows_per;
  colsum_split(M, N1 + N2, R, rows_per);
  const size_t bp = (size_t)R * (N1 + N2) * sizeof(float);
  return bp > b ? bp : b;
}

hipError_t colsum_launch(int dtype, const void* X, int M, int N, long ld, void* out, float* ws,
                         hipStream_t stream) {
  if (N <= 0) return hipSuccess;
  int R, rows_per;
  colsum_split(M, N, R, rows_per);
  const unsigned cblocks = (N + CB - 1) / CB;
  if (M > 0 && colsum_vec_ok(X, N, ld)) {
    const hipError_t e = vec_pass(dtype, single_job(X, ld, N, ws, out), (N + 511) / 512, R, M, rows_per, stream);
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

hipError_t colsum_pair_launch(int dtype, int M, const void* X1, int N1, long ld1, void* out1, const void* X2, int N2,
                              long ld2, void* out2, float* ws, hipStream_t stream) {
  if (out2 == nullptr || N2 <= 0) return colsum_launch(dtype, X1, M, N1, ld1, out1, ws, stream);
  if (N1 <= 0) return colsum_launch(dtype, X2, M, N2, ld2, out2, ws, stream);
  if (M <= 0 || !colsum_vec_ok(X1, N1, ld1) || !colsum_vec_ok(X2, N2, ld2)) {  // one after the other
    const hipError_t e = colsum_launch(dtype, X1, M, N1, ld1, out1, ws, stream);
    return e != hipSuccess ? e : colsum_launch(dtype, X2, M, N2, ld2, out2, ws, stream);
  }
  int R, rows_per;
  colsum_split(M, N1 + N2, R, rows_per);
  const unsigned vb1 = (N1 + 511) / 512, vb2 = (N2 + 511) / 512, fb1 = (N1 + FC - 1) / FC,
                 fb2 = (N2 + FC - 1) / FC;
  ColJobs jobs = single_job(X1, ld1, N1, ws, out1);
  jobs.j[1].X = X2; jobs.j[1].ld = ld2; jobs.j[1].N = N2;
  jobs.j[1].blk0 = (int)vb1; jobs.j[1].fblk0 = (int)fb1;
  jobs.j[1].part = ws + (size_t)R * N1;
  jobs.j[1].out = out2;
  const hipError_t e = vec_pass(dtype, jobs, vb1 + vb2, R, M, rows_per, stream);
  return e != hipSuccess ? e : final_pass(dtype, jobs, R, fb1 + fb2, stream);
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
  return final_pass(dtype, single_job(nullptr, 0, N, (float*)part, out), R, (N + FC - 1) / FC, stream);
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
