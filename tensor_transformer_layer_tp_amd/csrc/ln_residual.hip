// Residual add + LayerNorm after a tensor-parallel block, forward and backward.
//
// The layer wraps its attention and MLP blocks in residual connections and
// layer normalizations (Megatron-LM deep dive, Fig. 2); g completes each
// block's output before the residual add (same page, Fig. 4), and the
// Megatron-DeepSpeed blog (section 4.3) fuses the residual add into the
// LayerNorm kernel. Definitions (h = hidden, per token row t):
//
//   r    = resid_in + (sum_k parts[k] + bias)    stored in the storage type
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
// Forward: one workgroup of 256 threads per row (several rows in flight per
// CU); the row stays in registers between the two reductions (mean, then
// variance about the mean).
// Backward: one workgroup of 512 threads per run of rows; each thread owns
// the same columns in every row of its run and keeps fp32 column partials of
// dy xhat and dy in registers, and loads the next row while it reduces the
// current one; a second kernel adds the runs' partials in a fixed order (no
// atomics: results do not depend on scheduling). dbias, when asked for, is a
// column sum of dr.
//
// The workgroup reductions exchange values through LDS behind a barrier that
// waits only for LDS traffic, so loads and stores to memory stay in flight
// across it.
//
// Dropout variants (DO): the block output (sum of parts + bias) is multiplied
// by keep * scale before the residual add; element (t, j) draws 16-bit lane
// j % 16 of the Philox4x64-10 block at counter (t, j / 16, 0, 2) with key
// (seed, offset) -- no rank in it, so every rank draws the same mask -- and is
// kept iff that lane >= thr. The forward stores the 8 keep bits of each
// 8-element chunk as one byte; the backward also writes the gradient of the
// block output, d_block = dr * keep * scale.
#include "common.h"
#include "kernels.h"
#include "philox.h"
#include "rowops.h"

namespace tpk {
namespace {

constexpr int FWD_T = 256;
constexpr int BWD_T = 512;
constexpr int BWD_RUNS = 256;  // target number of row runs (one per CU)

struct PartPtrs {
  const void* p[64];
};

struct DropArgs {
  uint8_t* mask;  // [rows][h/8]
  uint32_t thr;
  float scale;
  uint64_t seed, offset;
};

// Keep bits (bit e = element 8c + e) of chunk c of row t.
__device__ __forceinline__ uint32_t residual_keep_byte(const DropArgs& d, long t, int c) {
  uint64_t x0 = (uint64_t)t, x1 = (uint64_t)(c >> 1), x2 = 0, x3 = 2;
  philox4x64_10(x0, x1, x2, x3, d.seed, d.offset);
  const uint64_t w[4] = {x0, x1, x2, x3};
  uint32_t bits = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) bits |= (uint32_t)(philox_lane16(w, 8 * (c & 1) + e) >= d.thr) << e;
  return bits;
}

// Keep byte from 8 16-bit lanes held in two Philox words (lanes 4e'..4e'+3
// in word e').
__device__ __forceinline__ uint32_t keep_byte_of(uint64_t w0, uint64_t w1, uint32_t thr) {
  uint32_t bits = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) bits |= (uint32_t)((((e < 4 ? w0 : w1) >> (16 * (e & 3))) & 0xFFFFull) >= thr) << e;
  return bits;
}

__device__ __forceinline__ uint64_t shfl_xor1_u64(uint64_t v) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, 1), hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), 1);
  return ((uint64_t)hi << 32) | lo;
}

// Keep bytes of this thread's chunks c_i = threadIdx.x + i FWD_T, i < NV.
// Chunks 2k and 2k+1 take lanes 0-7 and 8-15 of the block at counter
// (t, k), and all of a thread's chunks have its parity, so two neighbouring
// threads need the same block for every i. For each pair (i, i+1) the even
// thread draws the block of its chunk i, the odd thread that of its chunk
// i+1, and each hands the half it does not use to the other: one block per
// thread per two chunks instead of one per chunk. Counters come from the
// unclamped chunk index, so a thread past the row's end still draws the
// block its neighbour needs.
template <int NV>
__device__ __forceinline__ void residual_keep_bytes(const DropArgs& d, long t, uint32_t (&bits)[NV]) {
  const int odd = threadIdx.x & 1;
#pragma unroll
  for (int i = 0; i + 1 < NV; i += 2) {
    const int c = (int)threadIdx.x + (i + odd) * FWD_T;
    uint64_t x0 = (uint64_t)t, x1 = (uint64_t)(c >> 1), x2 = 0, x3 = 2;
    philox4x64_10(x0, x1, x2, x3, d.seed, d.offset);
    const uint64_t k0 = odd ? x2 : x0, k1 = odd ? x3 : x1;  // the half this thread uses
    const uint64_t r0 = shfl_xor1_u64(odd ? x0 : x2), r1 = shfl_xor1_u64(odd ? x1 : x3);
    bits[i] = odd ? keep_byte_of(r0, r1, d.thr) : keep_byte_of(k0, k1, d.thr);
    bits[i + 1] = odd ? keep_byte_of(k0, k1, d.thr) : keep_byte_of(r0, r1, d.thr);
  }
  if (NV & 1) bits[NV - 1] = residual_keep_byte(d, t, (int)threadIdx.x + (NV - 1) * FWD_T);
}

// Chunk i of this thread (8 elements at column 8c) is valid if c < nc; the
// loads use the clamped chunk min(c, nc - 1), always in range, so that no load
// waits behind a branch; only arithmetic that feeds a sum and the stores
// depend on validity.
template <typename T, int NV, bool DO>
__global__ __launch_bounds__(FWD_T) void ln_residual_fwd_kernel(const T* __restrict__ resid_in, PartPtrs parts,
                                                                int n_parts, const T* __restrict__ bias,
                                                                const T* __restrict__ gamma,
                                                                const T* __restrict__ beta, float eps, int h,
                                                                T* __restrict__ resid_out, T* __restrict__ y,
                                                                float* __restrict__ mean, float* __restrict__ rstd,
                                                                DropArgs da) {
  __shared__ float red[FWD_T / 64];
  const long base = (long)blockIdx.x * h;
  const int nc = h >> 3;
  int cl[NV];
  bool ok[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = threadIdx.x + i * FWD_T;
    ok[i] = c < nc;
    cl[i] = 8 * (ok[i] ? c : nc - 1);
  }
  // the block output (sum of parts + bias) first, then the residual input
  // (after dropout in the DO variant; at p = 0 both variants add identically)
  V8<T> rv[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) rv[i].load(resid_in + base + cl[i]);
  float v[NV][8];
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) v[i][e] = 0.f;
  for (int k = 0; k < n_parts; ++k) {
    const T* pk = (const T*)parts.p[k];
    V8<T> pv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) pv[i].load(pk + base + cl[i]);
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] += pv[i][e];
  }
  if (bias) {
    V8<T> bv[NV];
#pragma unroll
    for (int i = 0; i < NV; ++i) bv[i].load(bias + cl[i]);
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] += bv[i][e];
  }
  uint32_t kb[NV];
  if (DO) residual_keep_bytes<NV>(da, blockIdx.x, kb);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (DO) {
      const uint32_t bits = kb[i];
      if (ok[i]) da.mask[(long)blockIdx.x * (h >> 3) + (cl[i] >> 3)] = (uint8_t)bits;
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] = rv[i][e] + (((bits >> e) & 1u) ? v[i][e] * da.scale : 0.f);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[i][e] = rv[i][e] + v[i][e];
    }
  }
  float s[1] = {0.f};
#pragma unroll
  for (int i = 0; i < NV; ++i) {
#pragma unroll
    for (int e = 0; e < 8; ++e) v[i][e] = to_f(from_f<T>(v[i][e]));  // the value stored
    if (!ok[i]) continue;
    store8(resid_out + base + cl[i], v[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) s[0] += v[i][e];
  }
  block_sum<FWD_T, 1>(s, red);
  const float mu = s[0] / (float)h;
  float q[1] = {0.f};
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (!ok[i]) continue;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float d = v[i][e] - mu;
      q[0] += d * d;
    }
  }
  V8<T> gm[NV], bt[NV];  // loaded before the second reduction, in flight across it
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    gm[i].load(gamma + cl[i]);
    bt[i].load(beta + cl[i]);
  }
  block_sum<FWD_T, 1>(q, red);
  const float rs = 1.0f / sqrtf(q[0] / (float)h + eps);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (!ok[i]) continue;
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = (v[i][e] - mu) * rs * gm[i][e] + bt[i][e];
    store8(y + base + cl[i], o);
  }
  if (threadIdx.x == 0) {
    mean[blockIdx.x] = mu;
    rstd[blockIdx.x] = rs;
  }
}

// Rows [run * rows_per, ...) of the backward pass; writes dr and this run's
// column partials part[(2 run + j) h + col], j = 0: dy xhat, 1: dy. Loads use
// clamped chunks and rows (always in range) as in the forward kernel.
template <typename T, int NV, bool DO>
__global__ __launch_bounds__(BWD_T) void ln_residual_bwd_kernel(const T* __restrict__ r, const float* __restrict__ mean,
                                                                const float* __restrict__ rstd,
                                                                const T* __restrict__ gamma, const T* __restrict__ dy,
                                                                const T* __restrict__ dr_in, int h, long rows,
                                                                int rows_per, T* __restrict__ dr,
                                                                float* __restrict__ part, const uint8_t* __restrict__ mask,
                                                                T* __restrict__ d_block, float dscale) {
  __shared__ float red[2 * BWD_T / 64];
  const int nc = h >> 3;
  const long r0 = (long)blockIdx.x * rows_per;
  const long r1 = r0 + rows_per < rows ? r0 + rows_per : rows;
  uint32_t cl[NV];  // byte offset of this thread's chunk i in a row
  bool ok[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = threadIdx.x + i * BWD_T;
    ok[i] = c < nc;
    cl[i] = (uint32_t)(8 * (ok[i] ? c : nc - 1) * sizeof(T));
  }
  const uint32_t hb = (uint32_t)(h * sizeof(T));  // bytes per row
  V8<T> gm[NV], dyv[NV], rv[NV];
  float ag[NV][8], ab[NV][8];
  {
    const auto rg = row_rsrc(gamma, hb), rd = row_rsrc(dy + r0 * h, hb), rr = row_rsrc(r + r0 * h, hb);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      load8_buf(gm[i], rg, cl[i]);
      load8_buf(dyv[i], rd, cl[i]);
      load8_buf(rv[i], rr, cl[i]);
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
#pragma unroll
    for (int e = 0; e < 8; ++e) ag[i][e] = ab[i][e] = 0.f;
  }
  for (long t = r0; t < r1; ++t) {
    const long base = t * h;
    const float mu = mean[t], rs = rstd[t];
    float s[2] = {0.f, 0.f};
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      if (!ok[i]) continue;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float g = dyv[i][e] * gm[i][e];
        s[0] += g;
        s[1] += g * ((rv[i][e] - mu) * rs);
      }
    }
    // the next row's dy and r (this row again after the last), and this row's
    // residual gradient, in flight across the reduction
    const long nb = (t + 1 < r1 ? t + 1 : t) * h;
    V8<T> dyn[NV], rn[NV], din[NV];
    {
      const auto rd = row_rsrc(dy + nb, hb), rr = row_rsrc(r + nb, hb);
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        load8_buf(dyn[i], rd, cl[i]);
        load8_buf(rn[i], rr, cl[i]);
      }
    }
    if (dr_in) {
      const auto ri = row_rsrc(dr_in + base, hb);
#pragma unroll
      for (int i = 0; i < NV; ++i) load8_buf(din[i], ri, cl[i]);
    }
    uint32_t mb[NV];
    if (DO) {
      const auto rm = row_rsrc(mask + t * (h >> 3), (uint32_t)(h >> 3));
#pragma unroll
      for (int i = 0; i < NV; ++i)
        mb[i] = __builtin_amdgcn_raw_buffer_load_b8(rm, (int)(cl[i] / (8 * (uint32_t)sizeof(T))), 0, 0);
    }
    block_sum<BWD_T, 2>(s, red);
    const float a = s[0] / (float)h, b = s[1] / (float)h;
    const auto ro = row_rsrc(dr + base, hb);
    const auto rob = row_rsrc(DO ? d_block + base : dr + base, hb);
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      gm[i].opaque();
      dyv[i].opaque();
      rv[i].opaque();
      if (ok[i]) {
        float o[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float xh = (rv[i][e] - mu) * rs;
          o[e] = (dr_in ? din[i][e] : 0.f) + rs * (dyv[i][e] * gm[i][e] - a - xh * b);
          ag[i][e] += dyv[i][e] * xh;
          ab[i][e] += dyv[i][e];
        }
        store8_buf(T{}, ro, cl[i], o);
        if (DO) {
#pragma unroll
          for (int e = 0; e < 8; ++e) o[e] = ((mb[i] >> e) & 1u) ? o[e] * dscale : 0.f;
          store8_buf(T{}, rob, cl[i], o);
        }
      }
      dyv[i] = dyn[i];
      rv[i] = rn[i];
    }
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    if (!ok[i]) continue;
    float* p = part + (long)2 * blockIdx.x * h + cl[i] / sizeof(T);
    store8(p, ag[i]);
    store8(p + h, ab[i]);
  }
}

// out_j[col] = sum over runs of part[(2 run + j) h + col]: a workgroup covers
// 64 columns (16 threads x 4) and its 16 thread rows take the runs
// interleaved (four loads in flight each); the 16 row sums are then added in
// a fixed order.
template <typename T>
__global__ __launch_bounds__(256) void ln_residual_bwd_final_kernel(const float* __restrict__ part, int runs, int h,
                                                                    T* dgamma, T* dbeta) {
  __shared__ f32x4 red[16][16];
  const int j = blockIdx.y;
  T* out = j == 0 ? dgamma : dbeta;
  const int tc = threadIdx.x & 15, tr = threadIdx.x >> 4;
  const int col = 4 * (blockIdx.x * 16 + tc);
  f32x4 s = {0.f, 0.f, 0.f, 0.f};
  if (col < h) {
    for (int w = tr; w < runs; w += 64) {
      f32x4 x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (w + 16 * u < runs) x[u] = *(const f32x4*)(part + ((long)2 * (w + 16 * u) + j) * h + col);
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if (w + 16 * u < runs) s += x[u];
    }
  }
  red[tr][tc] = s;
  __syncthreads();
  if (tr == 0 && col < h) {
    f32x4 t = red[0][tc];
#pragma unroll
    for (int k = 1; k < 16; ++k) t += red[k][tc];
#pragma unroll
    for (int e = 0; e < 4; ++e) out[col + e] = from_f<T>(t[e]);
  }
}

int ln_runs(long long rows, int& rows_per) {
  rows_per = (int)((rows + BWD_RUNS - 1) / BWD_RUNS);
  if (rows_per < 1) rows_per = 1;
  return (int)((rows + rows_per - 1) / rows_per);
}

DropArgs drop_args(const LnDesc& d) {
  DropArgs a{};
  a.mask = d.mask;
  a.thr = (uint32_t)floorf(d.drop_p * 65536.0f + 0.5f);
  a.scale = 65536.0f / (65536.0f - (float)a.thr);
  a.seed = d.seed;
  a.offset = d.offset;
  return a;
}

template <typename T, int NV>
void fwd_nv(const LnDesc& d, const PartPtrs& ps, hipStream_t st) {
  const DropArgs da = drop_args(d);
  if (d.mask)
    hipLaunchKernelGGL((ln_residual_fwd_kernel<T, NV, true>), dim3((unsigned)d.T), dim3(FWD_T), 0, st,
                       (const T*)d.resid_in, ps, d.n_parts, (const T*)d.bias, (const T*)d.gamma, (const T*)d.beta,
                       d.eps, d.h, (T*)d.resid_out, (T*)d.y, d.mean, d.rstd, da);
  else
    hipLaunchKernelGGL((ln_residual_fwd_kernel<T, NV, false>), dim3((unsigned)d.T), dim3(FWD_T), 0, st,
                       (const T*)d.resid_in, ps, d.n_parts, (const T*)d.bias, (const T*)d.gamma, (const T*)d.beta,
                       d.eps, d.h, (T*)d.resid_out, (T*)d.y, d.mean, d.rstd, da);
}

template <typename T>
hipError_t fwd_t(const LnDesc& d, hipStream_t st) {
  PartPtrs ps{};
  for (int k = 0; k < d.n_parts; ++k) ps.p[k] = d.parts[k];
  const int nv = (d.h / 8 + FWD_T - 1) / FWD_T;
  if (nv <= 1) fwd_nv<T, 1>(d, ps, st);
  else if (nv <= 2) fwd_nv<T, 2>(d, ps, st);
  else if (nv <= 4) fwd_nv<T, 4>(d, ps, st);
  else if (nv <= 6) fwd_nv<T, 6>(d, ps, st);
  else if (nv <= 8) fwd_nv<T, 8>(d, ps, st);
  else if (nv <= 10) fwd_nv<T, 10>(d, ps, st);
  else if (nv <= 12) fwd_nv<T, 12>(d, ps, st);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

template <typename T, int NV>
void bwd_nv(const LnDesc& d, int runs, int rows_per, float* part, hipStream_t st) {
  const DropArgs da = drop_args(d);
  if (d.mask)
    hipLaunchKernelGGL((ln_residual_bwd_kernel<T, NV, true>), dim3(runs), dim3(BWD_T), 0, st, (const T*)d.resid_out,
                       (const float*)d.mean, (const float*)d.rstd, (const T*)d.gamma, (const T*)d.dy,
                       (const T*)d.dr_in, d.h, (long)d.T, rows_per, (T*)d.dr, part, (const uint8_t*)d.mask,
                       (T*)d.d_block, da.scale);
  else
    hipLaunchKernelGGL((ln_residual_bwd_kernel<T, NV, false>), dim3(runs), dim3(BWD_T), 0, st, (const T*)d.resid_out,
                       (const float*)d.mean, (const float*)d.rstd, (const T*)d.gamma, (const T*)d.dy,
                       (const T*)d.dr_in, d.h, (long)d.T, rows_per, (T*)d.dr, part, (const uint8_t*)nullptr,
                       (T*)nullptr, da.scale);
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
  const dim3 grid((unsigned)((d.h / 4 + 15) / 16), 2);
  hipLaunchKernelGGL(ln_residual_bwd_final_kernel<T>, grid, dim3(256), 0, st, (const float*)part, runs, d.h,
                     (T*)d.dgamma, (T*)d.dbeta);
  e = hipGetLastError();
  if (e != hipSuccess || !d.dbias) return e;
  return colsum_launch(sizeof(T) == 2 ? DT_BF16 : DT_F32, d.mask ? d.d_block : d.dr, (int)d.T, d.h, d.h, d.dbias,
                       part + (size_t)2 * runs * d.h, st);
}

}  // namespace

// Two fp32 partial rows (dgamma, dbeta) per run, then the column-sum
// workspace of dbias.
size_t ln_bwd_workspace_bytes(long long rows, int h) {
  if (rows <= 0) return 0;
  int rows_per = 1;
  return (size_t)ln_runs(rows, rows_per) * 2 * (size_t)h * sizeof(float) + colsum_workspace_bytes((int)rows, h);
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
