// Flash-style causal attention for bf16 on CDNA4 matrix cores
// (v_mfma_f32_32x32x16_bf16), head widths D in {64, 96, 128, 160}.
//
// Layout: per rank, qkv [T, 3*h_l] = [Q | K | V] in fp32; local head l uses
// columns l*D.. of each third; row t = b*seq + position. ctx [T, h_l] bf16, lse
// [batch, n_local, seq] (natural log, fp32).
//
// Precision: scores are formed from q and k split into bf16 high and low parts,
// S = q_hi k_hi + q_hi k_lo + q_lo k_hi (three products, error ~2^-16 |q||k|),
// because rows of large, nearly tied scores amplify bf16 rounding of q and k
// far beyond the rounding of the output. V, P, dS and dctx enter the products
// as bf16 (their rounding is not amplified).
//
// Forward (one workgroup = 4 waves = 128 queries of one head; each wave owns 32
// queries): per 64-key tile, K is staged in LDS row-major and V transposed; a
// wave computes S^T = K Q^T for 32 keys x its 32 queries, so each lane holds one
// query column and the softmax statistics (max, sum) are per lane, combined
// with the partner lane 32 away. P^T stays in registers and is fed straight
// back as the B operand of ctx^T += V^T P^T: the keys a lane holds in the S^T
// accumulator form, chunk by chunk, a fixed permutation of 16 consecutive keys,
// and the transposed V tile is stored in LDS in that same key order.
//
// Backward: dK/dV per 32-key wave (workgroup = 128 keys, looping over 64-query
// tiles), dQ per 32-query wave (looping over 64-key tiles); both recompute P
// from lse, dS = P (dP - delta) with delta = rowsum(dctx * ctx). No atomics.
#include "common.h"
#include "kernels.h"

namespace tpk {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

struct MP {
  int batch, seq, n_local, h_l, head0, n_heads, alibi;
  long ld;             // 3*h_l
  const float* qkv;
  bf16* ctx;
  float* lse;
  const bf16* dctx;
  const float* delta;
  bf16* dqkv;
  float scale_log2;    // log2(e) / sqrt(D)
  float scale;         // 1 / sqrt(D)
};

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

__device__ __forceinline__ float alibi_slope_log2(const MP& p, int l) {
  // global head k = head0 + l + 1 (1-based): slope 2^(-8k/n_heads), in log2 units
  return p.alibi ? exp2f(-8.0f * (float)(p.head0 + l + 1) / (float)p.n_heads) * kLog2e : 0.0f;
}

// 8 consecutive elements as packed bf16 (one 16-byte LDS chunk).
__device__ __forceinline__ u32x4 load8(const bf16* p) { return *(const u32x4*)p; }
__device__ __forceinline__ u32x4 load8(const float* p) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
  bf16x8 v;
  v[0] = (bf16)a[0]; v[1] = (bf16)a[1]; v[2] = (bf16)a[2]; v[3] = (bf16)a[3];
  v[4] = (bf16)b[0]; v[5] = (bf16)b[1]; v[6] = (bf16)b[2]; v[7] = (bf16)b[3];
  return __builtin_bit_cast(u32x4, v);
}
// 8 consecutive fp32 elements split into bf16 high and low parts.
__device__ __forceinline__ void load8_split(const float* p, bf16x8& hi, bf16x8& lo) {
  const f32x4 a = *(const f32x4*)p, b = *(const f32x4*)(p + 4);
  const float x[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hi[e] = (bf16)x[e];
    lo[e] = (bf16)(x[e] - (float)hi[e]);
  }
}

// Tile rows [row0, row0+64) of a [seq, *] slab, row-major in LDS with row
// stride D+8 (the padding spreads rows over the banks). Rows >= seq are zero.
template <int D, typename S>
__device__ __forceinline__ void stage_rows(bf16* s, const S* src, long ld, long grow0, int row0, int seq) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int it = 0; it < D / 32; ++it) {
    const int id = threadIdx.x + 256 * it;
    const int r = id / CPR, c = id - r * CPR;
    const int pos = row0 + r;
    u32x4 v = {0u, 0u, 0u, 0u};
    if (pos < seq) v = load8(src + (grow0 + pos) * ld + 8 * c);
    *(u32x4*)(s + r * (D + 8) + 8 * c) = v;
  }
}
// Same, fp32 source split into high and low bf16 tiles.
template <int D>
__device__ __forceinline__ void stage_rows_split(bf16* shi, bf16* slo, const float* src, long ld, long grow0,
                                                 int row0, int seq) {
  constexpr int CPR = D / 8;
#pragma unroll
  for (int it = 0; it < D / 32; ++it) {
    const int id = threadIdx.x + 256 * it;
    const int r = id / CPR, c = id - r * CPR;
    const int pos = row0 + r;
    bf16x8 hi = bf16x8{}, lo = bf16x8{};
    if (pos < seq) load8_split(src + (grow0 + pos) * ld + 8 * c, hi, lo);
    *(bf16x8*)(shi + r * (D + 8) + 8 * c) = hi;
    *(bf16x8*)(slo + r * (D + 8) + 8 * c) = lo;
  }
}

// The same 64 rows transposed: LDS [D][64], row d holds the 64 tile rows in
// the accumulator key order (inside each group of 16: position 8g + 4a + r for
// tile row 8a + 4g + r), 16-byte chunks XOR-swizzled by swz(d). Each of the
// first D threads transposes one 8x8 block in registers.
template <int D, typename S>
__device__ __forceinline__ void stage_trans(bf16* s, const S* src, long ld, long grow0, int row0, int seq) {
  const int id = threadIdx.x;
  if (id >= D) return;
  const int rb8 = id & 7, cb8 = id >> 3;
  u32x4 r[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int pos = row0 + 8 * rb8 + j;
    r[j] = pos < seq ? load8(src + (grow0 + pos) * ld + 8 * cb8) : u32x4{0u, 0u, 0u, 0u};
  }
  const int c16 = rb8 >> 1, a = rb8 & 1;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int dw = i >> 1;
    uint32_t o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t lo = r[2 * q][dw], hi = r[2 * q + 1][dw];
      o[q] = (i & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
    }
    const int d = 8 * cb8 + i, sw = swz(d);
    bf16* rowp = s + d * 64;
    *(u32x2*)(rowp + (((2 * c16) ^ sw) << 3) + 4 * a) = u32x2{o[0], o[1]};
    *(u32x2*)(rowp + (((2 * c16 + 1) ^ sw) << 3) + 4 * a) = u32x2{o[2], o[3]};
  }
}

// A-operand fragment from a transposed tile: row d, 16-row chunk kc of the tile.
__device__ __forceinline__ bf16x8 frag_trans(const bf16* s, int d, int kc, int g) {
  return *(const bf16x8*)(s + d * 64 + (((2 * kc + g) ^ swz(d)) << 3));
}

__device__ __forceinline__ bf16x8 pack8(const float* x) {
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (bf16)x[e];
  return v;
}

template <int D>
__global__ __launch_bounds__(256) void fwd_mfma(MP p) {
  constexpr int NC = D / 16, NB = D / 32;
  __shared__ __attribute__((aligned(16))) bf16 sK[64 * (D + 8)];
  __shared__ __attribute__((aligned(16))) bf16 sKl[64 * (D + 8)];
  __shared__ __attribute__((aligned(16))) bf16 sVt[D * 64];
  const int head = blockIdx.x;
  const int b = head / p.n_local, l = head - b * p.n_local;
  const int nqt = (p.seq + 127) / 128;
  const int qt = nqt - 1 - blockIdx.y;  // heaviest (longest causal prefix) first
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const long grow0 = (long)b * p.seq;
  const float* Qg = p.qkv + (long)l * D;
  const float* Kg = p.qkv + p.h_l + (long)l * D;
  const float* Vg = p.qkv + 2L * p.h_l + (long)l * D;
  const int q0w = qt * 128 + 32 * w;
  const int myq = q0w + l32;
  bf16x8 qf[NC], qfl[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    qf[c] = bf16x8{};
    qfl[c] = bf16x8{};
    if (myq < p.seq) load8_split(Qg + (grow0 + myq) * p.ld + 16 * c + 8 * g, qf[c], qfl[c]);
  }
  f32x16 o[NB];
#pragma unroll
  for (int db = 0; db < NB; ++db) o[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float slope2 = alibi_slope_log2(p, l);
  const int kv_end = min(p.seq, qt * 128 + 128);
  const int nkt = (kv_end + 63) / 64;
  for (int kt = 0; kt < nkt; ++kt) {
    const int kv0 = kt * 64;
    __syncthreads();
    stage_rows_split<D>(sK, sKl, Kg, p.ld, grow0, kv0, p.seq);
    stage_trans<D>(sVt, Vg, p.ld, grow0, kv0, p.seq);
    __syncthreads();
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int k0 = kv0 + 32 * sb;
      if (k0 > q0w + 31 || k0 >= p.seq) continue;  // wave-uniform: all masked
      f32x16 s = f32x16{};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int off = (32 * sb + l32) * (D + 8) + 16 * c + 8 * g;
        const bf16x8 kh = *(const bf16x8*)(sK + off), kl = *(const bf16x8*)(sKl + off);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kl, qf[c], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, qfl[c], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, qf[c], s, 0, 0, 0);
      }
      // s[q]: key k0 + 8(q>>2) + 4g + (q&3), query myq
      const bool need_mask = (k0 + 31 > q0w) || (k0 + 32 > p.seq);
      float x[16];
      float mloc = -INFINITY;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int key = k0 + 8 * (q >> 2) + 4 * g + (q & 3);
        float v = s[q] * p.scale_log2 - slope2 * (float)(myq - key);
        if (need_mask && (key > myq || key >= p.seq)) v = -INFINITY;
        x[q] = v;
        mloc = fmaxf(mloc, v);
      }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float m_new = fmaxf(m_run, mloc);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      float lloc = 0.f;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        x[q] = exp2f(x[q] - m_use);
        lloc += x[q];
      }
      lloc += __shfl_xor(lloc, 32);
      const float corr = exp2f(m_run - m_use);
      l_run = l_run * corr + lloc;
      m_run = m_new;
#pragma unroll
      for (int db = 0; db < NB; ++db) o[db] *= corr;
      const bf16x8 pf0 = pack8(x), pf1 = pack8(x + 8);
#pragma unroll
      for (int db = 0; db < NB; ++db) {
        const int d = 32 * db + l32;
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_trans(sVt, d, 2 * sb, g), pf0, o[db], 0, 0, 0);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_trans(sVt, d, 2 * sb + 1, g), pf1, o[db], 0, 0, 0);
      }
    }
  }
  if (myq < p.seq) {
    const float inv = 1.0f / l_run;
    bf16* dst = p.ctx + (grow0 + myq) * p.h_l + (long)l * D;
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (bf16)(o[db][4 * q4 + e] * inv);
        *(bf16x4*)(dst + 32 * db + 8 * q4 + 4 * g) = v;
      }
    if (g == 0) p.lse[(long)head * p.seq + myq] = (m_run + __log2f(l_run)) * (1.0f / kLog2e);
  }
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(1, 1))) void dkdv_mfma(MP p) {
  constexpr int NC = D / 16, NB = D / 32;
  __shared__ __attribute__((aligned(16))) bf16 sQ[64 * (D + 8)];
  __shared__ __attribute__((aligned(16))) bf16 sQl[64 * (D + 8)];
  __shared__ __attribute__((aligned(16))) bf16 sC[64 * (D + 8)];
  __shared__ __attribute__((aligned(16))) bf16 sQt[D * 64];
  __shared__ __attribute__((aligned(16))) bf16 sCt[D * 64];
  __shared__ __attribute__((aligned(16))) float sL[64];
  __shared__ __attribute__((aligned(16))) float sDl[64];
  const int head = blockIdx.x;
  const int b = head / p.n_local, l = head - b * p.n_local;
  const int kvt = blockIdx.y;  // 128-key tile; tile 0 sees the most queries
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const long grow0 = (long)b * p.seq;
  const float* Qg = p.qkv + (long)l * D;
  const float* Kg = p.qkv + p.h_l + (long)l * D;
  const float* Vg = p.qkv + 2L * p.h_l + (long)l * D;
  const bf16* Cg = p.dctx + (long)l * D;
  const int k0w = kvt * 128 + 32 * w;
  const int myk = k0w + l32;
  bf16x8 kf[NC], kfl[NC], vf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    kf[c] = bf16x8{};
    kfl[c] = bf16x8{};
    vf[c] = bf16x8{};
    if (myk < p.seq) {
      load8_split(Kg + (grow0 + myk) * p.ld + 16 * c + 8 * g, kf[c], kfl[c]);
      vf[c] = __builtin_bit_cast(bf16x8, load8(Vg + (grow0 + myk) * p.ld + 16 * c + 8 * g));
    }
  }
  f32x16 dv[NB], dk[NB];
#pragma unroll
  for (int db = 0; db < NB; ++db) { dv[db] = f32x16{}; dk[db] = f32x16{}; }
  const float slope2 = alibi_slope_log2(p, l);
  const int nqt = (p.seq + 63) / 64;
  for (int qt = (kvt * 128) / 64; qt < nqt; ++qt) {
    const int q0 = qt * 64;
    __syncthreads();
    stage_rows_split<D>(sQ, sQl, Qg, p.ld, grow0, q0, p.seq);
    stage_rows<D>(sC, Cg, p.h_l, grow0, q0, p.seq);
    stage_trans<D>(sQt, Qg, p.ld, grow0, q0, p.seq);
    stage_trans<D>(sCt, Cg, p.h_l, grow0, q0, p.seq);
    if (tid < 64) {
      const int pos = q0 + tid;
      sL[tid] = pos < p.seq ? p.lse[(long)head * p.seq + pos] * kLog2e : 0.f;
      sDl[tid] = pos < p.seq ? p.delta[(long)head * p.seq + pos] : 0.f;
    }
    __syncthreads();
    if (k0w >= p.seq) continue;
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const int qs0 = q0 + 32 * qs;
      if (qs0 + 31 < k0w || qs0 >= p.seq) continue;  // wave-uniform: all masked
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int off = (32 * qs + l32) * (D + 8) + 16 * c + 8 * g;
        const bf16x8 qh = *(const bf16x8*)(sQ + off), ql = *(const bf16x8*)(sQl + off);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ql, kf[c], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qh, kfl[c], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qh, kf[c], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(sC + off), vf[c], dp, 0, 0, 0);
      }
      // s[q], dp[q]: query qs0 + 8(q>>2) + 4g + (q&3), key myk
      const bool need_mask = (qs0 < k0w + 31) || (qs0 + 32 > p.seq);
      float pv[16], dsv[16];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const f32x4 L = *(const f32x4*)(sL + 32 * qs + 8 * q4 + 4 * g);
        const f32x4 Dl = *(const f32x4*)(sDl + 32 * qs + 8 * q4 + 4 * g);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int q = 4 * q4 + e;
          const int query = qs0 + 8 * q4 + 4 * g + e;
          float pp = exp2f(s[q] * p.scale_log2 - slope2 * (float)(query - myk) - L[e]);
          if (need_mask && (query < myk || query >= p.seq)) pp = 0.f;
          pv[q] = pp;
          dsv[q] = pp * (dp[q] - Dl[e]);
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const bf16x8 pf = pack8(pv + 8 * h), df = pack8(dsv + 8 * h);
#pragma unroll
        for (int db = 0; db < NB; ++db) {
          const int d = 32 * db + l32;
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_trans(sCt, d, 2 * qs + h, g), pf, dv[db], 0, 0, 0);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_trans(sQt, d, 2 * qs + h, g), df, dk[db], 0, 0, 0);
        }
      }
    }
  }
  if (myk < p.seq) {
    bf16* dK = p.dqkv + (grow0 + myk) * p.ld + p.h_l + (long)l * D;
    bf16* dV = p.dqkv + (grow0 + myk) * p.ld + 2L * p.h_l + (long)l * D;
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 a, c;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = (bf16)(dk[db][4 * q4 + e] * p.scale);
          c[e] = (bf16)dv[db][4 * q4 + e];
        }
        *(bf16x4*)(dK + 32 * db + 8 * q4 + 4 * g) = a;
        *(bf16x4*)(dV + 32 * db + 8 * q4 + 4 * g) = c;
      }
  }
}

template <int D>
__global__ __launch_bounds__(256) void dq_mfma(MP p) {
  constexpr int NC = D / 16, NB = D / 32;
  __shared__ __attribute__((aligned(16))) bf16 sK[64 * (D + 8)];
  __shared__ __attribute__((aligned(16))) bf16 sKl[64 * (D + 8)];
  __shared__ __attribute__((aligned(16))) bf16 sV[64 * (D + 8)];
  __shared__ __attribute__((aligned(16))) bf16 sKt[D * 64];
  const int head = blockIdx.x;
  const int b = head / p.n_local, l = head - b * p.n_local;
  const int nqt = (p.seq + 127) / 128;
  const int qt = nqt - 1 - blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;
  const long grow0 = (long)b * p.seq;
  const float* Qg = p.qkv + (long)l * D;
  const float* Kg = p.qkv + p.h_l + (long)l * D;
  const float* Vg = p.qkv + 2L * p.h_l + (long)l * D;
  const bf16* Cg = p.dctx + (long)l * D;
  const int q0w = qt * 128 + 32 * w;
  const int myq = q0w + l32;
  bf16x8 qf[NC], qfl[NC], cf[NC];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    qf[c] = bf16x8{};
    qfl[c] = bf16x8{};
    cf[c] = bf16x8{};
    if (myq < p.seq) {
      load8_split(Qg + (grow0 + myq) * p.ld + 16 * c + 8 * g, qf[c], qfl[c]);
      cf[c] = *(const bf16x8*)(Cg + (grow0 + myq) * p.h_l + 16 * c + 8 * g);
    }
  }
  const float L = myq < p.seq ? p.lse[(long)head * p.seq + myq] * kLog2e : 0.f;
  const float Dl = myq < p.seq ? p.delta[(long)head * p.seq + myq] : 0.f;
  f32x16 dq[NB];
#pragma unroll
  for (int db = 0; db < NB; ++db) dq[db] = f32x16{};
  const float slope2 = alibi_slope_log2(p, l);
  const int kv_end = min(p.seq, qt * 128 + 128);
  const int nkt = (kv_end + 63) / 64;
  for (int kt = 0; kt < nkt; ++kt) {
    const int kv0 = kt * 64;
    __syncthreads();
    stage_rows_split<D>(sK, sKl, Kg, p.ld, grow0, kv0, p.seq);
    stage_rows<D>(sV, Vg, p.ld, grow0, kv0, p.seq);
    stage_trans<D>(sKt, Kg, p.ld, grow0, kv0, p.seq);
    __syncthreads();
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int k0 = kv0 + 32 * sb;
      if (k0 > q0w + 31 || k0 >= p.seq) continue;
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const int off = (32 * sb + l32) * (D + 8) + 16 * c + 8 * g;
        const bf16x8 kh = *(const bf16x8*)(sK + off), kl = *(const bf16x8*)(sKl + off);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kl, qf[c], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, qfl[c], s, 0, 0, 0);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kh, qf[c], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*(const bf16x8*)(sV + off), cf[c], dp, 0, 0, 0);
      }
      // s[q]: key k0 + 8(q>>2) + 4g + (q&3), query myq
      const bool need_mask = (k0 + 31 > q0w) || (k0 + 32 > p.seq);
      float ds[16];
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int key = k0 + 8 * (q >> 2) + 4 * g + (q & 3);
        float pp = exp2f(s[q] * p.scale_log2 - slope2 * (float)(myq - key) - L);
        if (need_mask && (key > myq || key >= p.seq)) pp = 0.f;
        ds[q] = pp * (dp[q] - Dl);
      }
      const bf16x8 df0 = pack8(ds), df1 = pack8(ds + 8);
#pragma unroll
      for (int db = 0; db < NB; ++db) {
        const int d = 32 * db + l32;
        dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_trans(sKt, d, 2 * sb, g), df0, dq[db], 0, 0, 0);
        dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_trans(sKt, d, 2 * sb + 1, g), df1, dq[db], 0, 0, 0);
      }
    }
  }
  if (myq < p.seq) {
    bf16* dQ = p.dqkv + (grow0 + myq) * p.ld + (long)l * D;
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 a;
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = (bf16)(dq[db][4 * q4 + e] * p.scale);
        *(bf16x4*)(dQ + 32 * db + 8 * q4 + 4 * g) = a;
      }
  }
}

MP make_mp(const AttnDesc& a) {
  MP p{};
  p.batch = a.batch; p.seq = a.seq; p.n_local = a.n_local;
  p.h_l = a.n_local * a.head_dim; p.head0 = a.head0; p.n_heads = a.n_heads; p.alibi = a.alibi;
  p.ld = 3L * p.h_l;
  p.qkv = a.qkv; p.ctx = (bf16*)a.ctx; p.lse = a.lse;
  p.dctx = (const bf16*)a.dctx; p.delta = a.delta; p.dqkv = (bf16*)a.dqkv;
  p.scale = 1.0f / sqrtf((float)a.head_dim);
  p.scale_log2 = p.scale * kLog2e;
  return p;
}

template <int D>
hipError_t fwd_d(const MP& p, hipStream_t stream) {
  dim3 grid(p.batch * p.n_local, (p.seq + 127) / 128);
  hipLaunchKernelGGL(fwd_mfma<D>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}
template <int D>
hipError_t bwd_d(const MP& p, hipStream_t stream) {
  dim3 grid(p.batch * p.n_local, (p.seq + 127) / 128);
  hipLaunchKernelGGL(dkdv_mfma<D>, grid, dim3(256), 0, stream, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(dq_mfma<D>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

bool attn_mfma_supported(int dtype, int head_dim) {
  return dtype == DT_BF16 && (head_dim == 64 || head_dim == 96 || head_dim == 128 || head_dim == 160);
}

hipError_t attn_mfma_fwd(const AttnDesc& a, hipStream_t stream) {
  const MP p = make_mp(a);
  switch (a.head_dim) {
    case 64: return fwd_d<64>(p, stream);
    case 96: return fwd_d<96>(p, stream);
    case 128: return fwd_d<128>(p, stream);
    case 160: return fwd_d<160>(p, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t attn_mfma_bwd(const AttnDesc& a, hipStream_t stream) {
  const MP p = make_mp(a);
  switch (a.head_dim) {
    case 64: return bwd_d<64>(p, stream);
    case 96: return bwd_d<96>(p, stream);
    case 128: return bwd_d<128>(p, stream);
    case 160: return bwd_d<160>(p, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace tpk
