// bf16 GEMM on CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16), fp32 accumulation,
// with the layer's fused epilogues (bias, bias+GeLU, GeLU' scaling, fp32 out).
//
// Tiling: a 256x256 output tile per workgroup of 4 waves (2x2), each wave a
// 128x128 sub-tile = 4x4 MFMA blocks of 32x32 (256 fp32 accumulators per lane).
// K advances 64 at a time through two LDS stages (2 x 64 KiB): the next k-slab
// is fetched into registers while the current one feeds the MFMAs, then written
// to the other stage, one barrier per k-step.
//
// LDS layout: both operands are kept "k-inner": row r (an m or n index) holds
// its 64 k-values as eight 16-byte chunks; chunk c is stored at c ^ swz(r),
// swz(r) = (r ^ (r >> 3)) & 7, so the MFMA fragment reads (32 rows, one chunk)
// and the transposed writes (rows 8a+i for a run of a) hit distinct banks.
// Operands that are k-outer in memory (the weight of a forward product, both
// operands of a weight gradient) are transposed in registers, 8x8 bf16 blocks,
// on their way to LDS.
//
// Scheduling: data-parallel tiles, plus stream-K for the last partial wave when
// whole waves would leave many CUs idle: the leftover tiles' k-iterations are
// split evenly over all workgroups, each split tile's fp32 partials go to the
// workspace and a second kernel sums them in a fixed order and applies the
// epilogue (no inter-workgroup waiting inside a kernel).
#include "common.h"
#include "kernels.h"

namespace tpk {
namespace {

constexpr int BM = 256, BN = 256, BKK = 64, NTHR = 256;
constexpr int STAGE = BM * BKK;  // bf16 elements per operand per stage
constexpr int GMAX = 256;        // largest persistent grid (workspace sizing)
constexpr int GROUP_M = 8;       // tiles along M per raster group

struct KParams {
  const bf16* A; const bf16* B;
  long lda, ldb;
  int M, N, K;
  int tiles_m, tiles_n, iters;
  int grid;           // workgroups launched
  int dp_rounds;      // data-parallel tiles per workgroup
  int sk_grid;        // workgroups taking part in the stream-K phase
  long long sk_begin; // first stream-K iteration (= dp tiles * iters)
  long long sk_total; // stream-K iterations
  int epi;
  bf16* C; long ldc;
  bf16* C2; long ldc2;
  const bf16* bias;
  const bf16* aux; long ldaux;
  float* partials;    // [2*sk_grid][BM*BN]
};

__device__ __forceinline__ int logical_wg(int w, int g) {
  // Workgroups are dealt round-robin to the 8 XCDs; renumber so that
  // consecutive logical ids (neighbouring tiles) share an XCD and its L2.
  return (g % 8 == 0) ? (w % 8) * (g / 8) + (w / 8) : w;
}

__device__ __forceinline__ void tile_coords(const KParams& p, int t, int& tm, int& tn) {
  int group = GROUP_M * p.tiles_n;
  int g = t / group;
  int first_m = g * GROUP_M;
  int gm = min(p.tiles_m - first_m, GROUP_M);
  int r = t - g * group;
  tm = first_m + r % gm;
  tn = r / gm;
}

// ---- global -> registers (buffer loads, 32-bit offsets) -------------------
// A tile's operand panel is addressed through a buffer resource whose base is
// the panel's first row (k-inner) or first column (k-outer); loads whose
// offset is at or past num_records return zero, which covers ragged M/N edges
// and the k tail.
struct Panel {
  const bf16* base;  // workgroup-uniform
  uint32_t nrec;     // workgroup-uniform buffer size in bytes
  uint32_t kstep;    // workgroup-uniform bytes the panel advances per k-step
  uint32_t voff[8];  // per-thread byte offsets of its 8 loads (nrec = invalid)
  int kvalid_from;   // k-inner: this thread's k offset inside the slab (8*chunk)
};

__device__ __forceinline__ uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ const bf16* uni_ptr(const bf16* p) {
  const uint64_t v = (uint64_t)p;
  return (const bf16*)(((uint64_t)uni((uint32_t)(v >> 32)) << 32) | uni((uint32_t)v));
}

// k-inner operand X[r*ld + k], rows r0g.. of `rows`: thread owns chunk (tid&7)
// of rows (tid>>3)+32i.
__device__ __forceinline__ Panel panel_kinner(const bf16* X, long ld, int rows, int r0g) {
  Panel pn;
  const int tid = threadIdx.x, c = tid & 7, rr = tid >> 3;
  int nrows = rows - r0g;
  nrows = nrows < 256 ? nrows : 256;
  pn.base = uni_ptr(X + (long)r0g * ld);
  pn.nrec = uni((uint32_t)((long)nrows * ld * 2));
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int r = rr + 32 * i;
    pn.voff[i] = r < nrows ? (uint32_t)(((long)r * ld + 8 * c) * 2) : pn.nrec;
  }
  pn.kstep = BKK * 2;
  pn.kvalid_from = 8 * c;
  return pn;
}
// k-outer operand X[k*ld + r]: thread owns the 8x8 block (k-block tid>>5, r-block tid&31).
__device__ __forceinline__ Panel panel_kouter(const bf16* X, long ld, int rows, int K, int r0g) {
  Panel pn;
  const int tid = threadIdx.x, kb = tid >> 5, rb = tid & 31;
  pn.base = uni_ptr(X + r0g);
  pn.nrec = uni((uint32_t)(((long)K * ld - r0g) * 2));
  const bool colok = r0g + 8 * rb < rows;
#pragma unroll
  for (int j = 0; j < 8; ++j)
    pn.voff[j] = colok ? (uint32_t)(((long)(8 * kb + j) * ld + 8 * rb) * 2) : pn.nrec;
  pn.kstep = uni((uint32_t)(BKK * ld * 2));
  pn.kvalid_from = 0;
  return pn;
}

template <bool KIN>
__device__ __forceinline__ void load_panel(const Panel& pn, int kt, int K, u32x4 (&reg)[8]) {
  const int soff = (int)uni((uint32_t)kt * pn.kstep);
  __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)pn.base, (short)0, (int)pn.nrec, 0x00020000);
  if (KIN) {
    const bool kok = kt * BKK + pn.kvalid_from < K;
#pragma unroll
    for (int i = 0; i < 8; ++i) reg[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, kok ? pn.voff[i] : pn.nrec, soff, 0);
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) reg[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, pn.voff[i], soff, 0);
  }
}

// ---- registers -> LDS ----------------------------------------------------
// k-inner: row r = rr + 32i, swz(r) = (rr&7) ^ (rr>>3) ^ 4(i&1).
__device__ __forceinline__ void store_kinner(bf16* s, const u32x4 (&reg)[8]) {
  const int tid = threadIdx.x;
  const int c = tid & 7, rr = tid >> 3;
  const int s0 = (rr & 7) ^ (rr >> 3);
  bf16* b0 = s + rr * BKK + ((c ^ s0) << 3);
  bf16* b1 = s + rr * BKK + ((c ^ s0 ^ 4) << 3);
#pragma unroll
  for (int i = 0; i < 8; ++i) *(u32x4*)(((i & 1) ? b1 : b0) + i * 32 * BKK) = reg[i];
}
// k-outer: transpose the 8x8 block in registers. reg[j] is k-row j holding
// r = 8rb+0..7 as 4 dwords; output row r = 8rb+i takes element i of each reg[j].
__device__ __forceinline__ void store_kouter(bf16* s, const u32x4 (&reg)[8]) {
  const int tid = threadIdx.x;
  const int kb = tid >> 5, rb = tid & 31;
  const int t = kb ^ (rb & 7);
  bf16* base = s + rb * 8 * BKK;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int d = i >> 1;
    u32x4 o;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      uint32_t lo = reg[2 * q][d], hi = reg[2 * q + 1][d];
      o[q] = (i & 1) ? ((lo >> 16) | (hi & 0xFFFF0000u)) : ((lo & 0xFFFFu) | (hi << 16));
    }
    *(u32x4*)(base + i * BKK + ((t ^ i) << 3)) = o;
  }
}
template <bool KIN>
__device__ __forceinline__ void store_op(bf16* s, const u32x4 (&reg)[8]) {
  if (KIN) store_kinner(s, reg);
  else store_kouter(s, reg);
}

// ---- main loop over k-iterations [kb, ke) of one tile -------------------------
template <bool AK, bool BKM>
__device__ __forceinline__ void mainloop(const KParams& p, int tm, int tn, int kb, int ke,
                                         f32x16 (&acc)[4][4], bf16* sA, bf16* sB) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int g = lane >> 5, l32 = lane & 31;
  const int s1 = (l32 & 7) ^ (l32 >> 3);
  const bf16* fa = sA + (wm * 128 + l32) * BKK;
  const bf16* fb = sB + (wn * 128 + l32) * BKK;
  Panel pa, pb;
  if (AK) pa = panel_kinner(p.A, p.lda, p.M, tm * BM);
  else pa = panel_kouter(p.A, p.lda, p.M, p.K, tm * BM);
  if (BKM) pb = panel_kinner(p.B, p.ldb, p.N, tn * BN);
  else pb = panel_kouter(p.B, p.ldb, p.N, p.K, tn * BN);
  u32x4 ra[8], rb[8];
  load_panel<AK>(pa, kb, p.K, ra);
  load_panel<BKM>(pb, kb, p.K, rb);
  store_op<AK>(sA, ra);
  store_op<BKM>(sB, rb);
  __syncthreads();
  for (int kt = kb; kt < ke; ++kt) {
    const int cur = (kt - kb) & 1;
    const bool more = kt + 1 < ke;
    if (more) {
      load_panel<AK>(pa, kt + 1, p.K, ra);
      load_panel<BKM>(pb, kt + 1, p.K, rb);
    }
    const bf16* a = fa + cur * STAGE;
    const bf16* b = fb + cur * STAGE;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int e = (2 * kk) ^ g ^ s1;
      bf16x8 af[4], bfg[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) af[i] = *(const bf16x8*)(a + i * 32 * BKK + ((e ^ (4 * (i & 1))) << 3));
#pragma unroll
      for (int j = 0; j < 4; ++j) bfg[j] = *(const bf16x8*)(b + j * 32 * BKK + ((e ^ (4 * (j & 1))) << 3));
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          // operands swapped: D[n][m], so each lane ends up owning one m and
          // runs of 4 consecutive n (vector stores in the epilogue)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfg[j], af[i], acc[i][j], 0, 0, 0);
    }
    if (more) {
      store_op<AK>(sA + (cur ^ 1) * STAGE, ra);
      store_op<BKM>(sB + (cur ^ 1) * STAGE, rb);
    }
    __syncthreads();
  }
}

// ---- epilogue ---------------------------------------------------------------
// Lane owns m = base_m + (lane&31) and n = base_n + 8*q4 + 4*(lane>>5) + 0..3.
__device__ __forceinline__ void store_bf16x4(bf16* dst, const float (&v)[4]) {
  bf16x4 o;
  o[0] = (bf16)v[0]; o[1] = (bf16)v[1]; o[2] = (bf16)v[2]; o[3] = (bf16)v[3];
  *(bf16x4*)dst = o;
}

template <int EPI>
__device__ __forceinline__ void epilogue(const KParams& p, int tm, int tn, const f32x16 (&acc)[4][4]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = tm * BM + wm * 128 + i * 32 + (lane & 31);
    if (m >= p.M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int n = tn * BN + wn * 128 + j * 32 + q4 * 8 + (lane >> 5) * 4;
        if (n >= p.N) continue;
        float v[4] = {acc[i][j][4 * q4], acc[i][j][4 * q4 + 1], acc[i][j][4 * q4 + 2], acc[i][j][4 * q4 + 3]};
        if (EPI == EPI_BIAS || EPI == EPI_BIAS_GELU || EPI == EPI_BIAS_F32) {
          bf16x4 bb = *(const bf16x4*)(p.bias + n);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += (float)bb[e];
        }
        if (EPI == EPI_DGELU) {
          bf16x4 pa = *(const bf16x4*)(p.aux + (long)m * p.ldaux + n);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] *= gelu_grad_f((float)pa[e]);
        }
        if (EPI == EPI_BIAS_F32) {
          *(f32x4*)((float*)p.C + (long)m * p.ldc + n) = f32x4{v[0], v[1], v[2], v[3]};
          continue;
        }
        store_bf16x4(p.C + (long)m * p.ldc + n, v);
        if (EPI == EPI_BIAS_GELU) {
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = gelu_f(v[e]);
          store_bf16x4(p.C2 + (long)m * p.ldc2 + n, y);
        }
      }
    }
  }
}

// ---- stream-K bookkeeping -----------------------------------------------------
// The sk_total iterations are dealt in contiguous runs: workgroup c gets
// [c*base + min(c, rem), ... + base + (c < rem)).
__device__ __forceinline__ long long sk_start(long long c, long long base, long long rem) {
  return c * base + (c < rem ? c : rem);
}
__device__ __forceinline__ long long sk_owner(long long x, long long base, long long rem) {
  long long big = rem * (base + 1);
  return x < big ? x / (base + 1) : rem + (x - big) / base;
}

// Partial tiles are stored in accumulator order: float4 f4 of thread tid at
// (f4*256 + tid)*4, so each store/load instruction covers 4 KiB contiguously.
__device__ __forceinline__ void store_partial(float* slot, const f32x16 (&acc)[4][4]) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int f4 = (i * 4 + j) * 4 + q4;
        f32x4 v = {acc[i][j][4 * q4], acc[i][j][4 * q4 + 1], acc[i][j][4 * q4 + 2], acc[i][j][4 * q4 + 3]};
        *(f32x4*)(slot + ((long)f4 * NTHR + tid) * 4) = v;
      }
}

// One loop over this workgroup's work items: first its data-parallel tiles,
// then its run of stream-K iterations (whole tiles in the run are stored
// directly, partial tiles go to the workspace).
template <bool AK, bool BKM, int EPI>
__device__ __forceinline__ void gemm_body(const KParams& p, bf16* sA, bf16* sB) {
  const int lw = logical_wg(blockIdx.x, p.grid);
  const bool in_sk = p.sk_total > 0 && lw < p.sk_grid;
  long long base = 0, rem = 0, s = 0, e = 0;
  if (in_sk) {
    base = p.sk_total / p.sk_grid;
    rem = p.sk_total % p.sk_grid;
    s = sk_start(lw, base, rem);
    e = s + base + (lw < rem ? 1 : 0);
  }
  int r = 0;
  long long it = s;
  for (;;) {
    int t, kb, ke;
    if (r < p.dp_rounds) {
      t = r * p.grid + lw;
      kb = 0;
      ke = p.iters;
      ++r;
    } else if (it < e) {
      const long long ga = p.sk_begin + it;
      t = (int)(ga / p.iters);
      kb = (int)(ga - (long long)t * p.iters);
      ke = (int)min((long long)p.iters, kb + (e - it));
      it += ke - kb;
    } else {
      break;
    }
    int tm, tn;
    tile_coords(p, t, tm, tn);
    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
    mainloop<AK, BKM>(p, tm, tn, kb, ke, acc, sA, sB);
    if (kb == 0 && ke == p.iters) {
      epilogue<EPI>(p, tm, tn, acc);
    } else {
      const long long t0 = (long long)t * p.iters - p.sk_begin;  // tile start, SK-relative
      const int slot = 2 * lw + (s >= t0 ? 0 : 1);
      store_partial(p.partials + (long)slot * BM * BN, acc);
    }
  }
}

// One workgroup per stream-K tile: sum the contributors' partials in
// contributor order and apply the epilogue.
template <int EPI>
__device__ __forceinline__ void fixup_body(const KParams& p, int first_tile) {
  const int t = first_tile + blockIdx.x;
  const long long base = p.sk_total / p.sk_grid, rem = p.sk_total % p.sk_grid;
  const long long t0 = (long long)t * p.iters - p.sk_begin;
  const long long c0 = sk_owner(t0, base, rem), c1 = sk_owner(t0 + p.iters - 1, base, rem);
  if (c0 == c1) return;  // one workgroup covered the whole tile and stored it
  const int tid = threadIdx.x;
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};
  for (long long c = c0; c <= c1; ++c) {
    const int slot = (int)(2 * c + (sk_start(c, base, rem) >= t0 ? 0 : 1));
    const float* src = p.partials + (long)slot * BM * BN;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int f4 = (i * 4 + j) * 4 + q4;
          f32x4 v = *(const f32x4*)(src + ((long)f4 * NTHR + tid) * 4);
          acc[i][j][4 * q4] += v[0];
          acc[i][j][4 * q4 + 1] += v[1];
          acc[i][j][4 * q4 + 2] += v[2];
          acc[i][j][4 * q4 + 3] += v[3];
        }
  }
  int tm, tn;
  tile_coords(p, t, tm, tn);
  epilogue<EPI>(p, tm, tn, acc);
}

}  // namespace

// One kernel (and its stream-K fix-up kernel) per product of the layer, so
// that a trace attributes time to each step by name.
#define TP_GEMM_KERNELS(NAME, AKV, BKV, EV)                                           \
  __global__ __launch_bounds__(NTHR) __attribute__((amdgpu_waves_per_eu(1, 1)))     \
  void NAME(KParams p) {                                                            \
    __shared__ __attribute__((aligned(16))) bf16 sA[2 * STAGE];                     \
    __shared__ __attribute__((aligned(16))) bf16 sB[2 * STAGE];                     \
    gemm_body<AKV, BKV, EV>(p, sA, sB);                                             \
  }                                                                                 \
  __global__ __launch_bounds__(NTHR) void NAME##_fixup(KParams p, int first_tile) { \
    fixup_body<EV>(p, first_tile);                                                  \
  }

// forward products: A k-inner (activations), B k-outer (weights)
TP_GEMM_KERNELS(gemm_qkv_proj, true, false, EPI_BIAS_F32)
TP_GEMM_KERNELS(gemm_out_proj, true, false, EPI_STORE)
TP_GEMM_KERNELS(gemm_fc1_bias_gelu, true, false, EPI_BIAS_GELU)
TP_GEMM_KERNELS(gemm_fc2, true, false, EPI_STORE)
// input gradients: both k-inner (weights read transposed)
TP_GEMM_KERNELS(gemm_fc2_dgrad_gelu, true, true, EPI_DGELU)
TP_GEMM_KERNELS(gemm_fc1_dgrad, true, true, EPI_STORE)
TP_GEMM_KERNELS(gemm_out_dgrad, true, true, EPI_STORE)
TP_GEMM_KERNELS(gemm_qkv_dgrad, true, true, EPI_STORE)
// weight gradients: both k-outer (K = tokens)
TP_GEMM_KERNELS(gemm_fc2_wgrad, false, false, EPI_STORE)
TP_GEMM_KERNELS(gemm_fc1_wgrad, false, false, EPI_STORE)
TP_GEMM_KERNELS(gemm_out_wgrad, false, false, EPI_STORE)
TP_GEMM_KERNELS(gemm_qkv_wgrad, false, false, EPI_STORE)
#undef TP_GEMM_KERNELS

namespace {

struct Plan {
  int grid, dp_rounds, sk_grid, sk_first_tile, sk_tiles;
  long long sk_begin, sk_total;
};

Plan make_plan(int tiles, int iters, int ncu) {
  Plan pl{};
  ncu = ncu < GMAX ? ncu : GMAX;
  const int waves = (tiles + ncu - 1) / ncu;
  const double eff_dp = (double)tiles / ((double)waves * ncu);
  if (iters < 8 || eff_dp >= 0.9) {
    pl.grid = tiles; pl.dp_rounds = 1;
    return pl;
  }
  const int full = tiles / ncu;
  pl.grid = ncu;
  pl.dp_rounds = full;
  pl.sk_first_tile = full * ncu;
  pl.sk_tiles = tiles - pl.sk_first_tile;
  pl.sk_begin = (long long)pl.sk_first_tile * iters;
  pl.sk_total = (long long)pl.sk_tiles * iters;
  pl.sk_grid = (int)(pl.sk_total < ncu ? pl.sk_total : ncu);
  return pl;
}

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return GMAX;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = GMAX;
    cached[dev] = n;
  }
  return cached[dev];
}

}  // namespace

size_t gemm_mfma_workspace_bytes(int M, int N, int K) {
  const long long tiles = (long long)((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const long long iters = (K + BKK - 1) / BKK;
  if (iters < 8 || tiles <= 0) return 0;
  long long slots = 2LL * GMAX;
  if (slots > 2 * tiles * iters) slots = 2 * tiles * iters;
  return (size_t)slots * BM * BN * sizeof(float);
}

hipError_t gemm_mfma_launch(const GemmDesc& g, void* ws, size_t ws_bytes, hipStream_t stream) {
  KParams p{};
  p.A = (const bf16*)g.A; p.B = (const bf16*)g.B;
  p.lda = g.lda; p.ldb = g.ldb;
  p.M = g.M; p.N = g.N; p.K = g.K;
  p.tiles_m = (g.M + BM - 1) / BM;
  p.tiles_n = (g.N + BN - 1) / BN;
  p.iters = (g.K + BKK - 1) / BKK;
  p.epi = g.epi;
  p.C = (bf16*)g.C; p.ldc = g.ldc;
  p.C2 = (bf16*)g.C2; p.ldc2 = g.ldc2;
  p.bias = (const bf16*)g.bias;
  p.aux = (const bf16*)g.aux; p.ldaux = g.ldaux;
  p.partials = (float*)ws;
  const int tiles = p.tiles_m * p.tiles_n;
  Plan pl = make_plan(tiles, p.iters, device_cus());
  if (pl.sk_total > 0) {
    const size_t need = (size_t)2 * pl.sk_grid * BM * BN * sizeof(float);
    if (ws == nullptr || ws_bytes < need) pl = Plan{tiles, 1, 0, 0, 0, 0, 0};  // data-parallel only
  }
  p.grid = pl.grid; p.dp_rounds = pl.dp_rounds; p.sk_grid = pl.sk_grid;
  p.sk_begin = pl.sk_begin; p.sk_total = pl.sk_total;
  dim3 grid(pl.grid), block(NTHR);
  const int first = pl.sk_first_tile, nsk = pl.sk_tiles;
  const bool sk = pl.sk_total > 0;
  typedef void (*MainK)(KParams);
  typedef void (*FixK)(KParams, int);
  MainK mk = nullptr;
  FixK fk = nullptr;
  bool ak = true, bk = false;
  int ep = EPI_STORE;
#define TP_ROLE(R, NAME, AKV, BKV, EV) \
  case R: mk = NAME; fk = NAME##_fixup; ak = AKV; bk = BKV; ep = EV; break;
  switch (g.role) {
    TP_ROLE(GR_QKV_PROJ, gemm_qkv_proj, true, false, EPI_BIAS_F32)
    TP_ROLE(GR_OUT_PROJ, gemm_out_proj, true, false, EPI_STORE)
    TP_ROLE(GR_FC1, gemm_fc1_bias_gelu, true, false, EPI_BIAS_GELU)
    TP_ROLE(GR_FC2, gemm_fc2, true, false, EPI_STORE)
    TP_ROLE(GR_FC2_DGRAD, gemm_fc2_dgrad_gelu, true, true, EPI_DGELU)
    TP_ROLE(GR_FC1_DGRAD, gemm_fc1_dgrad, true, true, EPI_STORE)
    TP_ROLE(GR_OUT_DGRAD, gemm_out_dgrad, true, true, EPI_STORE)
    TP_ROLE(GR_QKV_DGRAD, gemm_qkv_dgrad, true, true, EPI_STORE)
    TP_ROLE(GR_FC2_WGRAD, gemm_fc2_wgrad, false, false, EPI_STORE)
    TP_ROLE(GR_FC1_WGRAD, gemm_fc1_wgrad, false, false, EPI_STORE)
    TP_ROLE(GR_OUT_WGRAD, gemm_out_wgrad, false, false, EPI_STORE)
    TP_ROLE(GR_QKV_WGRAD, gemm_qkv_wgrad, false, false, EPI_STORE)
    default: return hipErrorInvalidValue;
  }
#undef TP_ROLE
  if (g.a_kmajor != ak || g.b_kmajor != bk || g.epi != ep) return hipErrorInvalidValue;
  hipLaunchKernelGGL(mk, grid, block, 0, stream, p);
  hipError_t e1 = hipGetLastError();
  if (e1 != hipSuccess || !sk) return e1;
  hipLaunchKernelGGL(fk, dim3(nsk), block, 0, stream, p, first);
  return hipGetLastError();
}

}  // namespace tpk
