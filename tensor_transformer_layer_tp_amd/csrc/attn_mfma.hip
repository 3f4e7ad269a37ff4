// Flash-style causal attention for bf16 on CDNA4 matrix cores
// (v_mfma_f32_32x32x16_bf16), head widths D in {64, 96, 128, 160}.
//
// Inputs: per rank, the QKV projection's five 16-bit planes [T, h_l] (written
// by its GEMM epilogue; local head l uses columns l*D..; row t = b*seq +
// position): q16 = fp16(q log2(e) / sqrt(D)), k16 = fp16(k) for the scores,
// and qb = bf16(q), kb = bf16(k), v = bf16(v) for the gradient and value
// products. Outputs: ctx [T, h_l] bf16, lse [batch, n_local, seq] fp32
// (natural log); backward dqkv [T, 3*h_l] bf16.
//
// Precision: the scores are one fp16 product q16 k16^T (fp32 accumulation),
// already in log2 units. Rows of large, nearly tied scores amplify the
// rounding of q and k far beyond the rounding of the output: with bf16 q and
// k (8-bit significands) the 530B-like shard's input gradients move by 1.2e-2
// relative, with fp16 (11 bits) by 1.5e-3. fp16 holds the scaled q and k of
// these layers with room to spare (|q log2(e)/sqrt(D)|, |k| far below 65504;
// larger values saturate to +-65504). V, P, dS and dctx enter
// the products as bf16 (their rounding is not amplified, and bf16 keeps the
// gradients' fp32 range).
//
// Tiles of 64 rows x D columns are staged in LDS by buffer loads that write
// LDS directly, double-buffered (the next tile's loads are in flight while
// the current tile is used), row-major with a row stride of 192 bytes (D <=
// 96) or 320 (D >= 128; D = 64 and 128 leave 4 unused 16-byte chunks per
// row), so that each 1 KiB load takes whole row segments of a few rows
// rather than one 16-byte chunk of 64 rows (64 cache lines per
// instruction). Logical chunk c of row r sits at physical chunk
// 4(c/4) + ((c mod 4) xor s(r)), s(r) = 2 bit2(r) + bit3(r). A tile is read
// two ways, both free of bank conflicts by that swizzle (a CPU simulation of
// both reads under each lane grouping the hardware may use):
//  * as rows (MFMA A operand "rows x D"): one ds_read_b128 per lane, lanes
//    0..31 read 32 consecutive rows of one chunk;
//  * transposed (A operand "D x rows"): two ds_read_b64_tr_b16 per lane, the
//    gfx950 transposing read, each giving a lane 4 consecutive rows of its
//    column. The row order within 16-row groups follows the key/query order
//    the score accumulators produce, so P (or dS) is fed from registers as the
//    B operand without any shuffle.
//
// Forward (workgroup = 8 waves = 128 queries of one head; a pair of waves
// shares 32 queries and splits every 64-key tile into its two 32-key halves):
// S^T = K Q^T for 32 keys x the wave's 32 queries, so each lane holds one
// query column and the softmax statistics (max, sum) are per lane, combined
// with the partner lane 32 away; ctx^T += V^T P^T; the pair merges at the end.
//
// Backward (workgroup = 8 waves, two per SIMD): dK/dV of 128 keys looping
// over 64-query tiles, each 32-key pair of waves split into a role that
// recomputes P from lse and accumulates dV and a role that forms dP and
// dS = P (dP - delta) (delta = rowsum(dctx * ctx)) and accumulates dK; dQ of
// 128 queries looping over 64-key tiles, each 32-query pair splitting the key
// tiles' halves. No atomics.
//
// Dropout variants (DO): the forward draws, per lane and 32-key block, one
// Philox4x64-10 block at counter (query, key block, batch << 32 | global head,
// g) with key (seed, offset): 16 uniforms of 16 bits for the lane's 16 keys
// (key k0 + 8(q>>2) + 4g + (q&3) takes lane q), kept iff >= thr. It zeroes
// the dropped probabilities before the value product (the row sum keeps them
// all), scales the output by 65536 / (65536 - thr), and stores the 16 keep
// bits as one 16-bit word mask[batch][head][key block][g][query] (rows padded
// to a multiple of 8). The backward kernels read those words: dP and (for dV)
// P are multiplied by keep * scale.
#include "common.h"
#include "kernels.h"
#include "philox.h"

namespace tpk {
namespace {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int TROWS = 64;  // rows per staged tile

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void* lds_ptr;
typedef __attribute__((address_space(3))) i16x4* lds_i16x4;

struct MP {
  int batch, seq, n_local, h_l, head0, n_heads, alibi;
  long T;
  // [T, h_l] each: scaled fp16 q and fp16 k (scores), bf16 q, k, v
  const bf16* q16; const bf16* qb; const bf16* k16; const bf16* kb; const bf16* vh;
  bf16* ctx;
  float* lse;
  const bf16* dctx;    // [T, h_l]
  const float* delta;  // [batch, n_local, seq]
  bf16* dqkv;          // [T, 3*h_l]
  float scale;         // 1 / sqrt(D) (q16 carries log2(e) / sqrt(D) already)
  // dropout (DO kernels)
  uint16_t* mask;      // [batch][n_local][nkb][2][mstride] keep bits
  int nkb, mstride;    // ceil(seq / 32); seq rounded up to a multiple of 8
  uint32_t drop_thr;   // keep iff the 16-bit uniform >= drop_thr
  float drop_scale;    // 65536 / (65536 - drop_thr)
  uint64_t seed, offset;
  // forward key-split items: partial (output, max, sum) of each half,
  // [2][batch * n_local][seq][D] and [2][batch * n_local][seq]
  float* part_o;
  float* part_ml;
};

// Forward work items, heaviest first: item = qt << 2 | part, where part 0 is
// a whole 128-query tile and parts 1, 2 are the two halves of its key tiles.
// n == 0: no table, blockIdx.y = nqt - 1 - qt.
constexpr int kMaxFwdItems = 512;
struct FwdItems {
  int n;
  int qsplit;  // query tiles >= qsplit are split (== nqt: none)
  uint16_t it[kMaxFwdItems];
};

// Keep bits (bit q = lane q's key) of query i, key block kb, half g.
__device__ __forceinline__ uint32_t keep_bits(const MP& p, int b, int hk, int i, int kb, int g) {
  uint64_t x0 = (uint64_t)i, x1 = (uint64_t)kb, x2 = ((uint64_t)b << 32) | (uint64_t)hk, x3 = (uint64_t)g;
  philox4x64_10(x0, x1, x2, x3, p.seed, p.offset);
  const uint64_t w[4] = {x0, x1, x2, x3};
  uint32_t bits = 0;
#pragma unroll
  for (int q = 0; q < 16; ++q) bits |= (uint32_t)(((w[q >> 2] >> (16 * (q & 3))) & 0xFFFFull) >= p.drop_thr) << q;
  return bits;
}

__device__ __forceinline__ uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ const void* uni_ptr(const void* p) {
  const uint64_t v = (uint64_t)p;
  return (const void*)(((uint64_t)uni((uint32_t)(v >> 32)) << 32) | uni((uint32_t)v));
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, uint32_t nrec) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)uni_ptr(base), (short)0, (int)uni(nrec), 0x00020000);
}

__device__ __forceinline__ float alibi_slope_log2(const MP& p, int l) {
  // global head k = head0 + l + 1 (1-based): slope 2^(-8k/n_heads), in log2 units
  return p.alibi ? exp2f(-8.0f * (float)(p.head0 + l + 1) / (float)p.n_heads) * kLog2e : 0.0f;
}


// Row stride and size of a staged tile (see the layout above).
template <int D>
constexpr int tile_rs() { return D <= 96 ? 192 : 320; }
template <int D>
constexpr int tile_bytes() { return TROWS * tile_rs<D>(); }
__device__ __forceinline__ int lswz(int r) { return ((r >> 1) & 2) | ((r >> 3) & 1); }

// Per-lane source offsets of the 1 KiB blocks wave w fills in a tile:
// blocks j = w, w + NW, ... of the tile's tile_rs/16; lane i of block j
// writes bytes 1024 j + 16 i = row r, physical chunk q, which holds logical
// chunk c; off[k] = 2 (r h_l + 8 c) bytes from the tile's first element, or
// ~0 for an unused chunk.
template <int D, int NW>
struct TileLanes {
  static constexpr int S = tile_rs<D>() / 16;
  static constexpr int K = (S + NW - 1) / NW;
  uint32_t off[K];
};
template <int D, int NW>
__device__ __forceinline__ TileLanes<D, NW> tile_lanes(int h_l, int w, int lane) {
  TileLanes<D, NW> t;
#pragma unroll
  for (int k = 0; k < TileLanes<D, NW>::K; ++k) {
    const int o = 1024 * (w + NW * k) + 16 * lane;
    const int r = o / tile_rs<D>(), q = (o - r * tile_rs<D>()) >> 4;
    const int c = 4 * (q >> 2) + ((q & 3) ^ lswz(r));
    t.off[k] = c < D / 8 ? (uint32_t)(2 * (r * h_l + 8 * c)) : 0xffffffffu;
  }
  return t;
}

// Stage rows [row0, row0 + 64) of columns [col0, col0 + D) of a [T, h_l] bf16
// array into a tile. Rows at or past seq read zeros (offset beyond the
// buffer): a lane's row r is inside the sequence iff its offset is below
// 2 (seq - row0) h_l, as 16 c < 2 h_l.
template <int D, int NW = 4>
__device__ __forceinline__ void dma_tile(const bf16* arr, uint32_t nrec, char* tile, long grow0, int col0, int row0,
                                         int seq, int h_l, int w, const TileLanes<D, NW>& tl) {
  const __amdgpu_buffer_rsrc_t rs = rsrc(arr, nrec);
  const int rows = min(seq - row0, TROWS);
  const uint32_t lim = rows > 0 ? (uint32_t)(2 * rows * h_l) : 0u;
  const uint32_t base = (uint32_t)(((grow0 + row0) * h_l + col0) * 2);
#pragma unroll
  for (int k = 0; k < TileLanes<D, NW>::K; ++k) {
    const int j = w + NW * k;
    if (j < TileLanes<D, NW>::S) {
      const uint32_t o = tl.off[k];
      const uint32_t vo = o < lim ? base + o : nrec;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(tile + 1024 * j), 16, vo, 0, 0, 0);
    }
  }
}

// Row fragment for MFMA operand "rows x D": lane l reads row 32blk + (l & 31),
// columns 16c + 8(l >> 5) .. +7, i.e. logical chunk 2c + g, at physical chunk
// 4(c >> 1) + ((2(c & 1) + g) xor s(row)); s(row) = s(l & 31), so two
// per-lane offsets (c even, c odd) plus compile-time constants address every
// fragment.
struct RowOff {
  int e, o;
};
template <int D>
__device__ __forceinline__ RowOff row_offsets(int lane) {
  const int g = lane >> 5, l32 = lane & 31, f = lswz(l32);
  RowOff r;
  r.e = l32 * tile_rs<D>() + 16 * (g ^ f);
  r.o = l32 * tile_rs<D>() + 16 * ((2 + g) ^ f);
  return r;
}
template <int D>
__device__ __forceinline__ bf16x8 frag_row(const char* tile, int blk, int c, const RowOff& ro) {
  return *(const bf16x8*)(tile + ((c & 1) ? ro.o : ro.e) + 64 * (c >> 1) + blk * 32 * tile_rs<D>());
}

// 2^x by the hardware instruction (inputs here are <= 2^8 or far below 0;
// results below the normal range flush to 0, which softmax weights tolerate).
__device__ __forceinline__ float fexp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Transposed fragment: lane l gets column 32db + (l & 31) of rows
// 16kc + 4g + {0..3} and 16kc + 8 + 4g + {0..3} (g = l >> 5). In each 16-lane
// group, lane 4r + c fetches 4 columns of one of those rows; the per-lane
// byte offsets (relative to chunk 4db, row 16kc) are tr_offsets' a and b.
struct TrOff {
  int a, b;
};
template <int D>
__device__ __forceinline__ TrOff tr_offsets(int lane) {
  const int G = lane >> 4, r = (lane >> 2) & 3, c = lane & 3, g = lane >> 5;
  const int x = 2 * (G & 1) + (c >> 1);  // chunk within the 4-chunk (32-column) block
  const int ra = 4 * g + r, rb = 8 + ra;
  TrOff o;
  o.a = ra * tile_rs<D>() + 16 * (x ^ lswz(ra)) + 8 * (c & 1);
  o.b = rb * tile_rs<D>() + 16 * (x ^ lswz(rb)) + 8 * (c & 1);
  return o;
}
template <int D>
__device__ __forceinline__ bf16x8 frag_tr(const char* tile, int db, int kc, const TrOff& o) {
  const char* b = tile + 64 * db + kc * 16 * tile_rs<D>();
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(b + o.a));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(b + o.b));
  const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f16x8 as_f16(bf16x8 v) { return __builtin_bit_cast(f16x8, v); }
// score product of fp16 fragments (stored in 16-bit slots typed bf16x8)
__device__ __forceinline__ f32x16 mfma_f16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(as_f16(a), as_f16(b), c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 pack8(const float* x) {
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (bf16)x[e];
  return v;
}

__device__ __forceinline__ bf16x8 ld8(const bf16* p) { return *(const bf16x8*)p; }

// This wave's LDS reads and writes have completed, then the workgroup
// barrier (the LDS-only form: loads into LDS stay in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// This wave's loads into LDS have landed, then the workgroup barrier: after it
// every wave's loads have landed. (The barrier's own fence does not wait for
// loads that write LDS directly.)
__device__ __forceinline__ void loads_landed_barrier() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

// ---- forward ---------------------------------------------------------------------
template <int D>
struct FwdState {
  bf16x8 qf[D / 16];  // q16 fragments (fp16 bits)
  f32x16 o[D / 32];
  float m_run, l_run;
};

// Scores of one 32-key block in log2 units, masked to -inf where the key is
// after the query or past the sequence (MASK: only blocks on the diagonal or
// at the end need it).
template <bool MASK, bool AL>
__device__ __forceinline__ float fwd_scores(const f32x16& sa, float (&x)[16], float slope2, int k0, int g, int myq,
                                            int seq) {
  float mloc = -INFINITY;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int key = k0 + 8 * (q >> 2) + 4 * g + (q & 3);
    float v = sa[q];
    if (AL) v -= slope2 * (float)(myq - key);
    if (MASK && (key > myq || key >= seq)) v = -INFINITY;
    x[q] = v;
    mloc = fmaxf(mloc, v);
  }
  return mloc;
}

// Running softmax with a lazily moved reference: the reference max m_run only
// moves when a row's max exceeds it by more than 2^8, so weights stay below
// 2^8 (exact in fp32, in range for bf16) and the output accumulator is
// rescaled only when some row of the wave moves its reference.
constexpr float kLazy = 8.0f;

// One 32-key block (keys k0 .. k0 + 31, block sb of the 64-key tile in `cur`:
// K16 and V at 0 and TB) for this wave's 32 queries.
template <int D, bool AL, bool DO>
__device__ __forceinline__ void fwd_block(const MP& p, const char* __restrict__ cur, int k0, int sb, int g,
                                          int q0w, int myq, float slope2, const TrOff& tro, const RowOff& ro,
                                          int b, int head, int hk, FwdState<D>& st) {
  constexpr int NC = D / 16, NB = D / 32, TB = tile_bytes<D>();
  f32x16 sa = f32x16{};
#pragma unroll
  for (int c = 0; c < NC; ++c) sa = mfma_f16(frag_row<D>(cur, sb, c, ro), st.qf[c], sa);
  // s[q]: key k0 + 8(q>>2) + 4g + (q&3), query myq, in log2 units
  float x[16];
  float mloc;
  if ((k0 + 31 > q0w) || (k0 + 32 > p.seq))
    mloc = fwd_scores<true, AL>(sa, x, slope2, k0, g, myq, p.seq);
  else
    mloc = fwd_scores<false, AL>(sa, x, slope2, k0, g, myq, p.seq);
  mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
  const bool move = mloc > st.m_run + kLazy;  // also true on a row's first unmasked keys
  if (__ballot(move)) {                        // wave-uniform
    const float m_new = move ? mloc : st.m_run;
    const float corr = move ? fexp2(st.m_run - m_new) : 1.0f;
    st.l_run *= corr;
    st.m_run = m_new;
#pragma unroll
    for (int db = 0; db < NB; ++db) st.o[db] *= corr;
  }
  const float m_use = (st.m_run == -INFINITY) ? 0.f : st.m_run;
  float lloc = 0.f;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    x[q] = fexp2(x[q] - m_use);
    lloc += x[q];
  }
  st.l_run += lloc + __shfl_xor(lloc, 32);
  if (DO) {
    const int kb = k0 >> 5;
    const uint32_t bits = keep_bits(p, b, hk, myq, kb, g);
    if (myq < p.seq) p.mask[((long)(head * p.nkb + kb) * 2 + g) * p.mstride + myq] = (uint16_t)bits;
#pragma unroll
    for (int q = 0; q < 16; ++q) x[q] = ((bits >> q) & 1u) ? x[q] : 0.f;
  }
  const bf16x8 pf0 = pack8(x), pf1 = pack8(x + 8);
  const char* vt = cur + TB;
#pragma unroll
  for (int db = 0; db < NB; ++db) {
    st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_tr<D>(vt, db, 2 * sb, tro), pf0, st.o[db], 0, 0, 0);
    st.o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_tr<D>(vt, db, 2 * sb + 1, tro), pf1, st.o[db], 0, 0, 0);
  }
}

// Forward workgroup: 8 waves, two per SIMD. Wave w takes queries
// q0 + 32(w & 3) .. +31 and, of every 64-key tile, the 32-key half w >> 2, so
// the two waves of a pair see disjoint key sets with the same queries; each
// keeps its own running (max reference, sum, output), and the pair merges
// through LDS at the end. Two waves per SIMD let one wave's softmax
// arithmetic overlap the other's matrix products.
constexpr int FWD_WAVES = 8;

template <int D, bool AL, bool DO>
__global__ __launch_bounds__(64 * FWD_WAVES) void fwd_mfma(MP p, FwdItems items) {
  constexpr int NC = D / 16, NB = D / 32, TB = tile_bytes<D>();
  constexpr int NX = NB * 16 + 2;  // floats a wave hands to its partner, per lane
  // two stages of (K16, V) tiles; the pair merge at the end reuses the memory
  constexpr int SZ = 4 * TB > 4 * NX * 64 * 4 ? 4 * TB : 4 * NX * 64 * 4;
  __shared__ __attribute__((aligned(16))) char stage[SZ];
  const int head = blockIdx.x;
  const int b = head / p.n_local, l = head - b * p.n_local;
  const int nqt = (p.seq + 127) / 128;
  int qt = nqt - 1 - (int)blockIdx.y, part = 0;  // heaviest (longest causal prefix) first
  if (items.n) {
    const int it = items.it[blockIdx.y];
    qt = it >> 2;
    part = it & 3;
  }
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = (int)uni((uint32_t)(tid >> 6));
  const TileLanes<D, FWD_WAVES> tl = tile_lanes<D, FWD_WAVES>(p.h_l, w, lane);
  const int qw = w & 3, kh = w >> 2;
  const long grow0 = (long)b * p.seq;
  const int q0w = qt * 128 + 32 * qw;
  const int myq = q0w + l32;
  const uint32_t nrec = (uint32_t)(p.T * p.h_l * 2);
  const int kv_end = min(p.seq, qt * 128 + 128);
  const int nkt = (kv_end + TROWS - 1) / TROWS;
  // key tiles [ktb, kte): all of them, or one half of a split item (every
  // query of a split tile has keys in both halves)
  const int ktb = part == 2 ? nkt / 2 : 0, kte = part == 1 ? nkt / 2 : nkt;
  dma_tile<D, FWD_WAVES>(p.k16, nrec, stage, grow0, l * D, ktb * TROWS, p.seq, p.h_l, w, tl);
  dma_tile<D, FWD_WAVES>(p.vh, nrec, stage + TB, grow0, l * D, ktb * TROWS, p.seq, p.h_l, w, tl);
  FwdState<D> st;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    st.qf[c] = bf16x8{};
    if (myq < p.seq) st.qf[c] = ld8(p.q16 + (grow0 + myq) * p.h_l + (long)l * D + 16 * c + 8 * g);
  }
#pragma unroll
  for (int db = 0; db < NB; ++db) st.o[db] = f32x16{};
  st.m_run = -INFINITY;
  st.l_run = 0.f;
  const float slope2 = alibi_slope_log2(p, l);
  const TrOff tro = tr_offsets<D>(lane);
  const RowOff ro = row_offsets<D>(lane);
  for (int kt = ktb; kt < kte; ++kt) {
    loads_landed_barrier();  // tile kt is in LDS; tile kt-1 is no longer read
    const bool odd = (kt - ktb) & 1;
    const char* cur = odd ? stage + 2 * TB : stage;
    char* nxt = odd ? stage : stage + 2 * TB;
    const int kv0 = kt * TROWS;
    if (kt + 1 < kte) {
      dma_tile<D, FWD_WAVES>(p.k16, nrec, nxt, grow0, l * D, kv0 + TROWS, p.seq, p.h_l, w, tl);
      dma_tile<D, FWD_WAVES>(p.vh, nrec, nxt + TB, grow0, l * D, kv0 + TROWS, p.seq, p.h_l, w, tl);
    }
    const int k0 = kv0 + 32 * kh;
    if (k0 <= q0w + 31 && k0 < p.seq)  // wave-uniform; otherwise every key is masked
      fwd_block<D, AL, DO>(p, cur, k0, kh, g, q0w, myq, slope2, tro, ro, b, head, p.head0 + l, st);
  }
  // Pair merge. The last tile issued no loads, so after this barrier no wave
  // reads or writes the stages any more.
  __syncthreads();
  float* xs = (float*)stage + qw * NX * 64 + lane;
  if (kh) {
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) xs[(16 * db + i) * 64] = st.o[db][i];
    xs[NB * 16 * 64] = st.m_run;
    xs[(NB * 16 + 1) * 64] = st.l_run;
  }
  __syncthreads();
  if (kh || myq >= p.seq) return;
  const float m2 = xs[NB * 16 * 64], l2 = xs[(NB * 16 + 1) * 64];
  const float m = fmaxf(st.m_run, m2);  // finite: key myq is in one of the two halves
  const float f1 = st.m_run == -INFINITY ? 0.f : fexp2(st.m_run - m);
  const float f2 = m2 == -INFINITY ? 0.f : fexp2(m2 - m);
  const float lsum = st.l_run * f1 + l2 * f2;
  if (part) {
    // this half's output relative to its max m, with its sum; the merge
    // kernel combines the two halves
    const long row = ((long)(part - 1) * p.batch * p.n_local + head) * p.seq + myq;
    float* po = p.part_o + row * D;
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * q4 + e;
          v[e] = st.o[db][i] * f1 + xs[(16 * db + i) * 64] * f2;
        }
        *(f32x4*)(po + 32 * db + 8 * q4 + 4 * g) = v;
      }
    if (g == 0) {
      p.part_ml[2 * row] = m;
      p.part_ml[2 * row + 1] = lsum;
    }
    return;
  }
  const float inv = (DO ? p.drop_scale : 1.0f) / lsum;
  bf16* dst = p.ctx + (grow0 + myq) * p.h_l + (long)l * D;
#pragma unroll
  for (int db = 0; db < NB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * q4 + e;
        v[e] = (bf16)((st.o[db][i] * f1 + xs[(16 * db + i) * 64] * f2) * inv);
      }
      *(bf16x4*)(dst + 32 * db + 8 * q4 + 4 * g) = v;
    }
  if (g == 0) p.lse[(long)head * p.seq + myq] = (m + __log2f(lsum)) * (1.0f / kLog2e);
}

// Merge of the two key halves of each split query tile: per query, with
// m = max(m1, m2), ctx = (o1 2^(m1-m) + o2 2^(m2-m)) / (l1 2^(m1-m) + l2 2^(m2-m))
// (times the dropout scale) and lse = m + log2(sum), in natural log. One
// thread per query and 8 output columns.
template <int D, bool DO>
__global__ __launch_bounds__(256) void fwd_merge_kernel(MP p, int q_first) {
  constexpr int CH = D / 8;
  const int nq = p.seq - q_first, nh = p.batch * p.n_local;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)nh * nq * CH) return;
  const int ch = (int)(idx % CH);
  const long hq = idx / CH;
  const int head = (int)(hq / nq), q = q_first + (int)(hq % nq);
  const long r1 = (long)head * p.seq + q, r2 = ((long)nh + head) * p.seq + q;
  const float m1 = p.part_ml[2 * r1], l1 = p.part_ml[2 * r1 + 1];
  const float m2 = p.part_ml[2 * r2], l2 = p.part_ml[2 * r2 + 1];
  const float m = fmaxf(m1, m2);
  const float f1 = m1 == -INFINITY ? 0.f : fexp2(m1 - m);
  const float f2 = m2 == -INFINITY ? 0.f : fexp2(m2 - m);
  const float lsum = l1 * f1 + l2 * f2;
  const float inv = (DO ? p.drop_scale : 1.0f) / lsum;
  const float* o1 = p.part_o + r1 * D + 8 * ch;
  const float* o2 = p.part_o + r2 * D + 8 * ch;
  const f32x4 a0 = *(const f32x4*)o1, a1 = *(const f32x4*)(o1 + 4);
  const f32x4 b0 = *(const f32x4*)o2, b1 = *(const f32x4*)(o2 + 4);
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    v[e] = (bf16)((a0[e] * f1 + b0[e] * f2) * inv);
    v[4 + e] = (bf16)((a1[e] * f1 + b1[e] * f2) * inv);
  }
  const int b = head / p.n_local, l = head - b * p.n_local;
  *(bf16x8*)(p.ctx + ((long)b * p.seq + q) * p.h_l + (long)l * D + 8 * ch) = v;
  if (ch == 0) p.lse[(long)head * p.seq + q] = (m + __log2f(lsum)) * (1.0f / kLog2e);
}

// ---- backward ---------------------------------------------------------------------
// One launch, 8 waves (two per SIMD) per workgroup, two kinds of work item:
//  * dK/dV of 128 keys (tile kvt), looping over the 64-query tiles from the
//    diagonal on. Four key pairs of 32 keys; each pair is two waves with
//    split roles (waves p and p + 4, on one SIMD): role A holds K (fp16) and
//    the dV accumulator, forms S^T = K Q^T and P = 2^(S - lse), hands P to
//    role B through LDS and adds P^T dO into dV; role B holds V and the dK
//    accumulator, forms dP^T = V dO^T and, with A's P, dS = P (dP - delta),
//    and adds dS^T Q into dK. Each role keeps half the registers of a wave
//    that did all four products (which fit 256 only up to D = 96), so two
//    waves share each SIMD and one's softmax arithmetic overlaps the other's
//    matrix products.
//  * dQ of 128 queries (tile qt), looping over the 64-key tiles up to the
//    diagonal. Four query blocks of 32; each is two waves that take the two
//    32-key halves of every key tile and merge their dQ through LDS at the
//    end (as the forward's pairs do).
// P goes through LDS in fp32, so dS is formed from the same unrounded P as
// in a single wave. No atomics. Narrow heads (D <= 96) take bwd4_mfma below
// instead.

// lse and delta of a 64-query tile: 64 floats each, after the three tiles.
__device__ __forceinline__ void dma_stats(const MP& p, char* stage_stats, int head, int q0, int w, int lane) {
  if (w >= 2) return;
  const float* base = (w == 0 ? (const float*)p.lse : p.delta) + (long)head * p.seq;
  const uint32_t nrec = (uint32_t)(p.seq * 4);
  const __amdgpu_buffer_rsrc_t rs = rsrc(base, nrec);
  const uint32_t vo = q0 + lane < p.seq ? (uint32_t)((q0 + lane) * 4) : nrec;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)(stage_stats + 256 * w), 4, vo, 0, 0, 0);
}

constexpr int BWD_WAVES = 8;
// P hand-over: [key pair][query block][quad][lane][4] floats
constexpr int PBUF_BYTES = 4 * 2 * 4 * 64 * 4 * 4;
template <int D>
constexpr int bwd_stage_bytes() { return 3 * tile_bytes<D>() + 512; }  // three tiles + lse and delta of 64 queries
template <int D>
constexpr int bwd_lds_bytes() {
  // two stages and the P buffer; the dQ pairs' merge (4 x NB x 16 floats per
  // lane) reuses the stages
  return 2 * bwd_stage_bytes<D>() + PBUF_BYTES;
}
static_assert(2 * (3 * TROWS * 320 + 512) + PBUF_BYTES <= 160 * 1024, "LDS budget at D = 128 and 160");

// Keep bits of this lane's key for the 16 queries of a 32-query block: bit
// 4 q4 + e for query qs0 + 8 q4 + 4g + e (the order of the score
// accumulators), taken from the stored 16-bit words (rows padded: the 8-byte
// loads stay in the row; the key is bit qk of each word).
__device__ __forceinline__ uint32_t key_keep_bits(const MP& p, int head, int k0w, int qs0, int lane) {
  const int l32 = lane & 31, g = lane >> 5;
  const int qk = 4 * (l32 >> 3) + (l32 & 3);
  const uint16_t* mrow = p.mask + ((long)(head * p.nkb + (k0w >> 5)) * 2 + ((l32 >> 2) & 1)) * p.mstride;
  uint32_t bits = 0;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const int i0 = qs0 + 8 * q4 + 4 * g;
    const uint64_t wd = i0 < p.seq ? *(const uint64_t*)(mrow + i0) : 0ull;
#pragma unroll
    for (int e = 0; e < 4; ++e) bits |= (uint32_t)((wd >> (16 * e + qk)) & 1ull) << (4 * q4 + e);
  }
  return bits;
}

// Role A: P of one 32-query block for this lane's key (MASK as in
// fwd_scores).
template <bool MASK, bool AL>
__device__ __forceinline__ void a_probs(const f32x16& sa, const float* sL, float (&pr)[16], float slope2, int qs0,
                                        int g, int myk, int seq) {
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const f32x4 L = *(const f32x4*)(sL + 8 * q4 + 4 * g);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int q = 4 * q4 + e;
      const int query = qs0 + 8 * q4 + 4 * g + e;
      float v = sa[q] - L[e] * kLog2e;
      if (AL) v -= slope2 * (float)(query - myk);
      float pp = fexp2(v);
      if (MASK && (query < myk || query >= seq)) pp = 0.f;
      pr[q] = pp;
    }
  }
}

// 8 values packed to bf16, each times `scale` where its keep bit (bits >> q0) is set, else 0.
__device__ __forceinline__ bf16x8 pack8_keep(const float* x, uint32_t bits, int q0, float scale) {
  bf16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = (bf16)(((bits >> (q0 + e)) & 1u) ? x[e] * scale : 0.f);
  return v;
}

// dK/dV of the 128 keys of tile kvt of one head.
template <int D, bool AL, bool DO>
__device__ __forceinline__ void dkdv_item(const MP& p, int head, int kvt, char* __restrict__ st0,
                                          char* __restrict__ st1, float* __restrict__ pbuf) {
  constexpr int NC = D / 16, NB = D / 32, TB = tile_bytes<D>();
  const int b = head / p.n_local, l = head - b * p.n_local;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = (int)uni((uint32_t)(tid >> 6));
  const TileLanes<D, BWD_WAVES> tl = tile_lanes<D, BWD_WAVES>(p.h_l, w, lane);
  const int kp = w & 3;         // key pair
  const bool roleA = w < 4;     // wave-uniform
  const long grow0 = (long)b * p.seq;
  const int k0w = kvt * 128 + 32 * kp;
  const int myk = k0w + l32;
  const uint32_t nrec = (uint32_t)(p.T * p.h_l * 2);
  const int nqt = (p.seq + TROWS - 1) / TROWS;
  const int qt0 = (kvt * 128) / TROWS;
  dma_tile<D, BWD_WAVES>(p.q16, nrec, st0, grow0, l * D, qt0 * TROWS, p.seq, p.h_l, w, tl);
  dma_tile<D, BWD_WAVES>(p.qb, nrec, st0 + TB, grow0, l * D, qt0 * TROWS, p.seq, p.h_l, w, tl);
  dma_tile<D, BWD_WAVES>(p.dctx, nrec, st0 + 2 * TB, grow0, l * D, qt0 * TROWS, p.seq, p.h_l, w, tl);
  dma_stats(p, st0 + 3 * TB, head, qt0 * TROWS, w, lane);
  // A: K (fp16 bits) and dV; B: V and dK
  bf16x8 kv[NC];
  f32x16 acc[NB];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    kv[c] = bf16x8{};
    if (myk < p.seq) kv[c] = ld8((roleA ? p.k16 : p.vh) + (grow0 + myk) * p.h_l + (long)l * D + 16 * c + 8 * g);
  }
#pragma unroll
  for (int db = 0; db < NB; ++db) acc[db] = f32x16{};
  const float slope2 = alibi_slope_log2(p, l);
  const TrOff tro = tr_offsets<D>(lane);
  const RowOff ro = row_offsets<D>(lane);
  float* pb = pbuf + kp * (2 * 4 * 64 * 4) + 4 * lane;  // + (qs*4 + q4)*256
  for (int qt = qt0; qt < nqt; ++qt) {
    loads_landed_barrier();  // tile qt is in LDS; the other stage and the P buffer are free
    const bool odd = (qt - qt0) & 1;
    const char* cur = odd ? st1 : st0;
    char* nxt = odd ? st0 : st1;
    if (qt + 1 < nqt) {
      const int qn = (qt + 1) * TROWS;
      dma_tile<D, BWD_WAVES>(p.q16, nrec, nxt, grow0, l * D, qn, p.seq, p.h_l, w, tl);
      dma_tile<D, BWD_WAVES>(p.qb, nrec, nxt + TB, grow0, l * D, qn, p.seq, p.h_l, w, tl);
      dma_tile<D, BWD_WAVES>(p.dctx, nrec, nxt + 2 * TB, grow0, l * D, qn, p.seq, p.h_l, w, tl);
      dma_stats(p, nxt + 3 * TB, head, qn, w, lane);
    }
    const float* sL = (const float*)(cur + 3 * TB);
    const float* sDl = sL + 64;
    const int q0 = qt * TROWS;
    bf16x8 pf[2][2];  // A: P * keep * scale of both query blocks, packed
    f32x16 dp[2];     // B: dP^T of both query blocks
    // phase 1: A scores -> P (to LDS); B dP
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const int qs0 = q0 + 32 * qs;
      if (qs0 + 31 < k0w || qs0 >= p.seq || k0w >= p.seq) continue;  // wave-uniform: all masked
      if (roleA) {
        f32x16 sa = f32x16{};
#pragma unroll
        for (int c = 0; c < NC; ++c) sa = mfma_f16(frag_row<D>(cur, qs, c, ro), kv[c], sa);
        float pr[16];
        if ((qs0 < k0w + 31) || (qs0 + 32 > p.seq))
          a_probs<true, AL>(sa, sL + 32 * qs, pr, slope2, qs0, g, myk, p.seq);
        else
          a_probs<false, AL>(sa, sL + 32 * qs, pr, slope2, qs0, g, myk, p.seq);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4)
          *(__attribute__((address_space(3))) f32x4*)(pb + (qs * 4 + q4) * 256) =
              f32x4{pr[4 * q4], pr[4 * q4 + 1], pr[4 * q4 + 2], pr[4 * q4 + 3]};
        if (DO) {  // the value product takes P * keep * scale
          const uint32_t bits = key_keep_bits(p, head, k0w, qs0, lane);
          pf[qs][0] = pack8_keep(pr, bits, 0, p.drop_scale);
          pf[qs][1] = pack8_keep(pr + 8, bits, 8, p.drop_scale);
        } else {
          pf[qs][0] = pack8(pr);
          pf[qs][1] = pack8(pr + 8);
        }
      } else {
        f32x16 d = f32x16{};
#pragma unroll
        for (int c = 0; c < NC; ++c)
          d = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_row<D>(cur + 2 * TB, qs, c, ro), kv[c], d, 0, 0, 0);
        dp[qs] = d;
      }
    }
    lds_barrier();  // A's P of both blocks is in LDS
    // phase 2: A dV += P^T dO; B dS = P (dP - delta), dK += dS^T Q
#pragma unroll
    for (int qs = 0; qs < 2; ++qs) {
      const int qs0 = q0 + 32 * qs;
      if (qs0 + 31 < k0w || qs0 >= p.seq || k0w >= p.seq) continue;
      bf16x8 f0, f1;
      const char* tt;
      if (roleA) {
        f0 = pf[qs][0];
        f1 = pf[qs][1];
        tt = cur + 2 * TB;
      } else {
        const uint32_t bits = DO ? key_keep_bits(p, head, k0w, qs0, lane) : 0u;
        float ds[16];
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const f32x4 P = *(__attribute__((address_space(3))) const f32x4*)(pb + (qs * 4 + q4) * 256);
          const f32x4 Dl = *(const f32x4*)(sDl + 32 * qs + 8 * q4 + 4 * g);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int q = 4 * q4 + e;
            const float dpq = DO ? (((bits >> q) & 1u) ? dp[qs][q] * p.drop_scale : 0.f) : dp[qs][q];
            ds[q] = P[e] * (dpq - Dl[e]);
          }
        }
        f0 = pack8(ds);
        f1 = pack8(ds + 8);
        tt = cur + TB;
      }
#pragma unroll
      for (int db = 0; db < NB; ++db) {
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_tr<D>(tt, db, 2 * qs, tro), f0, acc[db], 0, 0, 0);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_tr<D>(tt, db, 2 * qs + 1, tro), f1, acc[db], 0, 0, 0);
      }
    }
  }
  if (myk < p.seq) {
    // A: dV; B: dK (times 1 / sqrt(D): the scores' scale)
    bf16* dst = p.dqkv + (grow0 + myk) * (3L * p.h_l) + (roleA ? 2L : 1L) * p.h_l + (long)l * D;
    const float sc = roleA ? 1.0f : p.scale;
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 a;
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = (bf16)(acc[db][4 * q4 + e] * sc);
        *(bf16x4*)(dst + 32 * db + 8 * q4 + 4 * g) = a;
      }
  }
}

// dS of one 32-key block for this lane's query (MASK as in fwd_scores).
// DO: bit q of `bits` keeps lane q's key; dP is multiplied by keep * scale.
template <bool MASK, bool AL, bool DO>
__device__ __forceinline__ void q_dscores(const f32x16& sa, const f32x16& dp, float (&ds)[16], float slope2, float L,
                                          float Dl, int k0, int g, int myq, int seq, uint32_t bits, float dscale) {
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    const int key = k0 + 8 * (q >> 2) + 4 * g + (q & 3);
    float v = sa[q] - L;
    if (AL) v -= slope2 * (float)(myq - key);
    float pp = fexp2(v);
    if (MASK && (key > myq || key >= seq)) pp = 0.f;
    const float dpq = DO ? (((bits >> q) & 1u) ? dp[q] * dscale : 0.f) : dp[q];
    ds[q] = pp * (dpq - Dl);
  }
}

// dQ of the 128 queries of tile qt of one head: wave w takes queries
// qt*128 + 32(w & 3) .. +31 and the 32-key half w >> 2 of every 64-key tile.
template <int D, bool AL, bool DO>
__device__ __forceinline__ void dq_item(const MP& p, int head, int qt, char* __restrict__ st0,
                                        char* __restrict__ st1) {
  constexpr int NC = D / 16, NB = D / 32, TB = tile_bytes<D>();
  const int b = head / p.n_local, l = head - b * p.n_local;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = (int)uni((uint32_t)(tid >> 6));
  const TileLanes<D, BWD_WAVES> tl = tile_lanes<D, BWD_WAVES>(p.h_l, w, lane);
  const int qw = w & 3, kh = w >> 2;
  const long grow0 = (long)b * p.seq;
  const int q0w = qt * 128 + 32 * qw;
  const int myq = q0w + l32;
  const uint32_t nrec = (uint32_t)(p.T * p.h_l * 2);
  const int kv_end = min(p.seq, qt * 128 + 128);
  const int nkt = (kv_end + TROWS - 1) / TROWS;
  dma_tile<D, BWD_WAVES>(p.k16, nrec, st0, grow0, l * D, 0, p.seq, p.h_l, w, tl);
  dma_tile<D, BWD_WAVES>(p.kb, nrec, st0 + TB, grow0, l * D, 0, p.seq, p.h_l, w, tl);
  dma_tile<D, BWD_WAVES>(p.vh, nrec, st0 + 2 * TB, grow0, l * D, 0, p.seq, p.h_l, w, tl);
  bf16x8 qf[NC], cf[NC];  // q16 (fp16 bits), dctx
  f32x16 dq[NB];
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    qf[c] = bf16x8{};
    cf[c] = bf16x8{};
    if (myq < p.seq) {
      const long off = (grow0 + myq) * p.h_l + (long)l * D + 16 * c + 8 * g;
      qf[c] = ld8(p.q16 + off);
      cf[c] = ld8(p.dctx + off);
    }
  }
  const float L = myq < p.seq ? p.lse[(long)head * p.seq + myq] * kLog2e : 0.f;
  const float Dl = myq < p.seq ? p.delta[(long)head * p.seq + myq] : 0.f;
#pragma unroll
  for (int db = 0; db < NB; ++db) dq[db] = f32x16{};
  const float slope2 = alibi_slope_log2(p, l);
  const TrOff tro = tr_offsets<D>(lane);
  const RowOff ro = row_offsets<D>(lane);
  for (int kt = 0; kt < nkt; ++kt) {
    loads_landed_barrier();
    const bool odd = kt & 1;
    const char* cur = odd ? st1 : st0;
    char* nxt = odd ? st0 : st1;
    if (kt + 1 < nkt) {
      const int kn = (kt + 1) * TROWS;
      dma_tile<D, BWD_WAVES>(p.k16, nrec, nxt, grow0, l * D, kn, p.seq, p.h_l, w, tl);
      dma_tile<D, BWD_WAVES>(p.kb, nrec, nxt + TB, grow0, l * D, kn, p.seq, p.h_l, w, tl);
      dma_tile<D, BWD_WAVES>(p.vh, nrec, nxt + 2 * TB, grow0, l * D, kn, p.seq, p.h_l, w, tl);
    }
    const int k0 = kt * TROWS + 32 * kh;
    if (k0 > q0w + 31 || k0 >= p.seq) continue;  // wave-uniform: every key masked
    f32x16 sa = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      sa = mfma_f16(frag_row<D>(cur, kh, c, ro), qf[c], sa);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_row<D>(cur + 2 * TB, kh, c, ro), cf[c], dp, 0, 0, 0);
    }
    // s[q]: key k0 + 8(q>>2) + 4g + (q&3), query myq
    uint32_t bits = 0;
    if (DO)  // this query's keep word of the block (a query past seq reads row seq - 1's, unused)
      bits = p.mask[((long)(head * p.nkb + (k0 >> 5)) * 2 + g) * p.mstride + min(myq, p.seq - 1)];
    float ds[16];
    if ((k0 + 31 > q0w) || (k0 + 32 > p.seq))
      q_dscores<true, AL, DO>(sa, dp, ds, slope2, L, Dl, k0, g, myq, p.seq, bits, p.drop_scale);
    else
      q_dscores<false, AL, DO>(sa, dp, ds, slope2, L, Dl, k0, g, myq, p.seq, bits, p.drop_scale);
    const bf16x8 df0 = pack8(ds), df1 = pack8(ds + 8);
    const char* kbt = cur + TB;
#pragma unroll
    for (int db = 0; db < NB; ++db) {
      dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_tr<D>(kbt, db, 2 * kh, tro), df0, dq[db], 0, 0, 0);
      dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_tr<D>(kbt, db, 2 * kh + 1, tro), df1, dq[db], 0, 0, 0);
    }
  }
  // pair merge: the last tile issued no loads, so after this barrier no wave
  // reads or writes the stages any more
  __syncthreads();
  float* xs = (float*)st0 + qw * (NB * 16 * 64) + lane;
  if (kh) {
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
      for (int i = 0; i < 16; ++i) xs[(16 * db + i) * 64] = dq[db][i];
  }
  __syncthreads();
  if (kh || myq >= p.seq) return;
  bf16* dQ = p.dqkv + (grow0 + myq) * (3L * p.h_l) + (long)l * D;
#pragma unroll
  for (int db = 0; db < NB; ++db)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      bf16x4 a;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 4 * q4 + e;
        a[e] = (bf16)((dq[db][i] + xs[(16 * db + i) * 64]) * p.scale);
      }
      *(bf16x4*)(dQ + 32 * db + 8 * q4 + 4 * g) = a;
    }
}

// Items are numbered heaviest first: the dK/dV item of key tile r and the dQ
// item of query tile nt-1-r both cover nt-r query/key tile pairs (the causal
// triangle makes tile costs range from 1 to nt); rank r's dK/dV items, then
// its dQ items, for every head, so workgroups freed by light items pick up
// the remaining ones instead of waiting, as two separate launches would, for
// each launch's heaviest tile.
template <int D, bool AL, bool DO>
__global__ __launch_bounds__(64 * BWD_WAVES) __attribute__((amdgpu_waves_per_eu(2, 2))) void bwd_mfma(MP p) {
  constexpr int SB = bwd_stage_bytes<D>();
  __shared__ __attribute__((aligned(16))) char smem[bwd_lds_bytes<D>()];
  static_assert(4 * (D / 32) * 16 * 64 * 4 <= 2 * SB, "dQ pair merge fits the stages");
  const int nh = p.batch * p.n_local, nt = (p.seq + 127) / 128;
  const int head = (int)(blockIdx.x % (unsigned)nh), rk = (int)(blockIdx.x / (unsigned)nh);
  const int r = rk >> 1;
  if (rk & 1) dq_item<D, AL, DO>(p, head, nt - 1 - r, smem, smem + SB);
  else dkdv_item<D, AL, DO>(p, head, r, smem, smem + SB, (float*)(smem + 2 * SB));
}

// ---- backward, 4 waves per workgroup (narrow heads) --------------------------------
// Up to D = 96 a wave that holds K, V and both accumulators of its 32 keys
// (and does all four dK/dV products itself) fits 256 registers, so two such
// workgroups share a CU, two waves per SIMD; there this form measured faster
// than the split roles above (0.215 vs 0.276 ms at the GPT-2-like shard,
// D = 96): no P hand-over through LDS and one barrier per tile instead of two.
template <int D>
struct KvState4 {
  bf16x8 kf[D / 16], vf[D / 16];  // k16 (fp16 bits), v
  f32x16 dv[D / 32], dk[D / 32];
};

// P and dS of one 32-query block for this lane's key (MASK as in fwd_scores).
// DO: kw[q4] holds the keep words of queries qs0 + 8 q4 + 4g + 0..3 (16 bits
// each); this key is bit qk; pv becomes P * keep * scale (for dV) and dP is
// multiplied by keep * scale.
template <bool MASK, bool AL, bool DO>
__device__ __forceinline__ void kv_probs(const f32x16& sa, const f32x16& dp, const float* sL, const float* sDl,
                                         float (&pv)[16], float (&dsv)[16], float slope2, int qs0, int g, int myk,
                                         int seq, const uint64_t (&kw)[4], int qk, float dscale) {
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const f32x4 L = *(const f32x4*)(sL + 8 * q4 + 4 * g);
    const f32x4 Dl = *(const f32x4*)(sDl + 8 * q4 + 4 * g);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int q = 4 * q4 + e;
      const int query = qs0 + 8 * q4 + 4 * g + e;
      float v = sa[q] - L[e] * kLog2e;
      if (AL) v -= slope2 * (float)(query - myk);
      float pp = fexp2(v);
      if (MASK && (query < myk || query >= seq)) pp = 0.f;
      if (DO) {
        const float kd = ((kw[q4] >> (16 * e + qk)) & 1ull) ? dscale : 0.f;
        pv[q] = pp * kd;
        dsv[q] = pp * (dp[q] * kd - Dl[e]);
      } else {
        pv[q] = pp;
        dsv[q] = pp * (dp[q] - Dl[e]);
      }
    }
  }
}

// One 64-query tile from stage `cur` (Q16, Q bf16, dctx, then lse, delta).
template <int D, bool AL, bool DO>
__device__ __forceinline__ void dkdv_tile4(const MP& p, const char* __restrict__ cur, char* __restrict__ nxt,
                                          bool issue, int q0, int head, int l, long grow0, int w, int lane, int k0w,
                                          int myk, float slope2, const TrOff& tro, const RowOff& ro,
                                          const TileLanes<D, 4>& tl, KvState4<D>& st) {
  constexpr int NC = D / 16, NB = D / 32, TB = tile_bytes<D>();
  const uint32_t nrec = (uint32_t)(p.T * p.h_l * 2);
  if (issue) {
    const int qn = q0 + TROWS;
    dma_tile<D>(p.q16, nrec, nxt, grow0, l * D, qn, p.seq, p.h_l, w, tl);
    dma_tile<D>(p.qb, nrec, nxt + TB, grow0, l * D, qn, p.seq, p.h_l, w, tl);
    dma_tile<D>(p.dctx, nrec, nxt + 2 * TB, grow0, l * D, qn, p.seq, p.h_l, w, tl);
    dma_stats(p, nxt + 3 * TB, head, qn, w, lane);
  }
  if (k0w >= p.seq) return;
  const int g = lane >> 5;
  const float* sL = (const float*)(cur + 3 * TB);
  const float* sDl = sL + 64;
#pragma unroll
  for (int qs = 0; qs < 2; ++qs) {
    const int qs0 = q0 + 32 * qs;
    if (qs0 + 31 < k0w || qs0 >= p.seq) continue;  // wave-uniform: all masked
    f32x16 sa = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      sa = mfma_f16(frag_row<D>(cur, qs, c, ro), st.kf[c], sa);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_row<D>(cur + 2 * TB, qs, c, ro), st.vf[c], dp, 0, 0, 0);
    }
    // s[q], dp[q]: query qs0 + 8(q>>2) + 4g + (q&3), key myk
    uint64_t kw[4] = {0, 0, 0, 0};
    int qk = 0;
    if (DO) {  // keep words of this key's block and half for the lane's 16 queries (rows padded: 8-byte loads stay in the row)
      const int l32 = lane & 31;
      qk = 4 * (l32 >> 3) + (l32 & 3);
      const uint16_t* mrow = p.mask + ((long)(head * p.nkb + (k0w >> 5)) * 2 + ((l32 >> 2) & 1)) * p.mstride;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int i0 = qs0 + 8 * q4 + 4 * g;
        if (i0 < p.seq) kw[q4] = *(const uint64_t*)(mrow + i0);
      }
    }
    float pv[16], dsv[16];
    if ((qs0 < k0w + 31) || (qs0 + 32 > p.seq))
      kv_probs<true, AL, DO>(sa, dp, sL + 32 * qs, sDl + 32 * qs, pv, dsv, slope2, qs0, g, myk, p.seq, kw, qk,
                             p.drop_scale);
    else
      kv_probs<false, AL, DO>(sa, dp, sL + 32 * qs, sDl + 32 * qs, pv, dsv, slope2, qs0, g, myk, p.seq, kw, qk,
                              p.drop_scale);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16x8 pf = pack8(pv + 8 * h), df = pack8(dsv + 8 * h);
#pragma unroll
      for (int db = 0; db < NB; ++db) {
        st.dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_tr<D>(cur + 2 * TB, db, 2 * qs + h, tro), pf,
                                                            st.dv[db], 0, 0, 0);
        st.dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_tr<D>(cur + TB, db, 2 * qs + h, tro), df, st.dk[db],
                                                            0, 0, 0);
      }
    }
  }
}

// dK and dV of the 128 keys of tile kvt of one head (4 waves of 32 keys),
// looping over the 64-query tiles from the diagonal on.
template <int D, bool AL, bool DO>
__device__ __forceinline__ void dkdv_item4(const MP& p, int head, int kvt, char* __restrict__ st0,
                                          char* __restrict__ st1) {
  constexpr int NC = D / 16, NB = D / 32, TB = tile_bytes<D>();
  const int b = head / p.n_local, l = head - b * p.n_local;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = (int)uni((uint32_t)(tid >> 6));
  const TileLanes<D, 4> tl = tile_lanes<D, 4>(p.h_l, w, lane);
  const long grow0 = (long)b * p.seq;
  const int k0w = kvt * 128 + 32 * w;
  const int myk = k0w + l32;
  const uint32_t nrec = (uint32_t)(p.T * p.h_l * 2);
  const int nqt = (p.seq + TROWS - 1) / TROWS;
  const int qt0 = (kvt * 128) / TROWS;
  dma_tile<D>(p.q16, nrec, st0, grow0, l * D, qt0 * TROWS, p.seq, p.h_l, w, tl);
  dma_tile<D>(p.qb, nrec, st0 + TB, grow0, l * D, qt0 * TROWS, p.seq, p.h_l, w, tl);
  dma_tile<D>(p.dctx, nrec, st0 + 2 * TB, grow0, l * D, qt0 * TROWS, p.seq, p.h_l, w, tl);
  dma_stats(p, st0 + 3 * TB, head, qt0 * TROWS, w, lane);
  KvState4<D> st;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    st.kf[c] = bf16x8{};
    st.vf[c] = bf16x8{};
    if (myk < p.seq) {
      const long off = (grow0 + myk) * p.h_l + (long)l * D + 16 * c + 8 * g;
      st.kf[c] = ld8(p.k16 + off);
      st.vf[c] = ld8(p.vh + off);
    }
  }
#pragma unroll
  for (int db = 0; db < NB; ++db) {
    st.dv[db] = f32x16{};
    st.dk[db] = f32x16{};
  }
  const float slope2 = alibi_slope_log2(p, l);
  const TrOff tro = tr_offsets<D>(lane);
  const RowOff ro = row_offsets<D>(lane);
  for (int qt = qt0; qt < nqt; ++qt) {
    loads_landed_barrier();
    const bool odd = (qt - qt0) & 1;
    dkdv_tile4<D, AL, DO>(p, odd ? st1 : st0, odd ? st0 : st1, qt + 1 < nqt, qt * TROWS, head, l, grow0, w, lane, k0w,
                     myk, slope2, tro, ro, tl, st);
  }
  if (myk < p.seq) {
    const long ld3 = 3L * p.h_l;
    bf16* dK = p.dqkv + (grow0 + myk) * ld3 + p.h_l + (long)l * D;
    bf16* dV = p.dqkv + (grow0 + myk) * ld3 + 2L * p.h_l + (long)l * D;
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 a, c;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          a[e] = (bf16)(st.dk[db][4 * q4 + e] * p.scale);
          c[e] = (bf16)st.dv[db][4 * q4 + e];
        }
        *(bf16x4*)(dK + 32 * db + 8 * q4 + 4 * g) = a;
        *(bf16x4*)(dV + 32 * db + 8 * q4 + 4 * g) = c;
      }
  }
}

// ---- backward: dQ ----------------------------------------------------------------
template <int D>
struct QState4 {
  bf16x8 qf[D / 16], cf[D / 16];  // q16 (fp16 bits), dctx
  f32x16 dq[D / 32];
  float L, Dl;
};

// One 64-key tile from stage `cur` (K16, K bf16, V).
template <int D, bool AL, bool DO>
__device__ __forceinline__ void dq_tile4(const MP& p, const char* __restrict__ cur, char* __restrict__ nxt, bool issue,
                                        int kv0, int l, long grow0, int w, int lane, int q0w, int myq, float slope2,
                                        const TrOff& tro, const RowOff& ro, int head, const TileLanes<D, 4>& tl,
                                        QState4<D>& st) {
  constexpr int NC = D / 16, NB = D / 32, TB = tile_bytes<D>();
  const uint32_t nrec = (uint32_t)(p.T * p.h_l * 2);
  if (issue) {
    dma_tile<D>(p.k16, nrec, nxt, grow0, l * D, kv0 + TROWS, p.seq, p.h_l, w, tl);
    dma_tile<D>(p.kb, nrec, nxt + TB, grow0, l * D, kv0 + TROWS, p.seq, p.h_l, w, tl);
    dma_tile<D>(p.vh, nrec, nxt + 2 * TB, grow0, l * D, kv0 + TROWS, p.seq, p.h_l, w, tl);
  }
  const int g = lane >> 5;
#pragma unroll
  for (int sb = 0; sb < 2; ++sb) {
    const int k0 = kv0 + 32 * sb;
    if (k0 > q0w + 31 || k0 >= p.seq) continue;
    f32x16 sa = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      sa = mfma_f16(frag_row<D>(cur, sb, c, ro), st.qf[c], sa);
      dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_row<D>(cur + 2 * TB, sb, c, ro), st.cf[c], dp, 0, 0, 0);
    }
    // s[q]: key k0 + 8(q>>2) + 4g + (q&3), query myq
    uint32_t bits = 0;
    if (DO)  // this query's keep word of the block (a query past seq reads row seq - 1's, unused)
      bits = p.mask[((long)(head * p.nkb + (k0 >> 5)) * 2 + g) * p.mstride + min(myq, p.seq - 1)];
    float ds[16];
    if ((k0 + 31 > q0w) || (k0 + 32 > p.seq))
      q_dscores<true, AL, DO>(sa, dp, ds, slope2, st.L, st.Dl, k0, g, myq, p.seq, bits, p.drop_scale);
    else
      q_dscores<false, AL, DO>(sa, dp, ds, slope2, st.L, st.Dl, k0, g, myq, p.seq, bits, p.drop_scale);
    const bf16x8 df0 = pack8(ds), df1 = pack8(ds + 8);
    const char* kbt = cur + TB;
#pragma unroll
    for (int db = 0; db < NB; ++db) {
      st.dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_tr<D>(kbt, db, 2 * sb, tro), df0, st.dq[db], 0, 0, 0);
      st.dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(frag_tr<D>(kbt, db, 2 * sb + 1, tro), df1, st.dq[db], 0, 0, 0);
    }
  }
}

// dQ of the 128 queries of tile qt of one head (4 waves of 32 queries),
// looping over the 64-key tiles up to the diagonal.
template <int D, bool AL, bool DO>
__device__ __forceinline__ void dq_item4(const MP& p, int head, int qt, char* __restrict__ st0,
                                        char* __restrict__ st1) {
  constexpr int NC = D / 16, NB = D / 32, TB = tile_bytes<D>();
  const int b = head / p.n_local, l = head - b * p.n_local;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = (int)uni((uint32_t)(tid >> 6));
  const TileLanes<D, 4> tl = tile_lanes<D, 4>(p.h_l, w, lane);
  const long grow0 = (long)b * p.seq;
  const int q0w = qt * 128 + 32 * w;
  const int myq = q0w + l32;
  const uint32_t nrec = (uint32_t)(p.T * p.h_l * 2);
  const int kv_end = min(p.seq, qt * 128 + 128);
  const int nkt = (kv_end + TROWS - 1) / TROWS;
  dma_tile<D>(p.k16, nrec, st0, grow0, l * D, 0, p.seq, p.h_l, w, tl);
  dma_tile<D>(p.kb, nrec, st0 + TB, grow0, l * D, 0, p.seq, p.h_l, w, tl);
  dma_tile<D>(p.vh, nrec, st0 + 2 * TB, grow0, l * D, 0, p.seq, p.h_l, w, tl);
  QState4<D> st;
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    st.qf[c] = bf16x8{};
    st.cf[c] = bf16x8{};
    if (myq < p.seq) {
      const long off = (grow0 + myq) * p.h_l + (long)l * D + 16 * c + 8 * g;
      st.qf[c] = ld8(p.q16 + off);
      st.cf[c] = ld8(p.dctx + off);
    }
  }
  st.L = myq < p.seq ? p.lse[(long)head * p.seq + myq] * kLog2e : 0.f;
  st.Dl = myq < p.seq ? p.delta[(long)head * p.seq + myq] : 0.f;
#pragma unroll
  for (int db = 0; db < NB; ++db) st.dq[db] = f32x16{};
  const float slope2 = alibi_slope_log2(p, l);
  const TrOff tro = tr_offsets<D>(lane);
  const RowOff ro = row_offsets<D>(lane);
  for (int kt = 0; kt < nkt; ++kt) {
    loads_landed_barrier();
    const bool odd = kt & 1;
    dq_tile4<D, AL, DO>(p, odd ? st1 : st0, odd ? st0 : st1, kt + 1 < nkt, kt * TROWS, l, grow0, w, lane, q0w, myq,
                       slope2, tro, ro, head, tl, st);
  }
  if (myq < p.seq) {
    bf16* dQ = p.dqkv + (grow0 + myq) * (3L * p.h_l) + (long)l * D;
#pragma unroll
    for (int db = 0; db < NB; ++db)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        bf16x4 a;
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = (bf16)(st.dq[db][4 * q4 + e] * p.scale);
        *(bf16x4*)(dQ + 32 * db + 8 * q4 + 4 * g) = a;
      }
  }
}

// Same items and order as bwd_mfma, 4 waves of 32 keys (or queries): two
// workgroups per CU without dropout; the dropout variants (which would
// spill at 256 registers) one. Both take this kernel for D <= 96, so that
// dropout with p = 0 repeats the plain path's arithmetic bit for bit.
template <int D, bool DO>
constexpr int bwd4_waves_per_simd() { return DO ? 1 : 2; }
template <int D, bool AL, bool DO>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(bwd4_waves_per_simd<D, DO>(),
                                                                     bwd4_waves_per_simd<D, DO>()))) void bwd4_mfma(MP p) {
  constexpr int SB = 3 * tile_bytes<D>() + 512;  // three tiles + lse and delta of 64 queries
  __shared__ __attribute__((aligned(16))) char st0[SB];
  __shared__ __attribute__((aligned(16))) char st1[SB];
  const int nh = p.batch * p.n_local, nt = (p.seq + 127) / 128;
  const int head = (int)(blockIdx.x % (unsigned)nh), rk = (int)(blockIdx.x / (unsigned)nh);
  const int r = rk >> 1;
  if (rk & 1) dq_item4<D, AL, DO>(p, head, nt - 1 - r, st0, st1);
  else dkdv_item4<D, AL, DO>(p, head, r, st0, st1);
}

MP make_mp(const AttnDesc& a) {
  MP p{};
  p.batch = a.batch; p.seq = a.seq; p.n_local = a.n_local;
  p.h_l = a.n_local * a.head_dim; p.head0 = a.head0; p.n_heads = a.n_heads; p.alibi = a.alibi;
  p.T = (long)a.batch * a.seq;
  const bf16* sp = (const bf16*)a.qkv;  // the five planes the QKV projection wrote
  const long plane = p.T * p.h_l;
  p.q16 = sp; p.qb = sp + plane; p.k16 = sp + 2 * plane; p.kb = sp + 3 * plane; p.vh = sp + 4 * plane;
  p.ctx = (bf16*)a.ctx; p.lse = a.lse;
  p.dctx = (const bf16*)a.dctx; p.delta = a.delta; p.dqkv = (bf16*)a.dqkv;
  p.scale = 1.0f / sqrtf((float)a.head_dim);
  p.mask = a.mask;
  p.nkb = (a.seq + 31) / 32;
  p.mstride = (a.seq + 7) & ~7;
  p.drop_thr = (uint32_t)floorf(a.drop_p * 65536.0f + 0.5f);
  p.drop_scale = 65536.0f / (65536.0f - (float)p.drop_thr);
  p.seed = a.seed;
  p.offset = a.offset;
  p.part_o = a.fwd_part;
  p.part_ml = a.fwd_part ? a.fwd_part + 2L * a.batch * a.n_local * a.seq * a.head_dim : nullptr;
  return p;
}

int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Forward items. With fewer than two 128-query tiles per CU the longest
// causal tiles decide the kernel's time (one workgroup per CU fits), so a
// tile with more than half the longest tile's key tiles (and at least 4) is
// split into two halves of its key tiles, merged afterwards; the items are
// dealt heaviest first (ties: later query tile first).
FwdItems fwd_items(const MP& p) {
  FwdItems fi{};
  const int nqt = (p.seq + 127) / 128, nh = p.batch * p.n_local;
  auto nkt = [&](int qt) { return ((p.seq < qt * 128 + 128 ? p.seq : qt * 128 + 128) + TROWS - 1) / TROWS; };
  fi.qsplit = nqt;
  if (p.part_o == nullptr || 2 * nqt > kMaxFwdItems || (long)nh * nqt >= 2L * device_cus()) return fi;
  const int kmax = nkt(nqt - 1);
  while (fi.qsplit > 0 && nkt(fi.qsplit - 1) >= 4 && 2 * nkt(fi.qsplit - 1) > kmax) --fi.qsplit;
  if (fi.qsplit == nqt) return fi;
  int wt[kMaxFwdItems];
  for (int qt = nqt - 1; qt >= 0; --qt) {
    const int k = nkt(qt);
    if (qt >= fi.qsplit) {
      fi.it[fi.n] = (uint16_t)(qt << 2 | 2); wt[fi.n++] = k - k / 2;
      fi.it[fi.n] = (uint16_t)(qt << 2 | 1); wt[fi.n++] = k / 2;
    } else {
      fi.it[fi.n] = (uint16_t)(qt << 2); wt[fi.n++] = k;
    }
  }
  // stable insertion sort by weight, descending
  for (int i = 1; i < fi.n; ++i) {
    const int w = wt[i];
    const uint16_t v = fi.it[i];
    int j = i - 1;
    while (j >= 0 && wt[j] < w) { wt[j + 1] = wt[j]; fi.it[j + 1] = fi.it[j]; --j; }
    wt[j + 1] = w;
    fi.it[j + 1] = v;
  }
  return fi;
}

template <int D, bool DO>
hipError_t fwd_d(const MP& p, hipStream_t stream) {
  const FwdItems fi = fwd_items(p);
  const int nqt = (p.seq + 127) / 128;
  dim3 grid(p.batch * p.n_local, fi.n ? fi.n : nqt);
  if (p.alibi) hipLaunchKernelGGL((fwd_mfma<D, true, DO>), grid, dim3(64 * FWD_WAVES), 0, stream, p, fi);
  else hipLaunchKernelGGL((fwd_mfma<D, false, DO>), grid, dim3(64 * FWD_WAVES), 0, stream, p, fi);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || fi.qsplit >= nqt) return e;
  const int q_first = fi.qsplit * 128;
  const long n = (long)p.batch * p.n_local * (p.seq - q_first) * (D / 8);
  hipLaunchKernelGGL((fwd_merge_kernel<D, DO>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, p, q_first);
  return hipGetLastError();
}
template <int D, bool DO>
hipError_t bwd_d(const MP& p, hipStream_t stream) {
  const dim3 grid((unsigned)(2 * ((p.seq + 127) / 128) * p.batch * p.n_local));
  if constexpr (D <= 96) {
    if (p.alibi) hipLaunchKernelGGL((bwd4_mfma<D, true, DO>), grid, dim3(256), 0, stream, p);
    else hipLaunchKernelGGL((bwd4_mfma<D, false, DO>), grid, dim3(256), 0, stream, p);
  } else {
    if (p.alibi) hipLaunchKernelGGL((bwd_mfma<D, true, DO>), grid, dim3(64 * BWD_WAVES), 0, stream, p);
    else hipLaunchKernelGGL((bwd_mfma<D, false, DO>), grid, dim3(64 * BWD_WAVES), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace

bool attn_mfma_supported(int dtype, int head_dim) {
  return dtype == DT_BF16 && (head_dim == 64 || head_dim == 96 || head_dim == 128 || head_dim == 160);
}

size_t attn_fwd_part_bytes(int dtype, int head_dim, int batch, int seq, int n_local) {
  if (!attn_mfma_supported(dtype, head_dim)) return 0;
  return (size_t)2 * batch * n_local * seq * (head_dim + 2) * sizeof(float);
}

size_t attn_dropout_mask_bytes(int batch, int seq, int n_local) {
  return (size_t)batch * n_local * ((seq + 31) / 32) * 2 * ((seq + 7) & ~7) * sizeof(uint16_t);
}

template <bool DO>
hipError_t fwd_dispatch(const MP& p, int head_dim, hipStream_t stream) {
  switch (head_dim) {
    case 64: return fwd_d<64, DO>(p, stream);
    case 96: return fwd_d<96, DO>(p, stream);
    case 128: return fwd_d<128, DO>(p, stream);
    case 160: return fwd_d<160, DO>(p, stream);
  }
  return hipErrorInvalidValue;
}
template <bool DO>
hipError_t bwd_dispatch(const MP& p, int head_dim, hipStream_t stream) {
  switch (head_dim) {
    case 64: return bwd_d<64, DO>(p, stream);
    case 96: return bwd_d<96, DO>(p, stream);
    case 128: return bwd_d<128, DO>(p, stream);
    case 160: return bwd_d<160, DO>(p, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t attn_mfma_fwd(const AttnDesc& a, hipStream_t stream) {
  const MP p = make_mp(a);
  return a.mask ? fwd_dispatch<true>(p, a.head_dim, stream) : fwd_dispatch<false>(p, a.head_dim, stream);
}

hipError_t attn_mfma_bwd(const AttnDesc& a, hipStream_t stream) {
  const MP p = make_mp(a);
  return a.mask ? bwd_dispatch<true>(p, a.head_dim, stream) : bwd_dispatch<false>(p, a.head_dim, stream);
}

}  // namespace tpk
