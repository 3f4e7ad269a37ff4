// bf16 GEMM on CDNA4 matrix cores (v_mfma_f32_32x32x16_bf16), fp32 accumulation,
// with the layer's fused epilogues (bias, bias+GeLU, GeLU' scaling, fp32 out).
//
// Tiling: a 256x256 output tile per workgroup. With 4 waves (2x2) each wave
// owns a 128x128 sub-tile = 4x4 MFMA blocks of 32x32 (256 fp32 accumulators
// per lane, one wave per SIMD); with 8 waves (2x4) each owns 128x64 (128
// accumulators, two waves per SIMD, so one wave's barrier and load waits are
// covered by the other's MFMAs, and twice as many loads are in flight per CU).
// Products with a k-inner B may take a 256x320 tile instead (8 waves, 4x2,
// 64x160 each, 160 accumulators); the output projection (k-outer B) takes
// a 256x320 tile on v_mfma_f32_16x16x32_bf16 (8 waves, 2x4, 128x80 each)
// when its tiles run in whole data-parallel rounds. Narrow layers' products
// may take a 256x192 tile (8 waves, 4x2, 64x96 each, either B layout) when it
// fills the CUs in whole rounds where 256-wide tiles would leave a stream-K
// tail. K advances 64 at a time through two LDS stages (2 x 64 KiB; 2 x 72
// KiB for the 320-wide tiles, 2 x 56 KiB for the 192-wide ones).
//
// Global -> LDS: buffer loads that write LDS directly (16 bytes per lane; one
// instruction fills 1 KiB in lane order), so no VGPRs stage the tiles. Each
// lane picks the global address whose data belongs at its LDS slot, which is
// how the swizzles below are applied. Loads of k-step t+1 are issued right
// after the barrier of step t and complete while step t's MFMAs run.
//
// LDS layouts (bf16):
//  * k-inner operand (memory holds rows with k contiguous: activations of a
//    forward product, both operands of an input gradient): [256 rows][64 k],
//    16-byte chunk c of row r stored at c ^ swz(r), swz(r) = (r ^ (r>>3)) & 7;
//    an MFMA fragment is one ds_read_b128 per lane.
//  * k-outer operand (memory holds k-rows with the m/n index contiguous: the
//    weight of a forward product, both operands of a weight gradient): kept in
//    memory order, [64 k][256 cols], chunk c of k-row q at c ^ 4(q & 3) (192
//    cols: [64 k][24 chunks], the swizzle of panel_kouter192); an
//    MFMA fragment is two ds_read_b64_tr_b16 per lane (the transposing LDS
//    read of gfx950: lane 4r+c of each 16-lane group fetches 4 columns of
//    k-row r, and lane i receives column i of the 4 rows).
// Both layouts make the fragment reads bank-conflict free.
//
// Scheduling: data-parallel tiles, plus stream-K for the last partial wave when
// whole waves would leave many CUs idle: the leftover tiles' k-iterations are
// split evenly over all workgroups, each split tile's fp32 partials go to the
// workspace and a second kernel sums them in a fixed order and applies the
// epilogue (no inter-workgroup waiting inside a kernel).
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace tpk {
namespace {

constexpr int BM = 256, BKK = 64;
// Wave layout of a workgroup of NW waves over a BM x BNV tile. 256 wide: 2
// waves along m (128 rows each) x NW/2 along n (4 waves: one per SIMD, 128x128
// each; 8 waves: two per SIMD, 128x64 each). 320 and 192 wide (8 waves,
// k-inner B only): 4 waves along m x 2 along n, 64x160 or 64x96 each. 320:
// 11% more flops per byte staged than 256x256, and 2048 x 10240 / 20480
// products fill 256 CUs in whole rounds; 192: 12% fewer, but products with
// N = 1536 or 384 (narrow layers) then fill the CUs in whole rounds (or an
// exact k-split) instead of a stream-K tail.
template <int NW, int BNV>
struct WC {
  static_assert((NW == 4 && BNV == 256) || (NW == 8 && (BNV == 192 || BNV == 256 || BNV == 320)), "tile shape");
  static constexpr int NTHR = 64 * NW;
  static constexpr int WMG = BNV == 256 ? 2 : 4;  // waves along m
  static constexpr int WNG = NW / WMG;            // waves along n
  static constexpr int WMW = BM / WMG;            // rows per wave
  static constexpr int MI = WMW / 32;             // 32-row MFMA blocks per wave
  static constexpr int WNW = BNV / WNG;           // columns per wave
  static constexpr int NJ = WNW / 32;             // 32-column MFMA blocks per wave
  static constexpr int NLA = BM * BKK * 2 / 1024 / NW;   // A loads (1 KiB each) per wave per k-step
  static constexpr int NLB = BNV * BKK * 2 / 1024 / NW;  // B loads per wave per k-step
};
constexpr int BN_MAX = 320;      // widest tile (workspace sizing)
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
  int qkv_hl; float qscale;  // EPI_QKV_PLANES
  float* partials;    // [2*sk_grid][BM*BNV] (split tail: [splits*split_tiles][BM*BNV])
  // Split tail (splits > 1, instead of stream-K): after the data-parallel
  // rounds, workgroup lw < splits*split_tiles takes k-range lw / split_tiles of
  // tile split_first + lw % split_tiles.
  int splits, split_first, split_tiles;
  // Phase-block tile numbering of a stream-K plan (blk_s > 0; see
  // phase_blocks): tile t is position t / blk_s of block t % blk_s, blocks of
  // blk_m x blk_n tiles; workgroups keep their hardware order
  int blk_s, blk_m, blk_n;
};

__device__ __forceinline__ int logical_wg(int w, int g) {
  // Workgroups are dealt round-robin to the 8 XCDs; renumber so that
  // consecutive logical ids (neighbouring tiles) share an XCD and its L2.
  return (g % 8 == 0) ? (w % 8) * (g / 8) + (w / 8) : w;
}

__device__ __forceinline__ void tile_coords(const KParams& p, int t, int& tm, int& tn) {
  if (p.blk_s > 0) {
    const int rho = t % p.blk_s, i = t / p.blk_s, nbn = p.tiles_n / p.blk_n;
    tm = (rho / nbn) * p.blk_m + i % p.blk_m;
    tn = (rho % nbn) * p.blk_n + i / p.blk_m;
    return;
  }
  int group = GROUP_M * p.tiles_n;
  int g = t / group;
  int first_m = g * GROUP_M;
  int gm = min(p.tiles_m - first_m, GROUP_M);
  int r = t - g * group;
  tm = first_m + r % gm;
  tn = r / gm;
}

// ---- global -> LDS (buffer loads writing LDS) ------------------------------
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr;

__device__ __forceinline__ uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ const bf16* uni_ptr(const bf16* p) {
  const uint64_t v = (uint64_t)p;
  return (const bf16*)(((uint64_t)uni((uint32_t)(v >> 32)) << 32) | uni((uint32_t)v));
}

// One operand panel of a tile: a buffer resource based at the panel's first
// row (k-inner) or first column (k-outer), and this lane's byte offsets for its
// NL load instructions (nrec = out of range: the load writes zeros).
template <int NL>
struct Panel {
  const bf16* base;  // workgroup-uniform
  uint32_t nrec;     // workgroup-uniform buffer size in bytes
  uint32_t kstep;    // workgroup-uniform bytes the panel advances per k-step
  uint32_t voff[NL];
};

// k-inner X[r*ld + k], rows r0g .. r0g+PR-1 of `rows`. Load i of wave w fills
// LDS block b = NLI*w + i = rows 8b .. 8b+7; lane l lands in row 8b+(l>>3),
// physical chunk l&7, so it loads logical chunk (l&7) ^ swz(row) =
// (l&7) ^ (l>>3) ^ (b&7).
template <int NLI, int PR>
__device__ __forceinline__ Panel<NLI> panel_kinner(const bf16* X, long ld, int rows, int r0g, int wave, int lane) {
  Panel<NLI> pn;
  int nrows = rows - r0g;
  nrows = nrows < PR ? nrows : PR;
  pn.base = uni_ptr(X + (long)r0g * ld);
  pn.nrec = uni((uint32_t)((long)nrows * ld * 2));
  pn.kstep = BKK * 2;
#pragma unroll
  for (int i = 0; i < NLI; ++i) {
    const int b = NLI * wave + i;
    const int r = 8 * b + (lane >> 3);
    const int c = (lane & 7) ^ (lane >> 3) ^ (b & 7);
    pn.voff[i] = r < nrows ? (uint32_t)(((long)r * ld + 8 * c) * 2) : pn.nrec;
  }
  return pn;
}
// k-outer X[k*ld + r], columns r0g.. of `rows`. Load i of wave w fills LDS
// block b = NLI*w + i = k-rows 2b, 2b+1; lane l lands in k-row 2b+(l>>5),
// physical chunk l&31, so it loads logical chunk (l&31) ^ 4(krow&3). Rows at
// or past K fall beyond nrec and load zeros.
template <int NLI>
__device__ __forceinline__ Panel<NLI> panel_kouter(const bf16* X, long ld, int rows, int K, int r0g, int wave,
                                                   int lane) {
  Panel<NLI> pn;
  pn.base = uni_ptr(X + r0g);
  pn.nrec = uni((uint32_t)(((long)K * ld - r0g) * 2));
  pn.kstep = uni((uint32_t)(BKK * ld * 2));
#pragma unroll
  for (int i = 0; i < NLI; ++i) {
    const int kr = 2 * (NLI * wave + i) + (lane >> 5);
    const int c = (lane & 31) ^ (4 * (kr & 3));
    pn.voff[i] = (r0g + 8 * c < rows) ? (uint32_t)(((long)kr * ld + 8 * c) * 2) : pn.nrec;
  }
  return pn;
}

// k-outer X[k*ld + c], the 192 columns c0g.. of `cols` (a 192-wide tile's
// B): the stage holds 64 k-rows of 24 chunks (384 bytes). Load i of wave w
// fills linear chunk q = 64(NLI*w + i) + lane, i.e. k-row q / 24, physical
// chunk q % 24, which holds logical chunk (q % 24) ^ kout192_swz(k-row). The
// XOR stays inside aligned groups of 8 chunks; with 384-byte rows it puts the
// 8 (k-row, 32-byte column pair) reads that one transposing read serves
// together (lanes 0-31, or lanes 0-15 with 32-47) in 8 different 32-byte
// bank groups (checked exhaustively on the CPU for both groupings).
__device__ __forceinline__ int kout192_swz(int kr) { return 4 * ((kr >> 1) & 1) + 2 * ((kr >> 3) & 1); }
template <int NLI>
__device__ __forceinline__ Panel<NLI> panel_kouter192(const bf16* X, long ld, int cols, int K, int c0g, int wave,
                                                      int lane) {
  Panel<NLI> pn;
  pn.base = uni_ptr(X + c0g);
  pn.nrec = uni((uint32_t)(((long)K * ld - c0g) * 2));
  pn.kstep = uni((uint32_t)(BKK * ld * 2));
#pragma unroll
  for (int i = 0; i < NLI; ++i) {
    const int q = 64 * (NLI * wave + i) + lane;
    const int kr = q / 24, pc = q - 24 * kr;
    const int lc = pc ^ kout192_swz(kr);
    pn.voff[i] = (c0g + 8 * lc < cols) ? (uint32_t)(((long)kr * ld + 8 * lc) * 2) : pn.nrec;
  }
  return pn;
}

// Issue the NLI loads of one operand for k-step kt into LDS stage `dst`.
// TAIL: k-step kt may be a partial one (k-inner chunks at or past K must
// read zeros, not the next row); the caller passes false for every k-step
// that is full or past the tile's end (whose data nobody uses).
template <int NLI, bool KIN, bool TAIL>
__device__ __forceinline__ void issue_panel(const Panel<NLI>& pn, int kt, int K, bf16* dst, int wave, int lane) {
  const int soff = (int)uni((uint32_t)kt * pn.kstep);
  __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)pn.base, (short)0, (int)pn.nrec, 0x00020000);
  const bool tail = KIN && TAIL && (kt + 1) * BKK > K;
#pragma unroll
  for (int i = 0; i < NLI; ++i) {
    const int b = NLI * wave + i;
    uint32_t vo = pn.voff[i];
    if (tail) {
      const int c = (lane & 7) ^ (lane >> 3) ^ (b & 7);
      if (kt * BKK + 8 * c >= K) vo = pn.nrec;
    }
    bf16* blk = dst + b * 512;  // 1 KiB block, wave-uniform
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)blk, 16, vo, soff, 0, 0);
  }
}

__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// ---- fragment reads ------------------------------------------------------------
// k-inner: 32-row block i of this wave's rows; lane owns row base+32i+(l&31)
// and k = 16kk + 8(l>>5) .. +7. The wave's first row `base` is a multiple of
// 32; pb = (base/32) & 1 is its contribution to bit 2 of the row swizzle.
__device__ __forceinline__ bf16x8 frag_kin(const bf16* s, int rowbase, int s1, int g, int kk, int i, int pb) {
  const int e = (2 * kk) ^ g ^ s1 ^ (4 * ((i + pb) & 1));
  return *(const bf16x8*)(s + rowbase + i * 32 * BKK + (e << 3));
}
// k-outer: per-lane byte offset of 32-column block jb inside a stage (see the
// layout note): k-row 8v + (j>>2) (+16kk + 4t), chunk ((col>>3) ^ 4(j>>2)),
// half (j&1); j = l&15, h = (l>>4)&1, v = l>>5, col = base + 32jb + 16h + 4(j&3).
__device__ __forceinline__ int kout_lane_off(int colbase, int jb, int lane) {
  const int j = lane & 15, h = (lane >> 4) & 1, v = lane >> 5;
  const int col = colbase + 32 * jb + 16 * h + 4 * (j & 3);
  const int chunk = (col >> 3) ^ (4 * (j >> 2));
  return (8 * v + (j >> 2)) * 512 + chunk * 16 + 8 * (j & 1);
}
// 192-wide k-outer stage (384-byte k-rows, swizzle kout192_swz): the same
// lane roles; the swizzle depends on bits 1 and 3 of the k-row, which the
// +16kk and +4 steps of the reads leave unchanged.
__device__ __forceinline__ int kout192_lane_off(int colbase, int jb, int lane) {
  const int j = lane & 15, h = (lane >> 4) & 1, v = lane >> 5;
  const int col = colbase + 32 * jb + 16 * h + 4 * (j & 3);
  const int kr = 8 * v + (j >> 2);
  return kr * 384 + ((col >> 3) ^ kout192_swz(kr)) * 16 + 8 * (j & 1);
}
// RS: bytes per k-row of the stage (512 for 256 columns, 384 for 192)
template <int RS>
__device__ __forceinline__ bf16x8 frag_kout(const bf16* s, int lane_off, int kk) {
  const char* b = (const char*)s + lane_off + kk * 16 * RS;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(b));
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(b + 4 * RS));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// ---- main loop over k-iterations [kb, ke) of one tile -------------------------
// One k-step: wait for this wave's loads into the current stage, barrier (all
// loads landed; everyone finished reading the other stage), issue the next
// k-step's loads into the other stage, then 4 sub-steps of 4 x NJ MFMAs from
// the current stage with the next sub-step's fragments read ahead. The stage
// pointers are __restrict__: the two stages never overlap, and the no-alias
// information lets the compiler's wait-count pass leave the in-flight LDS
// writes (other stage) outstanding while the fragment reads (this stage)
// proceed.
template <int NW, int BNV, bool AK, bool BKM, bool TAIL>
__device__ __forceinline__ void kstep(const KParams& p, const Panel<WC<NW, BNV>::NLA>& pa,
                                      const Panel<WC<NW, BNV>::NLB>& pb, int kt, const bf16* __restrict__ a,
                                      const bf16* __restrict__ b, bf16* __restrict__ na, bf16* __restrict__ nb,
                                      int wave, int lane, int rowA, int rowB, const int (&offA)[WC<NW, BNV>::MI],
                                      const int (&offB)[WC<NW, BNV>::NJ], int s1, int g, int pbA, int pbB,
                                      f32x16 (&acc)[WC<NW, BNV>::MI][WC<NW, BNV>::NJ]) {
  constexpr int MI = WC<NW, BNV>::MI, NJ = WC<NW, BNV>::NJ;
  constexpr int NLA = WC<NW, BNV>::NLA, NLB = WC<NW, BNV>::NLB;
  constexpr int NF = MI > NJ ? MI : NJ;
  wait_vmem();
  __syncthreads();
  // Next k-step's loads, unconditionally so that the whole step is one
  // scheduling region: past the last k-step of the tile they read either zeros
  // (k beyond K is out of the buffer's range) or in-range data nobody uses.
  issue_panel<NLA, AK, TAIL>(pa, kt + 1, p.K, na, wave, lane);
  issue_panel<NLB, BKM, TAIL>(pb, kt + 1, p.K, nb, wave, lane);
  // fragments read in the order a0, b0, a1, b1, ...
  bf16x8 af[2][MI], bfg[2][NJ];
#pragma unroll
  for (int i = 0; i < NF; ++i) {
    if (i < MI) af[0][i] = AK ? frag_kin(a, rowA, s1, g, 0, i, pbA) : frag_kout<2 * BM>(a, offA[i], 0);
    if (i < NJ) bfg[0][i] = BKM ? frag_kin(b, rowB, s1, g, 0, i, pbB) : frag_kout<2 * BNV>(b, offB[i], 0);
  }
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    const int c = kk & 1, n = c ^ 1;
    if (kk < 3) {
#pragma unroll
      for (int i = 0; i < NF; ++i) {
        if (i < MI) af[n][i] = AK ? frag_kin(a, rowA, s1, g, kk + 1, i, pbA) : frag_kout<2 * BM>(a, offA[i], kk + 1);
        if (i < NJ)
          bfg[n][i] = BKM ? frag_kin(b, rowB, s1, g, kk + 1, i, pbB) : frag_kout<2 * BNV>(b, offB[i], kk + 1);
      }
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j)
        // operands swapped: D[n][m], so each lane ends up owning one m and
        // runs of 4 consecutive n (vector stores in the epilogue)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfg[c][j], af[c][i], acc[i][j], 0, 0, 0);
  }
  // Instruction order for the step: the first sub-step's fragment reads, then
  // the MFMAs with the next sub-step's fragment reads spread evenly between
  // them and (in the first sub-step) the next k-step's NLA+NLB loads.
  constexpr int R = (AK ? MI : 2 * MI) + (BKM ? NJ : 2 * NJ);  // LDS reads per sub-step
  constexpr int NM = MI * NJ;                                  // MFMAs per sub-step
  constexpr int NL = NLA + NLB;                                // global->LDS loads per k-step
  __builtin_amdgcn_sched_group_barrier(0x100, R, 0);
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
#pragma unroll
    for (int m = 0; m < NM; ++m) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      const int nr = (R * (m + 1)) / NM - (R * m) / NM;
      if (kk < 3)
#pragma unroll
        for (int t = 0; t < nr; ++t) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      const int nv = (NL * (m + 1)) / NM - (NL * m) / NM;
      if (kk == 0)
#pragma unroll
        for (int t = 0; t < nv; ++t) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    }
}

// Stage s (0, 1) of the two: A at smem + s*BM*BKK, B after both A stages.
template <int BNV>
__device__ __forceinline__ bf16* stage_a(bf16* smem, int s) { return smem + s * BM * BKK; }
template <int BNV>
__device__ __forceinline__ bf16* stage_b(bf16* smem, int s) { return smem + 2 * BM * BKK + s * BNV * BKK; }

template <int NW, int BNV, bool AK, bool BKM>
__device__ __forceinline__ void mainloop(const KParams& p, int tm, int tn, int kb, int ke,
                                         f32x16 (&acc)[WC<NW, BNV>::MI][WC<NW, BNV>::NJ], bf16* smem) {
  using C = WC<NW, BNV>;
  constexpr int MI = C::MI, NJ = C::NJ, WNG = C::WNG, WMW = C::WMW, WNW = C::WNW;
  static_assert(BKM || BNV == 256 || BNV == 192, "k-outer B panels are 256 or 192 columns wide");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = (int)uni((uint32_t)(tid >> 6));
  const int wm = wave / WNG, wn = wave % WNG;
  const int g = lane >> 5, l32 = lane & 31;
  const int s1 = (l32 & 7) ^ (l32 >> 3);
  Panel<C::NLA> pa;
  Panel<C::NLB> pb;
  if (AK) pa = panel_kinner<C::NLA, BM>(p.A, p.lda, p.M, tm * BM, wave, lane);
  else pa = panel_kouter<C::NLA>(p.A, p.lda, p.M, p.K, tm * BM, wave, lane);
  if (BKM) pb = panel_kinner<C::NLB, BNV>(p.B, p.ldb, p.N, tn * BNV, wave, lane);
  else if (BNV == 192) pb = panel_kouter192<C::NLB>(p.B, p.ldb, p.N, p.K, tn * BNV, wave, lane);
  else pb = panel_kouter<C::NLB>(p.B, p.ldb, p.N, p.K, tn * BNV, wave, lane);
  const int rowA = (wm * WMW + l32) * BKK, rowB = (wn * WNW + l32) * BKK;
  const int pbA = (wm * WMW / 32) & 1, pbB = (wn * WNW / 32) & 1;
  int offA[MI], offB[NJ];
#pragma unroll
  for (int i = 0; i < MI; ++i) offA[i] = AK ? 0 : kout_lane_off(wm * WMW, i, lane);
#pragma unroll
  for (int j = 0; j < NJ; ++j)
    offB[j] = BKM ? 0 : BNV == 192 ? kout192_lane_off(wn * WNW, j, lane) : kout_lane_off(wn * WNW, j, lane);
  issue_panel<C::NLA, AK, true>(pa, kb, p.K, stage_a<BNV>(smem, 0), wave, lane);
  issue_panel<C::NLB, BKM, true>(pb, kb, p.K, stage_b<BNV>(smem, 0), wave, lane);
  // the one k-step that may be partial (none if K is a multiple of BKK); only
  // the step that loads it checks its chunks against K: the loop is split
  // around that step
  const int ktail = p.K % BKK ? p.iters - 1 : -1;
  const int kmid = ktail > kb && ktail - 1 < ke ? ktail - 1 : ke;
  // stage addresses from the step's parity (a select between four pointers
  // measured a little slower in the weight gradients' loop)
  int cur = 0, kt = kb;
  for (; kt < kmid; ++kt) {
    kstep<NW, BNV, AK, BKM, false>(p, pa, pb, kt, stage_a<BNV>(smem, cur), stage_b<BNV>(smem, cur),
                                   stage_a<BNV>(smem, cur ^ 1), stage_b<BNV>(smem, cur ^ 1), wave, lane, rowA, rowB,
                                   offA, offB, s1, g, pbA, pbB, acc);
    cur ^= 1;
  }
  if (kt < ke) {
    kstep<NW, BNV, AK, BKM, true>(p, pa, pb, kt, stage_a<BNV>(smem, cur), stage_b<BNV>(smem, cur),
                                  stage_a<BNV>(smem, cur ^ 1), stage_b<BNV>(smem, cur ^ 1), wave, lane, rowA, rowB,
                                  offA, offB, s1, g, pbA, pbB, acc);
    cur ^= 1;
    ++kt;
  }
  for (; kt < ke; ++kt) {
    kstep<NW, BNV, AK, BKM, false>(p, pa, pb, kt, stage_a<BNV>(smem, cur), stage_b<BNV>(smem, cur),
                                   stage_a<BNV>(smem, cur ^ 1), stage_b<BNV>(smem, cur ^ 1), wave, lane, rowA, rowB,
                                   offA, offB, s1, g, pbA, pbB, acc);
    cur ^= 1;
  }
  wait_vmem();      // the last step's read-ahead loads have landed
  __syncthreads();  // LDS is reused by the next work item
}

// ---- epilogue ---------------------------------------------------------------
// Lane owns m = base_m + (lane&31) and n = base_n + 8*q4 + 4*(lane>>5) + 0..3.
__device__ __forceinline__ void store_bf16x4(bf16* dst, const float (&v)[4]) {
  bf16x4 o;
  o[0] = (bf16)v[0]; o[1] = (bf16)v[1]; o[2] = (bf16)v[2]; o[3] = (bf16)v[3];
  *(bf16x4*)dst = o;
}

// Column block j (32 columns) of row block i (rows 32i..32i+31 of each
// wave's rows) of a tile, from its accumulators a.
template <int NW, int BNV, int EPI>
__device__ __forceinline__ void epilogue_block(const KParams& p, int tm, int tn, int i, int j, const f32x16& a) {
  constexpr int WNG = WC<NW, BNV>::WNG, WMW = WC<NW, BNV>::WMW, WNW = WC<NW, BNV>::WNW;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WNG, wn = wave % WNG;
  {
    const int m = tm * BM + wm * WMW + i * 32 + (lane & 31);
    if (m >= p.M) return;
    {
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int n = tn * BNV + wn * WNW + j * 32 + q4 * 8 + (lane >> 5) * 4;
        if (n >= p.N) continue;
        float v[4] = {a[4 * q4], a[4 * q4 + 1], a[4 * q4 + 2], a[4 * q4 + 3]};
        if (EPI == EPI_BIAS || EPI == EPI_BIAS_GELU || EPI == EPI_BIAS_F32 || EPI == EPI_QKV_PLANES) {
          bf16x4 bb = *(const bf16x4*)(p.bias + n);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += (float)bb[e];
        }
        if (EPI == EPI_QKV_PLANES) {
          // the 4 columns lie in one third (hl is a multiple of 8)
          const int part = n / p.qkv_hl, c = n - part * p.qkv_hl;
          const long plane = (long)p.M * p.qkv_hl, off = (long)m * p.qkv_hl + c;
          bf16x4 hb;
#pragma unroll
          for (int e = 0; e < 4; ++e) hb[e] = (bf16)v[e];
          *(bf16x4*)(p.C + (part == 2 ? 4 * plane : (2 * part + 1) * plane) + off) = hb;
          if (part < 2) {
            const float sc = part == 0 ? p.qscale : 1.0f;
            _Float16 h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) h[e] = (_Float16)fminf(fmaxf(v[e] * sc, -65504.0f), 65504.0f);
            *(bf16x4*)(p.C + 2 * part * plane + off) = __builtin_bit_cast(bf16x4, h);
          }
          continue;
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

// Row block i of a tile (all its column blocks).
template <int NW, int BNV, int EPI>
__device__ __forceinline__ void epilogue_rows(const KParams& p, int tm, int tn, int i,
                                              const f32x16 (&acc)[WC<NW, BNV>::NJ]) {
#pragma unroll
  for (int j = 0; j < WC<NW, BNV>::NJ; ++j) epilogue_block<NW, BNV, EPI>(p, tm, tn, i, j, acc[j]);
}

// Whole-tile epilogue through LDS (the stages are free once the main loop has
// ended). Storing straight from the accumulator layout writes 8 or 16 bytes
// into each of 32 rows per instruction; instead each wave applies the
// epilogue in registers and writes its results into a row-major image of the
// tile in LDS, and the workgroup then stores whole rows, NTHR*16 bytes per
// instruction. Image rows of RB bytes hold NCH 16-byte chunks, chunk c of
// image row r at (c + r) mod NCH, so the row-per-lane writes spread over the
// banks and the row-major reads do not conflict. An image larger than the
// stage memory (fp32 out, or 320 columns) goes in passes of PR rows; GeLU's
// two outputs go one after the other. The LDS-only barriers leave the global
// stores in flight.
__device__ __forceinline__ void lds_only_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <int NW, int BNV, int EPI>
__device__ __forceinline__ void epilogue_staged(const KParams& p, int tm, int tn,
                                                const f32x16 (&acc)[WC<NW, BNV>::MI][WC<NW, BNV>::NJ],
                                                bf16* smem) {
  using C = WC<NW, BNV>;
  constexpr int ES = EPI == EPI_BIAS_F32 ? 4 : 2;  // bytes per output element
  constexpr int RB = BNV * ES, NCH = RB / 16;
  constexpr int LDS_BYTES = 2 * (BM + BNV) * BKK * 2;
  constexpr int PR = 256 * RB <= LDS_BYTES ? 256 : 128 * RB <= LDS_BYTES ? 128 : 64;
  // two images: GeLU's pre and y; the projection planes' fp16 score copies
  // (and v) and then their bf16 copies
  constexpr int NPASS = BM / PR, NIMG = (EPI == EPI_BIAS_GELU || EPI == EPI_QKV_PLANES) ? 2 : 1;
  constexpr int ITERS = PR * NCH / C::NTHR;
  static_assert(PR * NCH % C::NTHR == 0 && NCH >= 24 && PR % 32 == 0, "image layout");
  typedef __attribute__((address_space(3))) char lds_char;
  lds_char* img = (lds_char*)smem;
  // an opaque copy of the thread id keeps the per-lane addresses below from
  // being hoisted out of the tile loop (they would be held, or spilled,
  // across the main loop)
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = (int)uni((uint32_t)(tid >> 6));
  const int wm = wave / C::WNG, wn = wave % C::WNG;
  const int l32 = lane & 31, hh = lane >> 5;
#pragma unroll
  for (int im = 0; im < NIMG; ++im) {
#pragma unroll
    for (int ps = 0; ps < NPASS; ++ps) {
#pragma unroll
      for (int i = 0; i < C::MI; ++i) {
        const int r0 = wm * C::WMW + 32 * i - ps * PR;  // wave-uniform
        if (NPASS > 1 && (r0 < 0 || r0 >= PR)) continue;
        const unsigned rl = (unsigned)(r0 + l32);
        const int m = tm * BM + ps * PR + (int)rl;
#pragma unroll
        for (int j = 0; j < C::NJ; ++j)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            const int nt = wn * C::WNW + j * 32 + q4 * 8 + 4 * hh, n = tn * BNV + nt;
            float v[4] = {acc[i][j][4 * q4], acc[i][j][4 * q4 + 1], acc[i][j][4 * q4 + 2], acc[i][j][4 * q4 + 3]};
            if (n < p.N) {
              if (EPI == EPI_BIAS || EPI == EPI_BIAS_GELU || EPI == EPI_BIAS_F32 || EPI == EPI_QKV_PLANES) {
                const bf16x4 bb = *(const bf16x4*)(p.bias + n);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] += (float)bb[e];
              }
              if (EPI == EPI_DGELU && m < p.M) {
                const bf16x4 pa = *(const bf16x4*)(p.aux + (long)m * p.ldaux + n);
#pragma unroll
                for (int e = 0; e < 4; ++e) v[e] *= gelu_grad_f((float)pa[e]);
              }
            }
            if (EPI == EPI_BIAS_GELU && im == 1) {
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = gelu_f(v[e]);
            }
            const unsigned c = (unsigned)(nt * ES / 16), pc = (c + rl) % NCH;
            lds_char* dst = img + rl * RB + pc * 16 + (nt * ES) % 16;
            if constexpr (ES == 4) {
              *(__attribute__((address_space(3))) f32x4*)dst = f32x4{v[0], v[1], v[2], v[3]};
            } else if (EPI == EPI_QKV_PLANES && im == 0 && n < 2 * p.qkv_hl) {
              // q and k columns, first image: fp16 score copies (q scaled)
              const float sc = n < p.qkv_hl ? p.qscale : 1.0f;
              _Float16 hv[4];
#pragma unroll
              for (int e = 0; e < 4; ++e) hv[e] = (_Float16)fminf(fmaxf(v[e] * sc, -65504.0f), 65504.0f);
              *(__attribute__((address_space(3))) bf16x4*)dst = __builtin_bit_cast(bf16x4, hv);
            } else {
              bf16x4 o;
#pragma unroll
              for (int e = 0; e < 4; ++e) o[e] = (bf16)v[e];
              *(__attribute__((address_space(3))) bf16x4*)dst = o;
            }
          }
      }
      lds_only_barrier();
      char* out = im == 0 ? (char*)p.C : (char*)p.C2;
      const long ld = im == 0 ? p.ldc : p.ldc2;
#pragma unroll
      for (int it = 0; it < ITERS; ++it) {
        const unsigned lin = (unsigned)(it * C::NTHR + tid), rl = lin / NCH, c = lin - rl * NCH;
        const u32x4 v = *(__attribute__((address_space(3))) const u32x4*)(img + rl * RB + ((c + rl) % NCH) * 16);
        const int gm = tm * BM + ps * PR + (int)rl, gn = tn * BNV + (int)c * (16 / ES);
        if (EPI == EPI_QKV_PLANES) {
          // 8 columns of one third: its plane for this image (v has none in the second)
          const int part = gn / p.qkv_hl, cc = gn - part * p.qkv_hl;
          const int pl = part < 2 ? 2 * part + im : (im == 0 ? 4 : -1);
          if (gm < p.M && gn < p.N && pl >= 0)
            *(u32x4*)(p.C + (long)pl * p.M * p.qkv_hl + (long)gm * p.qkv_hl + cc) = v;
          continue;
        }
        if (gm < p.M && gn < p.N) *(u32x4*)(out + ((long)gm * ld + gn) * ES) = v;
      }
      lds_only_barrier();  // the image (or the next tile's loads) overwrites this pass
    }
  }
}

// Whole-tile epilogue: through LDS, except the fp32 output (its direct stores
// already write 16 bytes per lane, and its image would take two passes). The
// projection's 16-bit planes go through LDS: stored straight from the
// accumulators they took 8-byte stores into five planes (+20% on the
// GPT-2-like projection).
template <int NW, int BNV, int EPI>
__device__ __forceinline__ void epilogue_tile(const KParams& p, int tm, int tn,
                                              const f32x16 (&acc)[WC<NW, BNV>::MI][WC<NW, BNV>::NJ], bf16* smem) {
  if constexpr (EPI == EPI_BIAS_F32) {
#pragma unroll
    for (int i = 0; i < WC<NW, BNV>::MI; ++i) epilogue_rows<NW, BNV, EPI>(p, tm, tn, i, acc[i]);
  } else {
    epilogue_staged<NW, BNV, EPI>(p, tm, tn, acc, smem);
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
// (f4*NTHR + tid)*4, so each store/load instruction covers NTHR*16 bytes
// contiguously.
template <int NW, int BNV>
__device__ __forceinline__ void store_partial(float* slot, const f32x16 (&acc)[WC<NW, BNV>::MI][WC<NW, BNV>::NJ]) {
  constexpr int MI = WC<NW, BNV>::MI, NJ = WC<NW, BNV>::NJ, NTHR = WC<NW, BNV>::NTHR;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < MI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int f4 = (i * NJ + j) * 4 + q4;
        f32x4 v = {acc[i][j][4 * q4], acc[i][j][4 * q4 + 1], acc[i][j][4 * q4 + 2], acc[i][j][4 * q4 + 3]};
        *(f32x4*)(slot + ((long)f4 * NTHR + tid) * 4) = v;
      }
}

// One loop over this workgroup's work items: first its data-parallel tiles,
// then its run of stream-K iterations (whole tiles in the run are stored
// directly, partial tiles go to the workspace).
template <int NW, int BNV, bool AK, bool BKM, int EPI>
__device__ __forceinline__ void gemm_body(const KParams& p, bf16* smem) {
  constexpr int MI = WC<NW, BNV>::MI, NJ = WC<NW, BNV>::NJ;
  const int lw = p.blk_s > 0 ? (int)blockIdx.x : logical_wg(blockIdx.x, p.grid);
  if (p.splits > 1) {
    // data-parallel rounds, then the split tail: consecutive workgroups (one
    // XCD) take the same k-range of neighbouring tiles, so they share panels
    // in L2
    for (int r = 0; r < p.dp_rounds; ++r) {
      const int t = r * p.grid + lw;
      int tm, tn;
      tile_coords(p, t, tm, tn);
      f32x16 acc[MI][NJ];
#pragma unroll
      for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};
      mainloop<NW, BNV, AK, BKM>(p, tm, tn, 0, p.iters, acc, smem);
      epilogue_tile<NW, BNV, EPI>(p, tm, tn, acc, smem);
    }
    if (lw >= p.splits * p.split_tiles) return;
    const int t = p.split_first + lw % p.split_tiles, sidx = lw / p.split_tiles;
    const int kb = (int)((long long)sidx * p.iters / p.splits);
    const int ke = (int)((long long)(sidx + 1) * p.iters / p.splits);
    int tm, tn;
    tile_coords(p, t, tm, tn);
    f32x16 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};
    mainloop<NW, BNV, AK, BKM>(p, tm, tn, kb, ke, acc, smem);
    store_partial<NW, BNV>(p.partials + (long)lw * BM * BNV, acc);
    return;
  }
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
    f32x16 acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
      for (int j = 0; j < NJ; ++j) acc[i][j] = f32x16{};
    mainloop<NW, BNV, AK, BKM>(p, tm, tn, kb, ke, acc, smem);
    if (kb == 0 && ke == p.iters) {
      epilogue_tile<NW, BNV, EPI>(p, tm, tn, acc, smem);
    } else {
      const long long t0 = (long long)t * p.iters - p.sk_begin;  // tile start, SK-relative
      const int slot = 2 * lw + (s >= t0 ? 0 : 1);
      store_partial<NW, BNV>(p.partials + (long)slot * BM * BNV, acc);
    }
  }
}

// Stream-K fix-up: sum each split tile's partials in contributor order and
// apply the epilogue. MI x NJ workgroups per tile, one per (row block i,
// column block j) of the waves' sub-tiles: each thread adds 4 float4 per
// contributor (a 320-wide tile split 4 ways over K, or a stream-K tile, is
// spread over 10 or 8 workgroups instead of 2 or 4, so the few split tiles
// still fill the CUs).
template <int NW, int BNV, int EPI>
__device__ __forceinline__ void fixup_body(const KParams& p, int first_tile) {
  constexpr int MI = WC<NW, BNV>::MI, NJ = WC<NW, BNV>::NJ, NTHR = WC<NW, BNV>::NTHR;
  const int t = first_tile + blockIdx.x / (MI * NJ), r = blockIdx.x % (MI * NJ), i = r / NJ, j = r % NJ;
  const int tid = threadIdx.x;
  f32x16 acc = f32x16{};
  auto add = [&](const float* src) {
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int f4 = (i * NJ + j) * 4 + q4;
      const f32x4 v = *(const f32x4*)(src + ((long)f4 * NTHR + tid) * 4);
      acc[4 * q4] += v[0];
      acc[4 * q4 + 1] += v[1];
      acc[4 * q4 + 2] += v[2];
      acc[4 * q4 + 3] += v[3];
    }
  };
  if (p.splits > 1) {  // split tail: tile t's partials are slots (t - first) + s*split_tiles
    for (int sidx = 0; sidx < p.splits; ++sidx)
      add(p.partials + (long)(sidx * p.split_tiles + t - p.split_first) * BM * BNV);
  } else {
    const long long base = p.sk_total / p.sk_grid, rem = p.sk_total % p.sk_grid;
    const long long t0 = (long long)t * p.iters - p.sk_begin;
    const long long c0 = sk_owner(t0, base, rem), c1 = sk_owner(t0 + p.iters - 1, base, rem);
    if (c0 == c1) return;  // one workgroup covered the whole tile and stored it
    for (long long c = c0; c <= c1; ++c)
      add(p.partials + (long)(2 * c + (sk_start(c, base, rem) >= t0 ? 0 : 1)) * BM * BNV);
  }
  int tm, tn;
  tile_coords(p, t, tm, tn);
  epilogue_block<NW, BNV, EPI>(p, tm, tn, i, j, acc);
}

// ---- 256x320 tiles for the output projection (k-outer B) ----------------------
// 8 waves, 2 along m x 4 along n (128 x 80 each) on v_mfma_f32_16x16x32_bf16:
// each wave reads its A rows (k-inner, the panel above) through ds_read_b128
// and its 80 B columns (k-outer: the weight) through the transposing reads,
// so the weight goes through the transposing reads twice per k-step (the 4x2
// layout of the 32x32 tile needs four). The B stage is [64 k-rows][40 chunks]
// (640 bytes per k-row); logical chunk lc of k-row kr sits at physical chunk
// 8(lc/8) + ((lc%8) ^ f(kr)), f(kr) = 2(((kr%8) + s(kr/8)) % 4) with
// s(G) = (G%4) ^ ((G%4)/2), so the four k-rows one 16-lane group of a
// transposing read touches land in four different 32-byte bank groups, and
// the k-rows of lane groups served together differ in f or in parity.
// Permuted k slots: lane group g of the 16x16x32 MFMA holds the 8 k of
// logical chunk 4kk + t(g) of the sub-step, t = (0, 2, 1, 3), in both
// operands (the sum over k is unchanged). A 128-bit LDS read serves lanes
// {s..s+7} and {s+32..s+39} together; with t(g) = g those lanes read the same
// eight A rows at chunks c and c ^ 2, which share banks (measured: 4 conflict
// cycles per read, twice the cycles of the 32x32 kernels' reads), with t they
// read chunks of opposite parity and do not conflict. Operands are
// swapped in the MFMA as in the 32x32 kernels: each lane owns one m and four
// consecutive n of a 16x16 block. Data-parallel plans only (N a multiple of
// 320, whole rounds of tiles); a K that is not a multiple of 64 ends in a
// partial k-step whose A chunks past K read zeros (the one k-step that loads
// it checks them). Other shapes take the 256-wide tile.
struct PanelB320 { const bf16* base; uint32_t nrec, kstep; uint32_t voff[5]; };
__device__ __forceinline__ int b320_swz(int kr) {
  const int G = (kr >> 3) & 3;
  return 2 * (((kr & 7) + (G ^ (G >> 1))) & 3);
}
__device__ __forceinline__ int kslot16(int g) { return ((g & 1) << 1) | (g >> 1); }  // t(g)
// physical chunk q of the stage (64 k-rows x 40 chunks) holds logical chunk lc of k-row kr
__device__ __forceinline__ PanelB320 panel_b320(const bf16* B, long ld, int N, int K, int n0, int wave, int lane) {
  PanelB320 pn;
  pn.base = uni_ptr(B + n0);
  pn.nrec = uni((uint32_t)(((long)K * ld - n0) * 2));
  pn.kstep = uni((uint32_t)(BKK * ld * 2));
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int q = 64 * (5 * wave + i) + lane;
    const int kr = q / 40, pc = q - kr * 40;
    const int lc = 8 * (pc >> 3) + ((pc & 7) ^ b320_swz(kr));
    pn.voff[i] = (n0 + 8 * lc < N) ? (uint32_t)(((long)kr * ld + 8 * lc) * 2) : pn.nrec;
  }
  return pn;
}
__device__ __forceinline__ void issue_b320(const PanelB320& pn, int kt, bf16* dst, int wave) {
  const int soff = (int)uni((uint32_t)kt * pn.kstep);
  __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc((void*)pn.base, (short)0, (int)pn.nrec, 0x00020000);
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    bf16* blk = dst + (5 * wave + i) * 512;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr)blk, 16, pn.voff[i], soff, 0, 0);
  }
}

// One k-step: wait for this wave's loads, barrier, issue the next k-step's
// loads, then two 32-deep sub-steps: the wave's five B fragments (two
// transposing reads each), and for each of its eight 16-row A blocks one
// ds_read_b128 and five MFMAs.
template <bool TAIL>
__device__ __forceinline__ void fwd320_kstep(const KParams& p, const Panel<4>& pa, const PanelB320& pb, int kt,
                                             const bf16* __restrict__ a, const bf16* __restrict__ b,
                                             bf16* __restrict__ na, bf16* __restrict__ nb, int wave, int lane,
                                             int aoff0, int abase, const int (&boff)[5], f32x4 (&acc)[8][5]) {
  wait_vmem();
  __syncthreads();
  issue_panel<4, true, TAIL>(pa, kt + 1, p.K, na, wave, lane);  // B rows past K read zeros
  issue_b320(pb, kt + 1, nb, wave);
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    bf16x8 bfr[5];
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const char* bb = (const char*)b + boff[j];
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(bb + (32 * kk) * 640));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(bb + (32 * kk + 4) * 640));
      typedef short i16x8 __attribute__((ext_vector_type(8)));
      const i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
      bfr[j] = __builtin_bit_cast(bf16x8, v);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int ch = abase ^ (4 * kk) ^ (2 * (i & 3));
      const bf16x8 af = *(const bf16x8*)((const char*)a + aoff0 + 2048 * i + (ch << 4));
#pragma unroll
      for (int j = 0; j < 5; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[j], af, acc[i][j], 0, 0, 0);
    }
  }
}

// bf16 output (EPI_STORE, EPI_BIAS) through a row-major LDS image, two passes
// of 128 rows (one per wave row), chunk c of image row r at (c + r) mod 40.
template <int EPI>
__device__ __forceinline__ void fwd320_epilogue(const KParams& p, int tm, int tn, const f32x4 (&acc)[8][5], bf16* smem) {
  static_assert(EPI == EPI_STORE || EPI == EPI_BIAS, "bf16 single-output epilogues");
  constexpr int RB = 640, NCH = 40, PR = 128, ITERS = PR * NCH / 512;
  typedef __attribute__((address_space(3))) char lds_char;
  lds_char* img = (lds_char*)smem;
  int tid = threadIdx.x;
  asm volatile("" : "+v"(tid));
  const int lane = tid & 63, wave = (int)uni((uint32_t)(tid >> 6));
  const int wm = wave >> 2, wn = wave & 3, l16 = lane & 15, g = lane >> 4;
#pragma unroll
  for (int ps = 0; ps < 2; ++ps) {
    if (wm == ps) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const unsigned rl = (unsigned)(16 * i + l16);
#pragma unroll
        for (int j = 0; j < 5; ++j) {
          const int nt = wn * 80 + 16 * j + 4 * g, n = tn * 320 + nt;
          float v[4] = {acc[i][j][0], acc[i][j][1], acc[i][j][2], acc[i][j][3]};
          if (EPI == EPI_BIAS && n < p.N) {
            const bf16x4 bb = *(const bf16x4*)(p.bias + n);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] += (float)bb[e];
          }
          const unsigned c = (unsigned)(nt >> 3), pc = (c + rl) % NCH;
          bf16x4 o;
#pragma unroll
          for (int e = 0; e < 4; ++e) o[e] = (bf16)v[e];
          *(__attribute__((address_space(3))) bf16x4*)(img + rl * RB + pc * 16 + (nt * 2) % 16) = o;
        }
      }
    }
    lds_only_barrier();
#pragma unroll
    for (int it = 0; it < ITERS; ++it) {
      const unsigned lin = (unsigned)(it * 512 + tid), rl = lin / NCH, c = lin - rl * NCH;
      const u32x4 v = *(__attribute__((address_space(3))) const u32x4*)(img + rl * RB + ((c + rl) % NCH) * 16);
      const int gm = tm * BM + ps * PR + (int)rl, gn = tn * 320 + (int)c * 8;
      if (gm < p.M && gn < p.N) *(u32x4*)((char*)p.C + ((long)gm * p.ldc + gn) * 2) = v;
    }
    lds_only_barrier();  // the next pass (or the next tile's loads) overwrites the image
  }
}

template <int EPI>
__device__ __forceinline__ void fwd320_body(const KParams& p, bf16* smem) {
  const int lw = logical_wg(blockIdx.x, p.grid);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = (int)uni((uint32_t)(tid >> 6));
  const int wm = wave >> 2, wn = wave & 3, l16 = lane & 15, g = lane >> 4;
  // A fragment of block i, sub-step kk: row wm*128 + 16i + l16, k chunk
  // 4kk + t(g), stored at chunk (4kk + t(g)) ^ swz(row) = abase ^ 4kk ^ 2(i & 3)
  // (the k-inner swizzle (r ^ r>>3) & 7 restricted to these rows)
  const int tg = kslot16(g);
  const int aoff0 = (wm * 128 + l16) * 128;
  const int abase = tg ^ ((l16 & 7) ^ (l16 >> 3));
  // B fragment of block j: this lane addresses k-row 8t(g) + r' (+ 32kk, + 4
  // for the second read) and column quad c' = l16 & 3, i.e. logical chunk
  // lc = wn*10 + 2j + c'/2 at physical 8(lc/8) + ((lc%8) ^ f), f = b320_swz of
  // that k-row, the same for every kk and read
  const int rp = l16 >> 2, cq = l16 & 3, f = b320_swz(8 * tg + rp);
  for (int r = 0; r < p.dp_rounds; ++r) {
    const int t = r * p.grid + lw;
    int tm, tn;
    tile_coords(p, t, tm, tn);
    f32x4 acc[8][5];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 5; ++j) acc[i][j] = f32x4{};
    const Panel<4> pa = panel_kinner<4, BM>(p.A, p.lda, p.M, tm * BM, wave, lane);
    const PanelB320 pb = panel_b320(p.B, p.ldb, p.N, p.K, tn * 320, wave, lane);
    issue_panel<4, true, true>(pa, 0, p.K, smem, wave, lane);
    issue_b320(pb, 0, smem + 2 * BM * BKK, wave);
    int boff[5];
#pragma unroll
    for (int j = 0; j < 5; ++j) {
      const int lc = wn * 10 + 2 * j + (cq >> 1);
      boff[j] = (8 * tg + rp) * 640 + (8 * (lc >> 3) + ((lc & 7) ^ f)) * 16 + 8 * (cq & 1);
    }
    // only the k-step that loads a partial last k-step (K not a multiple of
    // 64) checks the A chunks against K: the loop is split around it
    const int kload = p.K % BKK ? p.iters - 2 : -1;  // k-step whose loads are the partial one
    int cur = 0, kt = 0;
    auto step = [&](auto tail) {
      fwd320_kstep<decltype(tail)::value>(p, pa, pb, kt, smem + cur * BM * BKK, smem + 2 * BM * BKK + cur * 320 * BKK,
                                          smem + (cur ^ 1) * BM * BKK, smem + 2 * BM * BKK + (cur ^ 1) * 320 * BKK,
                                          wave, lane, aoff0, abase, boff, acc);
      cur ^= 1;
      ++kt;
    };
    const int kmid = kload >= 0 ? kload : p.iters;
    while (kt < kmid) step(std::false_type{});
    if (kt < p.iters && kt == kload) step(std::true_type{});
    while (kt < p.iters) step(std::false_type{});
    wait_vmem();
    __syncthreads();
    fwd320_epilogue<EPI>(p, tm, tn, acc, smem);
  }
}
}  // namespace

// One kernel (and its stream-K fix-up kernel) per product of the layer, so
// that a trace attributes time to each step by name.
#define TP_GEMM_KERNELS(NAME, NWV, BNV, AKV, BKV, EV)                                      \
  __global__ __launch_bounds__(64 * NWV)                                                   \
  __attribute__((amdgpu_waves_per_eu(NWV / 4, NWV / 4))) void NAME(KParams p) {            \
    __shared__ __attribute__((aligned(16))) bf16 smem[2 * (BM + BNV) * BKK];               \
    gemm_body<NWV, BNV, AKV, BKV, EV>(p, smem);                                            \
  }                                                                                        \
  __global__ __launch_bounds__(64 * NWV) void NAME##_fixup(KParams p, int first_tile) {    \
    fixup_body<NWV, BNV, EV>(p, first_tile);                                               \
  }

// Every layer product runs 8 waves per workgroup (two per SIMD). The weight
// gradients (K = tokens) take one operand as a transposed copy made just
// before them (k-inner, read by ds_read_b128) and the other as stored
// (k-outer, read through transposing LDS loads): with both operands k-outer
// the 8-wave tile reads 1.5x more LDS bytes-equivalent per flop than the
// forward products, and 4 waves (one per SIMD) left the matrix cores idle at
// every wait; the copies cost less than they save. Products with a k-inner B
// also have a 256x320-tile kernel (suffix _n320), taken when N is a multiple
// of 320. Only the vocabulary-parallel weight gradient keeps 4 waves with
// both operands k-outer.
// forward products: A k-inner (activations), B k-outer (weights)
// the QKV projection writes the attention's 16-bit operand planes (matrix-core
// attention) or fp32 q, k, v (the vector-ALU attention)
TP_GEMM_KERNELS(gemm_qkv_proj, 8, 256, true, false, EPI_QKV_PLANES)
TP_GEMM_KERNELS(gemm_qkv_proj_f32, 8, 256, true, false, EPI_BIAS_F32)
TP_GEMM_KERNELS(gemm_out_proj, 8, 256, true, false, EPI_STORE)
TP_GEMM_KERNELS(gemm_fc1_bias_gelu, 8, 256, true, false, EPI_BIAS_GELU)
TP_GEMM_KERNELS(gemm_fc2, 8, 256, true, false, EPI_STORE)
TP_GEMM_KERNELS(gemm_qkv_proj_n192, 8, 192, true, false, EPI_QKV_PLANES)
TP_GEMM_KERNELS(gemm_out_proj_n192, 8, 192, true, false, EPI_STORE)
TP_GEMM_KERNELS(gemm_fc1_bias_gelu_n192, 8, 192, true, false, EPI_BIAS_GELU)
TP_GEMM_KERNELS(gemm_fc2_n192, 8, 192, true, false, EPI_STORE)
// input gradients: both k-inner (weights read transposed)
TP_GEMM_KERNELS(gemm_fc2_dgrad_gelu, 8, 256, true, true, EPI_DGELU)
TP_GEMM_KERNELS(gemm_fc1_dgrad, 8, 256, true, true, EPI_STORE)
TP_GEMM_KERNELS(gemm_out_dgrad, 8, 256, true, true, EPI_STORE)
TP_GEMM_KERNELS(gemm_qkv_dgrad, 8, 256, true, true, EPI_STORE)
TP_GEMM_KERNELS(gemm_fc2_dgrad_gelu_n320, 8, 320, true, true, EPI_DGELU)
TP_GEMM_KERNELS(gemm_fc1_dgrad_n320, 8, 320, true, true, EPI_STORE)
TP_GEMM_KERNELS(gemm_out_dgrad_n320, 8, 320, true, true, EPI_STORE)
TP_GEMM_KERNELS(gemm_qkv_dgrad_n320, 8, 320, true, true, EPI_STORE)
TP_GEMM_KERNELS(gemm_fc2_dgrad_gelu_n192, 8, 192, true, true, EPI_DGELU)
TP_GEMM_KERNELS(gemm_fc1_dgrad_n192, 8, 192, true, true, EPI_STORE)
TP_GEMM_KERNELS(gemm_out_dgrad_n192, 8, 192, true, true, EPI_STORE)
TP_GEMM_KERNELS(gemm_qkv_dgrad_n192, 8, 192, true, true, EPI_STORE)
// weight gradients (K = tokens): dB_i = (y_i^T copy) dZ and dWo_i = (ctx_i^T
// copy) dO take a k-inner A and the stored gradient as a k-outer B; dA_i = X^T
// (dPre^T copy) and dWqkv_i = X^T (dqkv^T copy) take X as stored (k-outer A)
// and a k-inner B
TP_GEMM_KERNELS(gemm_fc2_wgrad, 8, 256, true, false, EPI_STORE)
TP_GEMM_KERNELS(gemm_out_wgrad, 8, 256, true, false, EPI_STORE)
TP_GEMM_KERNELS(gemm_fc1_wgrad, 8, 256, false, true, EPI_STORE)
TP_GEMM_KERNELS(gemm_qkv_wgrad, 8, 256, false, true, EPI_STORE)
TP_GEMM_KERNELS(gemm_fc1_wgrad_n320, 8, 320, false, true, EPI_STORE)
TP_GEMM_KERNELS(gemm_qkv_wgrad_n320, 8, 320, false, true, EPI_STORE)
// weight gradients of narrow layers, both operands read as stored (k-outer,
// 4 waves: with both through the transposing loads 8 waves measured slower);
// there a transposed copy costs more than the product gains
TP_GEMM_KERNELS(gemm_fc2_wgrad_ko, 4, 256, false, false, EPI_STORE)
TP_GEMM_KERNELS(gemm_out_wgrad_ko, 4, 256, false, false, EPI_STORE)
TP_GEMM_KERNELS(gemm_fc1_wgrad_ko, 4, 256, false, false, EPI_STORE)
TP_GEMM_KERNELS(gemm_qkv_wgrad_ko, 4, 256, false, false, EPI_STORE)
// the output projection on 256x320 tiles (16x16x32 MFMAs, data-parallel
// plans only, so no fix-up kernel). GEMM1 (bias + GeLU, two outputs) keeps
// the 256-wide tile: on that tile its step time was 30 us longer although the
// kernel alone ran 3% faster. GEMM2 and its weight gradient (same k-outer B)
// also keep it: on the 32x32x16 256-wide tile with a stream-K tail their
// kernels ran 0.06-0.09 ms faster each and the step 0.10-0.13 ms shorter on
// three of four GPUs (equal on the fourth).
#define TP_GEMM_FWD320(NAME, EV)                                                                \
  __global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(2, 2))) void NAME(KParams p) { \
    __shared__ __attribute__((aligned(16))) bf16 smem[2 * (BM + BN_MAX) * BKK];                 \
    fwd320_body<EV>(p, smem);                                                                   \
  }
TP_GEMM_FWD320(gemm_out_proj_n320, EPI_STORE)
#undef TP_GEMM_FWD320
// vocabulary-parallel output layer: logits = X W_i^T (the table slice W_i
// [V/p, h] is k-inner), dX = dlogits W_i, dW_i = dlogits^T X
TP_GEMM_KERNELS(gemm_logits, 8, 256, true, true, EPI_STORE)
TP_GEMM_KERNELS(gemm_logits_n320, 8, 320, true, true, EPI_STORE)
TP_GEMM_KERNELS(gemm_logits_dgrad, 8, 256, true, false, EPI_STORE)
TP_GEMM_KERNELS(gemm_logits_wgrad, 4, 256, false, false, EPI_STORE)
#undef TP_GEMM_KERNELS

namespace {

struct Plan {
  int grid, dp_rounds, sk_grid, sk_first_tile, sk_tiles;
  long long sk_begin, sk_total;
  int splits;
  int blk_s, blk_m, blk_n;  // phase blocks (0: raster order)
};

// Data-parallel rounds of ncu tiles; the remaining R tiles, if a partial
// round would leave many CUs idle, are either split evenly in K over
// S = ncu / R workgroups each (when that keeps >= 90% of the CUs busy and
// >= 8 k-steps per piece: better L2 reuse) or dealt out stream-K.
Plan make_plan(int tiles, int iters, int ncu) {
  Plan pl{};
  ncu = ncu < GMAX ? ncu : GMAX;
  pl.splits = 1;
  const int waves = (tiles + ncu - 1) / ncu;
  const double eff_dp = (double)tiles / ((double)waves * ncu);
  if (iters < 8 || eff_dp >= 0.9) {
    pl.grid = tiles; pl.dp_rounds = 1;
    return pl;
  }
  const int full0 = tiles / ncu, rem0 = tiles - full0 * ncu;
  if (rem0 > 0 && iters >= 16) {
    int sp = ncu / rem0;
    if (sp > iters / 8) sp = iters / 8;
    const double eff_tail = (double)(sp * rem0) / ncu;
    if (sp >= 2 && eff_tail >= 0.9) {
      pl.splits = sp;
      pl.dp_rounds = full0;
      pl.grid = full0 > 0 ? ncu : rem0 * sp;
      pl.sk_first_tile = full0 * ncu;  // first split tile (fix-up launch)
      pl.sk_tiles = rem0;
      return pl;
    }
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

// Stream-K over all tiles with the same whole number q of k-steps per
// workgroup: workgroup w starts at k-step (q w) mod iters of tile q w / iters,
// so the workgroups w = r (mod P), P = iters / gcd(q, iters), run in step
// (the same k-step at the same time) on tiles t_r + s i, i = 0 .. c-1, with
// c = grid / P and s = tiles / c. Workgroups are dealt round-robin to the 8
// XCDs: with P a multiple of 8 each such class sits on one XCD. Numbering the
// tiles so that each class's c tiles form a compact bm x bn block of the tile
// grid (tile t = position t / s of block t % s) lets the class share its
// operand panels in that XCD's L2: bm + bn panel loads per k-step instead of
// 2c. (In the raster order the workgroups of one XCD sit at up to 16
// different k-steps of their tiles, and the panels come from the
// memory-side cache at a lower rate.)
void phase_blocks(Plan& pl, int tiles_m, int tiles_n, int iters) {
  if (pl.sk_total == 0 || pl.splits > 1 || pl.dp_rounds > 0 || pl.sk_total % pl.sk_grid) return;
  const long long q = pl.sk_total / pl.sk_grid;
  long long a = q, b = iters;
  while (b) {
    const long long r = a % b;
    a = b;
    b = r;
  }
  const long long P = iters / a;
  if (P % 8 || pl.sk_grid % P) return;
  const int c = (int)(pl.sk_grid / P), tiles = tiles_m * tiles_n;
  if (tiles % c) return;
  int bm_best = 0, bn_best = 0;
  for (int bm = 1; bm <= c; ++bm) {
    if (c % bm || tiles_m % bm || tiles_n % (c / bm)) continue;
    if (bm_best == 0 || bm + c / bm < bm_best + bn_best) {
      bm_best = bm;
      bn_best = c / bm;
    }
  }
  if (bm_best == 0) return;
  pl.blk_s = tiles / c;
  pl.blk_m = bm_best;
  pl.blk_n = bn_best;
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

// Upper bound over the tile widths a product may run with.
size_t gemm_mfma_workspace_bytes(int M, int N, int K) {
  const long long iters = (K + BKK - 1) / BKK;
  size_t best = 0;
  for (int bn : {192, 256, BN_MAX}) {
    const long long tiles = (long long)((M + BM - 1) / BM) * ((N + bn - 1) / bn);
    if (iters < 8 || tiles <= 0) continue;
    long long slots = 2LL * GMAX;
    if (slots > 2 * tiles * iters) slots = 2 * tiles * iters;
    const size_t b = (size_t)slots * BM * bn * sizeof(float);
    best = b > best ? b : best;
  }
  return best;
}

namespace {

typedef void (*MainK)(KParams);
typedef void (*FixK)(KParams, int);
struct KRef {
  MainK mk = nullptr;
  FixK fk = nullptr;  // stream-K / k-split fix-up (none for the forward 320-wide kernels)
  const char* name = nullptr;
};
#define TP_K(NAME) KRef{NAME, NAME##_fixup, #NAME}
#define TP_KF(NAME) KRef{NAME, nullptr, #NAME}

// The kernels of one product: the 256-wide tile and the alternatives its
// role has (k-inner B on 320- or 192-wide tiles, the output projection's
// 16x16x32 320-wide tile, both operands k-outer on 4 waves), with the
// operand layouts and epilogue the kernels are compiled for.
struct RoleKernels {
  KRef base, w320, w192, f320, ko;
  int nw = 8;
  bool ak = true, bk = false;
  int ep = EPI_STORE;
};

bool role_kernels(const GemmDesc& g, RoleKernels& r) {
  switch (g.role) {
    case GR_QKV_PROJ:
      if (g.epi == EPI_QKV_PLANES) { r.base = TP_K(gemm_qkv_proj); r.w192 = TP_K(gemm_qkv_proj_n192); r.ep = EPI_QKV_PLANES; }
      else { r.base = TP_K(gemm_qkv_proj_f32); r.ep = EPI_BIAS_F32; }
      return true;
    case GR_OUT_PROJ:
      r.base = TP_K(gemm_out_proj); r.f320 = TP_KF(gemm_out_proj_n320); r.w192 = TP_K(gemm_out_proj_n192); return true;
    case GR_FC1:
      r.base = TP_K(gemm_fc1_bias_gelu); r.w192 = TP_K(gemm_fc1_bias_gelu_n192); r.ep = EPI_BIAS_GELU; return true;
    case GR_FC2: r.base = TP_K(gemm_fc2); r.w192 = TP_K(gemm_fc2_n192); return true;
    case GR_FC2_DGRAD:
      r.base = TP_K(gemm_fc2_dgrad_gelu); r.w320 = TP_K(gemm_fc2_dgrad_gelu_n320);
      r.w192 = TP_K(gemm_fc2_dgrad_gelu_n192); r.bk = true; r.ep = EPI_DGELU; return true;
    case GR_FC1_DGRAD:
      r.base = TP_K(gemm_fc1_dgrad); r.w320 = TP_K(gemm_fc1_dgrad_n320); r.w192 = TP_K(gemm_fc1_dgrad_n192);
      r.bk = true; return true;
    case GR_OUT_DGRAD:
      r.base = TP_K(gemm_out_dgrad); r.w320 = TP_K(gemm_out_dgrad_n320); r.w192 = TP_K(gemm_out_dgrad_n192);
      r.bk = true; return true;
    case GR_QKV_DGRAD:
      r.base = TP_K(gemm_qkv_dgrad); r.w320 = TP_K(gemm_qkv_dgrad_n320); r.w192 = TP_K(gemm_qkv_dgrad_n192);
      r.bk = true; return true;
    case GR_FC2_WGRAD:
      r.base = TP_K(gemm_fc2_wgrad); r.ko = TP_K(gemm_fc2_wgrad_ko); return true;
    case GR_FC1_WGRAD:
      r.base = TP_K(gemm_fc1_wgrad); r.w320 = TP_K(gemm_fc1_wgrad_n320); r.ko = TP_K(gemm_fc1_wgrad_ko);
      r.ak = false; r.bk = true; return true;
    case GR_OUT_WGRAD: r.base = TP_K(gemm_out_wgrad); r.ko = TP_K(gemm_out_wgrad_ko); return true;
    case GR_QKV_WGRAD:
      r.base = TP_K(gemm_qkv_wgrad); r.w320 = TP_K(gemm_qkv_wgrad_n320); r.ko = TP_K(gemm_qkv_wgrad_ko);
      r.ak = false; r.bk = true; return true;
    case GR_LOGITS: r.base = TP_K(gemm_logits); r.w320 = TP_K(gemm_logits_n320); r.bk = true; return true;
    case GR_LOGITS_DGRAD: r.base = TP_K(gemm_logits_dgrad); return true;
    case GR_LOGITS_WGRAD: r.base = TP_K(gemm_logits_wgrad); r.nw = 4; r.ak = false; return true;
  }
  return false;
}
#undef TP_K
#undef TP_KF

// Critical-path length of a plan, in k-steps of the plan's tile: data-parallel
// rounds, plus the longest k-split piece or stream-K run; a plan with a
// fix-up launch pays kFixSteps more (the fp32 partial tiles are written,
// read back and reduced: 16-38 us measured, 10-20 k-steps of a 256x256 tile).
// A 256x192 k-step takes about kStep192 of a 256x256 one (0.75 of the flops,
// 0.875 of the bytes staged through LDS).
constexpr double kStep192 = 0.85, kFixSteps = 20.0;
double plan_cost(const Plan& pl, int tiles, int iters, int ncu, double per_step) {
  ncu = ncu < GMAX ? ncu : GMAX;
  double steps;
  if (pl.splits > 1) steps = (double)pl.dp_rounds * iters + (iters + pl.splits - 1) / pl.splits;
  else if (pl.sk_total > 0) steps = (double)pl.dp_rounds * iters + (double)((pl.sk_total + pl.sk_grid - 1) / pl.sk_grid);
  else steps = (double)((tiles + ncu - 1) / ncu) * iters;
  return per_step * steps + ((pl.splits > 1 || pl.sk_total > 0) ? kFixSteps : 0.0);
}

// The kernel and schedule of one product.
struct Pick {
  KRef k;
  int bn = 256, nw = 8;
  int fix_per_tile = 8;  // fix-up workgroups per tile: MI x NJ blocks of the waves' sub-tiles
  bool fwd320 = false;  // the 16x16x32 320-wide kernel (data-parallel only)
  Plan pl{};
};

// Kernel choice, given ws_bytes of workspace for stream-K / k-split
// partials (too little: data-parallel only). False when the role, operand
// layouts and epilogue match no kernel.
bool pick(const GemmDesc& g, size_t ws_bytes, Pick& out) {
  RoleKernels r;
  if (!role_kernels(g, r)) return false;
  if (r.ko.mk != nullptr && !g.a_kmajor && !g.b_kmajor) {  // weight gradient without a transposed copy
    r.base = r.ko;
    r.w320 = r.w192 = r.f320 = KRef{};
    r.nw = 4; r.ak = false; r.bk = false;
  }
  if (g.a_kmajor != r.ak || g.b_kmajor != r.bk || g.epi != r.ep) return false;
  const int ncu = device_cus(), cus = ncu < GMAX ? ncu : GMAX;
  const int iters = (g.K + BKK - 1) / BKK, tm = (g.M + BM - 1) / BM;
  // the output projection (k-outer B): 256x320 tiles when N is a whole
  // number of them and the tiles run in data-parallel rounds (no k-split tail)
  if (r.f320.mk != nullptr && g.N % BN_MAX == 0) {
    const int tiles = tm * (g.N / BN_MAX);
    const Plan pl = make_plan(tiles, iters, ncu);
    if (pl.splits == 1 && pl.sk_total == 0) {
      out.k = r.f320; out.bn = BN_MAX; out.nw = 8; out.fwd320 = true; out.pl = pl;
      return true;
    }
  }
  // k-inner B: the 320-wide tile when N is a whole number of them and they
  // fill the CUs at least once, or, fewer, when their k-split covers every CU
  // exactly. Then (either B layout) the 192-wide tile when its plan is
  // shorter than the 256-wide one's (whole rounds or an exact k-split instead
  // of a stream-K tail and its fix-up)
  int bn = 256;
  if (r.w320.mk != nullptr && g.N % BN_MAX == 0) {
    const int t320 = tm * (g.N / BN_MAX);
    const Plan p320 = make_plan(t320, iters, ncu);
    if (t320 >= cus || (p320.splits > 1 && p320.dp_rounds == 0 && p320.splits * t320 == cus)) bn = BN_MAX;
  }
  if (bn == 256 && r.w192.mk != nullptr) {
    const int t256 = tm * ((g.N + 255) / 256), t192 = tm * ((g.N + 191) / 192);
    if (plan_cost(make_plan(t192, iters, ncu), t192, iters, ncu, kStep192) <
        plan_cost(make_plan(t256, iters, ncu), t256, iters, ncu, 1.0))
      bn = 192;
  }
  out.k = bn == BN_MAX ? r.w320 : bn == 192 ? r.w192 : r.base;
  out.bn = bn;
  out.nw = r.nw;
  out.fix_per_tile = bn == BN_MAX ? WC<8, BN_MAX>::MI * WC<8, BN_MAX>::NJ
                     : bn == 192  ? WC<8, 192>::MI * WC<8, 192>::NJ
                     : r.nw == 4  ? WC<4, 256>::MI * WC<4, 256>::NJ
                                  : WC<8, 256>::MI * WC<8, 256>::NJ;
  const int tn = (g.N + bn - 1) / bn, tiles = tm * tn;
  Plan pl = make_plan(tiles, iters, ncu);
  if (pl.sk_total > 0 || pl.splits > 1) {
    const size_t slots = pl.splits > 1 ? (size_t)pl.splits * pl.sk_tiles : (size_t)2 * pl.sk_grid;
    if (ws_bytes < slots * BM * bn * sizeof(float)) pl = Plan{tiles, 1, 0, 0, 0, 0, 0, 1};  // data-parallel only
  }
  phase_blocks(pl, tm, tn, iters);
  out.pl = pl;
  return true;
}

}  // namespace

const char* gemm_mfma_kernel_name(const GemmDesc& g) {
  Pick pk;
  return pick(g, (size_t)-1, pk) ? pk.k.name : nullptr;
}

hipError_t gemm_mfma_launch(const GemmDesc& g, void* ws, size_t ws_bytes, hipStream_t stream) {
  Pick pk;
  if (!pick(g, ws != nullptr ? ws_bytes : 0, pk)) return hipErrorInvalidValue;
  const Plan& pl = pk.pl;
  KParams p{};
  p.A = (const bf16*)g.A; p.B = (const bf16*)g.B;
  p.lda = g.lda; p.ldb = g.ldb;
  p.M = g.M; p.N = g.N; p.K = g.K;
  p.tiles_m = (g.M + BM - 1) / BM;
  p.tiles_n = (g.N + pk.bn - 1) / pk.bn;
  p.iters = (g.K + BKK - 1) / BKK;
  p.epi = g.epi;
  p.C = (bf16*)g.C; p.ldc = g.ldc;
  p.C2 = (bf16*)g.C2; p.ldc2 = g.ldc2;
  p.bias = (const bf16*)g.bias;
  p.aux = (const bf16*)g.aux; p.ldaux = g.ldaux;
  p.qkv_hl = g.qkv_hl; p.qscale = g.qscale;
  p.partials = (float*)ws;
  p.grid = pl.grid; p.dp_rounds = pl.dp_rounds; p.sk_grid = pl.sk_grid;
  p.sk_begin = pl.sk_begin; p.sk_total = pl.sk_total; p.splits = pl.splits;
  p.split_first = pl.sk_first_tile; p.split_tiles = pl.sk_tiles;
  p.blk_s = pl.blk_s; p.blk_m = pl.blk_m; p.blk_n = pl.blk_n;
  const dim3 block(64 * pk.nw);
  hipLaunchKernelGGL(pk.k.mk, dim3(pl.grid), block, 0, stream, p);
  hipError_t e1 = hipGetLastError();
  const bool sk = pl.sk_total > 0 || pl.splits > 1;
  if (e1 != hipSuccess || !sk || pk.fwd320) return e1;
  hipLaunchKernelGGL(pk.k.fk, dim3(pk.fix_per_tile * pl.sk_tiles), block, 0, stream, p, pl.sk_first_tile);
  return hipGetLastError();
}

}  // namespace tpk
