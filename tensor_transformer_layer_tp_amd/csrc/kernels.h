// Host-side launchers of the layer-shard kernels (internal C++ interface used
// by the C ABI in tp_layer.cpp). Every launcher enqueues on `stream` and
// returns the launch status; none allocates or synchronizes.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace tpk {

enum DType : int { DT_F32 = 0, DT_BF16 = 1 };

// Epilogues applied to an fp32 accumulator element C[m][n] before it is stored.
enum Epi : int {
  EPI_STORE = 0,      // out = acc
  EPI_BIAS_GELU = 1,  // pre = acc + bias[n]; out2 = gelu(pre); out = pre
  EPI_DGELU = 2,      // out = acc * gelu'(aux[m][n])
  EPI_BIAS = 3,       // out = acc + bias[n]
  EPI_BIAS_F32 = 4,   // out (fp32) = acc + bias[n]
  // x = acc + bias[n] of a [M, 3 h] projection [q | k | v] (h = qkv_hl) as
  // five 16-bit planes [M, h] at out + p*M*h: 0 fp16(q qscale), 1 bf16(q),
  // 2 fp16(k), 3 bf16(k), 4 bf16(v); fp16 values saturate at +-65504
  EPI_QKV_PLANES = 5,
};

// The layer's products; the numbers match the TP_STEP_* ids of the C ABI.
enum GemmRole : int {
  GR_QKV_PROJ = 1, GR_OUT_PROJ = 3, GR_FC1 = 4, GR_FC2 = 5, GR_FC2_DGRAD = 6, GR_FC2_WGRAD = 7,
  GR_FC1_WGRAD = 8, GR_FC1_DGRAD = 9, GR_OUT_DGRAD = 10, GR_OUT_WGRAD = 11, GR_QKV_WGRAD = 13,
  GR_QKV_DGRAD = 14, GR_LOGITS = 18, GR_LOGITS_DGRAD = 22, GR_LOGITS_WGRAD = 23,
};

// C[M,N] = op(A) op(B) with fp32 accumulation, then an epilogue.
//   A: a_kmajor ? A[m*lda + k] : A[k*lda + m]
//   B: b_kmajor ? B[n*ldb + k] : B[k*ldb + n]
// epi: one of Epi (C2 receives gelu(pre) for EPI_BIAS_GELU).
struct GemmDesc {
  int role = 0;  // GemmRole (selects the bf16 kernel; the fp32 path ignores it)
  int M = 0, N = 0, K = 0;
  const void* A = nullptr; long lda = 0; bool a_kmajor = true;
  const void* B = nullptr; long ldb = 0; bool b_kmajor = false;
  int epi = 0;
  void* C = nullptr; long ldc = 0;
  void* C2 = nullptr; long ldc2 = 0;
  const void* bias = nullptr;
  const void* aux = nullptr; long ldaux = 0;
  int qkv_hl = 0; float qscale = 0.f;  // EPI_QKV_PLANES only
};

// Workspace bytes gemm_launch needs for this problem (host only).
size_t gemm_workspace_bytes(int dtype, int M, int N, int K);
hipError_t gemm_launch(int dtype, const GemmDesc& g, void* ws, size_t ws_bytes, hipStream_t stream);
// Name of the main kernel gemm_launch runs for g (host only; null when it
// launches none: an empty product, or no kernel for g's layouts).
const char* gemm_kernel_name(int dtype, const GemmDesc& g);

// Attention on the per-rank projection [T, 3*h_l] = [Q | K | V]: qkv holds
// it in fp32 for the vector-ALU path, or as the five 16-bit planes of
// EPI_QKV_PLANES (T*h_l elements each) for the matrix-core path
// (attn_mfma_supported); ctx, dctx and dqkv use the storage type.
struct AttnDesc {
  int batch = 0, seq = 0, n_local = 0, head_dim = 0;
  int head0 = 0;       // 0-based global index of local head 0 (rank * n_local)
  int n_heads = 1;     // global head count (ALiBi slopes)
  int alibi = 0;
  const void* qkv = nullptr;  // fp32 [T, 3*h_l], or the five planes
  void* ctx = nullptr;        // [T, h_l]
  float* lse = nullptr;       // [batch, n_local, seq]
  // backward only
  const void* dctx = nullptr;  // [T, h_l]
  float* delta = nullptr;      // [batch, n_local, seq] scratch: rowsum(dctx * ctx)
  void* dqkv = nullptr;        // [T, 3*h_l]
  // attention-probability dropout (matrix-core path only; enabled when mask is
  // set): keep bits [batch][n_local][ceil(seq/32)][2][seq rounded up to 8],
  // written by the forward, read by the backward
  uint16_t* mask = nullptr;
  float drop_p = 0.f;
  uint64_t seed = 0, offset = 0;
  // matrix-core forward only: attn_fwd_part_bytes() bytes for the partial
  // results of query tiles whose keys are split over two workgroups (null:
  // no split)
  float* fwd_part = nullptr;
};
size_t attn_dropout_mask_bytes(int batch, int seq, int n_local);
size_t attn_fwd_part_bytes(int dtype, int head_dim, int batch, int seq, int n_local);
bool attn_mfma_supported(int dtype, int head_dim);
hipError_t attn_fwd_launch(int dtype, const AttnDesc& a, hipStream_t stream);
hipError_t attn_bwd_launch(int dtype, const AttnDesc& a, hipStream_t stream);

// out[n] = sum_m X[m*ld + n] for n < N (fp32 accumulation, fixed order).
size_t colsum_workspace_bytes(int M, int N);
hipError_t colsum_launch(int dtype, const void* X, int M, int N, long ld, void* out, float* ws,
                         hipStream_t stream);
// The same for two matrices with the same row count M (out1 from X1, out2
// from X2), each pass one launch for both; out2 null: X1 alone.
size_t colsum_pair_workspace_bytes(int M, int N1, int N2);
hipError_t colsum_pair_launch(int dtype, int M, const void* X1, int N1, long ld1, void* out1, const void* X2, int N2,
                              long ld2, void* out2, float* ws, hipStream_t stream);

// bf16 XT[c*ldt + r] = X[r*ldx + c] (r < R, c < C; the 8-row group holding
// row R-1 is written whole, zeros past R, so ldt must be a multiple of 8 and
// >= R), and, when part is not null, part[b*C + c] = sum of X[r][c] over the
// b-th run of 32 rows (fixed order) for b < transpose_part_rows(R). Needs C % 8 == 0,
// ldx % 8 == 0, 16-byte aligned X and XT.
int transpose_part_rows(int R);
hipError_t transpose_colsum_launch(const void* X, int R, int C, long ldx, void* XT, long ldt, float* part,
                                   hipStream_t stream);
// out[n] = sum over r < R of part[r*N + n], added in the order r = 0, 1, ...
hipError_t colsum_final_launch(int dtype, const float* part, int R, int N, void* out, hipStream_t stream);

// out[i] = sum_k parts[k][i] + bias[i % cols] over count elements.
hipError_t sum_partials_launch(int dtype, const void* const* parts, int n_parts, const void* bias,
                               void* out, long long count, int cols, hipStream_t stream);

// Residual add + LayerNorm around a tensor-parallel block (token rows of h
// elements; h a multiple of 8, at most kLnMaxHidden).
constexpr int kLnMaxHidden = 24576;
struct LnDesc {
  long long T = 0;  // rows
  int h = 0;
  float eps = 0.f;
  // forward: resid_out = resid_in + sum_k parts[k] + bias; y = LayerNorm(resid_out)
  const void* resid_in = nullptr;
  const void* const* parts = nullptr;  // host array of n_parts (<= 64) device pointers
  int n_parts = 0;
  const void* bias = nullptr;  // [h] or NULL
  const void* gamma = nullptr;
  const void* beta = nullptr;
  void* resid_out = nullptr;  // also the backward's input r
  void* y = nullptr;
  float* mean = nullptr;  // [T]
  float* rstd = nullptr;  // [T]
  // backward
  const void* dy = nullptr;
  const void* dr_in = nullptr;  // [T,h] or NULL
  void* dr = nullptr;
  void* dgamma = nullptr;
  void* dbeta = nullptr;
  void* dbias = nullptr;  // [h] or NULL
  // dropout on the block output before the residual add (enabled by mask):
  // keep bits [T][h/8] (bit e of byte c: element 8c + e); the backward also
  // writes d_block = dr * keep * scale and forms dbias from it
  uint8_t* mask = nullptr;
  void* d_block = nullptr;
  float drop_p = 0.f;
  uint64_t seed = 0, offset = 0;
};
size_t ln_bwd_workspace_bytes(long long rows, int h);
hipError_t ln_fwd_launch(int dtype, const LnDesc& d, hipStream_t stream);
hipError_t ln_bwd_launch(int dtype, const LnDesc& d, void* ws, hipStream_t stream);

// Vocabulary-parallel cross-entropy of one rank's slice [v0, v0 + n) of the
// vocabulary (n a multiple of 8, at most kCeMaxSlice).
constexpr int kCeMaxSlice = 32768;
struct CeDesc {
  long long T = 0;  // tokens
  int n = 0, v0 = 0;
  const void* logits = nullptr;  // [T, n]
  const int* labels = nullptr;   // [T] global token ids
  float* stats = nullptr;        // [3][T]: m, s, z (ce_stats)
  const float* lse = nullptr;    // [T] (ce_dlogits)
  const float* dloss = nullptr;  // [T]
};
hipError_t ce_stats_launch(int dtype, const CeDesc& d, hipStream_t stream);
hipError_t ce_combine_launch(const float* const* stats, int n_parts, long long rows, float* loss, float* lse,
                             hipStream_t stream);
hipError_t ce_dlogits_launch(int dtype, const CeDesc& d, void* dl, hipStream_t stream);

// Fill rows x cols (leading dimension ld) of dtype elements with zero.
hipError_t zero_launch(int dtype, void* p, long long rows, long long cols, long long ld,
                       hipStream_t stream);

}  // namespace tpk
