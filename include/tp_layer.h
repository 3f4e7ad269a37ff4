/*
 * tp_layer.h -- C ABI of one tensor-parallel rank's share of a Megatron-style
 * Transformer layer (MLP block + causal self-attention block), forward and
 * backward, for AMD Instinct MI355X (gfx950).
 *
 * The operations follow the tensor-parallel split of the Megatron-LM deep dive
 * (charles2530.github.io): "MLP: column parallel then row parallel" (Fig. 3a),
 * "Attention: split Q/K/V by head" (Fig. 3b) and the f / g operators (Fig. 4);
 * and the MT-NLG 530B deep dive (zzszmyf.github.io), section 2.4 (column and
 * row parallel linear layers).
 *
 * The caller passes ONE rank's shards; the library computes that rank's share
 * and never communicates. The g all-reduce of the forward pass and the f
 * all-reduce of the backward pass are left to the caller; on one device they
 * are emulated with tp_sum_partials over the ranks' partial outputs.
 *
 * Conventions (all calls):
 *   - Notation per rank r of p = tp_size: T = batch*seq tokens (row t =
 *     batch_index*seq + position), h = hidden, h_l = h/p, n_l = n_heads/p local
 *     heads of width d = head_dim, f_l = ffn/p.
 *   - Every matrix is row-major and contiguous. Every pointer is a device
 *     pointer, 16-byte aligned, except the tp_shape pointer (host memory) and
 *     tp_sum_partials' array of part pointers (a host array of device pointers).
 *   - Tensors are stored in shape->dtype (fp32 or bf16); products accumulate in
 *     fp32. lse is always fp32. bf16 results are rounded to nearest even once.
 *   - The caller allocates and owns every buffer, including the workspace
 *     (size from tp_*_workspace_bytes). The library never allocates, frees or
 *     synchronizes: work is enqueued on `stream` (a hipStream_t; NULL = the
 *     null stream) and the call returns.
 *   - Outputs (weight gradients included) are overwritten, never accumulated.
 *     Outputs must not alias inputs or each other.
 *   - Error behaviour: a non-zero return means nothing was enqueued, except
 *     TP_ERR_HIP (a launch failed part way; the outputs are undefined). The
 *     message is available from tp_last_error() on the calling thread.
 *     Device-side faults surface at the caller's next synchronization.
 *     No C++ exception crosses this interface.
 *   - Empty batches (batch == 0 or seq == 0) are valid: token-shaped outputs
 *     are empty and weight / bias gradients are written as zeros.
 */
#ifndef TP_LAYER_H
#define TP_LAYER_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TP_OK = 0,
  TP_ERR_NULL = -1,         /* a required pointer is NULL                       */
  TP_ERR_SHAPE = -2,        /* negative size, or a size limit exceeded          */
  TP_ERR_DIVISIBILITY = -3, /* n_heads or ffn not divisible by tp_size, or
                               n_heads*head_dim != hidden                       */
  TP_ERR_RANK = -4,         /* tp_rank outside [0, tp_size) or tp_size < 1      */
  TP_ERR_DTYPE = -5,        /* dtype not TP_FP32 / TP_BF16                      */
  TP_ERR_HEADDIM = -6,      /* head_dim outside the supported set               */
  TP_ERR_WORKSPACE = -7,    /* workspace NULL or smaller than required          */
  TP_ERR_ALIGN = -8,        /* pointer not 16-byte aligned, or (bf16) a weight
                               dimension not a multiple of 8                    */
  TP_ERR_HIP = -9           /* a HIP launch or query failed                     */
} tp_status;

typedef enum { TP_FP32 = 0, TP_BF16 = 1 } tp_dtype;

/* Full (unsharded) layer sizes plus the pages' (rank, degree) pair. */
typedef struct {
  int32_t batch, seq, hidden, ffn, n_heads, head_dim;
  int32_t tp_rank, tp_size; /* 0 <= tp_rank < tp_size                           */
  int32_t dtype;            /* tp_dtype: storage type; accumulation is fp32     */
  int32_t causal;           /* must be 1: left-to-right (autoregressive) mask,
                               key j attends to query i iff j <= i              */
  int32_t alibi;            /* 0/1: add -m_k*(i-j) to the scaled score of global
                               head k (1-based), m_k = 2^(-8k/n_heads)
                               (Megatron-DeepSpeed blog, section 4.3)           */
} tp_shape;

/* Supported sizes (else TP_ERR_SHAPE / TP_ERR_HEADDIM / TP_ERR_ALIGN):
 * head_dim a multiple of 8 in [8, 256]; batch <= 65535, seq <= 65536,
 * batch*seq < 2^22, hidden and ffn <= 2^22; every tensor (X, pre_i, qkv_i,
 * A_i, Wqkv_i, ...) below 2^30 elements; bf16 also needs hidden, ffn/p and
 * hidden/p to be multiples of 8. */

/* Workspace bytes the calls below need for this shape (0 on an invalid shape).
 * Host-only; no HIP call. */
size_t tp_mlp_workspace_bytes(const tp_shape* shape);
size_t tp_attn_workspace_bytes(const tp_shape* shape);

/* MLP forward (Megatron-LM deep dive, Fig. 3a; Megatron-DeepSpeed blog 2.1):
 *   pre_i = X A_i + b1_i         X [T,h] (replicated input), A_i [h,f_l]
 *                                (column shard), b1_i [f_l]
 *   y_i   = GeLU(pre_i)          tanh form: 0.5 x (1 + tanh(sqrt(2/pi)(x + 0.044715 x^3)))
 *   Z_i   = y_i B_i              B_i [f_l,h] (row shard); Z_i [T,h] is this
 *                                rank's PARTIAL sum; b2 is not added (the caller
 *                                adds it once after the sum over ranks).
 * Outputs pre_i, y_i [T,f_l] are saved for the backward pass. */
tp_status tp_mlp_fwd(const tp_shape* shape, const void* X, const void* A_i, const void* b1_i,
                     const void* B_i, void* pre_i, void* y_i, void* Z_i, void* workspace,
                     size_t workspace_bytes, void* stream);

/* MLP backward (Megatron-LM deep dive, Fig. 3a for the column / row split
 * and Fig. 4 for the conjugate operators: g's backward passes dZ through
 * unchanged, f's backward sums the ranks' input gradients): gradients of
 * <Z_i + b2, dZ> with dZ [T,h] replicated:
 *   dPre = (dZ B_i^T) * GeLU'(pre_i)
 *   dB_i = y_i^T dZ [f_l,h];  dA_i = X^T dPre [h,f_l];  db1_i = sum_t dPre [f_l]
 *   dX_i = dPre A_i^T [T,h]   this rank's PARTIAL input gradient (f's backward
 *                             sums it over ranks)
 *   db2  = sum_t dZ [h]       replicated bias; written only if db2_or_null != NULL */
tp_status tp_mlp_bwd(const tp_shape* shape, const void* X, const void* A_i, const void* B_i,
                     const void* pre_i, const void* y_i, const void* dZ, void* dX_i, void* dA_i,
                     void* db1_i, void* dB_i, void* db2_or_null, void* workspace,
                     size_t workspace_bytes, void* stream);

/* Attention forward (Megatron-LM deep dive, Fig. 3b):
 *   qkv_i = X Wqkv_i + bqkv_i    (saved in the form described below)
 *                                Wqkv_i [h,3h_l] = [Wq_i | Wk_i | Wv_i] (the
 *                                columns of this rank's heads), bqkv_i [3h_l];
 *                                local head l uses columns l*d..l*d+d-1 of each
 *                                third; rank r owns global heads r*n_l..r*n_l+n_l-1
 *   per batch element and local head: S = q k^T / sqrt(d) (+ ALiBi), causal
 *   mask, row softmax, ctx = softmax(S) v; lse = log-sum-exp of each row of S
 *   O_i = ctx_i Wo_i             Wo_i [h_l,h] (row shard); O_i [T,h] is this
 *                                rank's PARTIAL sum; bo is not added.
 * Saved for backward: qkv_i (tp_attn_qkv_bytes bytes), ctx_i [T,h_l] (heads
 * side by side), lse_i [batch, n_l, seq] fp32. The projection is saved at
 * more than storage precision, because the scores q.k/sqrt(d) can be large and
 * nearly tied (rows sharper than bf16 can resolve):
 *   - dtype TP_BF16 with head_dim 64, 96, 128 or 160 (the matrix-core path):
 *     five 16-bit planes [T,h_l] (x = the fp32 projection, rounded to
 *     nearest), plane k at byte offset 2*k*T*h_l: 0 fp16(q log2(e)/sqrt(d)),
 *     1 bf16(q), 2 fp16(k), 3 bf16(k), 4 bf16(v), where q, k, v are the three
 *     thirds of qkv_i; the scores are one matrix-core product of the fp16
 *     planes (11-bit significands; fp16 values saturate at +-65504), the
 *     bf16 planes feed the gradient and value products;
 *   - otherwise [T,3h_l] fp32.
 * The backward reads the buffer as the forward wrote it. */
size_t tp_attn_qkv_bytes(const tp_shape* shape);
tp_status tp_attn_fwd(const tp_shape* shape, const void* X, const void* Wqkv_i, const void* bqkv_i,
                      const void* Wo_i, void* qkv_i, void* ctx_i, float* lse_i, void* O_i,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Attention backward (Megatron-LM deep dive, Fig. 3b for the per-head split
 * and Fig. 4 for f and g in the backward pass: dO reaches every rank whole,
 * and the ranks' partial input gradients are summed by f's backward):
 * gradients of <O_i + bo, dO>, dO [T,h] replicated.
 *   dC = dO Wo_i^T;  dWo_i = ctx_i^T dO [h_l,h]
 *   per head: dV = P^T dC, dP = dC V^T, dS = P*(dP - rowsum(dC*ctx)),
 *             dQ = dS K / sqrt(d), dK = dS^T Q / sqrt(d)   (P recomputed from lse)
 *   dWqkv_i = X^T dqkv [h,3h_l];  dbqkv_i = sum_t dqkv [3h_l]
 *   dX_i = dqkv Wqkv_i^T [T,h]   PARTIAL input gradient
 *   dbo = sum_t dO [h]           replicated bias; written only if dbo_or_null != NULL */
tp_status tp_attn_bwd(const tp_shape* shape, const void* X, const void* Wqkv_i, const void* Wo_i,
                      const void* qkv_i, const void* ctx_i, const float* lse_i, const void* dO,
                      void* dX_i, void* dWqkv_i, void* dbqkv_i, void* dWo_i, void* dbo_or_null,
                      void* workspace, size_t workspace_bytes, void* stream);

/* Attention-probability dropout (Megatron-LM deep dive: dropout 0.1 in the
 * training setup; inside the model-parallel region each rank draws independent
 * random numbers). The variants below apply it inside the flash-style kernels
 * (bf16 matrix-core path only: shape->dtype TP_BF16 and head_dim 64, 96, 128
 * or 160, else TP_ERR_DTYPE / TP_ERR_HEADDIM):
 *   ctx = (softmax(S) * keep * scale) v,  lse as without dropout,
 * with keep drawn by Philox4x64-10 (Salmon et al., SC 2011) for element
 * (batch b, global head k, query i, key j) at counter
 * (i, j / 32, b * 2^32 + k, ((j % 32) / 4) % 2) with key (seed, offset): its
 * 16-bit lane 4 ((j % 32) / 8) + j % 4 is kept iff >= thr = round(65536 p),
 * scale = 65536 / (65536 - thr). Ranks own different global heads, so one
 * seed gives each rank independent numbers. The forward stores the keep bits
 * in mask_i (tp_attn_dropout_mask_bytes bytes, device memory, 16-byte
 * aligned; layout [batch][n_l][ceil(seq/32)][2][seq rounded up to 8] of
 * 16-bit words); the backward reads them (pass the same p). p = 0 gives the
 * results of tp_attn_fwd / tp_attn_bwd. p must keep thr below 65536 (at
 * least one 16-bit value kept, a finite scale): p outside [0, 1 - 2^-17) is
 * TP_ERR_SHAPE. */
typedef struct {
  float p;          /* drop probability, 0 <= p < 1 - 2^-17 */
  uint64_t seed;    /* Philox key word 0 */
  uint64_t offset;  /* Philox key word 1 (e.g. a step or layer counter) */
} tp_dropout;

size_t tp_attn_dropout_mask_bytes(const tp_shape* shape);
tp_status tp_attn_fwd_dropout(const tp_shape* shape, const tp_dropout* dropout, const void* X,
                              const void* Wqkv_i, const void* bqkv_i, const void* Wo_i, void* qkv_i,
                              void* ctx_i, float* lse_i, uint16_t* mask_i, void* O_i, void* workspace,
                              size_t workspace_bytes, void* stream);
tp_status tp_attn_bwd_dropout(const tp_shape* shape, const tp_dropout* dropout, const void* X,
                              const void* Wqkv_i, const void* Wo_i, const void* qkv_i,
                              const void* ctx_i, const float* lse_i, const uint16_t* mask_i,
                              const void* dO, void* dX_i, void* dWqkv_i, void* dbqkv_i, void* dWo_i,
                              void* dbo_or_null, void* workspace, size_t workspace_bytes, void* stream);

/* The f / g all-reduce emulated on one device (Megatron-LM deep dive, Fig. 4):
 *   out [T,h] = sum_{k < n_parts} parts[k] + bias   (fp32 accumulation, rounded
 * once). parts is a HOST array of n_parts (1..64) device pointers to [T,h]
 * tensors in shape->dtype; bias_or_null [h] may be NULL. out may alias parts[0]. */
tp_status tp_sum_partials(const tp_shape* shape, const void* const* parts, int32_t n_parts,
                          const void* bias_or_null, void* out, void* stream);

/* Residual add + LayerNorm after a block (Megatron-LM deep dive, Fig. 2: the
 * layer's residual connections and layer normalizations around the attention
 * and MLP blocks; Fig. 4: g completes the block output before the residual
 * add; Megatron-DeepSpeed blog, section 4.3: the residual add fused into the
 * LayerNorm kernel). Per token row t of h = hidden elements:
 *   resid_out = resid_in + sum_{k < n_parts} parts[k] + bias   (the new
 *               residual stream; with the ranks' partial block outputs as
 *               parts this is also g's sum, emulated on one device)
 *   mean, rstd: mean and 1/sqrt(biased variance + eps) of the row of
 *               resid_out as stored (fp32 [T] each, saved for the backward)
 *   ln_out    = (resid_out - mean) * rstd * gamma + beta   (the next block's input)
 * resid_in, parts[k], resid_out, ln_out [T,h]; bias_or_null, gamma, beta [h]
 * in shape->dtype (only batch, seq, hidden and dtype of shape are used, the
 * rest is validated as for every call). parts is a HOST array of n_parts
 * (0..64) device pointers (may be NULL when n_parts = 0). eps > 0 (the pages
 * give no value). Needs hidden % 8 == 0 (else TP_ERR_ALIGN) and hidden <=
 * 24576 (else TP_ERR_SHAPE). Outputs must not alias inputs. */
tp_status tp_ln_residual_fwd(const tp_shape* shape, const void* resid_in, const void* const* parts,
                             int32_t n_parts, const void* bias_or_null, const void* gamma,
                             const void* beta, float eps, void* resid_out, void* ln_out, float* mean,
                             float* rstd, void* stream);

/* Workspace bytes of tp_ln_residual_bwd (0 when none is needed, i.e. an empty
 * batch, or on an invalid shape). Host-only; no HIP call. */
size_t tp_ln_workspace_bytes(const tp_shape* shape);

/* Backward of tp_ln_residual_fwd: gradients of <ln_out, d_ln_out> +
 * <resid_out, d_resid_out> (d_resid_out_or_null: the gradient reaching
 * resid_out along the residual stream from later in the network; NULL = 0),
 * from the saved resid_out, mean, rstd:
 *   xhat = (resid_out - mean) * rstd,  g = d_ln_out * gamma
 *   d_resid = d_resid_out + rstd * (g - mean_j g - xhat * mean_j (g * xhat))   [T,h]
 *             (the gradient of resid_in, of every part and of the block output)
 *   dgamma = sum_t d_ln_out * xhat,  dbeta = sum_t d_ln_out   [h]
 *   dbias  = sum_t d_resid [h], written only if dbias_or_null != NULL
 * Column sums are formed from fixed-order fp32 partials (deterministic). */
tp_status tp_ln_residual_bwd(const tp_shape* shape, const void* resid_out, const float* mean,
                             const float* rstd, const void* gamma, const void* d_ln_out,
                             const void* d_resid_out_or_null, void* d_resid, void* dgamma,
                             void* dbeta, void* dbias_or_null, void* workspace,
                             size_t workspace_bytes, void* stream);

/* tp_ln_residual_bwd without a workspace argument, for callers that cannot
 * allocate device memory (code under stream capture, tight serving loops,
 * harnesses that forbid allocation). Same arguments, results and errors as
 * tp_ln_residual_bwd (bit-identical outputs), but the fp32 run partials live
 * in a scratch array of tp_ln_residual_bwd_noalloc_max_scratch_bytes() bytes
 * (48 MiB) that the library holds on each device it runs on until the
 * process ends; the call itself allocates nothing. A shape whose
 * tp_ln_workspace_bytes exceeds that size is TP_ERR_SHAPE (e.g. hidden 24576
 * with 256 or more rows; hidden 20480 fits). Every call on a device shares
 * that device's array: calls that overlap on one device (several streams or
 * threads) race and give undefined results; calls ordered on one stream are
 * safe. The first call on a device looks up the array's address
 * (hipGetSymbolAddress) and keeps it. */
size_t tp_ln_residual_bwd_noalloc_max_scratch_bytes(void);
tp_status tp_ln_residual_bwd_noalloc(const tp_shape* shape, const void* resid_out, const float* mean,
                                     const float* rstd, const void* gamma, const void* d_ln_out,
                                     const void* d_resid_out_or_null, void* d_resid, void* dgamma,
                                     void* dbeta, void* dbias_or_null, void* stream);

/* Vocabulary-parallel logits + cross-entropy of the output layer
 * (Megatron-LM deep dive, vocabulary-parallel loss fusion section: the
 * embedding table is split along the vocabulary, each rank computes the
 * logits of its slice, and the loss exchanges per-token aggregates instead
 * of the logits; the training-recipe table pads the GPT-2 vocabulary to
 * 51,200 so that it splits evenly). V = vocab (padded), n = V / tp_size,
 * rank r owns token ids [v0, v0 + n), v0 = r n. W_i [n, h] is rows v0.. of
 * the [V, h] table (tied to the input embedding; no bias). labels [T] int32
 * global token ids; a label outside [0, V) is owned by no rank (its loss is
 * the log-sum-exp). Needs V % tp_size == 0 (else TP_ERR_DIVISIBILITY), n a
 * multiple of 8 (else TP_ERR_ALIGN) and n <= 32768 (else TP_ERR_SHAPE); of
 * shape, batch, seq, hidden, tp_rank, tp_size and dtype are used (the rest is
 * validated as for every call). Workspace: tp_vocab_workspace_bytes.
 *
 * Forward, per rank:
 *   logits_i = X W_i^T   [T, n] (shape->dtype)    X [T, h]: final hidden states
 *   stats_i  [3][T] fp32: m = max_j logits_i[t, j], s = sum_j exp(logits_i - m),
 *            z = logits_i[t, label_t - v0] if the label is in the slice, else 0 */
size_t tp_vocab_workspace_bytes(const tp_shape* shape, int32_t vocab);
tp_status tp_vocab_ce_fwd(const tp_shape* shape, int32_t vocab, const void* X, const void* W_i,
                          const int32_t* labels, void* logits_i, float* stats_i, void* workspace,
                          size_t workspace_bytes, void* stream);

/* The exchange of the per-token aggregates, emulated on one device over the
 * ranks' stats (a HOST array of n_parts (1..64) device pointers to [3][T]
 * fp32): m = max_k m_k, S = sum_k s_k exp(m_k - m), z = sum_k z_k;
 * lse [T] = m + log S; loss [T] = lse - z (fp32, per token). */
tp_status tp_vocab_ce_combine(const tp_shape* shape, const float* const* stats, int32_t n_parts,
                              float* loss, float* lse, void* stream);

/* Backward for the loss sum_t dloss_t loss_t (dloss [T] fp32; 1/T for a mean):
 *   dlogits = (exp(logits_i - lse) - onehot(label - v0)) * dloss   (workspace)
 *   dX_i = dlogits W_i [T, h]   this rank's PARTIAL input gradient (f sums it)
 *   dW_i = dlogits^T X [n, h] */
tp_status tp_vocab_ce_bwd(const tp_shape* shape, int32_t vocab, const void* X, const void* W_i,
                          const int32_t* labels, const void* logits_i, const float* lse,
                          const float* dloss, void* dX_i, void* dW_i, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Residual add + LayerNorm with dropout on the block output (Megatron-LM deep
 * dive: dropout before the residual add lies outside the model-parallel
 * region and must be identical on the ranks of a model replica):
 *   resid_out = resid_in + keep * scale * (sum_k parts[k] + bias), then as in
 *   tp_ln_residual_fwd; element (t, j) is kept iff 16-bit lane j % 16 of the
 *   Philox4x64-10 block at counter (t, j / 16, 0, 2) with key (seed, offset)
 *   is >= thr = round(65536 p); scale = 65536 / (65536 - thr). No rank enters
 *   the counter, so every rank draws the same mask from the same (seed,
 *   offset). mask [T][hidden/8] bytes (bit e of byte c: element 8c + e,
 *   tp_ln_dropout_mask_bytes bytes) receives the keep bits. p outside
 *   [0, 1 - 2^-17) is TP_ERR_SHAPE; other arguments as in tp_ln_residual_fwd. */
size_t tp_ln_dropout_mask_bytes(const tp_shape* shape);
tp_status tp_ln_residual_fwd_dropout(const tp_shape* shape, const tp_dropout* dropout,
                                     const void* resid_in, const void* const* parts, int32_t n_parts,
                                     const void* bias_or_null, const void* gamma, const void* beta,
                                     float eps, void* resid_out, void* ln_out, float* mean, float* rstd,
                                     uint8_t* mask, void* stream);

/* Backward of tp_ln_residual_fwd_dropout: d_resid as in tp_ln_residual_bwd
 * (the gradient of resid_in), and d_block [T,h] = d_resid * keep * scale, the
 * gradient of the block output, of every part and (summed over tokens, into
 * dbias_or_null) of the bias. mask as written by the forward. */
tp_status tp_ln_residual_bwd_dropout(const tp_shape* shape, const tp_dropout* dropout,
                                     const void* resid_out, const float* mean, const float* rstd,
                                     const void* gamma, const void* d_ln_out,
                                     const void* d_resid_out_or_null, const uint8_t* mask,
                                     void* d_resid, void* d_block, void* dgamma, void* dbeta,
                                     void* dbias_or_null, void* workspace, size_t workspace_bytes,
                                     void* stream);

/* Steps of the path, for per-step timing. The id doubles as the bit position
 * in tp_profile_enable's mask. */
enum {
  TP_STEP_QKV_PROJ = 1,   /* qkv_i = X Wqkv_i + bqkv_i                       */
  TP_STEP_ATTN_FWD = 2,   /* per-head causal attention, forward              */
  TP_STEP_OUT_PROJ = 3,   /* O_i = ctx_i Wo_i                                */
  TP_STEP_FC1 = 4,        /* pre_i = X A_i + b1_i, y_i = GeLU(pre_i)         */
  TP_STEP_FC2 = 5,        /* Z_i = y_i B_i                                   */
  TP_STEP_FC2_DGRAD = 6,  /* dPre = (dZ B_i^T) * GeLU'(pre_i)                */
  TP_STEP_FC2_WGRAD = 7,  /* dB_i = y_i^T dZ                                 */
  TP_STEP_FC1_WGRAD = 8,  /* dA_i = X^T dPre                                 */
  TP_STEP_FC1_DGRAD = 9,  /* dX_i = dPre A_i^T                               */
  TP_STEP_OUT_DGRAD = 10, /* dC = dO Wo_i^T                                  */
  TP_STEP_OUT_WGRAD = 11, /* dWo_i = ctx_i^T dO                              */
  TP_STEP_ATTN_BWD = 12,  /* per-head causal attention, backward             */
  TP_STEP_QKV_WGRAD = 13, /* dWqkv_i = X^T dqkv                              */
  TP_STEP_QKV_DGRAD = 14, /* dX_i = dqkv Wqkv_i^T                            */
  TP_STEP_BIAS_GRADS = 15, /* column sums db1_i, db2, dbo, dbqkv_i           */
  TP_STEP_LN_FWD = 16,     /* residual add + LayerNorm, forward              */
  TP_STEP_LN_BWD = 17,     /* residual add + LayerNorm, backward             */
  TP_STEP_LOGITS = 18,     /* logits_i = X W_i^T                             */
  TP_STEP_CE_STATS = 19,   /* per-token aggregates of the vocabulary slice   */
  TP_STEP_CE_COMBINE = 20, /* exchange of the aggregates (emulated)          */
  TP_STEP_CE_DLOGITS = 21, /* dlogits = (softmax - onehot) dloss             */
  TP_STEP_LOGITS_DGRAD = 22, /* dX_i = dlogits W_i                           */
  TP_STEP_LOGITS_WGRAD = 23, /* dW_i = dlogits^T X                           */
  TP_STEP_TRANSPOSE = 24     /* bf16 backward: token-contiguous copies y_i^T,
                                dPre^T, ctx_i^T, dqkv^T read by the weight
                                gradients (the dPre^T and dqkv^T copies also
                                form db1_i's and dbqkv_i's column partials) */
};

/* Measurement aid (no passage of the pages; for benchmarks). This timing
 * state -- the step mask, the recorded events and the event pool, guarded by
 * one mutex -- is the library's only process-global state besides the
 * thread-local error message and a per-device cache of the compute-unit
 * count (read once, used to plan launches); the compute calls above keep no
 * data between calls. While bit k of
 * step_mask is set, every launch sequence of step k is bracketed by a pair of
 * hipEvents recorded on the caller's stream (the events are created on first
 * use and pooled). tp_profile_enable discards what was recorded and sets the
 * mask (0 turns timing off). tp_profile_collect waits for the recorded events
 * of one step, returns how many launch sequences were recorded and their total
 * GPU time in ms, and forgets them. Not for use under stream capture. */
tp_status tp_profile_enable(uint32_t step_mask);
tp_status tp_profile_collect(int32_t step, int32_t* launches, double* total_ms);

/* Measurement aid (no passage of the pages; for traces and roofline
 * records): the name of the main kernel that the GEMM step `step` (a
 * TP_STEP_* id of a product: QKV_PROJ, OUT_PROJ, FC1, FC2, the input and
 * weight gradients) launches for this shape on the current device, as a
 * kernel trace shows it (e.g. "gemm_fc1_bias_gelu"); a k-split or stream-K
 * plan adds the kernel of that name with the suffix "_fixup". The choice
 * depends on the shape and the device's compute-unit count only. Returns NULL
 * for an invalid shape, a step that is not a product, or an empty product
 * (no launch). The string is static; the call touches no device memory. */
const char* tp_step_kernel(const tp_shape* shape, int32_t step);

/* Message for the last non-OK status returned on the calling thread ("" if none). */
const char* tp_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* TP_LAYER_H */
