// C ABI of the tensor-parallel layer shard: argument validation, workspace
// planning and the launch sequence of each operation on the caller's stream.
// See include/tp_layer.h for the contract of every entry point.
#include "../../include/tp_layer.h"

#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "kernels.h"

using namespace tpk;

namespace {

thread_local std::string g_last_error;

tp_status fail(tp_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

tp_status hip_fail(hipError_t e, const char* where) {
  return fail(TP_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

// ---- per-step timing (tp_profile_enable / tp_profile_collect) -----------------
// While a step's bit is set, every launch sequence of that step is bracketed by
// a pair of hipEvents recorded on the caller's stream. Event pairs are pooled
// per device and reused after collection.
struct EvPair {
  hipEvent_t a, b;
  int dev;
};
struct Rec {
  int step;
  EvPair ev;
};
std::mutex g_prof_mu;
uint32_t g_prof_mask = 0;
std::vector<Rec> g_prof_recs;
std::vector<EvPair> g_prof_pool;

class StepTimer {
 public:
  StepTimer(int step, hipStream_t st) : step_(step), st_(st) {
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (!(g_prof_mask & (1u << step))) return;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return;
    for (size_t i = 0; i < g_prof_pool.size(); ++i)
      if (g_prof_pool[i].dev == dev) {
        ev_ = g_prof_pool[i];
        g_prof_pool.erase(g_prof_pool.begin() + i);
        active_ = true;
        break;
      }
    if (!active_) {
      if (hipEventCreate(&ev_.a) != hipSuccess) return;
      if (hipEventCreate(&ev_.b) != hipSuccess) { (void)hipEventDestroy(ev_.a); return; }
      ev_.dev = dev;
      active_ = true;
    }
    if (hipEventRecord(ev_.a, st_) != hipSuccess) {
      g_prof_pool.push_back(ev_);
      active_ = false;
    }
  }
  ~StepTimer() {
    if (!active_) return;
    std::lock_guard<std::mutex> lk(g_prof_mu);
    if (hipEventRecord(ev_.b, st_) == hipSuccess) g_prof_recs.push_back(Rec{step_, ev_});
    else g_prof_pool.push_back(ev_);
  }

 private:
  int step_;
  hipStream_t st_;
  EvPair ev_{};
  bool active_ = false;
};

constexpr long long kMaxElems = 1LL << 30;  // per tensor (32-bit byte offsets)
constexpr int kMaxDim = 1 << 22;

struct Dims {
  long long T, h, hl, fl, nl, d;
  long long batch, seq;
  int dtype;
  size_t esz;
};

tp_status check_shape(const tp_shape* s, Dims& dm) {
  if (!s) return fail(TP_ERR_NULL, "shape is NULL");
  if (s->tp_size < 1 || s->tp_rank < 0 || s->tp_rank >= s->tp_size)
    return fail(TP_ERR_RANK, "tp_rank %d outside [0, tp_size=%d)", s->tp_rank, s->tp_size);
  if (s->dtype != TP_FP32 && s->dtype != TP_BF16) return fail(TP_ERR_DTYPE, "dtype %d is not TP_FP32/TP_BF16", s->dtype);
  if (s->batch < 0 || s->seq < 0 || s->hidden <= 0 || s->ffn <= 0 || s->n_heads <= 0 || s->head_dim <= 0)
    return fail(TP_ERR_SHAPE, "sizes must be positive (batch, seq may be 0)");
  if (s->batch > 65535 || s->seq > 65536 || s->hidden > kMaxDim || s->ffn > kMaxDim)
    return fail(TP_ERR_SHAPE, "size limit exceeded (batch <= 65535, seq <= 65536, hidden/ffn <= 2^22)");
  if (s->causal != 1) return fail(TP_ERR_SHAPE, "only the causal (left-to-right) mask is supported");
  if (s->alibi != 0 && s->alibi != 1) return fail(TP_ERR_SHAPE, "alibi must be 0 or 1");
  if (s->n_heads % s->tp_size != 0) return fail(TP_ERR_DIVISIBILITY, "n_heads %d not divisible by tp_size %d", s->n_heads, s->tp_size);
  if (s->ffn % s->tp_size != 0) return fail(TP_ERR_DIVISIBILITY, "ffn %d not divisible by tp_size %d", s->ffn, s->tp_size);
  if ((long long)s->n_heads * s->head_dim != s->hidden)
    return fail(TP_ERR_DIVISIBILITY, "n_heads*head_dim = %lld != hidden %d", (long long)s->n_heads * s->head_dim, s->hidden);
  if (s->head_dim < 8 || s->head_dim > 256 || s->head_dim % 8 != 0)
    return fail(TP_ERR_HEADDIM, "head_dim %d not a multiple of 8 in [8, 256]", s->head_dim);
  dm.T = (long long)s->batch * s->seq;
  dm.batch = s->batch;
  dm.seq = s->seq;
  dm.h = s->hidden;
  dm.nl = s->n_heads / s->tp_size;
  dm.d = s->head_dim;
  dm.hl = dm.nl * dm.d;
  dm.fl = s->ffn / s->tp_size;
  dm.dtype = s->dtype;
  dm.esz = s->dtype == TP_BF16 ? 2 : 4;
  if (s->dtype == TP_BF16 && (dm.h % 8 || dm.fl % 8 || dm.hl % 8))
    return fail(TP_ERR_ALIGN, "bf16 needs hidden, ffn/tp and hidden/tp to be multiples of 8");
  const long long big[] = {dm.T * dm.h, dm.T * dm.fl, dm.T * 3 * dm.hl, dm.h * dm.fl, dm.h * 3 * dm.hl};
  for (long long v : big)
    if (v >= kMaxElems) return fail(TP_ERR_SHAPE, "a tensor of this shape has >= 2^30 elements");
  if (dm.T >= kMaxDim) return fail(TP_ERR_SHAPE, "batch*seq must be < 2^22");
  return TP_OK;
}

// Required pointer: non-NULL unless its tensor is empty; 16-byte aligned.
tp_status check_ptr(const void* p, const char* name, bool empty_ok) {
  if (!p) {
    if (empty_ok) return TP_OK;
    return fail(TP_ERR_NULL, "%s is NULL", name);
  }
  if (((uintptr_t)p) & 15u) return fail(TP_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return TP_OK;
}

#define TP_CHECK(expr)                 \
  do {                                 \
    tp_status _st = (expr);            \
    if (_st != TP_OK) return _st;      \
  } while (0)

#define TP_HIP(expr, where)                         \
  do {                                              \
    hipError_t _e = (expr);                         \
    if (_e != hipSuccess) return hip_fail(_e, where); \
  } while (0)

// TP_HIP for one step of the path, timed when profiling selects it.
#define TP_STEP(step, expr, where)                  \
  do {                                              \
    StepTimer _t((step), st);                       \
    hipError_t _e = (expr);                         \
    if (_e != hipSuccess) return hip_fail(_e, where); \
  } while (0)

// Bump allocation inside the caller's workspace (256-byte aligned pieces).
struct Bump {
  char* base;
  size_t off = 0;
  explicit Bump(void* b) : base((char*)b) {}
  void* take(size_t bytes) {
    off = (off + 255) & ~(size_t)255;
    void* p = base ? base + off : nullptr;
    off += bytes;
    return p;
  }
};

size_t max3(size_t a, size_t b, size_t c) { return a > b ? (a > c ? a : c) : (b > c ? b : c); }

// Row length of a transposed [*, T] copy: T rounded up to a multiple of 8
// (at least 8), so that every row starts 16-byte aligned.
long long t_ld(long long T) { return T < 8 ? 8 : (T + 7) / 8 * 8; }

// bf16 weight gradients of wide layers read one operand as a transposed copy
// (k = tokens contiguous). A weight gradient does h/2 flops per byte of its
// copied operand (M or N is h), and the copy moves each byte twice: below
// h = 8192 the copy costs more than the product gains (about 10%), and both
// operands are read as stored, as on the fp32 path.
constexpr long long kCopyMinHidden = 8192;
bool wgrad_copies(const Dims& dm) { return dm.dtype == DT_BF16 && dm.h >= kCopyMinHidden; }

struct MlpPlan {
  void *dpre, *gemm_ws, *col_ws;
  void *yT, *dpreT;  // [fl, t_ld(T)] transposed copies (bf16 backward)
  float* tpart;      // [transpose_part_rows(T), fl] column partials of dPre
  size_t gemm_bytes, col_bytes, total;
};

MlpPlan plan_mlp(const Dims& dm, void* ws, bool bwd) {
  Bump bp(ws);
  MlpPlan pl{};
  const int dt = dm.dtype;
  if (bwd) pl.dpre = bp.take((size_t)(dm.T * dm.fl) * dm.esz);
  if (bwd && wgrad_copies(dm) && dm.T > 0) {
    const size_t tbytes = (size_t)(dm.fl * t_ld(dm.T)) * dm.esz;
    pl.yT = bp.take(tbytes);
    pl.dpreT = bp.take(tbytes);
    pl.tpart = (float*)bp.take((size_t)transpose_part_rows((int)dm.T) * dm.fl * sizeof(float));
  }
  size_t g = gemm_workspace_bytes(dt, (int)dm.T, (int)dm.fl, (int)dm.h);
  g = max3(g, gemm_workspace_bytes(dt, (int)dm.T, (int)dm.h, (int)dm.fl), 0);
  if (bwd) {
    g = max3(g, gemm_workspace_bytes(dt, (int)dm.fl, (int)dm.h, (int)dm.T),
             gemm_workspace_bytes(dt, (int)dm.h, (int)dm.fl, (int)dm.T));
    pl.col_bytes = colsum_pair_workspace_bytes((int)dm.T, (int)dm.fl, (int)dm.h);
    pl.col_ws = bp.take(pl.col_bytes);
  }
  pl.gemm_bytes = g;
  pl.gemm_ws = bp.take(g);
  pl.total = bp.off;
  return pl;
}

struct AttnPlan {
  void *dctx, *dqkv, *delta, *gemm_ws, *col_ws;
  void* fwd_part;      // forward: partials of key-split query tiles
  void *ctxT, *dqkvT;  // [hl, t_ld(T)], [3hl, t_ld(T)] transposed copies (bf16 backward)
  float* tpart;        // [transpose_part_rows(T), 3hl] column partials of dqkv
  size_t gemm_bytes, col_bytes, total;
};

AttnPlan plan_attn(const Dims& dm, void* ws, bool bwd) {
  Bump bp(ws);
  AttnPlan pl{};
  const int dt = dm.dtype;
  const long long B = dm.T;
  if (!bwd) {
    const size_t fp = attn_fwd_part_bytes(dt, (int)dm.d, (int)dm.batch, (int)dm.seq, (int)dm.nl);
    pl.fwd_part = fp ? bp.take(fp) : nullptr;
  }
  size_t g = max3(gemm_workspace_bytes(dt, (int)B, (int)(3 * dm.hl), (int)dm.h),
                  gemm_workspace_bytes(dt, (int)B, (int)dm.h, (int)dm.hl), 0);
  if (bwd) {
    pl.dctx = bp.take((size_t)(dm.T * dm.hl) * dm.esz);
    pl.dqkv = bp.take((size_t)(dm.T * 3 * dm.hl) * dm.esz);
    pl.delta = bp.take((size_t)(dm.T * dm.nl) * sizeof(float));
    if (wgrad_copies(dm) && dm.T > 0) {
      pl.ctxT = bp.take((size_t)(dm.hl * t_ld(dm.T)) * dm.esz);
      pl.dqkvT = bp.take((size_t)(3 * dm.hl * t_ld(dm.T)) * dm.esz);
      pl.tpart = (float*)bp.take((size_t)transpose_part_rows((int)dm.T) * 3 * dm.hl * sizeof(float));
    }
    g = max3(g, gemm_workspace_bytes(dt, (int)B, (int)dm.hl, (int)dm.h),
             gemm_workspace_bytes(dt, (int)dm.hl, (int)dm.h, (int)B));
    g = max3(g, gemm_workspace_bytes(dt, (int)dm.h, (int)(3 * dm.hl), (int)B), 0);
    pl.col_bytes = colsum_pair_workspace_bytes((int)dm.T, (int)(3 * dm.hl), (int)dm.h);
    pl.col_ws = bp.take(pl.col_bytes);
  }
  pl.gemm_bytes = g;
  pl.gemm_ws = bp.take(g);
  pl.total = bp.off;
  return pl;
}

tp_status check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return TP_OK;
  if (!ws) return fail(TP_ERR_WORKSPACE, "workspace is NULL but %zu bytes are needed", need);
  if (have < need) return fail(TP_ERR_WORKSPACE, "workspace has %zu bytes, needs %zu", have, need);
  if (((uintptr_t)ws) & 255u) return fail(TP_ERR_ALIGN, "workspace is not 256-byte aligned");
  return TP_OK;
}

// Residual add + LayerNorm: row-vector kernels need 8 | hidden and keep a row
// (forward) or a thread's column partials (backward) in registers.
tp_status check_ln(const Dims& dm) {
  if (dm.h % 8) return fail(TP_ERR_ALIGN, "residual + LayerNorm needs hidden to be a multiple of 8");
  if (dm.h > kLnMaxHidden) return fail(TP_ERR_SHAPE, "residual + LayerNorm supports hidden <= %d", kLnMaxHidden);
  return TP_OK;
}

// Vocabulary-parallel output layer: the rank's slice [v0, v0 + n) of a vocab
// of V = vocab rows, n = V / tp_size.
struct VocabDims {
  int n, v0;
};
tp_status check_vocab(const tp_shape* s, const Dims& dm, int32_t vocab, VocabDims& vd) {
  if (vocab <= 0 || vocab > kMaxDim) return fail(TP_ERR_SHAPE, "vocab %d outside [1, 2^22]", vocab);
  if (vocab % s->tp_size) return fail(TP_ERR_DIVISIBILITY, "vocab %d not divisible by tp_size %d", vocab, s->tp_size);
  vd.n = vocab / s->tp_size;
  vd.v0 = s->tp_rank * vd.n;
  if (vd.n % 8) return fail(TP_ERR_ALIGN, "vocab / tp_size = %d is not a multiple of 8", vd.n);
  if (vd.n > kCeMaxSlice) return fail(TP_ERR_SHAPE, "vocab / tp_size = %d exceeds %d", vd.n, kCeMaxSlice);
  if (dm.T * vd.n >= kMaxElems || (long long)vd.n * dm.h >= kMaxElems)
    return fail(TP_ERR_SHAPE, "a tensor of this shape has >= 2^30 elements");
  return TP_OK;
}

struct VocabPlan {
  void *dl, *gemm_ws;
  size_t gemm_bytes, total;
};

VocabPlan plan_vocab(const Dims& dm, const VocabDims& vd, void* ws, bool bwd) {
  Bump bp(ws);
  VocabPlan pl{};
  const int dt = dm.dtype, T = (int)dm.T, h = (int)dm.h, n = vd.n;
  size_t g = gemm_workspace_bytes(dt, T, n, h);
  if (bwd) {
    pl.dl = bp.take((size_t)(dm.T * n) * dm.esz);
    g = max3(g, gemm_workspace_bytes(dt, T, h, n), gemm_workspace_bytes(dt, n, h, T));
  }
  pl.gemm_bytes = g;
  pl.gemm_ws = bp.take(g);
  pl.total = bp.off;
  return pl;
}

// Shape, operand layouts and epilogue of a GEMM step's product (the caller
// fills in the pointers): the wrappers below launch exactly these, and
// tp_step_kernel names the kernel each one runs. Weight gradients of wide
// layers read a transposed, token-contiguous copy of one operand (leading
// dimension t_ld(T)).
GemmDesc step_gemm(const Dims& dm, int step) {
  GemmDesc g;
  const int T = (int)dm.T, h = (int)dm.h, hl = (int)dm.hl, fl = (int)dm.fl;
  const bool cp = wgrad_copies(dm);
  const long ldt = (long)t_ld(T);
  auto set = [&](int role, int M, int N, int K, long lda, bool ak, long ldb, bool bk, int epi, long ldc) {
    g.role = role;
    g.M = M; g.N = N; g.K = K;
    g.lda = lda; g.a_kmajor = ak;
    g.ldb = ldb; g.b_kmajor = bk;
    g.epi = epi;
    g.ldc = ldc;
  };
  switch (step) {
    case TP_STEP_QKV_PROJ: {
      const bool planes = attn_mfma_supported(dm.dtype, (int)dm.d);
      set(GR_QKV_PROJ, T, 3 * hl, h, h, true, 3 * hl, false, planes ? EPI_QKV_PLANES : EPI_BIAS_F32,
          planes ? hl : 3 * hl);
      g.qkv_hl = hl;
      g.qscale = (float)(1.4426950408889634 / std::sqrt((double)dm.d));
      break;
    }
    case TP_STEP_OUT_PROJ: set(GR_OUT_PROJ, T, h, hl, hl, true, h, false, EPI_STORE, h); break;
    case TP_STEP_FC1: set(GR_FC1, T, fl, h, h, true, fl, false, EPI_BIAS_GELU, fl); g.ldc2 = fl; break;
    case TP_STEP_FC2: set(GR_FC2, T, h, fl, fl, true, h, false, EPI_STORE, h); break;
    case TP_STEP_FC2_DGRAD: set(GR_FC2_DGRAD, T, fl, h, h, true, h, true, EPI_DGELU, fl); g.ldaux = fl; break;
    case TP_STEP_FC2_WGRAD:
      if (cp) set(GR_FC2_WGRAD, fl, h, T, ldt, true, h, false, EPI_STORE, h);
      else set(GR_FC2_WGRAD, fl, h, T, fl, false, h, false, EPI_STORE, h);
      break;
    case TP_STEP_FC1_WGRAD:
      if (cp) set(GR_FC1_WGRAD, h, fl, T, h, false, ldt, true, EPI_STORE, fl);
      else set(GR_FC1_WGRAD, h, fl, T, h, false, fl, false, EPI_STORE, fl);
      break;
    case TP_STEP_FC1_DGRAD: set(GR_FC1_DGRAD, T, h, fl, fl, true, fl, true, EPI_STORE, h); break;
    case TP_STEP_OUT_DGRAD: set(GR_OUT_DGRAD, T, hl, h, h, true, h, true, EPI_STORE, hl); break;
    case TP_STEP_OUT_WGRAD:
      if (cp) set(GR_OUT_WGRAD, hl, h, T, ldt, true, h, false, EPI_STORE, h);
      else set(GR_OUT_WGRAD, hl, h, T, hl, false, h, false, EPI_STORE, h);
      break;
    case TP_STEP_QKV_WGRAD:
      if (cp) set(GR_QKV_WGRAD, h, 3 * hl, T, h, false, ldt, true, EPI_STORE, 3 * hl);
      else set(GR_QKV_WGRAD, h, 3 * hl, T, h, false, 3 * hl, false, EPI_STORE, 3 * hl);
      break;
    case TP_STEP_QKV_DGRAD: set(GR_QKV_DGRAD, T, h, 3 * hl, 3 * hl, true, 3 * hl, true, EPI_STORE, h); break;
    default: break;  // role 0: not a GEMM step
  }
  return g;
}

GemmDesc with_ptrs(GemmDesc g, const void* A, const void* B, void* C) {
  g.A = A; g.B = B; g.C = C;
  return g;
}

GemmDesc gd(int role, int M, int N, int K, const void* A, long lda, bool ak, const void* B, long ldb, bool bk,
            int epi, void* C, long ldc) {
  GemmDesc g;
  g.role = role;
  g.M = M; g.N = N; g.K = K;
  g.A = A; g.lda = lda; g.a_kmajor = ak;
  g.B = B; g.ldb = ldb; g.b_kmajor = bk;
  g.epi = epi;
  g.C = C; g.ldc = ldc;
  return g;
}

}  // namespace

extern "C" {

const char* tp_last_error(void) { return g_last_error.c_str(); }

const char* tp_step_kernel(const tp_shape* shape, int32_t step) {
  Dims dm;
  if (check_shape(shape, dm) != TP_OK) return nullptr;
  const GemmDesc g = step_gemm(dm, step);
  if (g.role == 0) return nullptr;
  return gemm_kernel_name(dm.dtype, g);
}

size_t tp_mlp_workspace_bytes(const tp_shape* shape) {
  Dims dm;
  if (check_shape(shape, dm) != TP_OK) return 0;
  const MlpPlan a = plan_mlp(dm, nullptr, false), b = plan_mlp(dm, nullptr, true);
  return a.total > b.total ? a.total : b.total;
}

size_t tp_attn_workspace_bytes(const tp_shape* shape) {
  Dims dm;
  if (check_shape(shape, dm) != TP_OK) return 0;
  const AttnPlan a = plan_attn(dm, nullptr, false), b = plan_attn(dm, nullptr, true);
  return a.total > b.total ? a.total : b.total;
}

tp_status tp_mlp_fwd(const tp_shape* shape, const void* X, const void* A_i, const void* b1_i, const void* B_i,
                     void* pre_i, void* y_i, void* Z_i, void* workspace, size_t workspace_bytes, void* stream) {
  Dims dm;
  TP_CHECK(check_shape(shape, dm));
  const bool e = dm.T == 0;
  TP_CHECK(check_ptr(X, "X", e));
  TP_CHECK(check_ptr(A_i, "A_i", false));
  TP_CHECK(check_ptr(b1_i, "b1_i", false));
  TP_CHECK(check_ptr(B_i, "B_i", false));
  TP_CHECK(check_ptr(pre_i, "pre_i", e));
  TP_CHECK(check_ptr(y_i, "y_i", e));
  TP_CHECK(check_ptr(Z_i, "Z_i", e));
  const MlpPlan need = plan_mlp(dm, nullptr, false);
  TP_CHECK(check_ws(workspace, workspace_bytes, need.total));
  if (e) return TP_OK;
  const MlpPlan pl = plan_mlp(dm, workspace, false);
  hipStream_t st = (hipStream_t)stream;
  const int dt = dm.dtype;
  GemmDesc g1 = with_ptrs(step_gemm(dm, TP_STEP_FC1), X, A_i, pre_i);
  g1.C2 = y_i; g1.bias = b1_i;
  TP_STEP(TP_STEP_FC1, gemm_launch(dt, g1, pl.gemm_ws, pl.gemm_bytes, st), "mlp GEMM1 (X A_i + b1_i, GeLU)");
  GemmDesc g2 = with_ptrs(step_gemm(dm, TP_STEP_FC2), y_i, B_i, Z_i);
  TP_STEP(TP_STEP_FC2, gemm_launch(dt, g2, pl.gemm_ws, pl.gemm_bytes, st), "mlp GEMM2 (y_i B_i)");
  return TP_OK;
}

tp_status tp_mlp_bwd(const tp_shape* shape, const void* X, const void* A_i, const void* B_i, const void* pre_i,
                     const void* y_i, const void* dZ, void* dX_i, void* dA_i, void* db1_i, void* dB_i,
                     void* db2_or_null, void* workspace, size_t workspace_bytes, void* stream) {
  Dims dm;
  TP_CHECK(check_shape(shape, dm));
  const bool e = dm.T == 0;
  TP_CHECK(check_ptr(X, "X", e));
  TP_CHECK(check_ptr(A_i, "A_i", false));
  TP_CHECK(check_ptr(B_i, "B_i", false));
  TP_CHECK(check_ptr(pre_i, "pre_i", e));
  TP_CHECK(check_ptr(y_i, "y_i", e));
  TP_CHECK(check_ptr(dZ, "dZ", e));
  TP_CHECK(check_ptr(dX_i, "dX_i", e));
  TP_CHECK(check_ptr(dA_i, "dA_i", false));
  TP_CHECK(check_ptr(db1_i, "db1_i", false));
  TP_CHECK(check_ptr(dB_i, "dB_i", false));
  TP_CHECK(check_ptr(db2_or_null, "db2", true));
  const MlpPlan need = plan_mlp(dm, nullptr, true);
  TP_CHECK(check_ws(workspace, workspace_bytes, need.total));
  const MlpPlan pl = plan_mlp(dm, workspace, true);
  hipStream_t st = (hipStream_t)stream;
  const int dt = dm.dtype;
  const int T = (int)dm.T, h = (int)dm.h, fl = (int)dm.fl;
  if (T > 0) {
    GemmDesc g = with_ptrs(step_gemm(dm, TP_STEP_FC2_DGRAD), dZ, B_i, pl.dpre);
    g.aux = pre_i;
    TP_STEP(TP_STEP_FC2_DGRAD, gemm_launch(dt, g, pl.gemm_ws, pl.gemm_bytes, st), "mlp dgrad (dZ B_i^T * GeLU'(pre_i))");
  }
  // weight gradients (K = T; T == 0 gives zeros)
  if (wgrad_copies(dm)) {
    // y_i^T and dPre^T copies (the latter with db1_i's column partials)
    const long ldt = (long)t_ld(T);
    TP_STEP(TP_STEP_TRANSPOSE, transpose_colsum_launch(y_i, T, fl, fl, pl.yT, ldt, nullptr, st), "mlp y_i^T copy");
    TP_STEP(TP_STEP_FC2_WGRAD, gemm_launch(dt, with_ptrs(step_gemm(dm, TP_STEP_FC2_WGRAD), pl.yT, dZ, dB_i), pl.gemm_ws, pl.gemm_bytes, st),
           "mlp wgrad dB_i = y_i^T dZ");
    TP_STEP(TP_STEP_TRANSPOSE, transpose_colsum_launch(pl.dpre, T, fl, fl, pl.dpreT, ldt, pl.tpart, st), "mlp dPre^T copy");
    TP_STEP(TP_STEP_FC1_WGRAD, gemm_launch(dt, with_ptrs(step_gemm(dm, TP_STEP_FC1_WGRAD), X, pl.dpreT, dA_i), pl.gemm_ws, pl.gemm_bytes, st),
           "mlp wgrad dA_i = X^T dPre");
    TP_STEP(TP_STEP_BIAS_GRADS, colsum_final_launch(dt, pl.tpart, transpose_part_rows(T), fl, db1_i, st), "mlp db1_i");
  } else {
    TP_STEP(TP_STEP_FC2_WGRAD, gemm_launch(dt, with_ptrs(step_gemm(dm, TP_STEP_FC2_WGRAD), y_i, dZ, dB_i), pl.gemm_ws, pl.gemm_bytes, st),
           "mlp wgrad dB_i = y_i^T dZ");
    TP_STEP(TP_STEP_FC1_WGRAD, gemm_launch(dt, with_ptrs(step_gemm(dm, TP_STEP_FC1_WGRAD), X, pl.dpre, dA_i), pl.gemm_ws, pl.gemm_bytes, st),
           "mlp wgrad dA_i = X^T dPre");
    // db1_i and db2 in one launch of each column-sum pass
    TP_STEP(TP_STEP_BIAS_GRADS,
            colsum_pair_launch(dt, T, pl.dpre, fl, fl, db1_i, dZ, h, h, db2_or_null,
                               (float*)pl.col_ws, st),
            "mlp db1_i, db2");
  }
  if (T > 0)
    TP_STEP(TP_STEP_FC1_DGRAD, gemm_launch(dt, with_ptrs(step_gemm(dm, TP_STEP_FC1_DGRAD), pl.dpre, A_i, dX_i), pl.gemm_ws, pl.gemm_bytes, st),
           "mlp dgrad dX_i = dPre A_i^T");
  if (db2_or_null && wgrad_copies(dm))
    TP_STEP(TP_STEP_BIAS_GRADS, colsum_launch(dt, dZ, T, h, h, db2_or_null, (float*)pl.col_ws, st), "mlp db2");
  return TP_OK;
}

}  // extern "C"

namespace {

// A drop probability the kernels can realize: p >= 0 and a keep threshold
// thr = round(65536 p) (computed as the kernels do) below 65536, so that at
// least one of the 65536 16-bit values is kept and the keep scale
// 65536 / (65536 - thr) is finite (p < 1 - 2^-17).
bool valid_drop_p(float p) {
  if (!(p >= 0.f && p < 1.f)) return false;
  return floorf(p * 65536.0f + 0.5f) < 65536.0f;
}

// Dropout arguments: bf16 matrix-core attention only, a realizable p.
tp_status check_dropout(const tp_shape* s, const tp_dropout* dr) {
  if (!dr) return fail(TP_ERR_NULL, "dropout is NULL");
  if (!valid_drop_p(dr->p)) return fail(TP_ERR_SHAPE, "dropout p must be in [0, 1 - 2^-17)");
  if (s->dtype != TP_BF16) return fail(TP_ERR_DTYPE, "attention dropout runs in bf16 only");
  if (!attn_mfma_supported(s->dtype, s->head_dim))
    return fail(TP_ERR_HEADDIM, "attention dropout supports head_dim 64, 96, 128, 160");
  return TP_OK;
}

tp_status attn_fwd_impl(const tp_shape* shape, const tp_dropout* dr, uint16_t* mask, const void* X,
                        const void* Wqkv_i, const void* bqkv_i, const void* Wo_i, void* qkv_i, void* ctx_i,
                        float* lse_i, void* O_i, void* workspace, size_t workspace_bytes, void* stream) {
  Dims dm;
  TP_CHECK(check_shape(shape, dm));
  if (dr) TP_CHECK(check_dropout(shape, dr));
  if (dr) TP_CHECK(check_ptr(mask, "mask_i", dm.T == 0));
  const bool e = dm.T == 0;
  TP_CHECK(check_ptr(X, "X", e));
  TP_CHECK(check_ptr(Wqkv_i, "Wqkv_i", false));
  TP_CHECK(check_ptr(bqkv_i, "bqkv_i", false));
  TP_CHECK(check_ptr(Wo_i, "Wo_i", false));
  TP_CHECK(check_ptr(qkv_i, "qkv_i", e));
  TP_CHECK(check_ptr(ctx_i, "ctx_i", e));
  TP_CHECK(check_ptr(lse_i, "lse_i", e));
  TP_CHECK(check_ptr(O_i, "O_i", e));
  const AttnPlan need = plan_attn(dm, nullptr, false);
  TP_CHECK(check_ws(workspace, workspace_bytes, need.total));
  if (e) return TP_OK;
  const AttnPlan pl = plan_attn(dm, workspace, false);
  hipStream_t st = (hipStream_t)stream;
  const int dt = dm.dtype;
  // the matrix-core attention takes the projection as its five 16-bit
  // operand planes, written by the GEMM epilogue; the vector-ALU path fp32
  GemmDesc g = with_ptrs(step_gemm(dm, TP_STEP_QKV_PROJ), X, Wqkv_i, qkv_i);
  g.bias = bqkv_i;
  TP_STEP(TP_STEP_QKV_PROJ, gemm_launch(dt, g, pl.gemm_ws, pl.gemm_bytes, st), "attn QKV projection");
  AttnDesc a;
  a.batch = shape->batch; a.seq = shape->seq; a.n_local = (int)dm.nl; a.head_dim = (int)dm.d;
  a.head0 = shape->tp_rank * (int)dm.nl; a.n_heads = shape->n_heads; a.alibi = shape->alibi;
  a.qkv = qkv_i; a.ctx = ctx_i; a.lse = lse_i; a.fwd_part = (float*)pl.fwd_part;
  if (dr) {
    a.mask = mask; a.drop_p = dr->p; a.seed = dr->seed; a.offset = dr->offset;
  }
  TP_STEP(TP_STEP_ATTN_FWD, attn_fwd_launch(dt, a, st), "attn forward");
  TP_STEP(TP_STEP_OUT_PROJ, gemm_launch(dt, with_ptrs(step_gemm(dm, TP_STEP_OUT_PROJ), ctx_i, Wo_i, O_i), pl.gemm_ws, pl.gemm_bytes, st),
         "attn output projection");
  return TP_OK;
}

tp_status attn_bwd_impl(const tp_shape* shape, const tp_dropout* dr, const uint16_t* mask, const void* X,
                        const void* Wqkv_i, const void* Wo_i, const void* qkv_i, const void* ctx_i,
                        const float* lse_i, const void* dO, void* dX_i, void* dWqkv_i, void* dbqkv_i, void* dWo_i,
                        void* dbo_or_null, void* workspace, size_t workspace_bytes, void* stream) {
  Dims dm;
  TP_CHECK(check_shape(shape, dm));
  if (dr) TP_CHECK(check_dropout(shape, dr));
  if (dr) TP_CHECK(check_ptr(mask, "mask_i", dm.T == 0));
  const bool e = dm.T == 0;
  TP_CHECK(check_ptr(X, "X", e));
  TP_CHECK(check_ptr(Wqkv_i, "Wqkv_i", false));
  TP_CHECK(check_ptr(Wo_i, "Wo_i", false));
  TP_CHECK(check_ptr(qkv_i, "qkv_i", e));
  TP_CHECK(check_ptr(ctx_i, "ctx_i", e));
  TP_CHECK(check_ptr(lse_i, "lse_i", e));
  TP_CHECK(check_ptr(dO, "dO", e));
  TP_CHECK(check_ptr(dX_i, "dX_i", e));
  TP_CHECK(check_ptr(dWqkv_i, "dWqkv_i", false));
  TP_CHECK(check_ptr(dbqkv_i, "dbqkv_i", false));
  TP_CHECK(check_ptr(dWo_i, "dWo_i", false));
  TP_CHECK(check_ptr(dbo_or_null, "dbo", true));
  const AttnPlan need = plan_attn(dm, nullptr, true);
  TP_CHECK(check_ws(workspace, workspace_bytes, need.total));
  const AttnPlan pl = plan_attn(dm, workspace, true);
  hipStream_t st = (hipStream_t)stream;
  const int dt = dm.dtype;
  const int T = (int)dm.T, h = (int)dm.h, hl = (int)dm.hl;
  if (T > 0)
    TP_STEP(TP_STEP_OUT_DGRAD, gemm_launch(dt, with_ptrs(step_gemm(dm, TP_STEP_OUT_DGRAD), dO, Wo_i, pl.dctx), pl.gemm_ws, pl.gemm_bytes, st),
           "attn dgrad dC = dO Wo_i^T");
  const bool copies = wgrad_copies(dm);
  const long ldt = (long)t_ld(T);
  if (copies) {
    TP_STEP(TP_STEP_TRANSPOSE, transpose_colsum_launch(ctx_i, T, hl, hl, pl.ctxT, ldt, nullptr, st), "attn ctx_i^T copy");
    TP_STEP(TP_STEP_OUT_WGRAD, gemm_launch(dt, with_ptrs(step_gemm(dm, TP_STEP_OUT_WGRAD), pl.ctxT, dO, dWo_i), pl.gemm_ws, pl.gemm_bytes, st),
           "attn wgrad dWo_i = ctx_i^T dO");
  } else {
    TP_STEP(TP_STEP_OUT_WGRAD, gemm_launch(dt, with_ptrs(step_gemm(dm, TP_STEP_OUT_WGRAD), ctx_i, dO, dWo_i), pl.gemm_ws, pl.gemm_bytes, st),
           "attn wgrad dWo_i = ctx_i^T dO");
  }
  if (dbo_or_null && copies)
    TP_STEP(TP_STEP_BIAS_GRADS, colsum_launch(dt, dO, T, h, h, dbo_or_null, (float*)pl.col_ws, st), "attn dbo");
  if (T > 0) {
    AttnDesc a;
    a.batch = shape->batch; a.seq = shape->seq; a.n_local = (int)dm.nl; a.head_dim = (int)dm.d;
    a.head0 = shape->tp_rank * (int)dm.nl; a.n_heads = shape->n_heads; a.alibi = shape->alibi;
    a.qkv = qkv_i; a.ctx = (void*)ctx_i; a.lse = (float*)lse_i;
    a.dctx = pl.dctx; a.delta = (float*)pl.delta; a.dqkv = pl.dqkv;
    if (dr) {
      a.mask = (uint16_t*)mask; a.drop_p = dr->p; a.seed = dr->seed; a.offset = dr->offset;
    }
    TP_STEP(TP_STEP_ATTN_BWD, attn_bwd_launch(dt, a, st), "attn backward");
  }
  if (copies) {
    // dqkv^T copy with dbqkv_i's column partials
    TP_STEP(TP_STEP_TRANSPOSE, transpose_colsum_launch(pl.dqkv, T, 3 * hl, 3 * hl, pl.dqkvT, ldt, pl.tpart, st), "attn dqkv^T copy");
    TP_STEP(TP_STEP_QKV_WGRAD, gemm_launch(dt, with_ptrs(step_gemm(dm, TP_STEP_QKV_WGRAD), X, pl.dqkvT, dWqkv_i), pl.gemm_ws,
                       pl.gemm_bytes, st),
           "attn wgrad dWqkv_i = X^T dqkv");
    TP_STEP(TP_STEP_BIAS_GRADS, colsum_final_launch(dt, pl.tpart, transpose_part_rows(T), 3 * hl, dbqkv_i, st), "attn dbqkv_i");
  } else {
    TP_STEP(TP_STEP_QKV_WGRAD, gemm_launch(dt, with_ptrs(step_gemm(dm, TP_STEP_QKV_WGRAD), X, pl.dqkv, dWqkv_i), pl.gemm_ws,
                       pl.gemm_bytes, st),
           "attn wgrad dWqkv_i = X^T dqkv");
    // dbqkv_i and dbo in one launch of each column-sum pass
    TP_STEP(TP_STEP_BIAS_GRADS,
            colsum_pair_launch(dt, T, pl.dqkv, 3 * hl, 3 * hl, dbqkv_i, dO, h, h, dbo_or_null,
                               (float*)pl.col_ws, st),
            "attn dbqkv_i, dbo");
  }
  if (T > 0)
    TP_STEP(TP_STEP_QKV_DGRAD, gemm_launch(dt, with_ptrs(step_gemm(dm, TP_STEP_QKV_DGRAD), pl.dqkv, Wqkv_i, dX_i), pl.gemm_ws,
                       pl.gemm_bytes, st),
           "attn dgrad dX_i = dqkv Wqkv_i^T");
  return TP_OK;
}

}  // namespace

extern "C" {

tp_status tp_attn_fwd(const tp_shape* shape, const void* X, const void* Wqkv_i, const void* bqkv_i, const void* Wo_i,
                      void* qkv_i, void* ctx_i, float* lse_i, void* O_i, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return attn_fwd_impl(shape, nullptr, nullptr, X, Wqkv_i, bqkv_i, Wo_i, qkv_i, ctx_i, lse_i, O_i, workspace,
                       workspace_bytes, stream);
}

tp_status tp_attn_bwd(const tp_shape* shape, const void* X, const void* Wqkv_i, const void* Wo_i, const void* qkv_i,
                      const void* ctx_i, const float* lse_i, const void* dO, void* dX_i, void* dWqkv_i, void* dbqkv_i,
                      void* dWo_i, void* dbo_or_null, void* workspace, size_t workspace_bytes, void* stream) {
  return attn_bwd_impl(shape, nullptr, nullptr, X, Wqkv_i, Wo_i, qkv_i, ctx_i, lse_i, dO, dX_i, dWqkv_i, dbqkv_i,
                       dWo_i, dbo_or_null, workspace, workspace_bytes, stream);
}

size_t tp_attn_qkv_bytes(const tp_shape* shape) {
  Dims dm;
  if (check_shape(shape, dm) != TP_OK) return 0;
  const size_t per = attn_mfma_supported(dm.dtype, (int)dm.d) ? 5 * 2 : 3 * 4;  // planes, or fp32 q | k | v
  return (size_t)(dm.T * dm.hl) * per;
}

size_t tp_attn_dropout_mask_bytes(const tp_shape* shape) {
  Dims dm;
  if (check_shape(shape, dm) != TP_OK) return 0;
  return attn_dropout_mask_bytes(shape->batch, shape->seq, (int)dm.nl);
}

tp_status tp_attn_fwd_dropout(const tp_shape* shape, const tp_dropout* dropout, const void* X, const void* Wqkv_i,
                              const void* bqkv_i, const void* Wo_i, void* qkv_i, void* ctx_i, float* lse_i,
                              uint16_t* mask_i, void* O_i, void* workspace, size_t workspace_bytes, void* stream) {
  if (!dropout) return fail(TP_ERR_NULL, "dropout is NULL");
  return attn_fwd_impl(shape, dropout, mask_i, X, Wqkv_i, bqkv_i, Wo_i, qkv_i, ctx_i, lse_i, O_i, workspace,
                       workspace_bytes, stream);
}

tp_status tp_attn_bwd_dropout(const tp_shape* shape, const tp_dropout* dropout, const void* X, const void* Wqkv_i,
                              const void* Wo_i, const void* qkv_i, const void* ctx_i, const float* lse_i,
                              const uint16_t* mask_i, const void* dO, void* dX_i, void* dWqkv_i, void* dbqkv_i,
                              void* dWo_i, void* dbo_or_null, void* workspace, size_t workspace_bytes, void* stream) {
  if (!dropout) return fail(TP_ERR_NULL, "dropout is NULL");
  return attn_bwd_impl(shape, dropout, mask_i, X, Wqkv_i, Wo_i, qkv_i, ctx_i, lse_i, dO, dX_i, dWqkv_i, dbqkv_i,
                       dWo_i, dbo_or_null, workspace, workspace_bytes, stream);
}

tp_status tp_sum_partials(const tp_shape* shape, const void* const* parts, int32_t n_parts, const void* bias_or_null,
                          void* out, void* stream) {
  Dims dm;
  TP_CHECK(check_shape(shape, dm));
  const bool e = dm.T == 0;
  if (!parts) return fail(TP_ERR_NULL, "parts is NULL");
  if (n_parts < 1 || n_parts > 64) return fail(TP_ERR_SHAPE, "n_parts %d outside [1, 64]", n_parts);
  for (int k = 0; k < n_parts; ++k) TP_CHECK(check_ptr(parts[k], "parts[k]", e));
  TP_CHECK(check_ptr(bias_or_null, "bias", true));
  TP_CHECK(check_ptr(out, "out", e));
  if (e) return TP_OK;
  TP_HIP(sum_partials_launch(dm.dtype, parts, n_parts, bias_or_null, out, dm.T * dm.h, (int)dm.h, (hipStream_t)stream),
         "sum of partials");
  return TP_OK;
}

size_t tp_ln_workspace_bytes(const tp_shape* shape) {
  Dims dm;
  if (check_shape(shape, dm) != TP_OK || check_ln(dm) != TP_OK) return 0;
  return ln_bwd_workspace_bytes(dm.T, (int)dm.h);
}

}  // extern "C"

namespace {

tp_status check_p(const tp_dropout* dr) {
  if (!dr) return fail(TP_ERR_NULL, "dropout is NULL");
  if (!valid_drop_p(dr->p)) return fail(TP_ERR_SHAPE, "dropout p must be in [0, 1 - 2^-17)");
  return TP_OK;
}

tp_status ln_fwd_impl(const tp_shape* shape, const tp_dropout* dr, uint8_t* mask, const void* resid_in,
                      const void* const* parts, int32_t n_parts, const void* bias_or_null, const void* gamma,
                      const void* beta, float eps, void* resid_out, void* ln_out, float* mean, float* rstd,
                      void* stream) {
  Dims dm;
  TP_CHECK(check_shape(shape, dm));
  TP_CHECK(check_ln(dm));
  if (dr) TP_CHECK(check_p(dr));
  if (dr) TP_CHECK(check_ptr(mask, "mask", dm.T == 0));
  if (!(eps > 0.f) || !std::isfinite(eps)) return fail(TP_ERR_SHAPE, "eps must be positive and finite");
  if (n_parts < 0 || n_parts > 64) return fail(TP_ERR_SHAPE, "n_parts %d outside [0, 64]", n_parts);
  if (n_parts > 0 && !parts) return fail(TP_ERR_NULL, "parts is NULL");
  const bool e = dm.T == 0;
  TP_CHECK(check_ptr(resid_in, "resid_in", e));
  for (int k = 0; k < n_parts; ++k) TP_CHECK(check_ptr(parts[k], "parts[k]", e));
  TP_CHECK(check_ptr(bias_or_null, "bias", true));
  TP_CHECK(check_ptr(gamma, "gamma", false));
  TP_CHECK(check_ptr(beta, "beta", false));
  TP_CHECK(check_ptr(resid_out, "resid_out", e));
  TP_CHECK(check_ptr(ln_out, "ln_out", e));
  TP_CHECK(check_ptr(mean, "mean", e));
  TP_CHECK(check_ptr(rstd, "rstd", e));
  if (e) return TP_OK;
  LnDesc d;
  d.T = dm.T; d.h = (int)dm.h; d.eps = eps;
  d.resid_in = resid_in; d.parts = parts; d.n_parts = n_parts; d.bias = bias_or_null;
  d.gamma = gamma; d.beta = beta; d.resid_out = resid_out; d.y = ln_out; d.mean = mean; d.rstd = rstd;
  if (dr) {
    d.mask = mask; d.drop_p = dr->p; d.seed = dr->seed; d.offset = dr->offset;
  }
  hipStream_t st = (hipStream_t)stream;
  TP_STEP(TP_STEP_LN_FWD, ln_fwd_launch(dm.dtype, d, st), "residual add + LayerNorm forward");
  return TP_OK;
}

// ---- scratch of the entry point that allocates nothing ---------------------
// tp_ln_residual_bwd_noalloc keeps the backward's fp32 run partials in this
// array instead of a caller workspace. Each device holds its own copy for the
// life of the process; host code uses only the device address that
// hipGetSymbolAddress returns for the current device (looked up on the first
// call on that device and kept per device), never the array's name.
constexpr size_t kNoallocScratchBytes = (size_t)48 << 20;
__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};

tp_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(TP_ERR_HIP, "device %d outside the %d devices the library tracks", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p) return fail(TP_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL on device %d", dev);
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return TP_OK;
}

// use_scratch: take the workspace from the library's scratch array (after all
// argument checks) instead of the caller's.
tp_status ln_bwd_impl(const tp_shape* shape, const tp_dropout* dr, const uint8_t* mask, void* d_block,
                      const void* resid_out, const float* mean, const float* rstd, const void* gamma,
                      const void* d_ln_out, const void* d_resid_out_or_null, void* d_resid, void* dgamma, void* dbeta,
                      void* dbias_or_null, void* workspace, size_t workspace_bytes, void* stream,
                      bool use_scratch = false) {
  Dims dm;
  TP_CHECK(check_shape(shape, dm));
  TP_CHECK(check_ln(dm));
  if (dr) TP_CHECK(check_p(dr));
  if (dr) TP_CHECK(check_ptr(mask, "mask", dm.T == 0));
  if (dr) TP_CHECK(check_ptr(d_block, "d_block", dm.T == 0));
  const bool e = dm.T == 0;
  TP_CHECK(check_ptr(resid_out, "resid_out", e));
  TP_CHECK(check_ptr(mean, "mean", e));
  TP_CHECK(check_ptr(rstd, "rstd", e));
  TP_CHECK(check_ptr(gamma, "gamma", false));
  TP_CHECK(check_ptr(d_ln_out, "d_ln_out", e));
  TP_CHECK(check_ptr(d_resid_out_or_null, "d_resid_out", true));
  TP_CHECK(check_ptr(d_resid, "d_resid", e));
  TP_CHECK(check_ptr(dgamma, "dgamma", false));
  TP_CHECK(check_ptr(dbeta, "dbeta", false));
  TP_CHECK(check_ptr(dbias_or_null, "dbias", true));
  const size_t need = ln_bwd_workspace_bytes(dm.T, (int)dm.h);
  if (use_scratch) {
    if (need > kNoallocScratchBytes)
      return fail(TP_ERR_SHAPE, "this shape needs %zu bytes of scratch; the allocation-free entry point holds %zu "
                  "(use tp_ln_residual_bwd with a workspace)", need, kNoallocScratchBytes);
    workspace = nullptr;
    workspace_bytes = kNoallocScratchBytes;
    if (need) TP_CHECK(scratch_address(&workspace));
  }
  TP_CHECK(check_ws(workspace, workspace_bytes, need));
  LnDesc d;
  d.T = dm.T; d.h = (int)dm.h;
  d.resid_out = (void*)resid_out; d.mean = (float*)mean; d.rstd = (float*)rstd; d.gamma = gamma;
  d.dy = d_ln_out; d.dr_in = d_resid_out_or_null; d.dr = d_resid;
  d.dgamma = dgamma; d.dbeta = dbeta; d.dbias = dbias_or_null;
  if (dr) {
    d.mask = (uint8_t*)mask; d.d_block = d_block; d.drop_p = dr->p; d.seed = dr->seed; d.offset = dr->offset;
  }
  hipStream_t st = (hipStream_t)stream;
  TP_STEP(TP_STEP_LN_BWD, ln_bwd_launch(dm.dtype, d, workspace, st), "residual add + LayerNorm backward");
  return TP_OK;
}

}  // namespace

extern "C" {

tp_status tp_ln_residual_fwd(const tp_shape* shape, const void* resid_in, const void* const* parts, int32_t n_parts,
                             const void* bias_or_null, const void* gamma, const void* beta, float eps, void* resid_out,
                             void* ln_out, float* mean, float* rstd, void* stream) {
  return ln_fwd_impl(shape, nullptr, nullptr, resid_in, parts, n_parts, bias_or_null, gamma, beta, eps, resid_out,
                     ln_out, mean, rstd, stream);
}

tp_status tp_ln_residual_bwd(const tp_shape* shape, const void* resid_out, const float* mean, const float* rstd,
                             const void* gamma, const void* d_ln_out, const void* d_resid_out_or_null, void* d_resid,
                             void* dgamma, void* dbeta, void* dbias_or_null, void* workspace, size_t workspace_bytes,
                             void* stream) {
  return ln_bwd_impl(shape, nullptr, nullptr, nullptr, resid_out, mean, rstd, gamma, d_ln_out, d_resid_out_or_null,
                     d_resid, dgamma, dbeta, dbias_or_null, workspace, workspace_bytes, stream);
}

size_t tp_ln_residual_bwd_noalloc_max_scratch_bytes(void) { return kNoallocScratchBytes; }

tp_status tp_ln_residual_bwd_noalloc(const tp_shape* shape, const void* resid_out, const float* mean,
                                     const float* rstd, const void* gamma, const void* d_ln_out,
                                     const void* d_resid_out_or_null, void* d_resid, void* dgamma, void* dbeta,
                                     void* dbias_or_null, void* stream) {
  return ln_bwd_impl(shape, nullptr, nullptr, nullptr, resid_out, mean, rstd, gamma, d_ln_out, d_resid_out_or_null,
                     d_resid, dgamma, dbeta, dbias_or_null, nullptr, 0, stream, /*use_scratch=*/true);
}

size_t tp_ln_dropout_mask_bytes(const tp_shape* shape) {
  Dims dm;
  if (check_shape(shape, dm) != TP_OK || check_ln(dm) != TP_OK) return 0;
  return (size_t)(dm.T * (dm.h / 8));
}

tp_status tp_ln_residual_fwd_dropout(const tp_shape* shape, const tp_dropout* dropout, const void* resid_in,
                                     const void* const* parts, int32_t n_parts, const void* bias_or_null,
                                     const void* gamma, const void* beta, float eps, void* resid_out, void* ln_out,
                                     float* mean, float* rstd, uint8_t* mask, void* stream) {
  if (!dropout) return fail(TP_ERR_NULL, "dropout is NULL");
  return ln_fwd_impl(shape, dropout, mask, resid_in, parts, n_parts, bias_or_null, gamma, beta, eps, resid_out,
                     ln_out, mean, rstd, stream);
}

tp_status tp_ln_residual_bwd_dropout(const tp_shape* shape, const tp_dropout* dropout, const void* resid_out,
                                     const float* mean, const float* rstd, const void* gamma, const void* d_ln_out,
                                     const void* d_resid_out_or_null, const uint8_t* mask, void* d_resid,
                                     void* d_block, void* dgamma, void* dbeta, void* dbias_or_null, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  if (!dropout) return fail(TP_ERR_NULL, "dropout is NULL");
  return ln_bwd_impl(shape, dropout, mask, d_block, resid_out, mean, rstd, gamma, d_ln_out, d_resid_out_or_null,
                     d_resid, dgamma, dbeta, dbias_or_null, workspace, workspace_bytes, stream);
}

size_t tp_vocab_workspace_bytes(const tp_shape* shape, int32_t vocab) {
  Dims dm;
  VocabDims vd;
  if (check_shape(shape, dm) != TP_OK || check_vocab(shape, dm, vocab, vd) != TP_OK) return 0;
  const VocabPlan a = plan_vocab(dm, vd, nullptr, false), b = plan_vocab(dm, vd, nullptr, true);
  return a.total > b.total ? a.total : b.total;
}

tp_status tp_vocab_ce_fwd(const tp_shape* shape, int32_t vocab, const void* X, const void* W_i, const int32_t* labels,
                          void* logits_i, float* stats_i, void* workspace, size_t workspace_bytes, void* stream) {
  Dims dm;
  VocabDims vd;
  TP_CHECK(check_shape(shape, dm));
  TP_CHECK(check_vocab(shape, dm, vocab, vd));
  const bool e = dm.T == 0;
  TP_CHECK(check_ptr(X, "X", e));
  TP_CHECK(check_ptr(W_i, "W_i", false));
  TP_CHECK(check_ptr(labels, "labels", e));
  TP_CHECK(check_ptr(logits_i, "logits_i", e));
  TP_CHECK(check_ptr(stats_i, "stats_i", e));
  TP_CHECK(check_ws(workspace, workspace_bytes, plan_vocab(dm, vd, nullptr, false).total));
  if (e) return TP_OK;
  const VocabPlan pl = plan_vocab(dm, vd, workspace, false);
  hipStream_t st = (hipStream_t)stream;
  const int dt = dm.dtype, T = (int)dm.T, h = (int)dm.h, n = vd.n;
  TP_STEP(TP_STEP_LOGITS, gemm_launch(dt, gd(GR_LOGITS, T, n, h, X, h, true, W_i, h, true, EPI_STORE, logits_i, n), pl.gemm_ws, pl.gemm_bytes, st),
         "vocab logits X W_i^T");
  CeDesc c;
  c.T = dm.T; c.n = n; c.v0 = vd.v0; c.logits = logits_i; c.labels = labels; c.stats = stats_i;
  TP_STEP(TP_STEP_CE_STATS, ce_stats_launch(dt, c, st), "cross-entropy slice aggregates");
  return TP_OK;
}

tp_status tp_vocab_ce_combine(const tp_shape* shape, const float* const* stats, int32_t n_parts, float* loss,
                              float* lse, void* stream) {
  Dims dm;
  TP_CHECK(check_shape(shape, dm));
  const bool e = dm.T == 0;
  if (!stats) return fail(TP_ERR_NULL, "stats is NULL");
  if (n_parts < 1 || n_parts > 64) return fail(TP_ERR_SHAPE, "n_parts %d outside [1, 64]", n_parts);
  for (int k = 0; k < n_parts; ++k) TP_CHECK(check_ptr(stats[k], "stats[k]", e));
  TP_CHECK(check_ptr(loss, "loss", e));
  TP_CHECK(check_ptr(lse, "lse", e));
  if (e) return TP_OK;
  hipStream_t st = (hipStream_t)stream;
  TP_STEP(TP_STEP_CE_COMBINE, ce_combine_launch(stats, n_parts, dm.T, loss, lse, st), "cross-entropy exchange (emulated)");
  return TP_OK;
}

tp_status tp_vocab_ce_bwd(const tp_shape* shape, int32_t vocab, const void* X, const void* W_i, const int32_t* labels,
                          const void* logits_i, const float* lse, const float* dloss, void* dX_i, void* dW_i,
                          void* workspace, size_t workspace_bytes, void* stream) {
  Dims dm;
  VocabDims vd;
  TP_CHECK(check_shape(shape, dm));
  TP_CHECK(check_vocab(shape, dm, vocab, vd));
  const bool e = dm.T == 0;
  TP_CHECK(check_ptr(X, "X", e));
  TP_CHECK(check_ptr(W_i, "W_i", false));
  TP_CHECK(check_ptr(labels, "labels", e));
  TP_CHECK(check_ptr(logits_i, "logits_i", e));
  TP_CHECK(check_ptr(lse, "lse", e));
  TP_CHECK(check_ptr(dloss, "dloss", e));
  TP_CHECK(check_ptr(dX_i, "dX_i", e));
  TP_CHECK(check_ptr(dW_i, "dW_i", false));
  TP_CHECK(check_ws(workspace, workspace_bytes, plan_vocab(dm, vd, nullptr, true).total));
  const VocabPlan pl = plan_vocab(dm, vd, workspace, true);
  hipStream_t st = (hipStream_t)stream;
  const int dt = dm.dtype, T = (int)dm.T, h = (int)dm.h, n = vd.n;
  if (T > 0) {
    CeDesc c;
    c.T = dm.T; c.n = n; c.v0 = vd.v0; c.logits = logits_i; c.labels = labels; c.lse = lse; c.dloss = dloss;
    TP_STEP(TP_STEP_CE_DLOGITS, ce_dlogits_launch(dt, c, pl.dl, st), "cross-entropy dlogits");
    TP_STEP(TP_STEP_LOGITS_DGRAD, gemm_launch(dt, gd(GR_LOGITS_DGRAD, T, h, n, pl.dl, n, true, W_i, h, false, EPI_STORE, dX_i, h), pl.gemm_ws, pl.gemm_bytes, st),
           "vocab dgrad dX_i = dlogits W_i");
  }
  TP_STEP(TP_STEP_LOGITS_WGRAD, gemm_launch(dt, gd(GR_LOGITS_WGRAD, n, h, T, pl.dl, n, false, X, h, false, EPI_STORE, dW_i, h), pl.gemm_ws, pl.gemm_bytes, st),
         "vocab wgrad dW_i = dlogits^T X");
  return TP_OK;
}

tp_status tp_profile_enable(uint32_t step_mask) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  for (const Rec& r : g_prof_recs) g_prof_pool.push_back(r.ev);
  g_prof_recs.clear();
  g_prof_mask = step_mask;
  return TP_OK;
}

tp_status tp_profile_collect(int32_t step, int32_t* launches, double* total_ms) {
  if (!launches || !total_ms) return fail(TP_ERR_NULL, "launches / total_ms is NULL");
  std::lock_guard<std::mutex> lk(g_prof_mu);
  int n = 0;
  double tot = 0.0;
  std::vector<Rec> keep;
  for (const Rec& r : g_prof_recs) {
    if (r.step != step) {
      keep.push_back(r);
      continue;
    }
    float ms = 0.f;
    hipError_t e = hipEventSynchronize(r.ev.b);
    if (e == hipSuccess) e = hipEventElapsedTime(&ms, r.ev.a, r.ev.b);
    if (e != hipSuccess) {
      g_prof_recs.clear();
      return hip_fail(e, "tp_profile_collect");
    }
    tot += ms;
    ++n;
    g_prof_pool.push_back(r.ev);
  }
  g_prof_recs.swap(keep);
  *launches = n;
  *total_ms = tot;
  return TP_OK;
}

}  // extern "C"
