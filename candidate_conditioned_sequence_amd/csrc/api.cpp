// libwhalefuse C ABI: argument validation, workspace sizing and dispatch.
// Every check runs on the host before anything is enqueued; no call reads
// device memory on the host or synchronises (the host shape hints max_L and
// total_L replace any read of the offsets: gist.science Technical Summary
// §2.2, "shape hint tensors").
#include <cmath>
#include <cstring>

#include "../../include/whalefuse.h"
#include "kernels.h"

namespace {

struct Shape {
  int64_t M, T;
  int B, C, n_q, d, h, dh, QR, max_L;
};

whale_status_t check_dims(const whale_dims_t* dims, whale_dtype_t dtype, Shape* s) {
  if (dims == nullptr) return WHALE_ERR_NULL;
  if (dtype != WHALE_F32 && dtype != WHALE_BF16) return WHALE_ERR_DTYPE;
  const whale_dims_t& x = *dims;
  if (x.B <= 0 || x.C <= 0 || x.n_q <= 0 || x.d <= 0 || x.h <= 0 || x.max_L < 0 || x.total_L < 0)
    return WHALE_ERR_SHAPE;
  if (x.d % x.h != 0) return WHALE_ERR_SHAPE;
  const int64_t QR = (int64_t)x.C * x.n_q;
  const int64_t M = QR * x.B;
  if (QR > (1 << 30) || M > ((int64_t)1 << 31) - 1) return WHALE_ERR_SHAPE;
  if ((int64_t)x.max_L > x.total_L) return WHALE_ERR_SHAPE;
  if (x.total_L > (int64_t)x.B * x.max_L) return WHALE_ERR_SHAPE;
  const int dh = x.d / x.h;
  if (dh != 32 && dh != 64 && dh != 128) return WHALE_ERR_UNSUPPORTED;
  if (x.d != 64 && x.d != 128 && x.d != 256 && x.d != 512) return WHALE_ERR_UNSUPPORTED;
  s->M = M;
  s->T = x.total_L;
  s->B = x.B; s->C = x.C; s->n_q = x.n_q; s->d = x.d; s->h = x.h; s->dh = dh;
  s->QR = (int)QR;
  s->max_L = x.max_L;
  return WHALE_OK;
}

bool norm_ok(whale_norm_t n) { return n == WHALE_NORM_LAYER || n == WHALE_NORM_RMS || n == WHALE_NORM_NONE; }

// Norm parameters required by a norm kind (gamma for layer/rms, beta for layer).
bool norm_params_ok(whale_norm_t n, const float* g, const float* b) {
  if (n == WHALE_NORM_NONE) return true;
  if (g == nullptr) return false;
  return n == WHALE_NORM_RMS || b != nullptr;
}

whale_status_t ret(hipError_t e) { return e == hipSuccess ? WHALE_OK : WHALE_ERR_LAUNCH; }
#define WHALE_TRY(expr)                       \
  do {                                        \
    hipError_t _e = (expr);                   \
    if (_e != hipSuccess) return WHALE_ERR_LAUNCH; \
  } while (0)

size_t esz(whale_dtype_t t) { return t == WHALE_BF16 ? 2 : 4; }

// Bump allocator over a caller-provided workspace (256-byte aligned pieces).
struct Carve {
  char* base;
  size_t used = 0;
  explicit Carve(void* p) : base((char*)p) {}
  void* take(size_t bytes) {
    void* p = base ? base + used : nullptr;
    used += (bytes + 255) / 256 * 256;
    return p;
  }
};

GemmArgs gemm_defaults() {
  GemmArgs a;
  std::memset(&a, 0, sizeof(a));
  a.norm_kind = 2;
  a.nsplit = 1 << 30;
  return a;
}

WgradArgs wgrad_defaults() {
  WgradArgs a;
  std::memset(&a, 0, sizeof(a));
  a.norm_kind = 2;
  return a;
}

size_t wgrad_partial_bytes(int64_t M, int N, int K, bool dual = false) {
  const int sp = wgrad_splits(M, N, K);
  return (sp > 1 || dual) ? (size_t)sp * N * K * 4 : 0;
}

struct Wg {
  WgradArgs a;
  Wg(const void* G, int ldg, const void* X, int ldx, int pro, int64_t M, int N, int K, float* dW, float* partial) {
    a = wgrad_defaults();
    a.G = G; a.ldg = ldg; a.X = X; a.ldx = ldx; a.pro = pro;
    a.M = M; a.N = N; a.K = K; a.dW = dW; a.partial = partial; a.splits = wgrad_splits(M, N, K);
  }
  Wg& norm(const float* stats, const float* g, const float* b, int kind) {
    a.stats = stats; a.gamma = g; a.beta = b; a.norm_kind = kind;
    if (kind == 2 && a.pro == WPRO_NORM) a.pro = WPRO_PLAIN;
    return *this;
  }
  Wg& concat(const void* X2, int ldx2, int ksplit) { a.X2 = X2; a.ldx2 = ldx2; a.ksplit = ksplit; return *this; }
  Wg& dual(const void* G2, int nsplit, float* dW2) { a.G2 = G2; a.nsplit = nsplit; a.dW2 = dW2; return *this; }
  Wg& gz(const void* Z) { a.Gz = Z; return *this; }
  Wg& gate(int H) { a.gate_H = H; return *this; }
  hipError_t run(bool bf, hipStream_t st) { return launch_wgrad(a, bf, st); }
};

size_t norm_part_bytes(int64_t M, int d) { return (size_t)gemm_norm_bwd_tiles(M) * 2 * d * 4; }

// dX = dY W (as an NT GEMM with the pre-transposed weight Wt [K_out, N_in]) followed,
// in the same kernel, by the norm backward: out = Norm backward(dX) + R.
hipError_t norm_bwd_gemm(const void* dY, int ldy_in, const void* dY2, int ksplit, const void* Wt, int ldw, int K,
                         const void* nx, const float* stats, const float* gamma, int norm_kind, const void* R,
                         void* out, float* part, int64_t M, int d, bool bf, hipStream_t st) {
  GemmArgs g = gemm_defaults();
  g.X = dY; g.ldx = ldy_in; g.X2 = dY2; g.ldx2 = ldy_in; g.ksplit = ksplit;
  g.W = Wt; g.ldw = ldw; g.Y = out; g.ldy = d; g.R = R; g.ldr = d;
  g.nx = nx; g.stats = stats; g.gamma = gamma; g.norm_kind = norm_kind; g.part = part;
  g.M = M; g.N = d; g.K = K; g.pro = dY2 ? PRO_CONCAT : PRO_PLAIN; g.epi = EPI_NORM_BWD;
  return launch_gemm_nt(g, bf, st);
}

}  // namespace

extern "C" {

const char* whale_status_string(whale_status_t s) {
  switch (s) {
    case WHALE_OK: return "WHALE_OK";
    case WHALE_ERR_NULL: return "WHALE_ERR_NULL: a required pointer is NULL";
    case WHALE_ERR_SHAPE: return "WHALE_ERR_SHAPE: inconsistent sizes or values";
    case WHALE_ERR_DTYPE: return "WHALE_ERR_DTYPE: unknown data type";
    case WHALE_ERR_UNSUPPORTED:
      return "WHALE_ERR_UNSUPPORTED: shape not implemented (d_h must be 32, 64 or 128, d one of 64, 128, 256, 512, "
             "H % 64 == 0)";
    case WHALE_ERR_WORKSPACE: return "WHALE_ERR_WORKSPACE: workspace too small";
    case WHALE_ERR_LAUNCH: return "WHALE_ERR_LAUNCH: kernel launch failed";
  }
  return "WHALE_ERR_UNKNOWN";
}

const char* whale_version(void) { return "0.2.0"; }

whale_status_t whale_validate_offsets(const whale_dims_t* dims, const int64_t* offsets, const int64_t* cand_offsets,
                                      int32_t* flag, hipStream_t stream) {
  // Only the sizes the check reads need to be sane here; widths do not matter.
  if (dims == nullptr || !offsets || !flag) return WHALE_ERR_NULL;
  const whale_dims_t& x = *dims;
  if (x.B <= 0 || x.C <= 0 || x.max_L < 0 || x.total_L < 0) return WHALE_ERR_SHAPE;
  return ret(launch_validate_offsets(offsets, cand_offsets, x.B, x.max_L, x.total_L, x.C, flag, nullptr, stream));
}

whale_status_t whale_validate_timestamps(const whale_dims_t* dims, const int64_t* offsets, const int64_t* timestamps,
                                         int32_t* flag, hipStream_t stream) {
  if (dims == nullptr || !offsets || !timestamps || !flag) return WHALE_ERR_NULL;
  const whale_dims_t& x = *dims;
  if (x.B <= 0 || x.C <= 0 || x.max_L < 0 || x.total_L < 0) return WHALE_ERR_SHAPE;
  WHALE_TRY(launch_validate_offsets(offsets, nullptr, x.B, x.max_L, x.total_L, x.C, flag, nullptr, stream));
  return ret(launch_validate_timestamps(offsets, timestamps, x.B, x.total_L, flag, nullptr, stream));
}

int32_t whale_debug_checks(int32_t enable) { return set_debug_checks(enable != 0); }

whale_status_t whale_debug_status(int32_t* flag, int32_t reset, hipStream_t stream) {
  if (!flag) return WHALE_ERR_NULL;
  return ret(launch_debug_status(flag, reset, stream));
}

// ------------------------------------------------------------------ forward

whale_status_t whale_proj_qkv(const whale_dims_t* dims, whale_dtype_t dtype, const void* H_w, const void* H_s,
                              whale_norm_t norm, float eps, const float* g_q, const float* b_q, const float* g_kv,
                              const float* b_kv, const void* W_Q, const void* W_K, const void* W_V, void* Q, void* K,
                              void* V, float* stats_q, float* stats_kv, void* X_q, void* X_s, hipStream_t stream) {
  Shape s;
  whale_status_t rc = check_dims(dims, dtype, &s);
  if (rc != WHALE_OK) return rc;
  if (!norm_ok(norm) || !(eps >= 0.f) || !std::isfinite(eps)) return WHALE_ERR_SHAPE;
  // Shared key-value form: no W_V and no V; K serves as both.
  const bool tied = !W_V && !V;
  if (!H_w || !W_Q || !W_K || (!W_V && !tied) || !Q) return WHALE_ERR_NULL;
  if (s.T > 0 && (!H_s || !K || (!V && !tied))) return WHALE_ERR_NULL;
  if (!norm_params_ok(norm, g_q, b_q) || !norm_params_ok(norm, g_kv, b_kv)) return WHALE_ERR_NULL;
  if (norm != WHALE_NORM_NONE && (!stats_q || (s.T > 0 && !stats_kv))) return WHALE_ERR_NULL;
  const bool bf = dtype == WHALE_BF16;
  const int nk = (int)norm;
  const bool nrm = norm != WHALE_NORM_NONE;
  const int nkv = tied ? s.d : 2 * s.d;   // history-side output columns
  if (bf && rs_fwd_ok(s.d, s.d) && rs_fwd_ok(s.d, nkv)) {
    // Row-streaming kernels: the norm (statistics, X_q / X_s) and the
    // projection in one pass over the rows; K and V together.
    RsFwdArgs q{};
    q.H = (const __bf16*)H_w; q.ldh = s.d; q.W = (const __bf16*)W_Q; q.W2 = (const __bf16*)W_Q; q.nsplit = s.d;
    q.Y = (__bf16*)Q; q.Y2 = (__bf16*)Q; q.ldy = s.d;
    q.Xn = nrm ? (__bf16*)X_q : nullptr; q.stats = nrm ? stats_q : nullptr;
    q.gamma = g_q; q.beta = b_q; q.M = s.M; q.kind = nk; q.eps = eps;
    q.gate = 0; q.ngroups = 1; q.Z = nullptr; q.ldz = 0;
    WHALE_TRY(launch_rs_fwd(q, s.d, s.d, stream));
    if (s.T > 0) {
      RsFwdArgs kv = q;
      kv.H = (const __bf16*)H_s; kv.W = (const __bf16*)W_K; kv.W2 = (const __bf16*)(tied ? W_K : W_V);
      kv.Y = (__bf16*)K; kv.Y2 = (__bf16*)(tied ? K : V);
      kv.Xn = nrm ? (__bf16*)X_s : nullptr; kv.stats = nrm ? stats_kv : nullptr;
      kv.gamma = g_kv; kv.beta = b_kv; kv.M = s.T;
      WHALE_TRY(launch_rs_fwd(kv, s.d, nkv, stream));
    }
    return WHALE_OK;
  }
  if (bf && s.d == 512 && rs_fwd_groups_ok(s.d, s.d) && rs_fwd_groups_ok(s.d, nkv)) {
    // d = 512: the same kernels in column groups of 256 (2 for Q, 4 for K
    // and V); the groups of one row block share an XCD, so the rows are read
    // from HBM once.  Group 0 writes X_q / X_s and the statistics.
    RsFwdArgs q{};
    q.H = (const __bf16*)H_w; q.ldh = s.d; q.W = (const __bf16*)W_Q; q.W2 = (const __bf16*)W_Q; q.nsplit = s.d;
    q.Y = (__bf16*)Q; q.Y2 = (__bf16*)Q; q.ldy = s.d;
    q.Xn = nrm ? (__bf16*)X_q : nullptr; q.stats = nrm ? stats_q : nullptr;
    q.gamma = g_q; q.beta = b_q; q.M = s.M; q.kind = nk; q.eps = eps;
    q.gate = 0; q.ngroups = s.d / 256; q.Z = nullptr; q.ldz = 0;
    WHALE_TRY(launch_rs_fwd(q, s.d, 256, stream));
    if (s.T > 0) {
      RsFwdArgs kv = q;
      kv.H = (const __bf16*)H_s; kv.W = (const __bf16*)W_K; kv.W2 = (const __bf16*)(tied ? W_K : W_V);
      kv.Y = (__bf16*)K; kv.Y2 = (__bf16*)(tied ? K : V);
      kv.Xn = nrm ? (__bf16*)X_s : nullptr; kv.stats = nrm ? stats_kv : nullptr;
      kv.gamma = g_kv; kv.beta = b_kv; kv.M = s.T; kv.ngroups = nkv / 256;
      WHALE_TRY(launch_rs_fwd(kv, s.d, 256, stream));
    }
    return WHALE_OK;
  }
  // Each input is normalised either once into X_q / X_s (statistics computed
  // in the same pass) or, without them, per tile in the GEMM prologue.
  const bool mq = nrm && X_q != nullptr, ms = nrm && X_s != nullptr && s.T > 0;
  if (nrm) {
    if (mq) WHALE_TRY(launch_norm_apply(H_w, nullptr, stats_q, g_q, b_q, X_q, s.M, s.d, nk, eps, bf, stream));
    else WHALE_TRY(launch_norm_stats(H_w, stats_q, s.M, s.d, nk, eps, bf, stream));
    if (ms) WHALE_TRY(launch_norm_apply(H_s, nullptr, stats_kv, g_kv, b_kv, X_s, s.T, s.d, nk, eps, bf, stream));
    else WHALE_TRY(launch_norm_stats(H_s, stats_kv, s.T, s.d, nk, eps, bf, stream));
  }
  GemmArgs a = gemm_defaults();
  a.X = mq ? X_q : H_w; a.ldx = s.d; a.stats = stats_q; a.gamma = g_q; a.beta = b_q; a.norm_kind = nk;
  a.W = W_Q; a.ldw = s.d; a.Y = Q; a.ldy = s.d; a.M = s.M; a.N = s.d; a.K = s.d;
  a.pro = (nrm && !mq) ? PRO_NORM : PRO_PLAIN; a.epi = EPI_STORE;
  WHALE_TRY(launch_gemm_nt(a, bf, stream));
  if (s.T > 0) {
    // K and V in one pass over the history rows: weight rows [0, d) from W_K, [d, 2d) from W_V
    // (K alone in the shared key-value form).
    GemmArgs b = a;
    b.X = ms ? X_s : H_s; b.stats = stats_kv; b.gamma = g_kv; b.beta = b_kv;
    b.pro = (nrm && !ms) ? PRO_NORM : PRO_PLAIN;
    b.W = W_K; b.Y = K; b.M = s.T; b.N = nkv;
    if (!tied) { b.W2 = W_V; b.nsplit = s.d; b.Y2 = V; }
    WHALE_TRY(launch_gemm_nt(b, bf, stream));
  }
  return WHALE_OK;
}

}  // extern "C"

namespace {

// Debug mode (WHALE_DEBUG_CHECKS, or whale_debug_checks(1)): validate the
// offsets against the hints into the library's flag on this GPU, and hand the
// flag to the kernels, which skip their work when it is set.  Off: *guard =
// nullptr and nothing is launched.
whale_status_t debug_guard(const Shape& s, const int64_t* offsets, const int64_t* cand_offsets,
                           const int32_t** guard, hipStream_t stream) {
  *guard = nullptr;
  if (!debug_checks_on()) return WHALE_OK;
  int32_t* f = debug_flags_device();
  if (f == nullptr) return WHALE_ERR_LAUNCH;
  WHALE_TRY(launch_validate_offsets(offsets, cand_offsets, s.B, s.max_L, s.T, s.C, f, f + 1, stream));
  *guard = f;
  return WHALE_OK;
}

// Both forward attention calls: cand_offsets null for C candidates per request.
// Longest-first order for jagged batches (see kRankMaxB): every L_b <= max_L
// and their sum total_L = B max_L mean all lengths are equal.
bool rank_order(const Shape& s) { return s.B <= kRankMaxB && s.T != (int64_t)s.B * s.max_L; }

whale_status_t xattn_fwd_call(const whale_dims_t* dims, whale_dtype_t dtype, const void* Q, const void* K,
                              const void* V, const int64_t* offsets, const int64_t* cand_offsets, float scale,
                              void* A, float* lse, hipStream_t stream) {
  Shape s;
  whale_status_t rc = check_dims(dims, dtype, &s);
  if (rc != WHALE_OK) return rc;
  if (!Q || !A || !offsets) return WHALE_ERR_NULL;
  if (s.T > 0 && (!K || !V)) return WHALE_ERR_NULL;
  if (!(scale >= 0.f) || !std::isfinite(scale)) return WHALE_ERR_SHAPE;
  XattnArgs a;
  a.Q = Q; a.K = K; a.V = V; a.offsets = offsets; a.A = A; a.lse = lse;
  a.B = s.B; a.QR = s.QR; a.d = s.d; a.h = s.h; a.dh = s.dh;
  a.scale = scale > 0.f ? scale : 1.f / std::sqrt((float)s.dh);
  a.cand_offsets = cand_offsets; a.n_q = s.n_q;
  a.rank_order = rank_order(s);
  whale_status_t g = debug_guard(s, offsets, cand_offsets, &a.guard, stream);
  if (g != WHALE_OK) return g;
  return ret(launch_xattn_fwd(a, dtype == WHALE_BF16, stream));
}

}  // namespace

extern "C" {

whale_status_t whale_jagged_xattn_fwd(const whale_dims_t* dims, whale_dtype_t dtype, const void* Q, const void* K,
                                      const void* V, const int64_t* offsets, float scale, void* A, float* lse,
                                      hipStream_t stream) {
  return xattn_fwd_call(dims, dtype, Q, K, V, offsets, nullptr, scale, A, lse, stream);
}

whale_status_t whale_jagged_xattn_fwd_varc(const whale_dims_t* dims, whale_dtype_t dtype, const void* Q,
                                           const void* K, const void* V, const int64_t* offsets,
                                           const int64_t* cand_offsets, float scale, void* A, float* lse,
                                           hipStream_t stream) {
  if (!cand_offsets) return WHALE_ERR_NULL;
  return xattn_fwd_call(dims, dtype, Q, K, V, offsets, cand_offsets, scale, A, lse, stream);
}

whale_status_t whale_hstu_attn_fwd(const whale_dims_t* dims, whale_dtype_t dtype, const void* Q, const void* K,
                                   const void* V, const int64_t* offsets, const int64_t* timestamps,
                                   const float* w_pos, int32_t n_pos, const float* w_time, int32_t n_time,
                                   float scale, void* A, hipStream_t stream) {
  Shape s;
  whale_status_t rc = check_dims(dims, dtype, &s);
  if (rc != WHALE_OK) return rc;
  if (!offsets || !w_pos || !w_time) return WHALE_ERR_NULL;
  if (s.T > 0 && (!Q || !K || !V || !A || !timestamps)) return WHALE_ERR_NULL;
  if (!(scale >= 0.f) || !std::isfinite(scale)) return WHALE_ERR_SHAPE;
  if (n_pos < 1 || n_pos > hstu_max_pos() || n_time < 1 || n_time > 32) return WHALE_ERR_UNSUPPORTED;
  HstuArgs a;
  a.Q = Q; a.K = K; a.V = V; a.offsets = offsets; a.timestamps = timestamps;
  a.w_pos = w_pos; a.n_pos = n_pos; a.w_time = w_time; a.n_time = n_time; a.A = A;
  a.B = s.B; a.d = s.d; a.h = s.h; a.dh = s.dh; a.max_L = s.max_L;
  a.scale = scale > 0.f ? scale : 1.f / std::sqrt((float)s.dh);
  whale_status_t g = debug_guard(s, offsets, nullptr, &a.guard, stream);
  if (g != WHALE_OK) return g;
  if (a.guard != nullptr)   // debug mode: the timestamps' contract too
    WHALE_TRY(launch_validate_timestamps(offsets, timestamps, s.B, s.T, const_cast<int32_t*>(a.guard),
                                         const_cast<int32_t*>(a.guard) + 1, stream));
  if (s.T == 0) return WHALE_OK;
  return ret(launch_hstu_fwd(a, dtype == WHALE_BF16, stream));
}

whale_status_t whale_fusion_mlp(const whale_dims_t* dims, whale_dtype_t dtype, const void* A, const void* H_w,
                                const void* W_F, whale_act_t act, void* F, void* Z_saved, hipStream_t stream) {
  Shape s;
  whale_status_t rc = check_dims(dims, dtype, &s);
  if (rc != WHALE_OK) return rc;
  if (act != WHALE_ACT_SILU && act != WHALE_ACT_NONE) return WHALE_ERR_SHAPE;
  if (!A || !H_w || !W_F || !F) return WHALE_ERR_NULL;
  if (dtype == WHALE_BF16 && act == WHALE_ACT_SILU && rs_fwd_ok(2 * s.d, s.d)) {
    // Row-streaming kernel: [A | H_w] W_F^T, SiLU and the residual H_w (read
    // from the staged rows) in one pass.
    RsFwdArgs r{};
    r.H = (const __bf16*)A; r.ldh = s.d; r.H2 = (const __bf16*)H_w; r.ldh2 = s.d;
    r.W = (const __bf16*)W_F; r.W2 = (const __bf16*)W_F; r.nsplit = s.d;
    r.Y = (__bf16*)F; r.Y2 = (__bf16*)F; r.ldy = s.d; r.M = s.M; r.kind = 2;
    r.gate = 4; r.ngroups = 1; r.Z = (__bf16*)Z_saved; r.ldz = s.d;
    return ret(launch_rs_fwd(r, 2 * s.d, s.d, stream));
  }
  GemmArgs a = gemm_defaults();
  a.X = A; a.ldx = s.d; a.X2 = H_w; a.ldx2 = s.d; a.ksplit = s.d;
  a.W = W_F; a.ldw = 2 * s.d; a.Y = F; a.ldy = s.d; a.R = H_w; a.ldr = s.d; a.Z = Z_saved; a.ldz = s.d;
  a.M = s.M; a.N = s.d; a.K = 2 * s.d; a.pro = PRO_CONCAT;
  a.epi = act == WHALE_ACT_SILU ? EPI_SILU_RESID : EPI_RESID;
  return ret(launch_gemm_nt(a, dtype == WHALE_BF16, stream));
}

static bool ffn_h_ok(int32_t H) { return H > 0 && H % 64 == 0 && H <= (1 << 16); }

size_t whale_swiglu_ffn_workspace_size(const whale_dims_t* dims, whale_dtype_t dtype, whale_gate_t gate, int32_t H) {
  Shape s;
  if (check_dims(dims, dtype, &s) != WHALE_OK || !ffn_h_ok(H)) return 0;
  (void)gate;
  Carve c(nullptr);
  c.take((size_t)s.M * H * esz(dtype));      // G
  c.take((size_t)s.M * s.d * esz(dtype));    // X_f = Norm_f(F)
  return c.used;
}

whale_status_t whale_swiglu_ffn(const whale_dims_t* dims, whale_dtype_t dtype, const void* F, whale_norm_t norm,
                                float eps, const float* g_f, const float* b_f, const void* W_U, whale_gate_t gate,
                                int32_t H, const void* W_D, void* Y, void* U_saved, float* stats_f, void* X_f,
                                void* workspace, size_t ws_bytes, hipStream_t stream) {
  Shape s;
  whale_status_t rc = check_dims(dims, dtype, &s);
  if (rc != WHALE_OK) return rc;
  if (!norm_ok(norm) || !(eps >= 0.f) || !std::isfinite(eps)) return WHALE_ERR_SHAPE;
  if (gate != WHALE_GATE_SHARED && gate != WHALE_GATE_SEPARATE) return WHALE_ERR_SHAPE;
  if (!ffn_h_ok(H)) return WHALE_ERR_UNSUPPORTED;
  if (!F || !W_U || !W_D || !Y) return WHALE_ERR_NULL;
  if (!norm_params_ok(norm, g_f, b_f)) return WHALE_ERR_NULL;
  if (norm != WHALE_NORM_NONE && !stats_f) return WHALE_ERR_NULL;
  const size_t need = whale_swiglu_ffn_workspace_size(dims, dtype, gate, H);
  if (!workspace) return WHALE_ERR_NULL;
  if (ws_bytes < need) return WHALE_ERR_WORKSPACE;
  const bool bf = dtype == WHALE_BF16;
  Carve c(workspace);
  void* G = c.take((size_t)s.M * H * esz(dtype));
  void* Xf = c.take((size_t)s.M * s.d * esz(dtype));
  GemmArgs b = gemm_defaults();
  b.X = G; b.ldx = H; b.W = W_D; b.ldw = H; b.Y = Y; b.ldy = s.d; b.R = F; b.ldr = s.d;
  b.M = s.M; b.N = s.d; b.K = H; b.pro = PRO_PLAIN; b.epi = EPI_RESID;
  // Up-projection columns per row-streaming workgroup.  (At d = 512 the
  // row-streaming kernel runs in column groups of 256 and measured no faster
  // than the tiled path once the down projection forms the gate in its
  // prologue, so d = 512 keeps the tiled path.)
  constexpr int kGroup = 512;
  if (bf && gate == WHALE_GATE_SHARED && rs_fwd_ok(s.d, kGroup) && H % kGroup == 0 && 256 % (8 * (H / kGroup)) == 0) {
    // Up projection by the row-streaming kernel: Norm_f (statistics saved
    // for the backward), F W_U^T and the tied gate in one pass over F.
    // Only the product U is written (to U_saved, else to the workspace); the
    // down projection forms the gate SiLU(U) U from it in its prologue.
    void* Ubuf = U_saved ? U_saved : G;
    RsFwdArgs u{};
    u.H = (const __bf16*)F; u.ldh = s.d; u.W = (const __bf16*)W_U; u.W2 = (const __bf16*)W_U; u.nsplit = kGroup;
    u.Y = nullptr; u.Y2 = nullptr; u.ldy = H; u.Xn = norm != WHALE_NORM_NONE ? (__bf16*)X_f : nullptr;
    u.stats = norm != WHALE_NORM_NONE ? stats_f : nullptr; u.gamma = g_f; u.beta = b_f;
    u.M = s.M; u.kind = (int)norm; u.eps = eps;
    u.gate = 1; u.ngroups = H / kGroup; u.Z = (__bf16*)Ubuf; u.ldz = H;
    WHALE_TRY(launch_rs_fwd(u, s.d, kGroup, stream));
    b.X = Ubuf; b.pro = PRO_GATE;
    return ret(launch_gemm_nt(b, bf, stream));
  }
  // X_f = Norm_f(F) once (statistics saved for the backward), so that the
  // up projection does not renormalise F for every block of its H columns.
  const void* Xin = F;
  if (norm != WHALE_NORM_NONE) {
    void* dst = X_f ? X_f : Xf;
    WHALE_TRY(launch_norm_apply(F, nullptr, stats_f, g_f, b_f, dst, s.M, s.d, (int)norm, eps, bf, stream));
    Xin = dst;
  }
  GemmArgs a = gemm_defaults();
  a.X = Xin; a.ldx = s.d;
  a.W = W_U; a.ldw = s.d; a.Y = G; a.ldy = H; a.Z = U_saved;
  a.M = s.M; a.K = s.d;
  a.pro = PRO_PLAIN;
  if (gate == WHALE_GATE_SHARED) { a.N = H; a.epi = EPI_GATE_TIED; a.ldz = H; }
  else { a.N = 2 * H; a.epi = EPI_GATE_SEP; a.ldz = 2 * H; }
  WHALE_TRY(launch_gemm_nt(a, bf, stream));
  return ret(launch_gemm_nt(b, bf, stream));
}

// ------------------------------------------------------------------ backward

size_t whale_jagged_xattn_bwd_workspace_size(const whale_dims_t* dims, whale_dtype_t dtype) {
  Shape s;
  if (check_dims(dims, dtype, &s) != WHALE_OK) return 0;
  Carve c(nullptr);
  c.take((size_t)s.M * s.h * 4);
  const int splits = xattn_bwd_splits(s.B, s.h, s.QR, s.max_L, s.dh);
  if (splits > 1) c.take((size_t)splits * 2 * s.T * s.d * 4);
  if (xattn_bwd_kv_schedule(s.max_L, s.dh, dtype == WHALE_BF16))
    c.take((size_t)xattn_bwd_kv_qpartial_floats(s.M, s.d, s.max_L) * 4);
  if (s.B <= kRankMaxB) c.take((size_t)s.B * 4);      // longest-first request order
  return c.used;
}

}  // extern "C"

namespace {

// Host checks of the attention backward, everything but the workspace.
whale_status_t xattn_bwd_check(const whale_dims_t* dims, whale_dtype_t dtype, const void* Q, const void* K,
                               const void* V, const int64_t* offsets, float scale, const void* A, const float* lse,
                               const void* dA, void* dQ, void* dK, void* dV, Shape* s) {
  whale_status_t rc = check_dims(dims, dtype, s);
  if (rc != WHALE_OK) return rc;
  if (!Q || !offsets || !A || !lse || !dA || !dQ) return WHALE_ERR_NULL;
  if (s->T > 0 && (!K || !V || !dK)) return WHALE_ERR_NULL;
  // dV = NULL: shared key-value form, V must be K; dK receives dK + dV.
  if (s->T > 0 && !dV && V != K) return WHALE_ERR_SHAPE;
  if (!(scale >= 0.f) || !std::isfinite(scale)) return WHALE_ERR_SHAPE;
  return WHALE_OK;
}

// The launches, with the workspace carved from `workspace` (already checked
// to hold whale_jagged_xattn_bwd_workspace_size bytes).  Every byte of it
// that a kernel reads is written earlier in the same call, so its previous
// contents never matter.
whale_status_t xattn_bwd_launch(const Shape& s, whale_dtype_t dtype, const void* Q, const void* K, const void* V,
                                const int64_t* offsets, float scale, const void* A, const float* lse,
                                const void* dA, void* dQ, void* dK, void* dV, void* workspace, hipStream_t stream) {
  Carve c(workspace);
  XattnBwdArgs a;
  a.Q = Q; a.K = K; a.V = V; a.offsets = offsets; a.A = A; a.lse = lse; a.dA = dA;
  a.dQ = dQ; a.dK = dK; a.dV = dV;
  a.Dbuf = (float*)c.take((size_t)s.M * s.h * 4);
  a.splits = xattn_bwd_splits(s.B, s.h, s.QR, s.max_L, s.dh);
  a.partial = a.splits > 1 ? (float*)c.take((size_t)a.splits * 2 * s.T * s.d * 4) : nullptr;
  a.kv_schedule = xattn_bwd_kv_schedule(s.max_L, s.dh, dtype == WHALE_BF16);
  if (a.kv_schedule) {
    const int64_t qf = xattn_bwd_kv_qpartial_floats(s.M, s.d, s.max_L);
    a.qpartial = qf > 0 ? (float*)c.take((size_t)qf * 4) : nullptr;
  }
  // written by the dQ kernel, read by the dK/dV kernel after it
  a.perm = rank_order(s) ? (int32_t*)c.take((size_t)s.B * 4) : nullptr;
  a.B = s.B; a.QR = s.QR; a.d = s.d; a.h = s.h; a.dh = s.dh; a.max_L = s.max_L; a.T = s.T;
  a.scale = scale > 0.f ? scale : 1.f / std::sqrt((float)s.dh);
  whale_status_t g = debug_guard(s, offsets, nullptr, &a.guard, stream);
  if (g != WHALE_OK) return g;
  return ret(launch_xattn_bwd(a, dtype == WHALE_BF16, stream));
}

}  // namespace

extern "C" {

whale_status_t whale_jagged_xattn_bwd(const whale_dims_t* dims, whale_dtype_t dtype, const void* Q, const void* K,
                                      const void* V, const int64_t* offsets, float scale, const void* A,
                                      const float* lse, const void* dA, void* dQ, void* dK, void* dV,
                                      void* workspace, size_t ws_bytes, hipStream_t stream) {
  Shape s;
  whale_status_t rc = xattn_bwd_check(dims, dtype, Q, K, V, offsets, scale, A, lse, dA, dQ, dK, dV, &s);
  if (rc != WHALE_OK) return rc;
  if (!workspace) return WHALE_ERR_NULL;
  if (ws_bytes < whale_jagged_xattn_bwd_workspace_size(dims, dtype)) return WHALE_ERR_WORKSPACE;
  return xattn_bwd_launch(s, dtype, Q, K, V, offsets, scale, A, lse, dA, dQ, dK, dV, workspace, stream);
}

whale_status_t whale_jagged_xattn_bwd_noalloc(const whale_dims_t* dims, whale_dtype_t dtype, const void* Q,
                                              const void* K, const void* V, const int64_t* offsets, float scale,
                                              const void* A, const float* lse, const void* dA, void* dQ, void* dK,
                                              void* dV, hipStream_t stream) {
  Shape s;
  whale_status_t rc = xattn_bwd_check(dims, dtype, Q, K, V, offsets, scale, A, lse, dA, dQ, dK, dV, &s);
  if (rc != WHALE_OK) return rc;
  // The shape's workspace must fit the library's static scratch; the size is
  // known from the dims alone, so this is decided before touching the device.
  if (whale_jagged_xattn_bwd_workspace_size(dims, dtype) > static_scratch_bytes()) return WHALE_ERR_WORKSPACE;
  void* ws = static_scratch_device();   // this GPU's copy (looked up once per GPU)
  if (ws == nullptr) return WHALE_ERR_LAUNCH;
  return xattn_bwd_launch(s, dtype, Q, K, V, offsets, scale, A, lse, dA, dQ, dK, dV, ws, stream);
}

size_t whale_fusion_mlp_bwd_workspace_size(const whale_dims_t* dims, whale_dtype_t dtype) {
  Shape s;
  if (check_dims(dims, dtype, &s) != WHALE_OK) return 0;
  Carve c(nullptr);
  c.take((size_t)2 * s.d * s.d * esz(dtype));        // W_F^T [2d, d]
  c.take(wgrad_partial_bytes(s.M, s.d, 2 * s.d));
  c.take((size_t)s.M * s.d * esz(dtype));            // dZ
  return c.used;
}

whale_status_t whale_fusion_mlp_bwd(const whale_dims_t* dims, whale_dtype_t dtype, const void* A, const void* H_w,
                                    const void* W_F, whale_act_t act, const void* Z_saved, const void* dF, void* dA,
                                    void* dH_w, float* dW_F, void* workspace, size_t ws_bytes, hipStream_t stream) {
  Shape s;
  whale_status_t rc = check_dims(dims, dtype, &s);
  if (rc != WHALE_OK) return rc;
  if (act != WHALE_ACT_SILU && act != WHALE_ACT_NONE) return WHALE_ERR_SHAPE;
  if (!A || !H_w || !W_F || !dF || !dA || !dH_w || !dW_F || !workspace) return WHALE_ERR_NULL;
  if (act == WHALE_ACT_SILU && !Z_saved) return WHALE_ERR_NULL;
  if (ws_bytes < whale_fusion_mlp_bwd_workspace_size(dims, dtype)) return WHALE_ERR_WORKSPACE;
  const bool bf = dtype == WHALE_BF16;
  const bool silu = act == WHALE_ACT_SILU;
  const int d = s.d;
  Carve c(workspace);
  void* WFt = c.take((size_t)2 * d * d * esz(dtype));
  float* part = (float*)c.take(wgrad_partial_bytes(s.M, d, 2 * d));
  void* dZw = c.take((size_t)s.M * d * esz(dtype));
  if (bf && silu && rs_fwd_ok(d, 2 * d)) {
    // Row-streaming kernel: dZ = dF * SiLU'(Z) (written for the weight
    // gradient) and [dA | dH_w - dF] = dZ W_F with the residual, in one pass.
    WHALE_TRY(launch_transpose(W_F, d, 2 * d, WFt, d, 0, bf, stream));
    RsFwdArgs r{};
    r.H = (const __bf16*)dF; r.ldh = d; r.W = (const __bf16*)WFt; r.W2 = (const __bf16*)WFt + (size_t)d * d;
    r.nsplit = d; r.Y = (__bf16*)dA; r.Y2 = (__bf16*)dH_w; r.ldy = d;
    r.Xn = (__bf16*)dZw; r.stats = nullptr; r.gamma = nullptr; r.beta = nullptr;
    r.M = s.M; r.kind = 2; r.eps = 0.f;
    r.gate = 3; r.ngroups = 1; r.Z = (__bf16*)Z_saved; r.ldz = d;
    WHALE_TRY(launch_rs_fwd(r, d, 2 * d, stream));
    Wg w(dZw, d, A, d, WPRO_CONCAT, s.M, d, 2 * d, dW_F, part);
    w.concat(H_w, d, d);
    return ret(w.run(bf, stream));
  }
  // dZ = dF * act'(Z) once; both products below read it.
  const void* dZ = dF;
  if (silu) {
    WHALE_TRY(launch_dact(dF, Z_saved, dZw, (int64_t)s.M * d, bf, stream));
    dZ = dZw;
  }
  // dW_F = dZ^T [A, H_w]
  Wg w(dZ, d, A, d, WPRO_CONCAT, s.M, d, 2 * d, dW_F, part);
  w.concat(H_w, d, d);
  WHALE_TRY(w.run(bf, stream));
  // [dA | dH_w - dF] = dZ W_F: one GEMM against W_F^T [2d, d]; columns >= d get the residual dF.
  WHALE_TRY(launch_transpose(W_F, d, 2 * d, WFt, d, 0, bf, stream));
  GemmArgs g = gemm_defaults();
  g.X = dZ; g.ldx = d;
  g.W = WFt; g.ldw = d; g.Y = dA; g.Y2 = dH_w; g.ldy = d; g.nsplit = d; g.R = dF; g.ldr = d;
  g.M = s.M; g.N = 2 * d; g.K = d; g.pro = PRO_PLAIN; g.epi = EPI_DUAL_RESID2;
  return ret(launch_gemm_nt(g, bf, stream));
}

size_t whale_swiglu_ffn_bwd_workspace_size(const whale_dims_t* dims, whale_dtype_t dtype, whale_gate_t gate,
                                           int32_t H) {
  Shape s;
  if (check_dims(dims, dtype, &s) != WHALE_OK || !ffn_h_ok(H)) return 0;
  const int Hu = gate == WHALE_GATE_SEPARATE ? 2 * H : H;
  Carve c(nullptr);
  c.take((size_t)H * s.d * esz(dtype));              // W_D^T [H, d]
  c.take((size_t)s.M * Hu * esz(dtype));             // dU
  c.take((size_t)s.d * Hu * esz(dtype));             // W_U^T [d, Hu]
  const size_t p1 = wgrad_partial_bytes(s.M, s.d, H), p2 = wgrad_partial_bytes(s.M, Hu, s.d);
  c.take(p1 > p2 ? p1 : p2);
  c.take(norm_part_bytes(s.M, s.d));
  c.take((size_t)colsum_scratch_floats(s.d) * 4);
  c.take((size_t)s.M * s.d * esz(dtype));            // X_f
  return c.used;
}

whale_status_t whale_swiglu_ffn_bwd(const whale_dims_t* dims, whale_dtype_t dtype, const void* F, whale_norm_t norm,
                                    float eps, const float* g_f, const float* b_f, const float* stats_f,
                                    const void* W_U, whale_gate_t gate, int32_t H, const void* W_D,
                                    const void* U_saved, const void* X_f, const void* dY, void* dF, float* dW_U,
                                    float* dW_D,
                                    float* dg_f, float* db_f, void* workspace, size_t ws_bytes, hipStream_t stream) {
  Shape s;
  whale_status_t rc = check_dims(dims, dtype, &s);
  if (rc != WHALE_OK) return rc;
  if (!norm_ok(norm) || !(eps >= 0.f) || !std::isfinite(eps)) return WHALE_ERR_SHAPE;
  if (gate != WHALE_GATE_SHARED && gate != WHALE_GATE_SEPARATE) return WHALE_ERR_SHAPE;
  if (!ffn_h_ok(H)) return WHALE_ERR_UNSUPPORTED;
  if (!F || !W_U || !W_D || !U_saved || !dY || !dF || !dW_U || !dW_D || !workspace) return WHALE_ERR_NULL;
  if (!norm_params_ok(norm, g_f, b_f)) return WHALE_ERR_NULL;
  if (norm != WHALE_NORM_NONE && (!stats_f || !dg_f || (norm == WHALE_NORM_LAYER && !db_f))) return WHALE_ERR_NULL;
  if (ws_bytes < whale_swiglu_ffn_bwd_workspace_size(dims, dtype, gate, H)) return WHALE_ERR_WORKSPACE;
  const bool bf = dtype == WHALE_BF16;
  const bool sep = gate == WHALE_GATE_SEPARATE;
  const int d = s.d, Hu = sep ? 2 * H : H, nk = (int)norm;
  Carve c(workspace);
  void* WDt = c.take((size_t)H * d * esz(dtype));
  void* dU = c.take((size_t)s.M * Hu * esz(dtype));
  void* WUt = c.take((size_t)d * Hu * esz(dtype));
  const size_t p1 = wgrad_partial_bytes(s.M, d, H), p2 = wgrad_partial_bytes(s.M, Hu, d);
  float* part = (float*)c.take(p1 > p2 ? p1 : p2);
  float* npart = (float*)c.take(norm_part_bytes(s.M, d));
  float* cscr = (float*)c.take((size_t)colsum_scratch_floats(d) * 4);
  void* Xf = c.take((size_t)s.M * d * esz(dtype));

  // dW_D = dY^T G, with G recomputed from U in the loader.
  Wg w1(dY, d, U_saved, Hu, sep ? WPRO_GATE_SEP : WPRO_GATE_TIED, s.M, d, H, dW_D, part);
  WHALE_TRY(w1.gate(H).run(bf, stream));
  // dU = (dY W_D) * gate'(U)
  WHALE_TRY(launch_transpose(W_D, d, H, WDt, d, 0, bf, stream));       // [H, d]
  constexpr int kGroup = 512;   // columns per row-streaming workgroup
  if (bf && !sep && rs_fwd_ok(d, kGroup) && H % kGroup == 0 && 256 % (8 * (H / kGroup)) == 0) {
    RsFwdArgs r{};
    r.H = (const __bf16*)dY; r.ldh = d; r.W = (const __bf16*)WDt; r.W2 = (const __bf16*)WDt; r.nsplit = kGroup;
    r.Y = (__bf16*)dU; r.Y2 = (__bf16*)dU; r.ldy = Hu; r.Xn = nullptr; r.stats = nullptr;
    r.gamma = nullptr; r.beta = nullptr; r.M = s.M; r.kind = 2; r.eps = 0.f;
    r.gate = 2; r.ngroups = H / kGroup; r.Z = (__bf16*)U_saved; r.ldz = Hu;
    WHALE_TRY(launch_rs_fwd(r, d, kGroup, stream));
  } else {
    GemmArgs g = gemm_defaults();
    g.X = dY; g.ldx = d; g.W = WDt; g.ldw = d; g.Y = dU; g.ldy = Hu; g.Z = (void*)U_saved; g.ldz = Hu;
    g.M = s.M; g.N = H; g.K = d; g.pro = PRO_PLAIN; g.epi = sep ? EPI_DGATE_SEP : EPI_DGATE_TIED;
    WHALE_TRY(launch_gemm_nt(g, bf, stream));
  }
  // dW_U = dU^T X_f, X_f = Norm_f(F) formed once from the saved statistics
  const void* Xin = F;
  if (norm != WHALE_NORM_NONE) {
    if (X_f) {
      Xin = X_f;
    } else {
      WHALE_TRY(launch_norm_apply(F, stats_f, nullptr, g_f, b_f, Xf, s.M, d, nk, eps, bf, stream));
      Xin = Xf;
    }
  }
  Wg w2(dU, Hu, Xin, d, WPRO_PLAIN, s.M, Hu, d, dW_U, part);
  WHALE_TRY(w2.run(bf, stream));
  // dF = dY + Norm_f backward(dU W_U), one kernel.
  WHALE_TRY(launch_transpose(W_U, Hu, d, WUt, Hu, 0, bf, stream));     // [d, Hu]
  WHALE_TRY(norm_bwd_gemm(dU, Hu, nullptr, 0, WUt, Hu, Hu, F, stats_f, g_f, nk, dY, dF, npart, s.M, d, bf, stream));
  if (norm != WHALE_NORM_NONE)
    WHALE_TRY(launch_colsum_reduce(npart, gemm_norm_bwd_tiles(s.M), d, dg_f,
                                   norm == WHALE_NORM_LAYER ? db_f : nullptr, cscr, stream));
  if (norm == WHALE_NORM_RMS && db_f) WHALE_TRY(launch_fill_zero(db_f, d, stream));
  return WHALE_OK;
}

size_t whale_proj_qkv_bwd_workspace_size(const whale_dims_t* dims, whale_dtype_t dtype) {
  Shape s;
  if (check_dims(dims, dtype, &s) != WHALE_OK) return 0;
  Carve c(nullptr);
  c.take((size_t)s.d * s.d * esz(dtype));            // W_Q^T
  c.take((size_t)2 * s.d * s.d * esz(dtype));        // [W_K^T | W_V^T]
  const size_t p1 = wgrad_partial_bytes(s.M, s.d, s.d), p2 = wgrad_partial_bytes(s.T, 2 * s.d, s.d, true);
  c.take(p1 > p2 ? p1 : p2);
  c.take(norm_part_bytes(s.M, s.d));
  c.take(norm_part_bytes(s.T, s.d));
  c.take((size_t)colsum_scratch_floats(s.d) * 4);
  c.take((size_t)s.M * s.d * esz(dtype));            // X_q
  c.take((size_t)s.T * s.d * esz(dtype));            // X_s
  return c.used;
}

whale_status_t whale_proj_qkv_bwd(const whale_dims_t* dims, whale_dtype_t dtype, const void* H_w, const void* H_s,
                                  whale_norm_t norm, float eps, const float* g_q, const float* b_q, const float* g_kv,
                                  const float* b_kv, const float* stats_q, const float* stats_kv, const void* X_q_in,
                                  const void* X_s_in, const void* W_Q,
                                  const void* W_K, const void* W_V, const void* dQ, const void* dK, const void* dV,
                                  const void* dH_w_in, void* dH_w, void* dH_s, float* dW_Q, float* dW_K, float* dW_V,
                                  float* dg_q, float* db_q, float* dg_kv, float* db_kv, void* workspace,
                                  size_t ws_bytes, hipStream_t stream) {
  Shape s;
  whale_status_t rc = check_dims(dims, dtype, &s);
  if (rc != WHALE_OK) return rc;
  if (!norm_ok(norm) || !(eps >= 0.f) || !std::isfinite(eps)) return WHALE_ERR_SHAPE;
  // Shared key-value form: no W_V, dV or dW_V; dK is the gradient of the one tensor.
  const bool tied = !W_V && !dV && !dW_V;
  if (!H_w || !W_Q || !W_K || (!W_V && !tied) || !dQ || !dH_w || !dW_Q || !dW_K || (!dW_V && !tied) || !workspace)
    return WHALE_ERR_NULL;
  if (s.T > 0 && (!H_s || !dK || (!dV && !tied) || !dH_s)) return WHALE_ERR_NULL;
  if (!norm_params_ok(norm, g_q, b_q) || !norm_params_ok(norm, g_kv, b_kv)) return WHALE_ERR_NULL;
  if (norm != WHALE_NORM_NONE) {
    if (!stats_q || (s.T > 0 && !stats_kv) || !dg_q || !dg_kv) return WHALE_ERR_NULL;
    if (norm == WHALE_NORM_LAYER && (!db_q || !db_kv)) return WHALE_ERR_NULL;
  }
  if (ws_bytes < whale_proj_qkv_bwd_workspace_size(dims, dtype)) return WHALE_ERR_WORKSPACE;
  const bool bf = dtype == WHALE_BF16;
  const int d = s.d, nk = (int)norm;
  Carve c(workspace);
  void* WQt = c.take((size_t)d * d * esz(dtype));
  void* WKVt = c.take((size_t)2 * d * d * esz(dtype));
  const size_t p1 = wgrad_partial_bytes(s.M, d, d), p2 = wgrad_partial_bytes(s.T, 2 * d, d, true);
  float* part = (float*)c.take(p1 > p2 ? p1 : p2);
  float* npq = (float*)c.take(norm_part_bytes(s.M, d));
  float* npk = (float*)c.take(norm_part_bytes(s.T, d));
  float* cscr = (float*)c.take((size_t)colsum_scratch_floats(d) * 4);
  void* Xq = c.take((size_t)s.M * d * esz(dtype));
  void* Xs = c.take((size_t)s.T * d * esz(dtype));

  // Weight gradients against the normalised inputs, formed once from the
  // saved statistics; dW_K and dW_V share one pass over X_s.
  const void* Xqin = H_w;
  const void* Xsin = H_s;
  if (norm != WHALE_NORM_NONE) {
    if (X_q_in) {
      Xqin = X_q_in;
    } else {
      WHALE_TRY(launch_norm_apply(H_w, stats_q, nullptr, g_q, b_q, Xq, s.M, d, nk, eps, bf, stream));
      Xqin = Xq;
    }
    if (s.T > 0) {
      if (X_s_in) {
        Xsin = X_s_in;
      } else {
        WHALE_TRY(launch_norm_apply(H_s, stats_kv, nullptr, g_kv, b_kv, Xs, s.T, d, nk, eps, bf, stream));
        Xsin = Xs;
      }
    }
  }
  Wg wq(dQ, d, Xqin, d, WPRO_PLAIN, s.M, d, d, dW_Q, part);
  WHALE_TRY(wq.run(bf, stream));
  if (s.T > 0 && tied) {
    Wg wk(dK, d, Xsin, d, WPRO_PLAIN, s.T, d, d, dW_K, part);
    WHALE_TRY(wk.run(bf, stream));
  } else if (s.T > 0) {
    Wg wkv(dK, d, Xsin, d, WPRO_PLAIN, s.T, 2 * d, d, dW_K, part);
    WHALE_TRY(wkv.dual(dV, d, dW_V).run(bf, stream));
  } else {
    WHALE_TRY(launch_fill_zero(dW_K, (int64_t)d * d, stream));
    if (!tied) WHALE_TRY(launch_fill_zero(dW_V, (int64_t)d * d, stream));
  }
  // dH_w = Norm_q backward(dQ W_Q) + dH_w_in ; dH_s = Norm_kv backward([dK, dV] [W_K; W_V])
  // bf16 at d = 256: the row-streaming kernels (weight slice resident, rows
  // streamed once); their dgamma / dbeta partials are one row per workgroup.
  const bool rs = bf && rs_bwd_ok(d, d) && rs_bwd_ok(2 * d, d);
  auto rs_args = [&](const void* X, const void* X2, const void* Wt, const void* nx, const float* st,
                     const float* g, const void* R, void* out, float* part, int64_t M) {
    RsBwdArgs r;
    r.X = (const __bf16*)X; r.X2 = (const __bf16*)X2; r.ldx = d; r.ldx2 = d; r.ksplit = d;
    r.W = (const __bf16*)Wt; r.nx = (const __bf16*)nx; r.stats = st; r.gamma = g; r.R = (const __bf16*)R;
    r.Y = (__bf16*)out; r.part = part; r.M = M; r.kind = nk;
    return r;
  };
  WHALE_TRY(launch_transpose(W_Q, d, d, WQt, d, 0, bf, stream));
  if (rs)
    WHALE_TRY(launch_rs_bwd(rs_args(dQ, nullptr, WQt, H_w, stats_q, g_q, dH_w_in, dH_w, npq, s.M), d, d, stream));
  else
    WHALE_TRY(norm_bwd_gemm(dQ, d, nullptr, 0, WQt, d, d, H_w, stats_q, g_q, nk, dH_w_in, dH_w, npq, s.M, d, bf,
                            stream));
  if (norm != WHALE_NORM_NONE)
    WHALE_TRY(launch_colsum_reduce(npq, rs ? rs_bwd_grid(s.M) : gemm_norm_bwd_tiles(s.M), d, dg_q,
                                   norm == WHALE_NORM_LAYER ? db_q : nullptr, cscr, stream));
  if (s.T > 0) {
    // dH_s = Norm_kv backward(dK W_K [+ dV W_V]): W^T is [d, 2d] ([d, d] when tied).
    const int kk = tied ? d : 2 * d;
    WHALE_TRY(launch_transpose(W_K, d, d, WKVt, kk, 0, bf, stream));
    if (!tied) WHALE_TRY(launch_transpose(W_V, d, d, WKVt, kk, d, bf, stream));
    if (rs)
      WHALE_TRY(launch_rs_bwd(rs_args(dK, tied ? nullptr : dV, WKVt, H_s, stats_kv, g_kv, nullptr, dH_s, npk, s.T),
                              kk, d, stream));
    else
      WHALE_TRY(norm_bwd_gemm(dK, d, tied ? nullptr : dV, tied ? 0 : d, WKVt, kk, kk, H_s, stats_kv, g_kv, nk,
                              nullptr, dH_s, npk, s.T, d, bf, stream));
    if (norm != WHALE_NORM_NONE)
      WHALE_TRY(launch_colsum_reduce(npk, rs ? rs_bwd_grid(s.T) : gemm_norm_bwd_tiles(s.T), d, dg_kv,
                                     norm == WHALE_NORM_LAYER ? db_kv : nullptr, cscr, stream));
  } else if (norm != WHALE_NORM_NONE) {
    WHALE_TRY(launch_fill_zero(dg_kv, d, stream));
    if (db_kv) WHALE_TRY(launch_fill_zero(db_kv, d, stream));
  }
  if (norm == WHALE_NORM_RMS) {
    if (db_q) WHALE_TRY(launch_fill_zero(db_q, d, stream));
    if (db_kv) WHALE_TRY(launch_fill_zero(db_kv, d, stream));
  }
  return WHALE_OK;
}

}  // extern "C"
