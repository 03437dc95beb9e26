/*
 * libwhalefuse -- the per-layer attention-fusion module of the WHALE
 * recommender on AMD MI355X (gfx950), as a C ABI.
 *
 * Sources (web pages about arXiv 2607.17017, "WHALE: A Scalable Unified Model
 * for Recommendation with Wukong-HSTU Architecture"):
 *   [GS 2.1]  gist.science explainer, Technical Summary §2.1 (Core
 *             Architecture, "Attention-Based Fusion Module")
 *   [GS 2.2]  gist.science explainer, Technical Summary §2.2 (Efficiency
 *             Optimizations: shared key-value, asymmetric backward
 *             variants, shared-gate SwiGLU, BF16 mixed precision, shape-hint
 *             tensors)
 *   [PD 2]    paper-daily.com deep reading of WHALE, §2 (method details;
 *             query-dimension split of the backward)
 *   [PV km]   pith.science verdict record, pith_extraction.key_machinery
 *   [PV ref]  pith.science verdict record, referee_report (minor comments on
 *             Eq. (4), Eq. (5); major comment on §5.1 / Footnote 1)
 *
 * Notation: B requests, C candidates per request, n_q query (interaction)
 * tokens per candidate, width d, h heads of width d_h = d / h, L_b the
 * history length of request b, T = sum_b L_b, M = B*C*n_q.  The FFN hidden
 * width is H.
 *
 * Layouts (all row-major, row-vector convention y = x W^T, every weight
 * stored [out, in] as in torch.nn.Linear):
 *   H_w, Q, A, F, Y, Z  [M, d]      row m = (b*C + c)*n_q + i
 *   H_s, K, V           [T, d]      request b owns rows offsets[b] .. offsets[b+1]-1
 *   offsets             int64 [B+1] offsets[0] = 0, non-decreasing, offsets[B] = T
 *   lse                 fp32 [M, h] natural log of each softmax denominator
 *   stats_*             fp32 [rows, 2]  (mean, 1/sqrt(var + eps)) per row;
 *                       mean is 0 for RMSNorm
 *   W_Q, W_K, W_V [d, d]; W_F [d, 2d]; W_U [H, d] (shared gate) or [2H, d]
 *   holding [W_G; W_U] (separate gate); W_D [d, H]; U [M, H] or [M, 2H]
 *   Head j of Q, K, V, A is the column slice j*d_h .. (j+1)*d_h - 1.
 *
 * Conventions common to every call:
 *   - Data pointers are device pointers; `dims` is host memory.  The data
 *     type of activations and weights is `dtype` (fp32 or bf16).  Norm
 *     parameters gamma/beta, lse, statistics and weight gradients are
 *     always fp32; workspaces are opaque device memory.
 *   - The caller allocates every buffer; the library allocates nothing and
 *     keeps no state besides its compiled kernels.  Outputs must not alias
 *     inputs.  Weight and gamma/beta gradients are written, not accumulated.
 *   - Every call only enqueues work on `stream` and returns; none reads
 *     device memory on the host or synchronises.  The host shape hints
 *     dims->max_L and dims->total_L stand in for any device-to-host read of
 *     the offsets ("shape hint tensors", [GS 2.2]).  The caller guarantees
 *     that the offsets are consistent with them (offsets[0] == 0,
 *     non-decreasing, every L_b <= max_L, offsets[B] == total_L).  Grids are
 *     sized from the hints and rows indexed by the offsets, so inconsistent
 *     offsets give wrong results or out-of-range reads.  whale_validate_offsets
 *     checks them on the device; in debug mode (below) every attention call
 *     checks them first and skips its kernels when they fail.
 *   - Errors found on the host return before anything is enqueued: a NULL
 *     required pointer (WHALE_ERR_NULL), inconsistent sizes (WHALE_ERR_SHAPE,
 *     e.g. d % h != 0, M == 0), an unknown dtype (WHALE_ERR_DTYPE), a shape
 *     the kernels do not implement (WHALE_ERR_UNSUPPORTED: d_h not in
 *     {32, 64, 128}, d not in {64, 128, 256, 512}, H not a multiple of 64), or a workspace
 *     smaller than the size query returns (WHALE_ERR_WORKSPACE).  A failed kernel launch returns WHALE_ERR_LAUNCH.
 *   - Results are bitwise reproducible for fixed inputs, dims and device:
 *     no atomics, every reduction runs in a fixed order.
 *   - Arithmetic: products accumulate in fp32 (bf16 MFMA operands for
 *     bf16, fp32 MFMA operands for fp32); softmax and norm statistics are
 *     fp32; every stored bf16 value is rounded to nearest even.
 */
#ifndef WHALEFUSE_H
#define WHALEFUSE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct whale_dims {
  int32_t B, C, n_q, d, h;
  int32_t max_L;    /* host shape hint: max over b of L_b */
  int64_t total_L;  /* host shape hint: T = offsets[B] */
} whale_dims_t;

typedef enum { WHALE_F32 = 0, WHALE_BF16 = 1 } whale_dtype_t;
typedef enum { WHALE_NORM_LAYER = 0, WHALE_NORM_RMS = 1, WHALE_NORM_NONE = 2 } whale_norm_t;
typedef enum { WHALE_ACT_SILU = 0, WHALE_ACT_NONE = 1 } whale_act_t;
typedef enum { WHALE_GATE_SHARED = 0, WHALE_GATE_SEPARATE = 1 } whale_gate_t;
typedef enum {
  WHALE_OK = 0,
  WHALE_ERR_NULL = 1,
  WHALE_ERR_SHAPE = 2,
  WHALE_ERR_DTYPE = 3,
  WHALE_ERR_UNSUPPORTED = 4,
  WHALE_ERR_WORKSPACE = 5,
  WHALE_ERR_LAUNCH = 6
} whale_status_t;

/* Human-readable name of a status code (static storage, never NULL). */
const char* whale_status_string(whale_status_t status);

/* Library version string, "major.minor.patch". */
const char* whale_version(void);

/* ------------------------------------------------- offset validation */

/* Bits of the validation flag (0: the offsets satisfy the hints). */
#define WHALE_BAD_FIRST 1        /* offsets[0] != 0 */
#define WHALE_BAD_ORDER 2        /* offsets[b+1] < offsets[b] for some b */
#define WHALE_BAD_MAX_L 4        /* offsets[b+1] - offsets[b] > max_L for some b */
#define WHALE_BAD_TOTAL 8        /* offsets[B] != total_L */
#define WHALE_BAD_CAND_FIRST 16  /* cand_offsets[0] != 0 */
#define WHALE_BAD_CAND_ORDER 32  /* cand_offsets decrease somewhere */
#define WHALE_BAD_MAX_C 64       /* cand_offsets[b+1] - cand_offsets[b] > C for some b */
#define WHALE_BAD_TIME 128       /* a timestamp differs from its request's first by 2^30 or more */

/*
 * Checks the jagged offsets [B+1] (and, if not NULL, the candidate offsets
 * [B+1] of the serving form) against the host shape hints dims->max_L,
 * dims->total_L and dims->C, on the device: the shape hints replace any read
 * of the offsets on the host ([GS 2.2], "shape hint tensors"), so their
 * consistency can only be checked there.  One small kernel on `stream`
 * writes the bitmask of the violations found (WHALE_BAD_*) to *flag, an
 * int32 in device memory owned by the caller (overwritten, not accumulated).
 * Only dims->B, C, max_L and total_L are read.  Asynchronous: read *flag
 * after synchronising the stream.  WHALE_ERR_NULL for a NULL dims, offsets
 * or flag; WHALE_ERR_SHAPE for B <= 0, C <= 0 or negative hints.
 */
whale_status_t whale_validate_offsets(const whale_dims_t* dims, const int64_t* offsets, const int64_t* cand_offsets,
                                      int32_t* flag, hipStream_t stream);

/*
 * The same check as whale_validate_offsets (without candidate offsets),
 * plus the contract of whale_hstu_attn_fwd on the timestamps [total_L]:
 * every timestamp of request b differs from the request's first one by less
 * than 2^30 (WHALE_BAD_TIME otherwise).  Rows outside [0, total_L) are never
 * read: offsets that leave it are reported by the offsets bits.  *flag
 * (device int32, caller-owned) is overwritten.  Asynchronous on `stream`.
 * WHALE_ERR_NULL for a NULL dims, offsets, timestamps or flag;
 * WHALE_ERR_SHAPE as whale_validate_offsets.
 */
whale_status_t whale_validate_timestamps(const whale_dims_t* dims, const int64_t* offsets, const int64_t* timestamps,
                                         int32_t* flag, hipStream_t stream);

/*
 * Debug mode, for all GPUs of the process: enable != 0 turns it on, 0 off;
 * returns the previous setting.  It starts on when the environment variable
 * WHALE_DEBUG_CHECKS is set to a value other than "" or "0" when the first
 * call is made.  In debug mode whale_jagged_xattn_fwd, _fwd_varc, _bwd and
 * whale_hstu_attn_fwd (which also checks its timestamps, as
 * whale_validate_timestamps) first run the check of whale_validate_offsets
 * into a flag the library
 * keeps on each GPU (a small static device array, the only state the library
 * holds), and their kernels return without touching any output when it
 * reports a violation: nothing is read past the buffers the hints describe,
 * and the outputs keep whatever they held.  Calls in debug mode on one GPU
 * share that flag, so they must not overlap across streams.
 */
int32_t whale_debug_checks(int32_t enable);

/*
 * Debug mode: writes the OR of every check made since the last reset to
 * *flag (device int32, caller-owned), then clears the library's flags when
 * reset != 0.  Asynchronous on `stream`.  WHALE_ERR_NULL for a NULL flag.
 */
whale_status_t whale_debug_status(int32_t* flag, int32_t reset, hipStream_t stream);

/* ---------------------------------------------------------------- forward */

/*
 * a1 + a2: Q = Norm_q(H_w) W_Q^T over the M query rows, and K = Norm_kv(H_s)
 * W_K^T, V = Norm_kv(H_s) W_V^T over the T history rows, once per history
 * row and shared by all C candidates of the request ([PV km]: the Wukong
 * output is normalised and projected into queries, the HSTU output into
 * shared keys and values; [PV ref] Footnote 1: K/V amortised per request).
 *
 * norm: LayerNorm (biased variance, eps inside the root, then gamma, beta),
 * RMSNorm (gamma only; beta ignored and may be NULL) or none (gamma, beta
 * ignored).  g_q/b_q and g_kv/b_kv are fp32 [d].  stats_q [M,2] and
 * stats_kv [T,2] receive the row statistics; both are required unless norm
 * is none (whale_proj_qkv_bwd consumes them).  T may be 0.
 *
 * X_q [M,d] and X_s [T,d] (data dtype, may be NULL; unused for norm none)
 * receive the normalised inputs Norm_q(H_w) and Norm_kv(H_s).  Given, they
 * are written once and the projections read them; NULL, the projections
 * normalise their input tiles on the fly.  Passing them on to
 * whale_proj_qkv_bwd saves the backward from forming them again.
 *
 * Shared key-value form ([GS 2.2]: one tensor serves as keys and values,
 * which halves the history-side memory traffic): W_V and V both NULL.  Only
 * K = Norm_kv(H_s) W_K^T is computed, and the caller passes K as both K and
 * V to the attention calls.  Exactly one of W_V, V NULL is WHALE_ERR_NULL.
 */
whale_status_t whale_proj_qkv(const whale_dims_t* dims, whale_dtype_t dtype,
                              const void* H_w, const void* H_s,
                              whale_norm_t norm, float eps,
                              const float* g_q, const float* b_q,
                              const float* g_kv, const float* b_kv,
                              const void* W_Q, const void* W_K, const void* W_V,
                              void* Q, void* K, void* V,
                              float* stats_q, float* stats_kv,
                              void* X_q, void* X_s, hipStream_t stream);

/*
 * a3, Eq. (4): jagged softmax cross-attention.  For request b, head j and
 * each of its C*n_q query rows m:  s_l = scale * <Q[m, j], K[l, j]> for
 * l in [offsets[b], offsets[b+1]),  A[m, j] = sum_l softmax(s)_l V[l, j],
 * lse[m, j] = log sum_l exp(s_l).  No mask besides the jagged length
 * ([PV km]: one history-derived vector per interaction token; [PD 2]:
 * dot-product attention; [GS 2.1]: Wukong queries, HSTU keys/values).
 * All C*n_q queries of a request read the same K/V rows: each K/V tile is
 * staged once per workgroup and reused by all of its queries.
 * scale == 0 selects 1/sqrt(d_h).  An empty history (L_b = 0) gives A = 0
 * and lse = -inf.  lse may be NULL.  K and V may be the same buffer (the
 * shared key-value form of whale_proj_qkv).
 */
whale_status_t whale_jagged_xattn_fwd(const whale_dims_t* dims, whale_dtype_t dtype,
                                      const void* Q, const void* K, const void* V,
                                      const int64_t* offsets, float scale,
                                      void* A, float* lse, hipStream_t stream);

/*
 * a3 for serving, with a different number of candidates per request
 * ([PV ref] major comment on §5.1 / Footnote 1: K/V are formed once per
 * request and amortised over however many candidates it scores).
 * cand_offsets (device int64 [B+1], cand_offsets[0] = 0, non-decreasing)
 * gives request b the C_b = cand_offsets[b+1] - cand_offsets[b] >= 0
 * candidates whose query rows are n_q*cand_offsets[b] .. n_q*cand_offsets[b+1]-1
 * of Q, A and lse ([n_q*cand_offsets[B], d] and [.., h]).  dims->C is a
 * host shape hint: the largest C_b (the caller guarantees every C_b <=
 * dims->C; rows of a larger request past it are not written).  Otherwise as
 * whale_jagged_xattn_fwd: the same kernels, each row attending its own
 * request's history.  A request with C_b = 0 has no rows; micro-batches of
 * one request's candidates can each be run against the same K/V.
 */
whale_status_t whale_jagged_xattn_fwd_varc(const whale_dims_t* dims, whale_dtype_t dtype,
                                           const void* Q, const void* K, const void* V,
                                           const int64_t* offsets, const int64_t* cand_offsets,
                                           float scale, void* A, float* lse, hipStream_t stream);

/*
 * a4, Eq. (5): F = H_w + act([A, H_w] W_F^T): one linear layer from the
 * concatenation (attended vector first) to d, plus the residual
 * ([GS 2.1]; [PV ref] minor comment on Eq. (5); [PV km]).  act is SiLU or
 * none.  Z_saved [M, d], when non-NULL and act is SiLU, receives the
 * pre-activation Z = [A, H_w] W_F^T (needed by whale_fusion_mlp_bwd).
 */
whale_status_t whale_fusion_mlp(const whale_dims_t* dims, whale_dtype_t dtype,
                                const void* A, const void* H_w, const void* W_F,
                                whale_act_t act, void* F, void* Z_saved, hipStream_t stream);

/*
 * a5: pre-norm SwiGLU FFN with residual: X_f = Norm_f(F), U = X_f W_U^T,
 * Y = F + G W_D^T, with G = SiLU(U) * U for the shared gate (W_gate = W_up,
 * two matrix products instead of three, [GS 2.2], [PD 2]) or
 * G = SiLU(U_g) * U_u for the separate gate (one merged product with the
 * stacked [W_G; W_U], 2H rows).  U_saved ([M, H] or [M, 2H], columns
 * [U_g | U_u] for the separate gate) is written when non-NULL; stats_f
 * ([M, 2]) is required unless norm is none.  The backward needs both.
 * X_f ([M, d], data type, may be NULL; unused for norm none) receives
 * Norm_f(F); passing it on to whale_swiglu_ffn_bwd saves the backward from
 * forming it again.
 * workspace: at least whale_swiglu_ffn_workspace_size(...) bytes of device
 * memory (holds G).  Requires H % 64 == 0.
 */
size_t whale_swiglu_ffn_workspace_size(const whale_dims_t* dims, whale_dtype_t dtype,
                                       whale_gate_t gate, int32_t H);
whale_status_t whale_swiglu_ffn(const whale_dims_t* dims, whale_dtype_t dtype,
                                const void* F, whale_norm_t norm, float eps,
                                const float* g_f, const float* b_f,
                                const void* W_U, whale_gate_t gate, int32_t H, const void* W_D,
                                void* Y, void* U_saved, float* stats_f, void* X_f,
                                void* workspace, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------- backward */

/*
 * a6: attention backward, split along the query dimension ([PD 2]: the
 * backward is split on the query axis; [GS 2.2]: Q-parallel and
 * KV-parallel schedules).  With P recomputed from lse:
 *   D_m = <dA[m, j], A[m, j]>,  dP = dA V^T,  dS = P * (dP - D),
 *   dQ = scale dS K,  dK = scale dS^T Q,  dV = P^T dA,
 * where dK and dV sum over all C*n_q queries of the request (the gradient
 * of K/V shared across candidates).  dQ comes from a Q-parallel kernel
 * with no reduction; dK/dV from a kernel parallel over K/V tiles and over
 * query splits, whose fp32 partials are summed in a fixed order.
 * lse must be the forward's.  workspace: at least
 * whale_jagged_xattn_bwd_workspace_size(dims, dtype) bytes of device memory
 * (contents on entry do not matter; it holds D, the fp32 partials and, for
 * jagged batches of at most 256 requests, their longest-first order).
 * Both attention calls run the work of such batches longest history first;
 * the order changes no result bit.
 * Shared key-value form: V == K and dV NULL; dK then receives the gradient
 * of the one tensor, scale dS^T Q + P^T dA, summed in fp32 and rounded
 * once.  dV NULL with V != K is WHALE_ERR_SHAPE.
 */
size_t whale_jagged_xattn_bwd_workspace_size(const whale_dims_t* dims, whale_dtype_t dtype);
whale_status_t whale_jagged_xattn_bwd(const whale_dims_t* dims, whale_dtype_t dtype,
                                      const void* Q, const void* K, const void* V,
                                      const int64_t* offsets, float scale,
                                      const void* A, const float* lse, const void* dA,
                                      void* dQ, void* dK, void* dV,
                                      void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * a7 (fusion MLP): chain rule of whale_fusion_mlp.  dZ = dF * act'(Z);
 * dW_F = dZ^T [A, H_w] (fp32 [d, 2d]); dA = dZ W_F[:, :d];
 * dH_w = dF + dZ W_F[:, d:].  Z_saved is required for SiLU, ignored for none.
 */
/* ------------------------------------------------- HSTU self-attention */

/*
 * NEXT f4: the HSTU module's jagged self-attention over each request's own
 * history, which produces the states H_s the fusion attention reads ([PV km]:
 * a sequential attention block with relative position-and-time biases;
 * [GS 2.1]).  The pages leave the bias rab(p, t) undefined (pith.science
 * review page, referee minor comment on Eq. (2), pointing to the HSTU paper,
 * their reference [34]); this call computes the reading
 *   A[lo_b + i, head] = (1 / L_b) * sum over j <= i of
 *                       SiLU(scale * <Q_i, K_j> + w_pos[min(i - j, n_pos - 1)]
 *                            + w_time[min(floor(log2(max(tau_i - tau_j, 1))), n_time - 1)]) * V_j
 * for rows i, j of request b (0 <= i, j < L_b; tau = timestamps), per head
 * (columns head*d_h .. head*d_h + d_h - 1), with both tables shared by all
 * heads: causal, pointwise (SiLU instead of a softmax), normalised by the
 * request's length.
 *
 * Q, K, V, A: [T, d] in dtype (T = dims->total_L; all rows are history rows);
 * offsets [B+1] int64; timestamps [T] int64; w_pos [n_pos] and w_time
 * [n_time] fp32.  scale == 0 selects 1/sqrt(d_h).  Only dims->B, d, h, max_L
 * and total_L are used (C and n_q must be positive; pass 1).  Contract:
 * every timestamp of a request differs from the request's first one by less
 * than 2^30 (time differences are exact in 32-bit integers).  1 <= n_pos <=
 * 4096 and 1 <= n_time <= 32, else WHALE_ERR_UNSUPPORTED.  An empty request
 * leaves no rows.  Forward only.
 */
whale_status_t whale_hstu_attn_fwd(const whale_dims_t* dims, whale_dtype_t dtype,
                                   const void* Q, const void* K, const void* V,
                                   const int64_t* offsets, const int64_t* timestamps,
                                   const float* w_pos, int32_t n_pos, const float* w_time,
                                   int32_t n_time, float scale, void* A, hipStream_t stream);

/*
 * For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): whale_jagged_xattn_bwd
 * without a workspace argument.  Same arguments otherwise, same kernels and
 * the same results bit for bit.  The workspace comes from a static device
 * array of 32 MiB (33554432 bytes) that each GPU the library runs on holds
 * from module load until the process ends; the call itself allocates
 * nothing.  A shape whose
 * whale_jagged_xattn_bwd_workspace_size exceeds that returns
 * WHALE_ERR_WORKSPACE before anything is enqueued (the fixed-count layout
 * needs M*h*4 bytes, plus S*2*T*d*4 when the dK/dV query split S > 1 is
 * chosen for short histories).  Every call on a GPU shares that GPU's array:
 * calls that overlap on one GPU (different streams, or graphs replayed
 * concurrently) race and give wrong results.  Nothing in the array needs to
 * start at zero: each byte a kernel reads is written earlier in the call.
 */
whale_status_t whale_jagged_xattn_bwd_noalloc(const whale_dims_t* dims, whale_dtype_t dtype,
                                              const void* Q, const void* K, const void* V,
                                              const int64_t* offsets, float scale, const void* A,
                                              const float* lse, const void* dA, void* dQ, void* dK,
                                              void* dV, hipStream_t stream);

size_t whale_fusion_mlp_bwd_workspace_size(const whale_dims_t* dims, whale_dtype_t dtype);
whale_status_t whale_fusion_mlp_bwd(const whale_dims_t* dims, whale_dtype_t dtype,
                                    const void* A, const void* H_w, const void* W_F,
                                    whale_act_t act, const void* Z_saved, const void* dF,
                                    void* dA, void* dH_w, float* dW_F,
                                    void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * a7 (FFN): chain rule of whale_swiglu_ffn.  dW_D = dY^T G; dG = dY W_D;
 * dU from the gate derivative; dW_U = dU^T X_f; dX_f = dU W_U;
 * dF = dY + Norm_f backward(dX_f); dg_f/db_f are the norm parameter
 * gradients (db_f is zero for RMSNorm; neither is written, and both may be
 * NULL, for norm none).  U_saved and stats_f come from the forward (stats_f
 * may be NULL only for norm none).  X_f: the forward's Norm_f(F) if it wrote
 * it, else NULL (it is then formed again in the workspace).  Weight and norm
 * parameter gradients are fp32.
 */
size_t whale_swiglu_ffn_bwd_workspace_size(const whale_dims_t* dims, whale_dtype_t dtype,
                                           whale_gate_t gate, int32_t H);
whale_status_t whale_swiglu_ffn_bwd(const whale_dims_t* dims, whale_dtype_t dtype,
                                    const void* F, whale_norm_t norm, float eps,
                                    const float* g_f, const float* b_f, const float* stats_f,
                                    const void* W_U, whale_gate_t gate, int32_t H, const void* W_D,
                                    const void* U_saved, const void* X_f, const void* dY,
                                    void* dF, float* dW_U, float* dW_D, float* dg_f, float* db_f,
                                    void* workspace, size_t ws_bytes, hipStream_t stream);

/*
 * a7 (projections): chain rule of whale_proj_qkv.  dW_Q = dQ^T X_q,
 * dW_K = dK^T X_s, dW_V = dV^T X_s (fp32 [d, d]); dX_q = dQ W_Q;
 * dX_s = dK W_K + dV W_V; dH_w = Norm_q backward(dX_q) (+ dH_w_in when
 * non-NULL: the caller passes the fusion-MLP part of dH_w here to get the
 * total), dH_s = Norm_kv backward(dX_s); norm parameter gradients fp32 [d].
 * stats_q / stats_kv come from the forward (may be NULL only for norm none;
 * the norm parameter gradients are then not written and may be NULL).
 * X_q / X_s: the forward's normalised inputs if it wrote them, else NULL
 * (they are then formed again in the workspace).
 * Shared key-value form: W_V, dV and dW_V all NULL; dK is then the gradient
 * of the one tensor (from whale_jagged_xattn_bwd with dV NULL), and
 * dW_K = dK^T X_s, dX_s = dK W_K.  Some but not all three NULL is
 * WHALE_ERR_NULL.
 */
size_t whale_proj_qkv_bwd_workspace_size(const whale_dims_t* dims, whale_dtype_t dtype);
whale_status_t whale_proj_qkv_bwd(const whale_dims_t* dims, whale_dtype_t dtype,
                                  const void* H_w, const void* H_s,
                                  whale_norm_t norm, float eps,
                                  const float* g_q, const float* b_q,
                                  const float* g_kv, const float* b_kv,
                                  const float* stats_q, const float* stats_kv,
                                  const void* X_q, const void* X_s,
                                  const void* W_Q, const void* W_K, const void* W_V,
                                  const void* dQ, const void* dK, const void* dV,
                                  const void* dH_w_in,
                                  void* dH_w, void* dH_s,
                                  float* dW_Q, float* dW_K, float* dW_V,
                                  float* dg_q, float* db_q, float* dg_kv, float* db_kv,
                                  void* workspace, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------- diagnostics */

/*
 * Matrix-core rate probe (not part of the module): blocks workgroups of 256
 * threads, each wave running iters steps of four independent
 * v_mfma_f32_32x32x16_bf16 chains on register operands, with no memory
 * traffic besides one float per thread written to out [blocks * 256].  It
 * does blocks * 4 * iters * 4 * 32768 FLOPs; timed by the caller, it gives
 * the bf16 MFMA rate the GPU sustains, a measured ceiling beside the
 * data-sheet peak.  WHALE_ERR_NULL for out NULL, WHALE_ERR_SHAPE for
 * iters < 1 or blocks < 1.
 */
whale_status_t whale_mfma_peak_probe(float* out, int32_t iters, int32_t blocks, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* WHALEFUSE_H */
