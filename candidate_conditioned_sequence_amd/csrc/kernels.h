// Internal launcher interface between the C ABI (api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// ---------------------------------------------------------------- attention
struct XattnArgs {
  const void* Q; const void* K; const void* V; const int64_t* offsets;
  void* A; float* lse;
  int B, QR /* C*n_q (the largest over requests with cand_offsets) */, d, h, dh;
  float scale;
  // Optional candidate offsets [B+1]: request b owns query rows
  // n_q*cand_offsets[b] .. n_q*cand_offsets[b+1]-1 (nullptr: b*QR .. (b+1)*QR-1).
  const int64_t* cand_offsets;
  int n_q;
  // Debug mode: a device flag written by the offset validator just before;
  // every kernel of the call returns at once when it is non-zero.  nullptr
  // otherwise.
  const int32_t* guard = nullptr;
  // Run the work longest history first (set for batches of at most
  // kRankMaxB requests whose lengths are not all equal).
  bool rank_order = false;
};
hipError_t launch_xattn_fwd(const XattnArgs& a, bool bf16_data, hipStream_t st);

// Jagged batches of at most kRankMaxB requests run the attention kernels'
// work longest history first: the forward and dQ kernels rank the requests
// in each workgroup, and the dQ kernel leaves the order in perm for the
// dK/dV kernel.  The shape hints tell the host when every history has the
// same length (total_L = B max_L), and then the index order is kept.
constexpr int kRankMaxB = 256;

struct XattnBwdArgs {
  const void* Q; const void* K; const void* V; const int64_t* offsets;
  const void* A; const float* lse; const void* dA;
  void* dQ; void* dK; void* dV;
  float* Dbuf;          // [M, h] fp32: rowsum(dA * A) per head
  float* partial;       // [S, T, 2, d] fp32 dK/dV partials (S > 1 only)
  int B, QR, d, h, dh, max_L, splits;
  int64_t T;
  float scale;
  const int32_t* guard = nullptr;   // as in XattnArgs
  // KV-parallel schedule of the whole backward (one kernel forms dK, dV and
  // dQ); qpartial [nkt, M, d] fp32 holds its dQ block partials when a
  // history spans more than one 128-row block.
  bool kv_schedule = false;
  float* qpartial = nullptr;
  int32_t* perm = nullptr;   // [B] longest-first order, written by the dQ kernel (nullptr: index order)
};
hipError_t launch_xattn_bwd(const XattnBwdArgs& a, bool bf16_data, hipStream_t st);
int xattn_bwd_splits(int B, int h, int QR, int max_L, int dh);
// Schedule choice (env WHALE_XATTN_BWD_SCHEDULE = "kv" / "q" forces one).
bool xattn_bwd_kv_schedule(int max_L, int dh, bool bf16_data);
int64_t xattn_bwd_kv_qpartial_floats(int64_t M, int d, int max_L);

// ------------------------------------------------ HSTU self-attention
// A [T, d] = causal SiLU self-attention with relative position / time bias
// per request and head (see hstu.hip).  n_pos <= hstu_max_pos(),
// 1 <= n_time <= 32.
struct HstuArgs {
  const void* Q; const void* K; const void* V; const int64_t* offsets; const int64_t* timestamps;
  const float* w_pos; int n_pos; const float* w_time; int n_time;
  void* A;
  int B, d, h, dh, max_L;
  float scale;
  const int32_t* guard = nullptr;   // as in XattnArgs
};
hipError_t launch_hstu_fwd(const HstuArgs& a, bool bf16_data, hipStream_t st);
int hstu_max_pos();

// ---------------------------------------------------------------- norms
// Row statistics (mean, rstd) of x [rows, n]; mean = 0 for RMSNorm.
// kind: 0 LayerNorm, 1 RMSNorm.
// y = Norm(x) (gamma, beta applied; beta ignored for RMSNorm).  stats_in
// given: use those statistics; else compute them (and write stats_out if
// given).  kind: 0 LayerNorm, 1 RMSNorm.
hipError_t launch_norm_apply(const void* x, const float* stats_in, float* stats_out, const float* gamma,
                             const float* beta, void* y, int64_t rows, int n, int kind, float eps, bool bf16_data,
                             hipStream_t st);
// dZ = dF * SiLU'(Z) over n elements (n % 8 == 0).
hipError_t launch_dact(const void* dF, const void* Z, void* dZ, int64_t n, bool bf16_data, hipStream_t st);
hipError_t launch_norm_stats(const void* x, float* stats, int64_t rows, int n, int kind, float eps,
                             bool bf16_data, hipStream_t st);
// Column sums of per-tile partials part [nblk, 2, n] (row 0: dgamma terms,
// row 1: dbeta terms) in a fixed order; scratch holds colsum_scratch_floats(n).
hipError_t launch_colsum_reduce(const float* part, int64_t nblk, int n, float* dgamma, float* dbeta,
                                float* scratch, hipStream_t st);
int64_t colsum_scratch_floats(int n);

// ---------------------------------------------------------------- GEMMs
// Y[M,N] = op(X)[M,K] * W[N,K]^T with optional prologue on X and epilogue.
enum GemmPro {
  PRO_PLAIN = 0,
  PRO_NORM = 1,          // X rows normalised with stats + gamma/beta (norm_kind 0/1; 2 = none)
  PRO_CONCAT = 2,        // columns >= ksplit come from X2 (multiple of 64)
  PRO_DACT = 3,          // X = X * SiLU'(X2) elementwise (dZ from dF and Z)
  PRO_GATE = 4           // X = SiLU(X) * X elementwise (the tied gate from its saved product; EPI_RESID only)
};
enum GemmEpi {
  EPI_STORE = 0,         // Y = acc; with Y2: columns >= nsplit go to Y2 (column - nsplit)
  EPI_RESID = 1,         // Y = R + acc
  EPI_SILU_RESID = 2,    // Y = R + silu(acc); Z = acc (optional)
  EPI_GATE_TIED = 3,     // Y = silu(acc) * acc; Z = acc (optional)
  EPI_GATE_SEP = 4,      // W has N = 2H rows [W_G; W_U]: Y = silu(acc_g) * acc_u; Z = [acc_g | acc_u] (optional)
  EPI_DGATE_TIED = 5,    // Y = acc * (silu'(u) u + silu(u)), u = Z (input)
  EPI_DGATE_SEP = 6,     // Y[:, :N] = acc * u_u * silu'(u_g), Y[:, N:2N] = acc * silu(u_g), Z = [u_g | u_u]
  EPI_DUAL_RESID2 = 7,   // columns < nsplit: Y = acc; columns >= nsplit: Y2 = R + acc
  EPI_NORM_BWD = 8       // row-complete tiles: acc = dL/d(norm output); Y = norm backward (+ R);
                         // per-tile column partials of dgamma/dbeta into part [tiles_m, 2, N]
};
struct GemmArgs {
  const void* X; int ldx;          // plain / norm source, or first half of a concat
  const void* X2; int ldx2; int ksplit;   // concat second half, or Z for PRO_DACT
  const float* stats; const float* gamma; const float* beta; int norm_kind;  // PRO_NORM / EPI_NORM_BWD
  const void* W; int ldw;          // [N, K] row-major
  const void* W2; int nsplit;      // rows >= nsplit come from W2 (row - nsplit)
  void* Y; int ldy; bool y_f32;    // output (fp32 or data type)
  void* Y2;                        // second output (EPI_STORE / EPI_DUAL_RESID2)
  const void* R; int ldr;          // residual
  void* Z; int ldz;                // saved pre-activation (output) or gate input (DGATE)
  const void* nx;                  // EPI_NORM_BWD: the norm's input rows [M, N]
  float* part;                     // EPI_NORM_BWD: column partials [tiles_m, 2, N]
  int64_t M; int N; int K;
  int pro, epi;
};
hipError_t launch_gemm_nt(const GemmArgs& a, bool bf16_data, hipStream_t st);
inline int64_t gemm_norm_bwd_tiles(int64_t M) { return (M + 63) / 64; }

// ------------------------------------------------ row-streaming projections
// bf16 only.  Forward: Y = Norm(H) W^T for H [M, K] (row stride ldh); weight
// rows [0, nsplit) come from W and write Y, rows [nsplit, N) come from W2
// and write Y2 (both [*, K]; outputs with row stride ldy).  With kind 0/1
// the rows are normalised (gamma, beta over K; beta unused for kind 1) and
// the normalised rows go to Xn [M, K] and (mean, rstd) to stats [M, 2] when
// those are given (by column group 0); kind 2 multiplies H as it is.
// Shapes: rs_fwd_ok(K, N); at K = 512 (gate 0, norm allowed) also N = 256
// per column group with ngroups > 1 (rs_fwd_groups_ok(K, ngroups N)).
struct RsFwdArgs {
  const __bf16* H; int64_t ldh;
  const __bf16* H2; int64_t ldh2;   // gate = 4: columns [256, 512) of the rows
  const __bf16* W; const __bf16* W2; int nsplit;
  __bf16* Y; __bf16* Y2; int64_t ldy;
  __bf16* Xn; float* stats;
  const float* gamma; const float* beta;
  int64_t M; int kind; float eps;
  // gate = 1: the tied SwiGLU gate.  W has ngroups * N rows (N per column
  // group), Z [M, ngroups N] (row stride ldz) receives the product and Y the
  // gated U = SiLU(Z) Z; either may be null; W2 / Y2 / nsplit unused
  // (nsplit = N).
  // gate = 2: its backward (kind 2): Y = (H W^T) * (SiLU'(Z) Z + SiLU(Z))
  // with Z the saved product (input, required); the product is rounded to
  // bf16 once before the scaling.
  // gate = 3: the fusion MLP's backward (kind 2, ngroups 1): H = dF, Z the
  // saved pre-activation (input, row stride ldz); Xn receives dZ = dF SiLU'(Z)
  // (required), Y = dZ W^T for rows < nsplit of W, Y2 = dF + dZ W2^T.
  // gate = 4: the fusion MLP (K = 512, N = 256, kind 2): P = [H | H2] W^T,
  // Y = H2 + SiLU(P), Z = P when non-null.  Shapes for gate 0 to 3:
  // K = 256; gate 4: K = 512, N = 256.
  int gate; int ngroups; __bf16* Z; int64_t ldz;
};
// Backward: dX [M, N] = Norm backward(dY W^T) + R with dY = [X | X2] split at
// ksplit = 256 along K (X2 only for K = 512), W [N, K] (the transposed forward weight),
// nx [M, N] the norm's input, stats its (mean, rstd), gamma [N]; R [M, N] may
// be null (and must be at K = 512).  Column partials of dgamma / dbeta go to part [rs_bwd_grid(M), 2, N]
// (kind 0/1).  Shapes: rs_bwd_ok(K, N).
struct RsBwdArgs {
  const __bf16* X; const __bf16* X2; int64_t ldx, ldx2; int ksplit;
  const __bf16* W;
  const __bf16* nx; const float* stats; const float* gamma;
  const __bf16* R;
  __bf16* Y; float* part;
  int64_t M; int kind;
};
bool rs_fwd_ok(int K, int N);
bool rs_fwd_groups_ok(int K, int Ntot);   // K = 512, Ntot a multiple of 256 (column groups of 256)
bool rs_bwd_ok(int K, int N);
int64_t rs_bwd_grid(int64_t M);
hipError_t launch_rs_fwd(const RsFwdArgs& a, int K, int N, hipStream_t st);
hipError_t launch_rs_bwd(const RsBwdArgs& a, int K, int N, hipStream_t st);

// dW[N,K] = sum_m G[m,n] * Xop[m,k], fp32, with optional prologue on Xop
// (norm of X, concat [X | X2], or tied/separate gate recomputed from U) and
// on G (G * SiLU'(Gz) when Gz is set).  With G2, columns >= nsplit of G come
// from G2 and rows >= nsplit of the result go to dW2.
enum WgradPro { WPRO_PLAIN = 0, WPRO_NORM = 1, WPRO_CONCAT = 2, WPRO_GATE_TIED = 3, WPRO_GATE_SEP = 4 };
struct WgradArgs {
  const void* G; int ldg;          // [M, N]
  const void* G2; int nsplit;      // dual G
  const void* Gz;                  // G prologue: G * SiLU'(Gz)
  const void* X; int ldx;          // [M, K] (or U for the gate prologues)
  const void* X2; int ldx2; int ksplit;
  const float* stats; const float* gamma; const float* beta; int norm_kind;
  int gate_H;                      // WPRO_GATE_SEP: gate columns [0,H), up columns [H,2H) of X
  float* dW; float* dW2;           // [N, K] fp32 (split at nsplit rows with dW2)
  float* partial;                  // [max(splits, 1), N, K] fp32 workspace
  int64_t M; int N; int K; int splits;
  int pro;
};
hipError_t launch_wgrad(const WgradArgs& a, bool bf16_data, hipStream_t st);
int wgrad_splits(int64_t M, int N, int K);

// ------------------------------------------------- offset validation (debug)
// Bits of the validator's flag (0 = the offsets satisfy the hints).
enum : int32_t {
  kBadFirst = 1,        // offsets[0] != 0
  kBadOrder = 2,        // offsets decrease somewhere
  kBadMaxL = 4,         // some L_b > max_L
  kBadTotal = 8,        // offsets[B] != total_L
  kBadCandFirst = 16,   // cand_offsets[0] != 0
  kBadCandOrder = 32,   // cand_offsets decrease somewhere
  kBadMaxC = 64,        // some C_b > C
  kBadTime = 128        // a timestamp differs from its request's first by 2^30 or more
};
// One workgroup: flag[0] = violations found; sticky[0] |= the same (sticky may
// be null).  cand_offsets may be null.
// Timestamps [total_L] of the HSTU call: every row of request b against the
// request's first (rows outside [0, total_L) are not read: offsets that leave
// it are the offsets check's to report).  ORs kBadTime into flag[0] (and
// sticky[0] when not null).
hipError_t launch_validate_timestamps(const int64_t* offsets, const int64_t* ts, int B, int64_t total_L,
                                      int32_t* flag, int32_t* sticky, hipStream_t st);
hipError_t launch_validate_offsets(const int64_t* offsets, const int64_t* cand_offsets, int B, int max_L,
                                   int64_t total_L, int C, int32_t* flag, int32_t* sticky, hipStream_t st);
// The library's debug flags on the current GPU ([0] last check, [1] sticky),
// or nullptr if the address cannot be obtained.
int32_t* debug_flags_device();
// dst[0] = sticky flag; reset != 0 clears both flags afterwards.
hipError_t launch_debug_status(int32_t* dst, int reset, hipStream_t st);
bool debug_checks_on();
int set_debug_checks(int on);

// ------------------------------------------- static scratch (no-alloc call)
// Size of the static device scratch, and its address on the current GPU
// (looked up once per GPU; nullptr if the lookup fails).
size_t static_scratch_bytes();
void* static_scratch_device();

// ---------------------------------------------------------------- misc
// dst[c][col0 + r] = src[r][c] for a [rows, cols] matrix (data type), dst row stride ldd.
hipError_t launch_transpose(const void* src, int rows, int cols, void* dst, int ldd, int col0,
                            bool bf16_data, hipStream_t st);
// x[0..n) = 0 (a kernel, so that callers may capture it in a graph).
hipError_t launch_fill_zero(float* x, int64_t n, hipStream_t st);
