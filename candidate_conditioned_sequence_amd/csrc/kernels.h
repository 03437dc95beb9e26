// Internal launcher interface between the C ABI (api.cpp) and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// ---------------------------------------------------------------- attention
struct XattnArgs {
  const void* Q; const void* K; const void* V; const int64_t* offsets;
  void* A; float* lse;
  int B, QR /* C*n_q */, d, h, dh;
  float scale;
};
hipError_t launch_xattn_fwd(const XattnArgs& a, bool bf16_data, hipStream_t st);

struct XattnBwdArgs {
  const void* Q; const void* K; const void* V; const int64_t* offsets;
  const void* A; const float* lse; const void* dA;
  void* dQ; void* dK; void* dV;
  float* Dbuf;          // [M, h] fp32: rowsum(dA * A) per head
  float* partial;       // [S, T, 2, d] fp32 dK/dV partials (S > 1 only)
  int B, QR, d, h, dh, max_L, splits;
  int64_t T;
  float scale;
};
hipError_t launch_xattn_bwd(const XattnBwdArgs& a, bool bf16_data, hipStream_t st);
int xattn_bwd_splits(int B, int h, int QR, int max_L, int dh);

// ---------------------------------------------------------------- norms
// Row statistics (mean, rstd) of x [rows, n]; mean = 0 for RMSNorm.
hipError_t launch_norm_stats(const void* x, float* stats, int64_t rows, int n, int kind, float eps,
                             bool bf16_data, hipStream_t st);

// Norm backward for rows of x [rows, n] given dxn = dL/d(norm output) in fp32:
// dx = rstd * (g*dxn - mean(g*dxn) - xhat * mean(g*dxn * xhat))   (LayerNorm)
// dx = rstd * (g*dxn - xhat * mean(g*dxn * xhat))                  (RMSNorm)
// plus an optional residual `add` (data type), written as data type.
// Per-block partial column sums of dxn*xhat and dxn go to part [nblk, 2, n];
// launch_colsum_reduce then sums them in a fixed order.
hipError_t launch_norm_bwd(const void* x, const float* stats, const float* gamma, const float* dxn,
                           const void* add, void* dx, float* part, int64_t rows, int n, int kind,
                           bool bf16_data, int* nblk_out, hipStream_t st);
hipError_t launch_colsum_reduce(const float* part, int nblk, int n, float* dgamma, float* dbeta,
                                hipStream_t st);
int norm_bwd_blocks(int64_t rows);

// ---------------------------------------------------------------- GEMMs
// Y[M,N] = op(X)[M,K] * W[N,K]^T with optional prologue on X and epilogue.
enum GemmPro { PRO_PLAIN = 0, PRO_NORM = 1, PRO_CONCAT = 2 };
enum GemmEpi {
  EPI_STORE = 0,        // Y = acc
  EPI_RESID = 1,        // Y = R + acc
  EPI_SILU_RESID = 2,   // Y = R + silu(acc); Z = acc (optional)
  EPI_GATE_TIED = 3,    // Y = silu(acc) * acc; Z = acc (optional)
  EPI_GATE_SEP = 4,     // N' = N/2 outputs: Y = silu(acc_g) * acc_u; Z = [acc_g | acc_u] (optional)
  EPI_DGATE_TIED = 5,   // Y = acc * (silu'(u) u + silu(u)), u = Z (input)
  EPI_DGATE_SEP = 6,    // Y[:, :N] = acc * u_u * silu'(u_g), Y[:, N:] = acc * silu(u_g), Z = [u_g | u_u] (input)
  EPI_DACT_SILU = 7     // Y = acc * silu'(Z) (Z input)   [unused: fusion bwd uses elementwise]
};
struct GemmArgs {
  const void* X; int ldx;          // plain / norm source, or first half of a concat
  const void* X2; int ldx2; int ksplit;   // concat: columns >= ksplit come from X2
  const float* stats; const float* gamma; const float* beta; int norm_kind;  // PRO_NORM
  const void* W; int ldw;          // [N, K] row-major
  void* Y; int ldy; bool y_f32;    // output (fp32 or data type)
  const void* R; int ldr;          // residual
  void* Z; int ldz;                // saved pre-activation (output) or gate input (DGATE)
  int64_t M; int N; int K;
  int pro, epi;
};
hipError_t launch_gemm_nt(const GemmArgs& a, bool bf16_data, hipStream_t st);
// Same, with weight rows n >= nsplit taken from W2 (row n - nsplit) and their
// outputs written to Y2 (EPI_STORE only): two projections of one input in one pass.
hipError_t launch_gemm_nt_dual(const GemmArgs& a, int nsplit, const void* W2, void* Y2, bool bf16_data,
                               hipStream_t st);

// dW[N,K] = sum_m G[m,n] * Xop[m,k], fp32, with optional prologue on Xop
// (norm of X, concat [X | X2], or tied/separate gate recomputed from U).
enum WgradPro { WPRO_PLAIN = 0, WPRO_NORM = 1, WPRO_CONCAT = 2, WPRO_GATE_TIED = 3, WPRO_GATE_SEP = 4 };
struct WgradArgs {
  const void* G; int ldg;          // [M, N]
  const void* X; int ldx;          // [M, K] (or U for the gate prologues)
  const void* X2; int ldx2; int ksplit;
  const float* stats; const float* gamma; const float* beta; int norm_kind;
  int gate_H;                      // WPRO_GATE_SEP: gate columns [0,H), up columns [H,2H) of X
  float* dW;                       // [N, K] fp32
  float* partial;                  // [splits, N, K] fp32 workspace
  int64_t M; int N; int K; int splits;
  int pro;
};
hipError_t launch_wgrad(const WgradArgs& a, bool bf16_data, hipStream_t st);
int wgrad_splits(int64_t M, int N, int K);

// ---------------------------------------------------------------- misc
// dst[c][r] = src[r][c] for a [rows, cols] matrix (data type), into dst with row stride ldd,
// written at column offset col0.
hipError_t launch_transpose(const void* src, int rows, int cols, void* dst, int ldd, int col0,
                            bool bf16_data, hipStream_t st);
// x[0..n) = 0 (a kernel, so that callers may capture it in a graph).
hipError_t launch_fill_zero(float* x, int64_t n, hipStream_t st);
// dZ = dF * act'(Z) (SiLU) or dF (none); data type in and out.
hipError_t launch_dact(const void* dF, const void* Z, void* dZ, int64_t n, int act, bool bf16_data,
                       hipStream_t st);
