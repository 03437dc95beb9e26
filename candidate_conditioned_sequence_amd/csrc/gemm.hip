// Projection, fusion-MLP and FFN GEMMs (gfx950 MFMA, fp32 accumulation).
//
//  * gemm_nt: Y[M,N] = op(X)[M,K] W[N,K]^T.  Both operands are
//    K-contiguous, so the 32x32x16 MFMA operands are 16-byte rows of the LDS
//    tiles.  The X tile loader can apply the row norm (stats + gamma/beta)
//    or read the concatenation [X | X2]; W rows may come from two matrices
//    (K and V projections in one pass over H_s, or the gate and up halves of
//    a separate-gate SwiGLU side by side).  Epilogues fuse the residual,
//    SiLU, the shared-gate SwiGLU product G = SiLU(U) U (gist.science
//    Technical Summary §2.2; paper-daily.com deep reading §2), and the
//    gate derivatives of the backward.
//  * wgrad: dW[N,K] = sum_m G[m,n] X[m,k] (the weight gradients).  The
//    contraction runs over rows of both operands, so both tiles are stored
//    transposed in LDS.  M is split into fixed chunks whose fp32 partials a
//    second kernel sums in a fixed order: deterministic, no atomics.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace {

constexpr int BM = 128, BN = 128, BK = 32, LDT = BK + 8;

template <typename T>
WHALE_DEV x8_t<T> norm8(const x8_t<T>& v, float mean, float rstd, const float* g, const float* bt, int kind) {
  x8_t<T> o;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    float x = (to_f(v[u]) - mean) * rstd * g[u];
    if (kind == 0) x += bt[u];
    o[u] = from_f<T>(x);
  }
  return o;
}

template <typename T, int PRO, int EPI, bool YF32>
__global__ __launch_bounds__(256, 2) void gemm_nt_kernel(GemmArgs a, int tiles_n, int ntiles, int nsplit,
                                                         const T* __restrict__ W2, void* __restrict__ Y2) {
  __shared__ __attribute__((aligned(32))) T As[2][BM * LDT];
  __shared__ __attribute__((aligned(32))) T Bs[2][BN * LDT];
  typedef typename std::conditional<YF32, float, T>::type YT;

  const int lid = xcd_remap(blockIdx.x, ntiles);
  const int tn = lid % tiles_n, tm = lid / tiles_n;
  const int64_t m0 = (int64_t)tm * BM;
  const int n0 = tn * BN;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wm = w >> 1, wn = w & 1;
  const int64_t M = a.M;
  const int N = a.N, K = a.K;
  const T* X = (const T*)a.X;
  const T* X2 = (const T*)a.X2;
  const T* W = (const T*)a.W;
  const int Hs = N / 2;   // EPI_GATE_SEP: number of gate rows

  // Loader assignment: 2 chunks of 8 elements per thread per operand.
  int arow[2], ak0[2];
  float amean[2], arstd[2];
  const T* brow_ptr[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ch = tid + 256 * i;
    arow[i] = ch >> 2;
    ak0[i] = 8 * (ch & 3);
    const int64_t m = m0 + arow[i];
    amean[i] = 0.f;
    arstd[i] = 1.f;
    if (PRO == PRO_NORM && m < M && a.norm_kind != 2) {
      amean[i] = a.stats[2 * m];
      arstd[i] = a.stats[2 * m + 1];
    }
    // weight row for tile row arow[i]
    const int tr = arow[i];
    int n;
    if (EPI == EPI_GATE_SEP) {
      const int wn_ = tr >> 6, jj = (tr >> 5) & 1, rr = tr & 31;
      n = n0 / 2 + wn_ * 32 + rr;                 // output column
      brow_ptr[i] = (n < Hs) ? W + (int64_t)(jj ? Hs + n : n) * a.ldw : nullptr;
    } else {
      n = n0 + tr;
      if (n >= N) brow_ptr[i] = nullptr;
      else if (W2 != nullptr && n >= nsplit) brow_ptr[i] = W2 + (int64_t)(n - nsplit) * a.ldw;
      else brow_ptr[i] = W + (int64_t)n * a.ldw;
    }
  }

  x8_t<T> ar[2], br[2];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int64_t m = m0 + arow[i];
      const int k = k0 + ak0[i];
      if (m < M) {
        if (PRO == PRO_CONCAT && k >= a.ksplit) ar[i] = ld8<T>(X2 + m * a.ldx2 + (k - a.ksplit));
        else ar[i] = ld8<T>(X + m * a.ldx + k);
        if (PRO == PRO_NORM && a.norm_kind != 2)
          ar[i] = norm8<T>(ar[i], amean[i], arstd[i], a.gamma + k, a.beta + k, a.norm_kind);
      } else {
        ar[i] = zero8<T>();
      }
      br[i] = brow_ptr[i] ? ld8<T>(brow_ptr[i] + k) : zero8<T>();
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      st8<T>(&As[buf][arow[i] * LDT + ak0[i]], ar[i]);
      st8<T>(&Bs[buf][arow[i] * LDT + ak0[i]], br[i]);
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) acc[i][jj] = zero16();

  const int nk = K / BK;
  load(0);
  store(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) load((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      x8_t<T> af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = ld8<T>(&As[buf][(wm * 64 + 32 * i + l32) * LDT + 16 * ks + 8 * hh]);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) bf[jj] = ld8<T>(&Bs[buf][(wn * 64 + 32 * jj + l32) * LDT + 16 * ks + 8 * hh]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) mma32(acc[i][jj], af[i], bf[jj]);
    }
    if (kt + 1 < nk) store(buf ^ 1);
    __syncthreads();
  }

  // Epilogue.
  YT* Y = (YT*)a.Y;
  const T* R = (const T*)a.R;
  T* Z = (T*)a.Z;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int64_t m = m0 + wm * 64 + 32 * i + acc_row(r, hh);
      if (m >= M) continue;
      if (EPI == EPI_GATE_SEP) {
        const int n = n0 / 2 + wn * 32 + l32;
        if (n >= Hs) continue;
        const float g = acc[i][0][r], u = acc[i][1][r];
        Y[m * a.ldy + n] = from_f<YT>(siluf_(g) * u);
        if (Z) { Z[m * a.ldz + n] = from_f<T>(g); Z[m * a.ldz + Hs + n] = from_f<T>(u); }
        continue;
      }
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int n = n0 + wn * 64 + 32 * jj + l32;
        if (n >= N) continue;
        const float v = acc[i][jj][r];
        if (EPI == EPI_STORE) {
          if (Y2 != nullptr && n >= nsplit) ((YT*)Y2)[m * a.ldy + (n - nsplit)] = from_f<YT>(v);
          else Y[m * a.ldy + n] = from_f<YT>(v);
        } else if (EPI == EPI_RESID) {
          Y[m * a.ldy + n] = from_f<YT>(to_f(R[m * a.ldr + n]) + v);
        } else if (EPI == EPI_SILU_RESID) {
          Y[m * a.ldy + n] = from_f<YT>(to_f(R[m * a.ldr + n]) + siluf_(v));
          if (Z) Z[m * a.ldz + n] = from_f<T>(v);
        } else if (EPI == EPI_GATE_TIED) {
          Y[m * a.ldy + n] = from_f<YT>(siluf_(v) * v);
          if (Z) Z[m * a.ldz + n] = from_f<T>(v);
        } else if (EPI == EPI_DGATE_TIED) {
          const float u = to_f(Z[m * a.ldz + n]);
          Y[m * a.ldy + n] = from_f<YT>(v * (dsiluf_(u) * u + siluf_(u)));
        } else if (EPI == EPI_DGATE_SEP) {
          const float ug = to_f(Z[m * a.ldz + n]), uu = to_f(Z[m * a.ldz + N + n]);
          Y[m * a.ldy + n] = from_f<YT>(v * uu * dsiluf_(ug));
          Y[m * a.ldy + N + n] = from_f<YT>(v * siluf_(ug));
        }
      }
    }
  }
}

template <typename T, int PRO, int EPI>
hipError_t gemm_go(const GemmArgs& a, hipStream_t st, int nsplit, const void* W2, void* Y2) {
  const int Nrows = a.N;     // rows of W (2H for EPI_GATE_SEP)
  const int tiles_n = (Nrows + BN - 1) / BN;
  const int64_t tiles_m = (a.M + BM - 1) / BM;
  const int64_t nt = tiles_m * tiles_n;
  if (nt == 0) return hipSuccess;
  if (a.y_f32)
    hipLaunchKernelGGL((gemm_nt_kernel<T, PRO, EPI, true>), dim3((unsigned)nt), dim3(256), 0, st, a, tiles_n, (int)nt,
                       nsplit, (const T*)W2, Y2);
  else
    hipLaunchKernelGGL((gemm_nt_kernel<T, PRO, EPI, false>), dim3((unsigned)nt), dim3(256), 0, st, a, tiles_n, (int)nt,
                       nsplit, (const T*)W2, Y2);
  return hipGetLastError();
}

template <typename T, int PRO>
hipError_t gemm_epi(const GemmArgs& a, hipStream_t st, int nsplit, const void* W2, void* Y2) {
  switch (a.epi) {
    case EPI_STORE: return gemm_go<T, PRO, EPI_STORE>(a, st, nsplit, W2, Y2);
    case EPI_RESID: return gemm_go<T, PRO, EPI_RESID>(a, st, nsplit, W2, Y2);
    case EPI_SILU_RESID: return gemm_go<T, PRO, EPI_SILU_RESID>(a, st, nsplit, W2, Y2);
    case EPI_GATE_TIED: return gemm_go<T, PRO, EPI_GATE_TIED>(a, st, nsplit, W2, Y2);
    case EPI_GATE_SEP: return gemm_go<T, PRO, EPI_GATE_SEP>(a, st, nsplit, W2, Y2);
    case EPI_DGATE_TIED: return gemm_go<T, PRO, EPI_DGATE_TIED>(a, st, nsplit, W2, Y2);
    case EPI_DGATE_SEP: return gemm_go<T, PRO, EPI_DGATE_SEP>(a, st, nsplit, W2, Y2);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t gemm_pro(const GemmArgs& a, hipStream_t st, int nsplit, const void* W2, void* Y2) {
  switch (a.pro) {
    case PRO_PLAIN: return gemm_epi<T, PRO_PLAIN>(a, st, nsplit, W2, Y2);
    case PRO_NORM: return gemm_epi<T, PRO_NORM>(a, st, nsplit, W2, Y2);
    case PRO_CONCAT: return gemm_epi<T, PRO_CONCAT>(a, st, nsplit, W2, Y2);
  }
  return hipErrorInvalidValue;
}

// ------------------------------------------------------------------ wgrad

constexpr int WN = 128, WK = 128, WM = 32, LDW = WM + 8;

template <typename T, int PRO>
__global__ __launch_bounds__(256, 2) void wgrad_kernel(WgradArgs a, int tiles_k, int ntiles, int64_t chunk) {
  __shared__ __attribute__((aligned(32))) T Gt[2][WN * LDW];   // [n][m]
  __shared__ __attribute__((aligned(32))) T Xt[2][WK * LDW];   // [k][m]
  const int split = blockIdx.y;
  const int lid = xcd_remap(blockIdx.x, ntiles);
  const int tk = lid % tiles_k, tnn = lid / tiles_k;
  const int n0 = tnn * WN, k0 = tk * WK;
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, l32 = lane & 31, hh = lane >> 5;
  const int wm = w >> 1, wn = w & 1;
  const int N = a.N, K = a.K;
  const int64_t mb = (int64_t)split * chunk;
  const int64_t me = min(a.M, mb + chunk);
  const T* G = (const T*)a.G;
  const T* X = (const T*)a.X;
  const T* X2 = (const T*)a.X2;

  // Each thread loads 2 chunks of 8 consecutive columns of one row per operand.
  x8_t<T> gr[2], xr[2];
  auto load = [&](int64_t mbase) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ch = tid + 256 * i;
      const int mr = ch >> 4, c0 = 8 * (ch & 15);
      const int64_t m = mbase + mr;
      const bool mok = m < me;
      const int n = n0 + c0, k = k0 + c0;
      gr[i] = (mok && n < N) ? ld8<T>(G + m * a.ldg + n) : zero8<T>();
      if (!mok || k >= K) { xr[i] = zero8<T>(); continue; }
      if (PRO == WPRO_CONCAT && k >= a.ksplit) {
        xr[i] = ld8<T>(X2 + m * a.ldx2 + (k - a.ksplit));
      } else if (PRO == WPRO_GATE_TIED) {
        const x8_t<T> u = ld8<T>(X + m * a.ldx + k);
#pragma unroll
        for (int e = 0; e < 8; ++e) { const float uf = to_f(u[e]); xr[i][e] = from_f<T>(siluf_(uf) * uf); }
      } else if (PRO == WPRO_GATE_SEP) {
        const x8_t<T> ug = ld8<T>(X + m * a.ldx + k);
        const x8_t<T> uu = ld8<T>(X + m * a.ldx + a.gate_H + k);
#pragma unroll
        for (int e = 0; e < 8; ++e) xr[i][e] = from_f<T>(siluf_(to_f(ug[e])) * to_f(uu[e]));
      } else {
        xr[i] = ld8<T>(X + m * a.ldx + k);
        if (PRO == WPRO_NORM && a.norm_kind != 2)
          xr[i] = norm8<T>(xr[i], a.stats[2 * m], a.stats[2 * m + 1], a.gamma + k, a.beta + k, a.norm_kind);
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ch = tid + 256 * i;
      const int mr = ch >> 4, c0 = 8 * (ch & 15);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        Gt[buf][(c0 + e) * LDW + mr] = gr[i][e];
        Xt[buf][(c0 + e) * LDW + mr] = xr[i][e];
      }
    }
  };

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) acc[i][jj] = zero16();

  const int64_t nsteps = (me - mb + WM - 1) / WM;
  if (nsteps > 0) {
    load(mb);
    store(0);
  }
  __syncthreads();
  for (int64_t s = 0; s < nsteps; ++s) {
    const int buf = s & 1;
    if (s + 1 < nsteps) load(mb + (s + 1) * WM);
#pragma unroll
    for (int ks = 0; ks < WM / 16; ++ks) {
      x8_t<T> af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) af[i] = ld8<T>(&Gt[buf][(wm * 64 + 32 * i + l32) * LDW + 16 * ks + 8 * hh]);
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) bf[jj] = ld8<T>(&Xt[buf][(wn * 64 + 32 * jj + l32) * LDW + 16 * ks + 8 * hh]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < 2; ++jj) mma32(acc[i][jj], af[i], bf[jj]);
    }
    if (s + 1 < nsteps) store(buf ^ 1);
    __syncthreads();
  }

  float* out = a.splits > 1 ? a.partial + (int64_t)split * N * K : a.dW;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int n = n0 + wm * 64 + 32 * i + acc_row(r, hh);
        const int k = k0 + wn * 64 + 32 * jj + l32;
        if (n < N && k < K) out[(int64_t)n * K + k] = acc[i][jj][r];
      }
}

__global__ __launch_bounds__(256) void split_reduce_kernel(const float* __restrict__ part, int splits, int64_t n,
                                                           float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.f;
  for (int k = 0; k < splits; ++k) s += part[(int64_t)k * n + i];
  out[i] = s;
}

template <typename T>
hipError_t wgrad_t(const WgradArgs& a, hipStream_t st) {
  const int tiles_k = (a.K + WK - 1) / WK, tiles_n = (a.N + WN - 1) / WN;
  const int nt = tiles_k * tiles_n;
  int64_t chunk = (a.M + a.splits - 1) / a.splits;
  chunk = (chunk + WM - 1) / WM * WM;
  dim3 grid(nt, a.splits);
  switch (a.pro) {
    case WPRO_PLAIN: hipLaunchKernelGGL((wgrad_kernel<T, WPRO_PLAIN>), grid, dim3(256), 0, st, a, tiles_k, nt, chunk); break;
    case WPRO_NORM: hipLaunchKernelGGL((wgrad_kernel<T, WPRO_NORM>), grid, dim3(256), 0, st, a, tiles_k, nt, chunk); break;
    case WPRO_CONCAT: hipLaunchKernelGGL((wgrad_kernel<T, WPRO_CONCAT>), grid, dim3(256), 0, st, a, tiles_k, nt, chunk); break;
    case WPRO_GATE_TIED: hipLaunchKernelGGL((wgrad_kernel<T, WPRO_GATE_TIED>), grid, dim3(256), 0, st, a, tiles_k, nt, chunk); break;
    case WPRO_GATE_SEP: hipLaunchKernelGGL((wgrad_kernel<T, WPRO_GATE_SEP>), grid, dim3(256), 0, st, a, tiles_k, nt, chunk); break;
    default: return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || a.splits == 1) return e;
  const int64_t n = (int64_t)a.N * a.K;
  hipLaunchKernelGGL(split_reduce_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a.partial, a.splits, n, a.dW);
  return hipGetLastError();
}

// ------------------------------------------------------------------ misc

template <typename T>
__global__ __launch_bounds__(256) void transpose_kernel(const T* __restrict__ src, int rows, int cols, T* __restrict__ dst,
                                                        int ldd, int col0) {
  __shared__ T tile[32][33];
  const int bx = blockIdx.x * 32, by = blockIdx.y * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;
  for (int yy = ty; yy < 32; yy += 8) {
    const int r = by + yy, c = bx + tx;
    if (r < rows && c < cols) tile[yy][tx] = src[(int64_t)r * cols + c];
  }
  __syncthreads();
  for (int yy = ty; yy < 32; yy += 8) {
    const int c = bx + yy, r = by + tx;
    if (r < rows && c < cols) dst[(int64_t)c * ldd + col0 + r] = tile[tx][yy];
  }
}

template <typename T>
__global__ __launch_bounds__(256) void dact_kernel(const T* __restrict__ dF, const T* __restrict__ Z, T* __restrict__ dZ,
                                                   int64_t n, int act) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const float g = to_f(dF[i]);
  dZ[i] = from_f<T>(act == 0 ? g * dsiluf_(to_f(Z[i])) : g);
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ x, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) x[i] = 0.f;
}

}  // namespace

hipError_t launch_fill_zero(float* x, int64_t n, hipStream_t st) {
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, x, n);
  return hipGetLastError();
}

hipError_t launch_gemm_nt(const GemmArgs& a, bool bf16_data, hipStream_t st) {
  return bf16_data ? gemm_pro<bf16>(a, st, a.N, nullptr, nullptr) : gemm_pro<float>(a, st, a.N, nullptr, nullptr);
}

hipError_t launch_gemm_nt_dual(const GemmArgs& a, int nsplit, const void* W2, void* Y2, bool bf16_data, hipStream_t st) {
  return bf16_data ? gemm_pro<bf16>(a, st, nsplit, W2, Y2) : gemm_pro<float>(a, st, nsplit, W2, Y2);
}

int wgrad_splits(int64_t M, int N, int K) {
  const int tiles = ((N + WN - 1) / WN) * ((K + WK - 1) / WK);
  int64_t s = (1024 + tiles - 1) / tiles;
  const int64_t maxs = (M + 255) / 256;
  if (s > maxs) s = maxs;
  if (s < 1) s = 1;
  return (int)s;
}

hipError_t launch_wgrad(const WgradArgs& a, bool bf16_data, hipStream_t st) {
  return bf16_data ? wgrad_t<bf16>(a, st) : wgrad_t<float>(a, st);
}

hipError_t launch_transpose(const void* src, int rows, int cols, void* dst, int ldd, int col0, bool bf16_data,
                            hipStream_t st) {
  dim3 grid((cols + 31) / 32, (rows + 31) / 32);
  if (bf16_data)
    hipLaunchKernelGGL(transpose_kernel<bf16>, grid, dim3(256), 0, st, (const bf16*)src, rows, cols, (bf16*)dst, ldd, col0);
  else
    hipLaunchKernelGGL(transpose_kernel<float>, grid, dim3(256), 0, st, (const float*)src, rows, cols, (float*)dst, ldd, col0);
  return hipGetLastError();
}

hipError_t launch_dact(const void* dF, const void* Z, void* dZ, int64_t n, int act, bool bf16_data, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)((n + 255) / 256);
  if (bf16_data)
    hipLaunchKernelGGL(dact_kernel<bf16>, dim3(grid), dim3(256), 0, st, (const bf16*)dF, (const bf16*)Z, (bf16*)dZ, n, act);
  else
    hipLaunchKernelGGL(dact_kernel<float>, dim3(grid), dim3(256), 0, st, (const float*)dF, (const float*)Z, (float*)dZ, n, act);
  return hipGetLastError();
}
