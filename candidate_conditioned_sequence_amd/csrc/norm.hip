// Row normalisation (statistics, and the normalised rows for the GEMMs that
// consume them), the SiLU derivative product of the fusion MLP backward, and
// the column reduction of the norm parameter gradients.
//
// The pages normalise the Wukong output before the query projection, the
// HSTU output before the key/value projections, and the fused stream before
// the FFN (pith.science verdict record, pith_extraction.key_machinery;
// gist.science Technical Summary §2.1, pre-norm SwiGLU FFN).  LayerNorm uses
// the biased variance with eps inside the root; RMSNorm the mean square.  The
// norm backward runs in the epilogue of the GEMM that produces dX; the
// kernels here reduce its per-tile dgamma/dbeta partials.  All are HBM-bound:
// 16-byte loads, every byte read once.
#include "common.h"
#include "kernels.h"

namespace {

// A group of n/8 lanes owns one row, each lane 8 contiguous elements; every
// group handles kRows rows (loads for all of them issued first), so a block
// of 4 waves covers 4 * (64 / (n/8)) * kRows rows.
constexpr int kRows = 4;

// Row statistics of kRows rows, each held as 8 values per lane of a group of
// lpr lanes; the cross-lane sums of all rows advance together, so their
// shuffles are in flight at the same time.
WHALE_DEV void row_stats(const float (&v)[kRows][8], int lpr, int n, int kind, float eps, float (&mean)[kRows],
                         float (&rstd)[kRows]) {
  float s[kRows], q[kRows];
#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    s[k] = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) s[k] += v[k][u];
  }
  for (int o = 1; o < lpr; o <<= 1)
#pragma unroll
    for (int k = 0; k < kRows; ++k) s[k] += __shfl_xor(s[k], o);
#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    mean[k] = kind == 0 ? s[k] / n : 0.f;
    q[k] = 0.f;
#pragma unroll
    for (int u = 0; u < 8; ++u) { const float dl = v[k][u] - mean[k]; q[k] += dl * dl; }
  }
  for (int o = 1; o < lpr; o <<= 1)
#pragma unroll
    for (int k = 0; k < kRows; ++k) q[k] += __shfl_xor(q[k], o);
#pragma unroll
  for (int k = 0; k < kRows; ++k) rstd[k] = 1.f / sqrtf(q[k] / n + eps);
}

// Rows past the end read the last row (unmasked loads, all in flight at
// once); their results are never stored.
template <typename T>
WHALE_DEV void load_rows(const T* __restrict__ x, int64_t row0, int64_t rstep, int64_t rows, int n, int cl,
                         float (&v)[kRows][8]) {
  x8_t<T> r[kRows];
#pragma unroll
  for (int k = 0; k < kRows; ++k) r[k] = ld8<T>(x + min(row0 + k * rstep, rows - 1) * n + 8 * cl);
#pragma unroll
  for (int k = 0; k < kRows; ++k)
#pragma unroll
    for (int u = 0; u < 8; ++u) v[k][u] = to_f(r[k][u]);
}

template <typename T>
__global__ __launch_bounds__(256) void norm_stats_kernel(const T* __restrict__ x, float* __restrict__ stats,
                                                         int64_t rows, int n, int kind, float eps) {
  const int lpr = n / 8;                   // power of two, 8..64
  const int rpw = 64 / lpr;                // rows per wave and pass
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t rstep = 4 * rpw;           // rows per block and pass
  const int64_t row0 = (int64_t)blockIdx.x * rstep * kRows + w * rpw + lane / lpr;
  const int cl = lane % lpr;
  float v[kRows][8], mean[kRows], rstd[kRows];
  load_rows<T>(x, row0, rstep, rows, n, cl, v);
  row_stats(v, lpr, n, kind, eps, mean, rstd);
#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    const int64_t row = row0 + k * rstep;
    if (row < rows && cl == 0) {
      stats[2 * row] = mean[k];
      stats[2 * row + 1] = rstd[k];
    }
  }
}

// Normalised rows y = (x - mean) * rstd * gamma + beta (beta = 0 for RMSNorm)
// for the GEMMs that consume them, with the statistics computed here
// (stats_in == nullptr, written to stats_out if given) or read from a
// previous pass.  Same layout as norm_stats_kernel; HBM-bound.
template <typename T>
__global__ __launch_bounds__(256) void norm_apply_kernel(const T* __restrict__ x, const float* __restrict__ stats_in,
                                                         float* __restrict__ stats_out, const float* __restrict__ gamma,
                                                         const float* __restrict__ beta, T* __restrict__ y,
                                                         int64_t rows, int n, int kind, float eps) {
  const int lpr = n / 8;
  const int rpw = 64 / lpr;
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t rstep = 4 * rpw;
  const int64_t row0 = (int64_t)blockIdx.x * rstep * kRows + w * rpw + lane / lpr;
  const int cl = lane % lpr;
  float gm[8], bt[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    gm[u] = gamma[8 * cl + u];
    bt[u] = 0.f;
    if (kind == 0) bt[u] = beta[8 * cl + u];          // beta may be null for RMSNorm
  }
  float v[kRows][8], mean[kRows], rstd[kRows];
  load_rows<T>(x, row0, rstep, rows, n, cl, v);
  if (stats_in != nullptr) {
#pragma unroll
    for (int k = 0; k < kRows; ++k) {
      const int64_t row = min(row0 + k * rstep, rows - 1);
      mean[k] = stats_in[2 * row];
      rstd[k] = stats_in[2 * row + 1];
    }
  } else {
    row_stats(v, lpr, n, kind, eps, mean, rstd);
  }
#pragma unroll
  for (int k = 0; k < kRows; ++k) {
    const int64_t row = row0 + k * rstep;
    if (row >= rows) continue;
    if (stats_in == nullptr && cl == 0 && stats_out != nullptr) {
      stats_out[2 * row] = mean[k];
      stats_out[2 * row + 1] = rstd[k];
    }
    x8_t<T> o;
#pragma unroll
    for (int u = 0; u < 8; ++u) o[u] = from_f<T>((v[k][u] - mean[k]) * rstd[k] * gm[u] + bt[u]);
    st8<T>(y + row * n + 8 * cl, o);
  }
}

// dZ = dF * SiLU'(Z), elementwise (8 per thread).
template <typename T>
__global__ __launch_bounds__(256) void dact_kernel(const T* __restrict__ dF, const T* __restrict__ Z, T* __restrict__ dZ,
                                                   int64_t n8) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const x8_t<T> g = ld8<T>(dF + 8 * i), z = ld8<T>(Z + 8 * i);
  x8_t<T> o;
#pragma unroll
  for (int u = 0; u < 8; ++u) o[u] = from_f<T>(to_f(g[u]) * dsiluf_(to_f(z[u])));
  st8<T>(dZ + 8 * i, o);
}

// Level 1: block (column group cg of 64 columns, row split s) sums rows
// [s*R/S, (s+1)*R/S) of part [R, 2n]; 4 row phases combined in a fixed order.
__global__ __launch_bounds__(256) void colsum1_kernel(const float* __restrict__ part, int64_t R, int n2, int S,
                                                      float* __restrict__ out) {
  __shared__ float red[4][64];
  const int cg = blockIdx.x, s = blockIdx.y;
  const int ph = threadIdx.x >> 6, c = cg * 64 + (threadIdx.x & 63);
  const int64_t r0 = (int64_t)s * R / S, r1 = (int64_t)(s + 1) * R / S;
  // Four partial sums per thread (rows r, r+4, r+8, r+12 of each group of
  // 16), four loads in flight, combined in a fixed order.
  float a4[4] = {0.f, 0.f, 0.f, 0.f};
  if (c < n2) {
    int64_t r = r0 + ph;
    for (; r + 12 < r1; r += 16) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = part[(r + 4 * u) * n2 + c];
#pragma unroll
      for (int u = 0; u < 4; ++u) a4[u] += v[u];
    }
    for (int u = 0; r < r1; r += 4, ++u) a4[u & 3] += part[r * n2 + c];
  }
  const float acc = (a4[0] + a4[1]) + (a4[2] + a4[3]);
  red[ph][threadIdx.x & 63] = acc;
  __syncthreads();
  if (ph == 0 && c < n2) out[(int64_t)s * n2 + c] = ((red[0][threadIdx.x] + red[1][threadIdx.x]) + red[2][threadIdx.x]) +
                                                    red[3][threadIdx.x];
}

// Level 2: sum the S level-1 rows in order.
__global__ __launch_bounds__(256) void colsum2_kernel(const float* __restrict__ p2, int S, int n,
                                                      float* __restrict__ dgamma, float* __restrict__ dbeta) {
  const int c = blockIdx.x * 256 + threadIdx.x;
  if (c >= 2 * n) return;
  // Eight partial sums (row s goes to sum s % 8), combined in a fixed order.
  float a8[8];
#pragma unroll
  for (int u = 0; u < 8; ++u) a8[u] = 0.f;
  int s = 0;
  for (; s + 8 <= S; s += 8) {
    float v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = p2[(int64_t)(s + u) * 2 * n + c];
#pragma unroll
    for (int u = 0; u < 8; ++u) a8[u] += v[u];
  }
  for (; s < S; ++s) a8[s & 7] += p2[(int64_t)s * 2 * n + c];
  const float acc = ((a8[0] + a8[1]) + (a8[2] + a8[3])) + ((a8[4] + a8[5]) + (a8[6] + a8[7]));
  if (c < n) { if (dgamma) dgamma[c] = acc; }
  else if (dbeta) dbeta[c - n] = acc;
}

constexpr int kColsumSplits = 64;

}  // namespace

hipError_t launch_norm_stats(const void* x, float* stats, int64_t rows, int n, int kind, float eps,
                             bool bf16_data, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int rpb = 4 * (64 / (n / 8)) * kRows;   // rows per block
  const unsigned grid = (unsigned)((rows + rpb - 1) / rpb);
  if (bf16_data)
    hipLaunchKernelGGL(norm_stats_kernel<bf16>, dim3(grid), dim3(256), 0, st, (const bf16*)x, stats, rows, n, kind, eps);
  else
    hipLaunchKernelGGL(norm_stats_kernel<float>, dim3(grid), dim3(256), 0, st, (const float*)x, stats, rows, n, kind, eps);
  return hipGetLastError();
}

hipError_t launch_norm_apply(const void* x, const float* stats_in, float* stats_out, const float* gamma,
                             const float* beta, void* y, int64_t rows, int n, int kind, float eps, bool bf16_data,
                             hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int rpb = 4 * (64 / (n / 8)) * kRows;
  const unsigned grid = (unsigned)((rows + rpb - 1) / rpb);
  if (bf16_data)
    hipLaunchKernelGGL(norm_apply_kernel<bf16>, dim3(grid), dim3(256), 0, st, (const bf16*)x, stats_in, stats_out,
                       gamma, beta, (bf16*)y, rows, n, kind, eps);
  else
    hipLaunchKernelGGL(norm_apply_kernel<float>, dim3(grid), dim3(256), 0, st, (const float*)x, stats_in, stats_out,
                       gamma, beta, (float*)y, rows, n, kind, eps);
  return hipGetLastError();
}

hipError_t launch_dact(const void* dF, const void* Z, void* dZ, int64_t n, bool bf16_data, hipStream_t st) {
  if (n == 0) return hipSuccess;
  const int64_t n8 = n / 8;
  const unsigned grid = (unsigned)((n8 + 255) / 256);
  if (bf16_data)
    hipLaunchKernelGGL(dact_kernel<bf16>, dim3(grid), dim3(256), 0, st, (const bf16*)dF, (const bf16*)Z, (bf16*)dZ, n8);
  else
    hipLaunchKernelGGL(dact_kernel<float>, dim3(grid), dim3(256), 0, st, (const float*)dF, (const float*)Z,
                       (float*)dZ, n8);
  return hipGetLastError();
}

int64_t colsum_scratch_floats(int n) { return (int64_t)kColsumSplits * 2 * n; }

hipError_t launch_colsum_reduce(const float* part, int64_t nblk, int n, float* dgamma, float* dbeta, float* scratch,
                                hipStream_t st) {
  const int n2 = 2 * n;
  int S = (int)((nblk + 63) / 64);
  if (S > kColsumSplits) S = kColsumSplits;
  if (S < 1) S = 1;
  hipLaunchKernelGGL(colsum1_kernel, dim3((n2 + 63) / 64, S), dim3(256), 0, st, part, nblk, n2, S, scratch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(colsum2_kernel, dim3((n2 + 255) / 256), dim3(256), 0, st, scratch, S, n, dgamma, dbeta);
  return hipGetLastError();
}
