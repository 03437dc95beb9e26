// Row normalisation statistics and the column reduction of the norm
// parameter gradients.
//
// The pages normalise the Wukong output before the query projection, the
// HSTU output before the key/value projections, and the fused stream before
// the FFN (pith.science verdict record, pith_extraction.key_machinery;
// gist.science Technical Summary §2.1, pre-norm SwiGLU FFN).  LayerNorm uses
// the biased variance with eps inside the root; RMSNorm the mean square.  The
// affine gamma/beta is applied in the GEMM prologue that consumes each row and
// the norm backward runs in the epilogue of the GEMM that produces dX, so
// these kernels only produce (mean, rstd) per row and reduce the per-tile
// dgamma/dbeta partials.  Both are HBM-bound: 16-byte loads, every byte read
// once.
#include "common.h"
#include "kernels.h"

namespace {

// A group of n/8 lanes owns one row, each lane 8 contiguous elements.
template <typename T>
__global__ __launch_bounds__(256) void norm_stats_kernel(const T* __restrict__ x, float* __restrict__ stats,
                                                         int64_t rows, int n, int kind, float eps) {
  const int lpr = n / 8;                   // power of two, 8..64
  const int rpw = 64 / lpr;                // rows per wave
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = ((int64_t)blockIdx.x * 4 + w) * rpw + lane / lpr;
  const int cl = lane % lpr;
  const bool ok = row < rows;
  float v[8];
  if (ok) {
    const x8_t<T> r = ld8<T>(x + row * n + 8 * cl);
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = to_f(r[u]);
  } else {
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = 0.f;
  }
  float s = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) s += v[u];
  for (int o = 1; o < lpr; o <<= 1) s += __shfl_xor(s, o);
  const float mean = kind == 0 ? s / n : 0.f;
  float q = 0.f;
#pragma unroll
  for (int u = 0; u < 8; ++u) { const float dl = v[u] - mean; q += dl * dl; }
  for (int o = 1; o < lpr; o <<= 1) q += __shfl_xor(q, o);
  if (ok && cl == 0) {
    stats[2 * row] = mean;
    stats[2 * row + 1] = 1.f / sqrtf(q / n + eps);
  }
}

// Level 1: block (column group cg of 64 columns, row split s) sums rows
// [s*R/S, (s+1)*R/S) of part [R, 2n]; 4 row phases combined in a fixed order.
__global__ __launch_bounds__(256) void colsum1_kernel(const float* __restrict__ part, int64_t R, int n2, int S,
                                                      float* __restrict__ out) {
  __shared__ float red[4][64];
  const int cg = blockIdx.x, s = blockIdx.y;
  const int ph = threadIdx.x >> 6, c = cg * 64 + (threadIdx.x & 63);
  const int64_t r0 = (int64_t)s * R / S, r1 = (int64_t)(s + 1) * R / S;
  float acc = 0.f;
  if (c < n2)
    for (int64_t r = r0 + ph; r < r1; r += 4) acc += part[r * n2 + c];
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
  float acc = 0.f;
  for (int s = 0; s < S; ++s) acc += p2[(int64_t)s * 2 * n + c];
  if (c < n) { if (dgamma) dgamma[c] = acc; }
  else if (dbeta) dbeta[c - n] = acc;
}

constexpr int kColsumSplits = 64;

}  // namespace

hipError_t launch_norm_stats(const void* x, float* stats, int64_t rows, int n, int kind, float eps,
                             bool bf16_data, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const int rpb = 4 * (64 / (n / 8));      // rows per block
  const unsigned grid = (unsigned)((rows + rpb - 1) / rpb);
  if (bf16_data)
    hipLaunchKernelGGL(norm_stats_kernel<bf16>, dim3(grid), dim3(256), 0, st, (const bf16*)x, stats, rows, n, kind, eps);
  else
    hipLaunchKernelGGL(norm_stats_kernel<float>, dim3(grid), dim3(256), 0, st, (const float*)x, stats, rows, n, kind, eps);
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
