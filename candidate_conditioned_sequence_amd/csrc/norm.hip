// kind: 0 LayerNorm, 1 RMSNorm, 2 none (backward is then dx = dxn + add).
//
// Row normalisation (the "normalised" Wukong/HSTU outputs and the pre-norm of
// the FFN: pith.science verdict record, pith_extraction.key_machinery;
// gist.science Technical Summary §2.1).  LayerNorm uses the biased variance
// with eps inside the root; RMSNorm uses the mean square.  The affine
// gamma/beta is applied inside the GEMM prologue that consumes the row, so
// these kernels only produce (mean, rstd) per row, and the backward.
// HBM-bound: one wave per row, every row read once.
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kMaxPerLane = 8;   // n <= 512

template <typename T>
__global__ __launch_bounds__(256) void norm_stats_kernel(const T* __restrict__ x, float* __restrict__ stats,
                                                         int64_t rows, int n, int kind, float eps) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= rows) return;
  const T* xr = x + row * n;
  float v[kMaxPerLane];
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int k = lane + 64 * i;
    v[i] = k < n ? to_f(xr[k]) : 0.f;
    s += v[i];
  }
  float mean = 0.f, var;
  if (kind == 0) {
    mean = wave_sum(s) / n;
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int k = lane + 64 * i;
      const float dlt = k < n ? v[i] - mean : 0.f;
      q += dlt * dlt;
    }
    var = wave_sum(q) / n;
  } else {
    float q = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) q += v[i] * v[i];
    var = wave_sum(q) / n;
  }
  if (lane == 0) {
    stats[2 * row] = mean;
    stats[2 * row + 1] = 1.f / sqrtf(var + eps);
  }
}

// One workgroup of 4 waves handles a contiguous range of rows, one wave per
// row at a time; per-column partial sums of dxn*xhat and dxn stay in
// registers (lane owns columns lane + 64 i) and are combined across the 4
// waves in a fixed order through LDS.
template <typename T>
__global__ __launch_bounds__(256) void norm_bwd_kernel(const T* __restrict__ x, const float* __restrict__ stats,
                                                       const float* __restrict__ gamma,
                                                       const float* __restrict__ dxn, const T* __restrict__ add,
                                                       T* __restrict__ dx, float* __restrict__ part,
                                                       int64_t rows, int n, int kind, int64_t rows_per_blk) {
  __shared__ float red[4][2][512];
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_blk;
  const int64_t r1 = min(rows, r0 + rows_per_blk);
  float g[kMaxPerLane], pg[kMaxPerLane], pb[kMaxPerLane];
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int k = lane + 64 * i;
    g[i] = k < n ? (gamma != nullptr ? gamma[k] : 1.f) : 0.f;
    pg[i] = 0.f;
    pb[i] = 0.f;
  }
  for (int64_t row = r0 + w; row < r1; row += 4) {
    const float mean = kind == 2 ? 0.f : stats[2 * row];
    const float rstd = kind == 2 ? 1.f : stats[2 * row + 1];
    float xh[kMaxPerLane], dy[kMaxPerLane];
    float s1 = 0.f, s2 = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int k = lane + 64 * i;
      const bool ok = k < n;
      xh[i] = ok ? (to_f(x[row * n + k]) - mean) * rstd : 0.f;
      dy[i] = ok ? dxn[row * n + k] : 0.f;
      const float gd = dy[i] * g[i];
      s1 += gd;
      s2 += gd * xh[i];
      pg[i] += dy[i] * xh[i];
      pb[i] += dy[i];
    }
    s1 = wave_sum(s1) / n;
    s2 = wave_sum(s2) / n;
    if (kind != 0) s1 = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPerLane; ++i) {
      const int k = lane + 64 * i;
      if (k < n) {
        float v = kind == 2 ? dy[i] : rstd * (dy[i] * g[i] - s1 - xh[i] * s2);
        if (add != nullptr) v += to_f(add[row * n + k]);
        dx[row * n + k] = from_f<T>(v);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < kMaxPerLane; ++i) {
    const int k = lane + 64 * i;
    if (k < n) { red[w][0][k] = pg[i]; red[w][1][k] = pb[i]; }
  }
  __syncthreads();
  for (int k = threadIdx.x; k < n; k += 256) {
    part[((int64_t)blockIdx.x * 2 + 0) * n + k] = ((red[0][0][k] + red[1][0][k]) + red[2][0][k]) + red[3][0][k];
    part[((int64_t)blockIdx.x * 2 + 1) * n + k] = ((red[0][1][k] + red[1][1][k]) + red[2][1][k]) + red[3][1][k];
  }
}

__global__ __launch_bounds__(256) void colsum_reduce_kernel(const float* __restrict__ part, int nblk, int n,
                                                            float* __restrict__ dgamma, float* __restrict__ dbeta) {
  const int k = blockIdx.x * 256 + threadIdx.x;
  if (k >= n) return;
  float sg = 0.f, sb = 0.f;
  for (int bk = 0; bk < nblk; ++bk) {
    sg += part[((int64_t)bk * 2 + 0) * n + k];
    sb += part[((int64_t)bk * 2 + 1) * n + k];
  }
  if (dgamma) dgamma[k] = sg;
  if (dbeta) dbeta[k] = sb;
}

}  // namespace

hipError_t launch_norm_stats(const void* x, float* stats, int64_t rows, int n, int kind, float eps,
                             bool bf16_data, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const unsigned grid = (unsigned)((rows + 3) / 4);
  if (bf16_data)
    hipLaunchKernelGGL(norm_stats_kernel<bf16>, dim3(grid), dim3(256), 0, st, (const bf16*)x, stats, rows, n, kind, eps);
  else
    hipLaunchKernelGGL(norm_stats_kernel<float>, dim3(grid), dim3(256), 0, st, (const float*)x, stats, rows, n, kind, eps);
  return hipGetLastError();
}

int norm_bwd_blocks(int64_t rows) {
  int64_t nb = (rows + 63) / 64;
  if (nb > 1024) nb = 1024;
  if (nb < 1) nb = 1;
  return (int)nb;
}

hipError_t launch_norm_bwd(const void* x, const float* stats, const float* gamma, const float* dxn,
                           const void* add, void* dx, float* part, int64_t rows, int n, int kind,
                           bool bf16_data, int* nblk_out, hipStream_t st) {
  const int nblk = norm_bwd_blocks(rows);
  const int64_t rpb = (rows + nblk - 1) / nblk;
  *nblk_out = nblk;
  if (bf16_data)
    hipLaunchKernelGGL(norm_bwd_kernel<bf16>, dim3(nblk), dim3(256), 0, st, (const bf16*)x, stats, gamma, dxn,
                       (const bf16*)add, (bf16*)dx, part, rows, n, kind, rpb);
  else
    hipLaunchKernelGGL(norm_bwd_kernel<float>, dim3(nblk), dim3(256), 0, st, (const float*)x, stats, gamma, dxn,
                       (const float*)add, (float*)dx, part, rows, n, kind, rpb);
  return hipGetLastError();
}

hipError_t launch_colsum_reduce(const float* part, int nblk, int n, float* dgamma, float* dbeta, hipStream_t st) {
  hipLaunchKernelGGL(colsum_reduce_kernel, dim3((n + 255) / 256), dim3(256), 0, st, part, nblk, n, dgamma, dbeta);
  return hipGetLastError();
}
