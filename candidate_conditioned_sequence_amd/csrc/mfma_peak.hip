// Matrix-core rate probe: the bf16 MFMA throughput this GPU sustains with no
// memory traffic, the practical ceiling against which the attention and GEMM
// kernels are measured beside the data-sheet peak.  Each wave runs four
// independent accumulator chains of v_mfma_f32_32x32x16_bf16 on register
// operands; the sums are stored so that nothing is optimised away.

#include "common.h"
#include "whalefuse.h"

namespace {

__global__ __launch_bounds__(256) void mfma_peak_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  bf16x8 a, b;
#pragma unroll
  for (int u = 0; u < 8; ++u) {
    a[u] = from_f<bf16>(1e-3f * (float)(lane + u));
    b[u] = from_f<bf16>(1e-3f * (float)(lane - u));
  }
  f32x16 acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) acc[k] = zero16();
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int k = 0; k < 4; ++k) mma32(acc[k], a, b);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < 4; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[k][r];
  out[(int64_t)blockIdx.x * 256 + threadIdx.x] = s;
}

}  // namespace

extern "C" whale_status_t whale_mfma_peak_probe(float* out, int32_t iters, int32_t blocks, hipStream_t stream) {
  if (out == nullptr) return WHALE_ERR_NULL;
  if (iters < 1 || blocks < 1) return WHALE_ERR_SHAPE;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, out, (int)iters);
  return hipGetLastError() == hipSuccess ? WHALE_OK : WHALE_ERR_LAUNCH;
}
