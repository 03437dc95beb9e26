// Device-side validation of the jagged offsets against the host shape hints.
//
// Every call takes the history lengths as device offsets plus two host hints,
// max_L and total_L, so that nothing is read back to the host (the pages
// credit "shape hint tensors" with avoiding GPU-to-CPU syncs: gist.science
// Technical Summary §2.2).  The kernels trust the hints: grids are sized from
// them and rows are indexed by the offsets.  This file checks that contract
// on the device, without a sync:
//  * validate_kernel: one workgroup scans the offsets (and the candidate
//    offsets) and writes a bitmask of the violations found;
//  * the debug flags: a small static device array per GPU.  In debug mode
//    the attention calls run the validator into flag 0 first and pass its
//    address to their kernels, which return at once when it is non-zero;
//    flag 1 accumulates (OR) every check since the last reset.
#include <atomic>
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace {

// [0]: the last debug-mode check; [1]: OR of all checks since the last reset.
// Each GPU holds its own copy; host code reaches it only through the address
// hipGetSymbolAddress returns on that GPU.
__device__ __align__(256) int32_t whale_debug_flags[64];

__global__ __launch_bounds__(256) void validate_kernel(const int64_t* __restrict__ offsets,
                                                       const int64_t* __restrict__ coffs, int B, int max_L,
                                                       int64_t total_L, int C, int32_t* __restrict__ flag,
                                                       int32_t* __restrict__ sticky) {
  __shared__ int32_t part[4];
  int32_t bad = 0;
  for (int b = threadIdx.x; b < B; b += 256) {
    const int64_t lo = offsets[b], hi = offsets[b + 1];
    if (b == 0 && lo != 0) bad |= kBadFirst;
    if (hi < lo) bad |= kBadOrder;
    else if (hi - lo > (int64_t)max_L) bad |= kBadMaxL;
    if (b == B - 1 && hi != total_L) bad |= kBadTotal;
    if (coffs != nullptr) {
      const int64_t c0 = coffs[b], c1 = coffs[b + 1];
      if (b == 0 && c0 != 0) bad |= kBadCandFirst;
      if (c1 < c0) bad |= kBadCandOrder;
      else if (c1 - c0 > (int64_t)C) bad |= kBadMaxC;
    }
  }
  // OR over the workgroup: within each wave by lane exchanges, then across
  // the four waves through LDS.
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) bad |= __shfl_xor(bad, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = bad;
  __syncthreads();
  if (threadIdx.x == 0) {
    const int32_t all = part[0] | part[1] | part[2] | part[3];
    flag[0] = all;
    if (sticky != nullptr) sticky[0] |= all;
  }
}

// One workgroup per request (a stride over requests past the grid): each
// timestamp against the request's first, as unsigned differences (no
// overflow for any int64 values).  Only the kBadTime bit is set, so the
// unsynchronised read-modify-write of the flags by several workgroups loses
// nothing: every writer ORs in the same bit, after validate_kernel has
// written the rest in stream order.
__global__ __launch_bounds__(256) void validate_times_kernel(const int64_t* __restrict__ offsets,
                                                             const int64_t* __restrict__ ts, int B, int64_t total_L,
                                                             int32_t* __restrict__ flag,
                                                             int32_t* __restrict__ sticky) {
  __shared__ int32_t part[4];
  int32_t bad = 0;
  for (int b = blockIdx.x; b < B; b += gridDim.x) {
    const int64_t lo = offsets[b], hi = offsets[b + 1];
    if (lo < 0 || hi <= lo || hi > total_L) continue;
    const int64_t t0 = ts[lo];
    for (int64_t i = lo + threadIdx.x; i < hi; i += 256) {
      const int64_t t = ts[i];
      const uint64_t dist = t >= t0 ? (uint64_t)t - (uint64_t)t0 : (uint64_t)t0 - (uint64_t)t;
      if (dist >= (uint64_t{1} << 30)) bad = kBadTime;
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) bad |= __shfl_xor(bad, o);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = bad;
  __syncthreads();
  if (threadIdx.x == 0 && (part[0] | part[1] | part[2] | part[3]) != 0) {
    flag[0] |= kBadTime;
    if (sticky != nullptr) sticky[0] |= kBadTime;
  }
}

__global__ void debug_status_kernel(int32_t* __restrict__ flags, int32_t* __restrict__ dst, int reset) {
  if (threadIdx.x == 0) {
    dst[0] = flags[1];
    if (reset) { flags[0] = 0; flags[1] = 0; }
  }
}

std::atomic<int> g_debug{-1};   // -1: not yet read from the environment

}  // namespace

hipError_t launch_validate_offsets(const int64_t* offsets, const int64_t* cand_offsets, int B, int max_L,
                                   int64_t total_L, int C, int32_t* flag, int32_t* sticky, hipStream_t st) {
  hipLaunchKernelGGL(validate_kernel, dim3(1), dim3(256), 0, st, offsets, cand_offsets, B, max_L, total_L, C, flag,
                     sticky);
  return hipGetLastError();
}

hipError_t launch_validate_timestamps(const int64_t* offsets, const int64_t* ts, int B, int64_t total_L,
                                      int32_t* flag, int32_t* sticky, hipStream_t st) {
  if (B <= 0 || total_L <= 0) return hipSuccess;
  const int g = B < 65536 ? B : 65536;
  hipLaunchKernelGGL(validate_times_kernel, dim3(g), dim3(256), 0, st, offsets, ts, B, total_L, flag, sticky);
  return hipGetLastError();
}

int32_t* debug_flags_device() {
  static std::mutex mu;
  static int32_t* ptrs[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(whale_debug_flags)) != hipSuccess) return nullptr;
    ptrs[dev] = (int32_t*)p;
  }
  return ptrs[dev];
}

hipError_t launch_debug_status(int32_t* dst, int reset, hipStream_t st) {
  int32_t* f = debug_flags_device();
  if (f == nullptr) return hipErrorInvalidSymbol;
  hipLaunchKernelGGL(debug_status_kernel, dim3(1), dim3(64), 0, st, f, dst, reset);
  return hipGetLastError();
}

bool debug_checks_on() {
  int v = g_debug.load(std::memory_order_relaxed);
  if (v < 0) {
    const char* e = getenv("WHALE_DEBUG_CHECKS");
    v = (e != nullptr && e[0] != '\0' && e[0] != '0') ? 1 : 0;
    int expect = -1;
    g_debug.compare_exchange_strong(expect, v);
    v = g_debug.load(std::memory_order_relaxed);
  }
  return v == 1;
}

int set_debug_checks(int on) {
  const int prev = debug_checks_on() ? 1 : 0;
  g_debug.store(on ? 1 : 0, std::memory_order_relaxed);
  return prev;
}
