// Static device scratch for the call that allocates nothing
// (whale_jagged_xattn_bwd_noalloc).
//
// The array below is device memory the code object defines: each GPU the
// library runs on holds its own copy, from module load until the process
// ends.  In host code its name is only a host-side stand-in, not a device
// address; its address on a GPU comes from hipGetSymbolAddress with that GPU
// current, looked up once per GPU and kept here.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace {

constexpr size_t kScratchBytes = (size_t)32 << 20;   // 32 MiB per GPU
__device__ __align__(256) unsigned char scratch[kScratchBytes];

}  // namespace

size_t static_scratch_bytes() { return kScratchBytes; }

void* static_scratch_device() {
  static std::mutex mu;
  static void* ptrs[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
    ptrs[dev] = p;
  }
  return ptrs[dev];
}
