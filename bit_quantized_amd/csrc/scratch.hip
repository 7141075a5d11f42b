// Library-held device scratch for the entry point that allocates nothing
// (fourtune_linear_fwd_noalloc): a file-scope device array, one copy per
// GPU, located once per device through hipGetSymbolAddress.  In host code
// the array's name is a host-side stand-in, not a device address, so only
// the looked-up pointer is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "ft_kernels.h"

namespace ft {

namespace {

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
std::atomic<void*> g_ptr[kMaxDevices];

}  // namespace

// The current device's copy of the scratch array, looked up on the first
// call made with that device current and kept for the life of the process.
// nullptr if the device cannot be queried or the lookup fails.
void* noalloc_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  void* p = g_ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lk(g_mu);
  p = g_ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    void* q = nullptr;
    if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return nullptr;
    p = q;
    g_ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace ft
