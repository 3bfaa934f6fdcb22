// Device memory of the batched AllReduce entry point that allocates
// nothing (coll_allreduce_batch_noalloc): its descriptor table lives in a
// static device array instead of a buffer the library allocates, for
// callers that cannot call hipMalloc.  Every GPU the library runs on holds
// its own copy of the array until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernel_args.h"

// The table (call records, then per-call pointer lists).  In host code this
// name is only a stand-in for the symbol: the device address comes from
// hipGetSymbolAddress, per device, below.
static __device__ __align__(256) unsigned char scratch[coll::kNoAllocScratchBytes];

namespace coll {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

int noalloc_scratch(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!ptr) return (int)hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return 0;
}

}  // namespace coll
