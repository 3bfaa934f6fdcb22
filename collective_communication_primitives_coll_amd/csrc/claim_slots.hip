// Counter slots for the claimed tails of the streaming kernels: each slot
// holds a claim counter, zero at launch and zeroed again by the worker that
// makes the launch's last claim.  A static device array, so that no call
// allocates; every GPU the library runs on holds its own copy until the
// process ends.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernel_args.h"

// In host code this name is only a stand-in for the symbol: the device
// address comes from hipGetSymbolAddress, per device, below.
static __device__ __align__(256) unsigned long long claim_slots[coll::kClaimSlots * coll::kClaimSlotWords];

namespace coll {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_slots_mu;
unsigned long long* g_slots_ptr[kMaxDevices] = {};
}  // namespace

int claim_slots_base(int dev, unsigned long long** out) {
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_slots_mu);
  if (!g_slots_ptr[dev]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(claim_slots));
    if (e != hipSuccess) return (int)e;
    if (!ptr) return (int)hipErrorInvalidSymbol;
    g_slots_ptr[dev] = (unsigned long long*)ptr;
  }
  *out = g_slots_ptr[dev];
  return 0;
}

}  // namespace coll
