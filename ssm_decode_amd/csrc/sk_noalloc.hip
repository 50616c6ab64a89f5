// The scratch memory of sketchssm_read_noalloc: the read's workspace held in
// a device array of the library itself, for callers that cannot allocate.
//
// Each GPU the library runs on holds its own copy of the array (a device
// global of the code object) until the process ends.  In host code the
// array's name is only a stand-in; its device address on the current device
// comes from hipGetSymbolAddress, taken once per device and kept.
#include <atomic>
#include <mutex>

#include <hip/hip_runtime.h>

#include "sketchssm.h"

namespace sk {

static __device__ __align__(256) unsigned char scratch[SKSSM_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_mu;
}  // namespace

// Device address of the current device's scratch array: 0, or -5
// (SKSSM_ELAUNCH) when the device or the symbol cannot be resolved.
int noalloc_scratch(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return SKSSM_ELAUNCH;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* q = nullptr;
      if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || q == nullptr) {
        (void)hipGetLastError();             // leave no sticky error for the caller's next call
        return SKSSM_ELAUNCH;
      }
      g_scratch[dev].store(q, std::memory_order_release);
      p = q;
    }
  }
  *out = p;
  return SKSSM_OK;
}

}  // namespace sk
