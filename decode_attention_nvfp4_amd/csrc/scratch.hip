// scratch.hip -- the fixed device scratch behind nvfp4_decode_attn_noalloc.
//
// The array lives in the code object, so every device the library runs on
// holds its own copy from the first use until the process ends.  Host code
// never passes the array's name to a kernel (on the host it only names a
// stand-in); it takes the device address from hipGetSymbolAddress, once per
// device with that device current, and hands that address to the kernels as
// it hands them a caller's workspace.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "internal.h"

namespace nvfp4 {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_addr[kMaxDevices];
std::mutex g_mu;
}  // namespace

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_addr[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lk(g_mu);
    p = g_addr[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_addr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace nvfp4
