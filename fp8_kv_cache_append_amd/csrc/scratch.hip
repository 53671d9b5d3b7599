// Library-owned device scratch for fp8kv_decode_noalloc: the split partials
// of a decode call that brings no workspace.  The array is a file-scope
// device symbol, so every GPU the library runs on holds its own copy (loaded
// with the code object, kept until the process ends) and no call allocates.
// Host code never passes the symbol's name to a kernel (on the host it is a
// stand-in, not a device address): the address is resolved once per device
// with hipGetSymbolAddress, with that device current, and kept.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "launch.h"

namespace fp8kv {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 128;
std::atomic<void*> g_scratch[kMaxScratchDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t scratch_address(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace fp8kv
