// Scratch space for mla_decode_noalloc: a fixed device array owned by the library, for callers that
// cannot allocate (code under HIP graph capture, serving loops, harnesses that forbid hipMalloc).
//
// The array is a file-scope __device__ object, so every GPU the library runs on holds its own copy,
// at its own address, from the moment the code object is loaded until the process ends.  In host
// code its name is only a stand-in for the symbol: its device address is looked up once per device
// (hipGetSymbolAddress, with that device current) and only that address is ever passed to a kernel.
#include <atomic>
#include <mutex>

#include "mla_device.h"

namespace mla {
namespace {

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_lookup;

}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_lookup);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!p) return hipErrorInvalidSymbol;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace mla
