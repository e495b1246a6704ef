// m3_noalloc.hip -- the device-resident scratch buffer behind
// m3_scan_prefill_noalloc (include/m3.h): the prefill's chunk hand-off space
// for callers that cannot allocate device memory.
//
// The buffer is a file-scope __device__ array, one copy per GPU the library
// runs on, held until the process ends.  In host code its name is only a
// host-side stand-in, so its device address is looked up here, once per device
// with that device current (hipGetSymbolAddress), and that address is what
// every launch uses.
#include <atomic>

#include "m3_internal.h"

namespace m3 {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];   // device address per device (null: not looked up)

}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    // (two threads racing here both store the same address)
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace m3
