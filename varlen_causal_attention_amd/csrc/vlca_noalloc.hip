// Scratch memory of varlen_causal_attn_fwd_noalloc: a fixed array per device, so
// that the entry point never allocates (for callers that cannot: code under
// graph capture, serving loops that forbid allocation).  Every call on a device
// shares that device's array: calls that overlap on one device race on it.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>

#include "vlca_internal.h"

namespace vlca {
namespace {

// Split pool, its arrival counters (zero when the code object is loaded; every
// call leaves them zero, and the scheduler kernel clears them), then the
// worklist with its count and work counters.  About 27 MB per device.
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

std::mutex g_mu;
std::map<int, char*> g_ptr;  // device -> device address of its scratch array

}  // namespace

hipError_t noalloc_scratch(char** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_ptr.find(dev);
  if (it == g_ptr.end()) {
    // The array's name in host code stands for a host-side shadow; the device
    // copy's address (one per device, the current one here) comes from the runtime.
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return e != hipSuccess ? e : hipErrorInvalidSymbol;
    it = g_ptr.emplace(dev, static_cast<char*>(p)).first;
  }
  *ptr = it->second;
  return hipSuccess;
}

}  // namespace vlca
