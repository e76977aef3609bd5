// Stand-in HIP runtime and kernel launchers for host-only tests of vlca_api.cpp
// (see hip_stub.h).  Allocations are plain host memory; a "kernel" writes the
// first and last bytes of the worklist it is given, so that a use of a freed
// buffer shows up under the address sanitizer.
#include "hip_stub.h"

#include <cstdlib>
#include <cstring>

namespace stub {
State g;
void reset() {
  const bool dev = g.has_device;
  g = State();
  g.has_device = dev;
}
}  // namespace stub

using stub::g;

extern "C" {

hipError_t hipGetDevice(int* dev) {
  if (!g.has_device) return hipErrorNoDevice;
  *dev = 0;
  return hipSuccess;
}

hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t attr, int) {
  if (attr != hipDeviceAttributeMultiprocessorCount) return hipErrorInvalidValue;
  *v = g.cus;
  return hipSuccess;
}

hipError_t hipStreamIsCapturing(hipStream_t s, hipStreamCaptureStatus* st) {
  *st = (g.capturing != nullptr && s == g.capturing) ? hipStreamCaptureStatusActive : hipStreamCaptureStatusNone;
  return hipSuccess;
}

hipError_t hipThreadExchangeStreamCaptureMode(hipStreamCaptureMode* mode) {
  const hipStreamCaptureMode old = g.mode;
  g.mode = *mode;
  *mode = old;
  return hipSuccess;
}

// As the runtime does: an allocation while a stream is captured in global mode
// is refused unless this thread has relaxed its capture mode.
hipError_t hipMalloc(void** p, size_t n) {
  if (g.capturing != nullptr && g.mode != hipStreamCaptureModeRelaxed) {
    ++g.capture_violations;
    return hipErrorStreamCaptureUnsupported;
  }
  *p = std::malloc(n == 0 ? 1 : n);
  if (*p == nullptr) return hipErrorOutOfMemory;
  std::memset(*p, 0xA5, n);  // garbage, as fresh device memory may hold
  ++g.allocs;
  return hipSuccess;
}

hipError_t hipFree(void* p) {
  std::free(p);
  ++g.frees;
  return hipSuccess;
}

hipError_t hipMemsetAsync(void* p, int v, size_t n, hipStream_t s) {
  ++g.memsets;
  if (g.capturing != nullptr && s == g.capturing) {
    ++g.captured_memsets;  // would become a memset node of the graph
    return hipSuccess;
  }
  std::memset(p, v, n);
  return hipSuccess;
}

hipError_t hipStreamCreateWithFlags(hipStream_t* s, unsigned int) {
  static char fake[16];
  *s = reinterpret_cast<hipStream_t>(&fake[++g.streams_created % 16]);
  return hipSuccess;
}

hipError_t hipStreamSynchronize(hipStream_t s) {
  if (g.capturing != nullptr && (s == g.capturing || g.mode != hipStreamCaptureModeRelaxed)) {
    ++g.capture_violations;
    return hipErrorStreamCaptureUnsupported;
  }
  ++g.syncs;
  g.synced.push_back(s);
  return hipSuccess;
}

}  // extern "C"

namespace vlca {

namespace {
int64_t touch(const int4* items, const int32_t* count) {
  if (items == nullptr || count == nullptr) return 0;
  // The count word sits right after the worklist's items: write both ends.
  const int64_t bytes = reinterpret_cast<const char*>(count) - reinterpret_cast<const char*>(items) + 4;
  char* b = const_cast<char*>(reinterpret_cast<const char*>(items));
  b[0] = 1;
  b[bytes - 1] = 1;
  return bytes;
}
// The split pool's arrival counters must read zero when a kernel that may split starts.
void check_counters(const SplitArgs& split) {
  if (split.p <= 1) return;
  for (int i = 0; i < kPoolMaxSlots; ++i)
    if (split.ctr[i * kSplitCtrStride] != 0) ++g.dirty_counters;
}
}  // namespace

hipError_t launch_schedule(const int32_t*, int num_users, int max_tiles, int4* items, int32_t* count, int32_t*,
                           const SplitArgs& split, hipStream_t stream) {
  g.launches.push_back({'s', items, touch(items, count), num_users, max_tiles, 0, 1, -1, split, stream});
  return hipSuccess;
}

hipError_t launch_attention(const void*, const int4* items, const int32_t* count, int32_t*, int n_heads, float,
                            const SplitArgs& split, void*, int grid, int layer_log2, hipStream_t stream) {
  g.launches.push_back({'a', items, touch(items, count), 0, 0, n_heads, grid, layer_log2, split, stream});
  check_counters(split);
  return hipSuccess;
}

hipError_t launch_attention_fused(const void*, const int32_t*, int num_users, int max_tiles, int n_heads, float,
                                  const SplitArgs& split, void*, int grid, int layer_log2, hipStream_t stream) {
  g.launches.push_back({'f', nullptr, 0, num_users, max_tiles, n_heads, grid, layer_log2, split, stream});
  check_counters(split);
  return hipSuccess;
}

int attention_blocks_per_cu(bool) { return g.blocks_per_cu; }

hipError_t noalloc_scratch(char** ptr) {
  static char* scratch = static_cast<char*>(std::calloc(kNoAllocScratchBytes, 1));
  ++g.scratch_lookups;
  *ptr = scratch;
  return scratch != nullptr ? hipSuccess : hipErrorOutOfMemory;
}

}  // namespace vlca
