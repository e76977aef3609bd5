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
  // Distinct handles for the whole run (the library keys its state by stream).
  static char fake[64];
  static int next = 0;
  if (next == 64) return hipErrorOutOfMemory;
  *s = reinterpret_cast<hipStream_t>(&fake[next++]);
  ++g.streams_created;
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

hipError_t hipMemset(void* p, int v, size_t n) {
  if (g.capturing != nullptr && g.mode != hipStreamCaptureModeRelaxed) {
    ++g.capture_violations;
    return hipErrorStreamCaptureUnsupported;
  }
  std::memset(p, v, n);
  ++g.memsets;
  return hipSuccess;
}

hipError_t hipMemcpyAsync(void*, const void*, size_t n, hipMemcpyKind, hipStream_t s) {
  if (g.capturing != nullptr && s == g.capturing) ++g.captured_memsets;
  ++g.copies;
  g.copied_bytes += static_cast<int64_t>(n);
  return hipSuccess;
}

hipError_t hipStreamDestroy(hipStream_t) {
  ++g.streams_destroyed;
  return hipSuccess;
}

hipError_t hipDeviceSynchronize() {
  ++g.device_syncs;
  return hipSuccess;
}

hipError_t hipStreamBeginCapture(hipStream_t s, hipStreamCaptureMode) {
  if (g.capturing != nullptr) return hipErrorIllegalState;
  g.capturing = s;
  return hipSuccess;
}

hipError_t hipStreamEndCapture(hipStream_t s, hipGraph_t* graph) {
  if (g.capturing != s) return hipErrorIllegalState;
  g.capturing = nullptr;
  ++g.captures;
  *graph = reinterpret_cast<hipGraph_t>(new int(g.captures));
  return hipSuccess;
}

hipError_t hipGraphInstantiate(hipGraphExec_t* exec, hipGraph_t graph, hipGraphNode_t*, char*, size_t) {
  *exec = reinterpret_cast<hipGraphExec_t>(new int(*reinterpret_cast<int*>(graph)));
  return hipSuccess;
}

hipError_t hipGraphLaunch(hipGraphExec_t exec, hipStream_t s) {
  ++g.graph_launches;
  g.launches.push_back({'g', nullptr, *reinterpret_cast<int*>(exec), 0, 0, 0, 0, -1, {0, 0, 0, nullptr, nullptr}, s});
  return hipSuccess;
}

hipError_t hipGraphExecDestroy(hipGraphExec_t exec) {
  delete reinterpret_cast<int*>(exec);
  ++g.execs_destroyed;
  return hipSuccess;
}

hipError_t hipGraphDestroy(hipGraph_t graph) {
  delete reinterpret_cast<int*>(graph);
  ++g.graphs_destroyed;
  return hipSuccess;
}

}  // extern "C"

namespace vlca {

hipError_t launch_pad_offsets(const int32_t*, int num_users, int total, int32_t*, int max_users, hipStream_t) {
  ++g.pads;
  g.last_pad_users = num_users;
  g.last_pad_total = total;
  g.last_pad_max = max_users;
  return hipSuccess;
}


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
// Zero the work counters a kernel would (sets of kQueues counters kQueueStride
// apart, `sets` of them kBwdDqQueue apart): the address sanitizer flags a
// workspace tail too short for them.
void zero_queue(int32_t* queue, int sets) {
  if (queue == nullptr) return;
  for (int q = 0; q < kQueues; ++q)
    for (int k = 0; k < sets; ++k) queue[q * kQueueStride + k * kBwdDqQueue] = 0;
}
// The split pool's arrival counters must read zero when a kernel that may split starts.
void check_counters(const SplitArgs& split) {
  if (split.p <= 1) return;
  for (int i = 0; i < kPoolMaxSlots; ++i)
    if (split.ctr[i * kSplitCtrStride] != 0) ++g.dirty_counters;
}
}  // namespace

hipError_t launch_schedule(const int32_t*, int num_users, int max_tiles, int4* items, int32_t* count,
                           int32_t* queue, const SplitArgs& split, hipStream_t stream) {
  zero_queue(queue, 1);
  g.launches.push_back({'s', items, touch(items, count), num_users, max_tiles, 0, 1, -1, split, stream});
  return hipSuccess;
}

hipError_t launch_attention(const void*, const int4* items, const int32_t* count, int32_t*, int n_heads, float,
                            const SplitArgs& split, void*, float*, int grid, int layer_log2, hipStream_t stream) {
  g.launches.push_back({'a', items, touch(items, count), 0, 0, n_heads, grid, layer_log2, split, stream});
  check_counters(split);
  return hipSuccess;
}

hipError_t launch_attention_fused(const void*, const int32_t*, int num_users, int max_tiles, int n_heads, float,
                                  const SplitArgs& split, void*, float*, int grid, int layer_log2,
                                  hipStream_t stream) {
  g.launches.push_back({'f', nullptr, 0, num_users, max_tiles, n_heads, grid, layer_log2, split, stream});
  check_counters(split);
  return hipSuccess;
}

hipError_t launch_bwd_prepare(const void*, const void*, const float*, const int32_t*, int num_users, int max_tiles,
                              int4* items, int32_t* count, int32_t* queue, int n_heads, void*, int,
                              hipStream_t stream) {
  zero_queue(queue, 2);
  g.launches.push_back({'p', items, touch(items, count), num_users, max_tiles, n_heads, 0, -1,
                        {0, 0, 0, nullptr, nullptr}, stream});
  return hipSuccess;
}

hipError_t launch_backward(const void*, const void*, const float*, const int4* items, const int32_t* count,
                           int32_t*, int64_t max_items, int n_heads, float, void*, int, hipStream_t stream) {
  g.launches.push_back({'b', items, touch(items, count), 0, (int)max_items, n_heads, 0, -1,
                        {0, 0, 0, nullptr, nullptr}, stream});
  return hipSuccess;
}

hipError_t launch_masked_attention(const void*, const int4* items, const int32_t* count, int32_t*, int n_heads,
                                   float, const int32_t*, const int32_t*, int group, int wl, int wr, void*, int grid,
                                   hipStream_t stream) {
  g.launches.push_back({'m', items, touch(items, count), group, wl, n_heads, grid, wr, {0, 0, 0, nullptr, nullptr},
                        stream});
  return hipSuccess;
}

hipError_t launch_masked_attention_fused(const void*, const int32_t*, int num_users, int max_tiles, int n_heads, float,
                                         const int32_t*, const int32_t*, int, int, int, void*, int grid,
                                         int layer_log2, hipStream_t stream) {
  g.launches.push_back({'M', nullptr, 0, num_users, max_tiles, n_heads, grid, layer_log2,
                        {0, 0, 0, nullptr, nullptr}, stream});
  return hipSuccess;
}

int masked_blocks_per_cu(bool) { return g.blocks_per_cu; }

hipError_t launch_ln_qkv(const void*, const void*, const void*, float, const void*, const void*, int T, int N, void*,
                         int, hipStream_t stream) {
  g.launches.push_back({'l', nullptr, 0, T, N, 0, 0, -1, {0, 0, 0, nullptr, nullptr}, stream});
  return hipSuccess;
}

hipError_t launch_out_residual(const void*, const void*, const void*, const void*, int T, int N, void*, int,
                               hipStream_t stream) {
  g.launches.push_back({'o', nullptr, 0, T, N, 0, 0, -1, {0, 0, 0, nullptr, nullptr}, stream});
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
