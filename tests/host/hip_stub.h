// A stand-in for the few HIP runtime calls and kernel launchers that the C ABI
// (vlca_api.cpp) makes, so that its host logic -- argument checks, launch plan,
// per-stream worklist and split-pool bookkeeping, allocation while a stream is
// being captured -- runs on a machine without a GPU, under the address and
// undefined-behaviour sanitizers.  Test infrastructure only.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <vector>

#include "vlca_internal.h"

namespace stub {

struct Launch {
  char kind;  // 's' scheduler, 'a' attention over a worklist, 'f' single kernel, 'g' graph launch
  const void* items;
  int64_t touched;  // bytes of `items` the stand-in kernel wrote
  int num_users, max_tiles, n_heads, grid, layer_log2;
  vlca::SplitArgs split;
  hipStream_t stream;
};

struct State {
  bool has_device = true;
  int cus = 256;
  int blocks_per_cu = 4;
  hipStream_t capturing = nullptr;             // the stream being captured (global mode), if any
  hipStreamCaptureMode mode = hipStreamCaptureModeGlobal;  // this thread's capture mode
  int allocs = 0, frees = 0, syncs = 0, streams_created = 0;
  int memsets = 0, captured_memsets = 0, capture_violations = 0, dirty_counters = 0, scratch_lookups = 0;
  int captures = 0, graph_launches = 0, graphs_destroyed = 0, execs_destroyed = 0, copies = 0, pads = 0;
  int device_syncs = 0, streams_destroyed = 0;
  int64_t copied_bytes = 0;
  int last_pad_users = -1, last_pad_total = -1, last_pad_max = -1;
  std::vector<hipStream_t> synced;
  std::vector<Launch> launches;
};

extern State g;
void reset();

}  // namespace stub
