// C ABI of the varlen causal attention library: argument checks (all on the
// host, before any HIP call), the per-(device, stream) scheduler workspace and
// split-state pool, and the launches.  Declarations and the full contract are in
// include/varlen_causal_attn.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <map>
#include <mutex>
#include <utility>

#include "varlen_causal_attn.h"
#include "vlca_internal.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;
// Bytes after the workspace's items: the count, then from the next 256-byte
// boundary the work counters (kQueueStride int32 apart).
constexpr size_t kWorkspaceTail = (1 + vlca::kQueues) * vlca::kQueueStride * sizeof(int32_t);

struct Workspace {
  int4* items = nullptr;     // capacity items, the int32 count, then the work counters
  int64_t capacity = 0;
};

// Key-range splitting in the single-kernel plan: an item of a user of t q-tiles
// with more than max(ceil(t / 2), kSplitMinWidth) key tiles runs as two parts on
// different workgroups, when the batch's split list fits in one round of the
// grid (the kernel decides from the batch's own lengths).  The parts' softmax
// states meet in a pool of kPoolSlots slots per (device, stream), shared by the
// heads.
constexpr int kSplitParts = vlca::kMaxSplitParts;
constexpr int kSplitMinWidth = 4;
constexpr int kPoolSlots = 2048;

struct SplitPool {
  float* pool = nullptr;    // kPoolSlots slots of kPoolSlotFloats floats
  int32_t* ctr = nullptr;   // kPoolSlots arrival counters, kSplitCtrStride apart
};

std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Workspace> g_workspaces;
std::map<std::pair<int, hipStream_t>, SplitPool> g_pools;
std::map<int, int> g_resident;  // 2*device + fused -> resident attention workgroups
std::map<int, int> g_cus;       // device -> compute units

int64_t max_tiles_of(int max_seqlen) { return (static_cast<int64_t>(max_seqlen) + vlca::kTileRows - 1) / vlca::kTileRows; }

int64_t required_capacity(int num_users, int max_seqlen) {
  return static_cast<int64_t>(num_users) * max_tiles_of(max_seqlen);
}

// Size and scalar checks shared by every entry point.
int check_sizes(int num_users, int max_seqlen) {
  if (num_users < 0 || max_seqlen < 0) return VLCA_ERR_NEGATIVE_SIZE;
  if (max_seqlen > VLCA_MAX_SEQLEN) return VLCA_ERR_TOO_LARGE;
  if (required_capacity(num_users, max_seqlen) > INT32_MAX) return VLCA_ERR_TOO_LARGE;
  return VLCA_OK;
}

int check_attention_args(const void* qkv, const int32_t* cu_seqlens, int num_users, int max_seqlen, int n_heads,
                         int head_dim, float scale, const void* out) {
  int rc = check_sizes(num_users, max_seqlen);
  if (rc != VLCA_OK) return rc;
  if (head_dim != vlca::kHeadDim) return VLCA_ERR_HEAD_DIM;
  if (n_heads < 1 || n_heads > 65536) return VLCA_ERR_N_HEADS;
  if (!std::isfinite(scale) || !(scale > 0.f)) return VLCA_ERR_SCALE;
  if (num_users > 0 && (qkv == nullptr || cu_seqlens == nullptr || out == nullptr)) return VLCA_ERR_NULL_POINTER;
  if (qkv != nullptr && qkv == out) return VLCA_ERR_ALIAS;
  return VLCA_OK;
}

// Compute units of a device.
int cu_count(int dev) {
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_cus.find(dev);
  if (it != g_cus.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  g_cus[dev] = n;
  return n;
}

// Resident attention workgroups per device: CUs x workgroups per CU, for the
// kernel over a worklist or the single-kernel variant.
int resident_blocks(int dev, bool fused) {
  const int n = cu_count(dev);
  std::lock_guard<std::mutex> lk(g_mu);
  const int key = 2 * dev + (fused ? 1 : 0);
  auto it = g_resident.find(key);
  if (it != g_resident.end()) return it->second;
  const int r = n * vlca::attention_blocks_per_cu(fused);
  g_resident[key] = r;
  return r;
}

// Persistent grid for `work` (unit, head) pairs: the resident workgroups, capped
// by the work.
int grid_size(int dev, int64_t work, bool fused) {
  int64_t g = resident_blocks(dev, fused);
  if (g > vlca::kMaxGrid) g = vlca::kMaxGrid;
  g -= g % 8;  // keeps w % 8 == blockIdx.x % 8 (one head per XCD when H = 8)
  if (g < 8) g = 8;
  if (work < g) g = work;
  return static_cast<int>(g);
}

// The kernel's `layer_log2` argument.  With every unit in one round of the
// fixed assignment (at most max_units units per head), log2 of the slots between
// workgroups that share a CU (workgroups g and g + CUs in launch order; a
// workgroup's slot is g / H with the grid a multiple of H, else g), when that is
// a power of two smaller than the slots; -1 otherwise (plain snake).
int snake_layer_log2(int dev, int grid, int n_heads, int64_t max_units) {
  const bool by_head = grid % n_heads == 0;
  const int64_t slots = by_head ? grid / n_heads : grid;
  if ((by_head ? max_units : max_units * n_heads) > slots) return -1;
  const int cus = cu_count(dev);
  if (by_head && cus % n_heads != 0) return -1;
  const int layer = by_head ? cus / n_heads : cus;
  if (layer < 1 || (layer & (layer - 1)) != 0 || layer >= slots) return -1;
  return __builtin_ctz(static_cast<unsigned>(layer));
}

int64_t item_pairs(int num_users, int max_seqlen, int n_heads) {
  return static_cast<int64_t>(num_users) * max_tiles_of(max_seqlen) * n_heads;
}

// Workspace for (device, stream), grown when a call needs more items.  Growth
// synchronises `stream` before freeing the old buffer, so it is refused while
// the stream is capturing.
int get_workspace(int dev, hipStream_t stream, int64_t capacity, Workspace** out) {
  std::lock_guard<std::mutex> lk(g_mu);
  Workspace& ws = g_workspaces[std::make_pair(dev, stream)];
  if (ws.capacity < capacity) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &st) != hipSuccess) return VLCA_ERR_HIP;
    if (st != hipStreamCaptureStatusNone) return VLCA_ERR_WORKSPACE;
    int64_t cap = ws.capacity > 0 ? ws.capacity : 16384;
    while (cap < capacity) cap *= 2;
    if (ws.items != nullptr) {
      if (hipStreamSynchronize(stream) != hipSuccess) return VLCA_ERR_HIP;
      (void)hipFree(ws.items);
      ws.items = nullptr;
      ws.capacity = 0;
    }
    void* p = nullptr;
    if (hipMalloc(&p, static_cast<size_t>(cap) * sizeof(int4) + kWorkspaceTail) != hipSuccess)
      return VLCA_ERR_WORKSPACE;
    ws.items = static_cast<int4*>(p);
    ws.capacity = cap;
  }
  *out = &ws;
  return VLCA_OK;
}

int32_t* workspace_count(const Workspace* ws) { return reinterpret_cast<int32_t*>(ws->items + ws->capacity); }

// Split-state pool for (device, stream), allocated by the first call that splits
// (fixed size, never grown); its counters are zeroed in stream order before that
// call and every call leaves them zero.  *capturing = true (and no pool) when it
// does not exist yet and the stream is being captured: that call runs unsplit.
int get_split_pool(int dev, hipStream_t stream, SplitPool** out, bool* capturing) {
  std::lock_guard<std::mutex> lk(g_mu);
  *capturing = false;
  SplitPool& sp = g_pools[std::make_pair(dev, stream)];
  if (sp.pool == nullptr) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &st) != hipSuccess) return VLCA_ERR_HIP;
    if (st != hipStreamCaptureStatusNone) {
      *capturing = true;
      return VLCA_OK;
    }
    const size_t pool_bytes = static_cast<size_t>(kPoolSlots) * vlca::kPoolSlotFloats * sizeof(float);
    const size_t ctr_bytes = static_cast<size_t>(kPoolSlots) * vlca::kSplitCtrStride * sizeof(int32_t);
    void* p = nullptr;
    if (hipMalloc(&p, pool_bytes + ctr_bytes) != hipSuccess) return VLCA_ERR_WORKSPACE;
    int32_t* ctr = reinterpret_cast<int32_t*>(static_cast<char*>(p) + pool_bytes);
    if (hipMemsetAsync(ctr, 0, ctr_bytes, stream) != hipSuccess) {
      (void)hipFree(p);
      return VLCA_ERR_HIP;
    }
    sp.pool = static_cast<float*>(p);
    sp.ctr = ctr;
  }
  *out = &sp;
  return VLCA_OK;
}

// Scheduler (when schedule) then attention.  queue: the library workspace's work
// counters (dynamic assignment, zeroed by the scheduler), or null for a caller's
// worklist (fixed assignment).  split: key-range splitting (fwd's scheduler plan
// only; a caller's worklist always holds whole items).
int launch_pair(const void* qkv, const int32_t* cu_seqlens, int num_users, int max_seqlen, int n_heads, float scale,
                int4* items, int32_t* count, int32_t* queue, const vlca::SplitArgs& split, void* out,
                hipStream_t stream, bool schedule) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return VLCA_ERR_HIP;
  const int max_tiles = static_cast<int>(max_tiles_of(max_seqlen));
  if (schedule) {
    if (vlca::launch_schedule(cu_seqlens, num_users, max_tiles, items, count, queue, split, stream) != hipSuccess)
      return VLCA_ERR_HIP;
  }
  int64_t pairs = item_pairs(num_users, max_seqlen, n_heads);
  if (split.p > 1) pairs *= kSplitParts;
  const int grid = grid_size(dev, pairs, false);
  const int layer_log2 =
      queue ? -1 : snake_layer_log2(dev, grid, n_heads, static_cast<int64_t>(num_users) * max_tiles);
  if (vlca::launch_attention(qkv, items, count, queue, n_heads, scale * kLog2e, split, out, grid, layer_log2,
                             stream) != hipSuccess)
    return VLCA_ERR_HIP;
  return VLCA_OK;
}

}  // namespace

extern "C" {

int varlen_causal_attn_fwd(const void* qkv, const int32_t* cu_seqlens, int num_users, int max_seqlen, int n_heads,
                           int head_dim, float scale, void* out, hipStream_t stream) {
  int rc = check_attention_args(qkv, cu_seqlens, num_users, max_seqlen, n_heads, head_dim, scale, out);
  if (rc != VLCA_OK) return rc;
  if (num_users == 0 || max_seqlen == 0) return VLCA_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return VLCA_ERR_HIP;
  // Small batches: one kernel that locates its own work (no worklist buffer).
  const int max_tiles = static_cast<int>(max_tiles_of(max_seqlen));
  const int64_t pairs = item_pairs(num_users, max_seqlen, n_heads);
  int grid = grid_size(dev, pairs, true);
  // Key-range splitting: both plans take the same decision from the batch's own
  // lengths (split when the list with split items has at most upr units, one
  // round of the single-kernel grid), so max_seqlen, which picks the plan, does
  // not change the bits.  Batches of more than kFusedUsers users never split.
  // Only users of more than kSplitMinWidth q-tiles have split items.
  vlca::SplitArgs split{0, 0, 0, 0, nullptr, nullptr};
  const int cap = kPoolSlots / n_heads;
  if (num_users <= vlca::kFusedUsers && max_tiles > kSplitMinWidth && cap >= kSplitParts) {
    SplitPool* sp = nullptr;
    bool capturing = false;
    rc = get_split_pool(dev, stream, &sp, &capturing);
    if (rc != VLCA_OK) return rc;
    if (!capturing) {
      const int upr = std::max(1, grid_size(dev, INT64_MAX, true) / n_heads);
      split = vlca::SplitArgs{kSplitParts, kSplitMinWidth, upr, cap, sp->pool, sp->ctr};
    }
  }
  if (vlca::fused_fits(num_users, max_tiles, n_heads, grid)) {
    if (split.p > 1) grid = grid_size(dev, pairs * kSplitParts, true);
    const int layer_log2 = snake_layer_log2(dev, grid, n_heads, static_cast<int64_t>(num_users) * max_tiles);
    if (vlca::launch_attention_fused(qkv, cu_seqlens, num_users, max_tiles, n_heads, scale * kLog2e, split, out,
                                     grid, layer_log2, stream) != hipSuccess)
      return VLCA_ERR_HIP;
    return VLCA_OK;
  }
  // The worklist may hold split units: at most upr more than the whole items.
  const int64_t need = required_capacity(num_users, max_seqlen);
  Workspace* ws = nullptr;
  rc = get_workspace(dev, stream, split.p > 1 ? need + std::min<int64_t>(need, split.upr) : need, &ws);
  if (rc == VLCA_ERR_WORKSPACE && split.p > 1) {
    // E.g. a stream being captured whose workspace only holds whole items: run them whole.
    split = vlca::SplitArgs{0, 0, 0, 0, nullptr, nullptr};
    rc = get_workspace(dev, stream, need, &ws);
  }
  if (rc != VLCA_OK) return rc;
  return launch_pair(qkv, cu_seqlens, num_users, max_seqlen, n_heads, scale, ws->items, workspace_count(ws),
                     workspace_count(ws) + vlca::kQueueStride, split, out, stream, true);
}

int varlen_causal_attn_worklist_capacity(int num_users, int max_seqlen, int64_t* capacity) {
  int rc = check_sizes(num_users, max_seqlen);
  if (rc != VLCA_OK) return rc;
  if (capacity == nullptr) return VLCA_ERR_NULL_POINTER;
  *capacity = required_capacity(num_users, max_seqlen);
  return VLCA_OK;
}

int varlen_causal_attn_build_worklist(const int32_t* cu_seqlens, int num_users, int max_seqlen, int32_t* items,
                                      int64_t capacity, int32_t* count, hipStream_t stream) {
  int rc = check_sizes(num_users, max_seqlen);
  if (rc != VLCA_OK) return rc;
  const int64_t need = required_capacity(num_users, max_seqlen);
  if (count == nullptr || (need > 0 && items == nullptr) || (num_users > 0 && cu_seqlens == nullptr))
    return VLCA_ERR_NULL_POINTER;
  if (capacity < need) return VLCA_ERR_CAPACITY;
  const int max_tiles = static_cast<int>(max_tiles_of(max_seqlen));
  if (vlca::launch_schedule(cu_seqlens, num_users, max_tiles, reinterpret_cast<int4*>(items), count, nullptr,
                            vlca::SplitArgs{0, 0, 0, 0, nullptr, nullptr}, stream) != hipSuccess)
    return VLCA_ERR_HIP;
  return VLCA_OK;
}

int varlen_causal_attn_fwd_worklist(const void* qkv, const int32_t* cu_seqlens, int num_users, int max_seqlen,
                                    int n_heads, int head_dim, float scale, const int32_t* items, int64_t capacity,
                                    const int32_t* count, void* out, hipStream_t stream) {
  int rc = check_attention_args(qkv, cu_seqlens, num_users, max_seqlen, n_heads, head_dim, scale, out);
  if (rc != VLCA_OK) return rc;
  if (num_users > 0 && (items == nullptr || count == nullptr)) return VLCA_ERR_NULL_POINTER;
  if (num_users > 0 && capacity < required_capacity(num_users, max_seqlen)) return VLCA_ERR_CAPACITY;
  if (num_users == 0 || max_seqlen == 0) return VLCA_OK;
  return launch_pair(qkv, cu_seqlens, num_users, max_seqlen, n_heads, scale,
                     reinterpret_cast<int4*>(const_cast<int32_t*>(items)), const_cast<int32_t*>(count), nullptr,
                     vlca::SplitArgs{0, 0, 0, 0, nullptr, nullptr}, out, stream, false);
}

int varlen_causal_attn_single_kernel(int num_users, int max_seqlen, int n_heads, int* single_kernel) {
  int rc = check_sizes(num_users, max_seqlen);
  if (rc != VLCA_OK) return rc;
  if (single_kernel == nullptr) return VLCA_ERR_NULL_POINTER;
  if (n_heads < 1 || n_heads > 65536) return VLCA_ERR_N_HEADS;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return VLCA_ERR_HIP;
  const int max_tiles = static_cast<int>(max_tiles_of(max_seqlen));
  const int grid = grid_size(dev, item_pairs(num_users, max_seqlen, n_heads), true);
  *single_kernel = (num_users > 0 && max_seqlen > 0 && vlca::fused_fits(num_users, max_tiles, n_heads, grid)) ? 1 : 0;
  return VLCA_OK;
}

int varlen_causal_attn_tile_rows(void) { return vlca::kTileRows; }

const char* varlen_causal_attn_strerror(int code) {
  switch (code) {
    case VLCA_OK: return "success";
    case VLCA_ERR_NULL_POINTER: return "a required pointer is NULL";
    case VLCA_ERR_NEGATIVE_SIZE: return "num_users or max_seqlen is negative";
    case VLCA_ERR_HEAD_DIM: return "head_dim must be 64";
    case VLCA_ERR_N_HEADS: return "n_heads must be in [1, 65536]";
    case VLCA_ERR_SCALE: return "scale must be finite and > 0";
    case VLCA_ERR_TOO_LARGE: return "max_seqlen exceeds VLCA_MAX_SEQLEN or the worklist exceeds 2^31 items";
    case VLCA_ERR_CAPACITY: return "worklist buffer is smaller than varlen_causal_attn_worklist_capacity()";
    case VLCA_ERR_ALIAS: return "qkv and out must not be the same buffer";
    case VLCA_ERR_WORKSPACE: return "library workspace could not be allocated (or must grow during stream capture)";
    case VLCA_ERR_HIP: return "HIP runtime call or kernel launch failed";
    default: return "unknown error code";
  }
}

}  // extern "C"
