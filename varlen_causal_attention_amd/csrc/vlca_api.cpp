// C ABI of the varlen causal attention library: argument checks (all on the
// host, before any HIP call), the per-(device, stream) scheduler worklist and
// split-state pool, and the launches.  Declarations and the full contract are in
// include/varlen_causal_attn.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "varlen_causal_attn.h"
#include "vlca_internal.h"

namespace {

constexpr float kLog2e = 1.4426950408889634f;
// Bytes after the workspace's items: the count, then from the next 256-byte
// boundary the work counters (kQueueStride int32 apart).
constexpr size_t kWorkspaceTail = (1 + vlca::kQueues) * vlca::kQueueStride * sizeof(int32_t);

// Key-range splitting: an item of a user of t q-tiles with more than
// max(ceil(t / 2), kSplitMinWidth) key tiles runs as two parts on different
// workgroups, when the batch's split list fits in one round of the single-kernel
// grid (at most upr units per head; the kernels decide from the lengths of the
// batch's non-empty users).  The parts' softmax states meet in a pool of
// vlca::kPoolMaxSlots slots per (device, stream), shared by the heads.
constexpr int kSplitParts = vlca::kMaxSplitParts;
constexpr int kSplitMinWidth = 4;
constexpr size_t kPoolBytes = static_cast<size_t>(vlca::kPoolMaxSlots) * vlca::kPoolSlotFloats * sizeof(float);
constexpr size_t kPoolCtrBytes = static_cast<size_t>(vlca::kPoolMaxSlots) * vlca::kSplitCtrStride * sizeof(int32_t);

// Library state of one (device, stream): the scheduler's worklist (capacity
// items, then the int32 count and the work counters) and the split-state pool
// (then its arrival counters).  Calls on one stream run in stream order and
// share it; so does every graph captured on that stream.  Nothing is ever
// freed: a worklist that has to grow is replaced and the old one kept, since
// graphs captured earlier may still launch kernels that use it.
struct StreamState {
  int4* items = nullptr;
  int64_t capacity = 0;
  float* pool = nullptr;
  int32_t* ctr = nullptr;
};

std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, StreamState> g_states;
std::vector<void*> g_retired;   // replaced worklists, kept for graphs that still refer to them
std::map<int, hipStream_t> g_zero_streams;  // per device: clears new pools while another stream captures
std::map<int, int> g_resident;  // 2*device + fused -> resident attention workgroups
std::map<int, int> g_cus;       // device -> compute units

int64_t max_tiles_of(int max_seqlen) { return (static_cast<int64_t>(max_seqlen) + vlca::kTileRows - 1) / vlca::kTileRows; }

int64_t required_capacity(int num_users, int max_seqlen) {
  return static_cast<int64_t>(num_users) * max_tiles_of(max_seqlen);
}

// Alignment of a pointer the kernels read or write in chunks of `bytes` (a null
// pointer passes: the null checks come first where it matters).
bool aligned(const void* p, uintptr_t bytes) { return (reinterpret_cast<uintptr_t>(p) & (bytes - 1)) == 0; }

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
  if (!aligned(qkv, 16) || !aligned(out, 16) || !aligned(cu_seqlens, 4)) return VLCA_ERR_ALIGN;
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

// Units per head that one round of the single-kernel grid runs (at most the
// pool's slots per head): a batch splits only if its split list fits.  Depends
// on the device and n_heads only.
int split_units_per_round(int dev, int n_heads) {
  const int g = std::min(grid_size(dev, INT64_MAX, true), vlca::kPoolMaxSlots);
  return std::max(1, g / n_heads);
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

// Whether `stream` is being captured into a graph.
int capturing(hipStream_t stream, bool* cap) {
  hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &st) != hipSuccess) return VLCA_ERR_HIP;
  *cap = st != hipStreamCaptureStatusNone;
  return VLCA_OK;
}

// Allocates device memory now, also while a stream is being captured: the
// calling thread's capture mode is relaxed for the call (an allocation is not a
// stream operation, so nothing is recorded into the graph).
hipError_t alloc_now(void** p, size_t bytes) {
  hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
  if (hipThreadExchangeStreamCaptureMode(&mode) != hipSuccess) return hipErrorUnknown;
  const hipError_t e = hipMalloc(p, bytes);
  (void)hipThreadExchangeStreamCaptureMode(&mode);
  return e;
}

// Zeroes new memory before its first use on `stream`: in stream order, or --
// while `stream` is being captured, where a memset would be recorded -- on a
// library stream of the device, waited for here (once per new pool).
int zero_before_use(int dev, void* p, size_t bytes, hipStream_t stream, bool cap) {
  if (!cap) return hipMemsetAsync(p, 0, bytes, stream) == hipSuccess ? VLCA_OK : VLCA_ERR_HIP;
  hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
  if (hipThreadExchangeStreamCaptureMode(&mode) != hipSuccess) return VLCA_ERR_HIP;
  int rc = VLCA_OK;
  hipStream_t& zs = g_zero_streams[dev];  // g_mu is held by the caller
  if (zs == nullptr && hipStreamCreateWithFlags(&zs, hipStreamNonBlocking) != hipSuccess) {
    zs = nullptr;
    rc = VLCA_ERR_HIP;
  }
  if (rc == VLCA_OK && (hipMemsetAsync(p, 0, bytes, zs) != hipSuccess || hipStreamSynchronize(zs) != hipSuccess))
    rc = VLCA_ERR_HIP;
  (void)hipThreadExchangeStreamCaptureMode(&mode);
  return rc;
}

// Worklist of (device, stream) with room for `capacity` items.  A larger one
// replaces it without synchronising the stream; the old one is kept (kernels in
// flight and captured graphs may still use it).
int get_workspace(int dev, hipStream_t stream, int64_t capacity, StreamState* out) {
  std::lock_guard<std::mutex> lk(g_mu);
  StreamState& st = g_states[std::make_pair(dev, stream)];
  if (st.capacity < capacity) {
    int64_t n = st.capacity > 0 ? st.capacity : 16384;
    while (n < capacity) n *= 2;
    void* p = nullptr;
    if (alloc_now(&p, static_cast<size_t>(n) * sizeof(int4) + kWorkspaceTail) != hipSuccess)
      return VLCA_ERR_WORKSPACE;
    if (st.items != nullptr) g_retired.push_back(st.items);
    st.items = static_cast<int4*>(p);
    st.capacity = n;
  }
  *out = st;
  return VLCA_OK;
}

int32_t* workspace_count(const StreamState* st) { return reinterpret_cast<int32_t*>(st->items + st->capacity); }

// Split-state pool of (device, stream), allocated by the first call that may
// split (fixed size); its arrival counters are zeroed before that call and
// every call leaves them zero.
int get_split_pool(int dev, hipStream_t stream, StreamState* out) {
  std::lock_guard<std::mutex> lk(g_mu);
  StreamState& st = g_states[std::make_pair(dev, stream)];
  if (st.pool == nullptr) {
    bool cap = false;
    if (capturing(stream, &cap) != VLCA_OK) return VLCA_ERR_HIP;
    void* p = nullptr;
    if (alloc_now(&p, kPoolBytes + kPoolCtrBytes) != hipSuccess) return VLCA_ERR_WORKSPACE;
    int32_t* ctr = reinterpret_cast<int32_t*>(static_cast<char*>(p) + kPoolBytes);
    const int rc = zero_before_use(dev, ctr, kPoolCtrBytes, stream, cap);
    if (rc != VLCA_OK) {
      g_retired.push_back(p);  // never freed while a capture may be under way
      return rc;
    }
    st.pool = static_cast<float*>(p);
    st.ctr = ctr;
  }
  *out = st;
  return VLCA_OK;
}

// Scheduler (when schedule) then attention.  queue: the library workspace's work
// counters (dynamic assignment, zeroed by the scheduler), or null for a caller's
// worklist (fixed assignment).  split: key-range splitting (fwd's scheduler plan
// only; a caller's worklist always holds whole items).
int launch_pair(const void* qkv, const int32_t* cu_seqlens, int num_users, int max_seqlen, int n_heads, float scale,
                int4* items, int32_t* count, int32_t* queue, const vlca::SplitArgs& split, void* out, float* lse,
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
  if (vlca::launch_attention(qkv, items, count, queue, n_heads, scale * kLog2e, split, out, lse, grid, layer_log2,
                             stream) != hipSuccess)
    return VLCA_ERR_HIP;
  return VLCA_OK;
}

// The forward pass; lse: null, or [T, n_heads] fp32 log-sum-exp output.
int fwd_impl(const void* qkv, const int32_t* cu_seqlens, int num_users, int max_seqlen, int n_heads, int head_dim,
             float scale, void* out, float* lse, hipStream_t stream) {
  int rc = check_attention_args(qkv, cu_seqlens, num_users, max_seqlen, n_heads, head_dim, scale, out);
  if (rc != VLCA_OK) return rc;
  if (num_users == 0 || max_seqlen == 0) return VLCA_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return VLCA_ERR_HIP;
  const int max_tiles = static_cast<int>(max_tiles_of(max_seqlen));
  const int64_t pairs = item_pairs(num_users, max_seqlen, n_heads);
  // Key-range splitting: both plans take the same decision from the lengths of
  // the batch's non-empty users (split when the list with split items has at
  // most upr units per head, one round of the single-kernel grid), so neither
  // max_seqlen (which picks the plan) nor zero-length users change the bits.
  // Only users of more than kSplitMinWidth q-tiles have split items.
  vlca::SplitArgs split{0, 0, 0, nullptr, nullptr};
  const int upr = split_units_per_round(dev, n_heads);
  if (max_tiles > kSplitMinWidth && upr >= kSplitParts) {
    StreamState st;
    rc = get_split_pool(dev, stream, &st);
    if (rc != VLCA_OK) return rc;
    split = vlca::SplitArgs{kSplitParts, kSplitMinWidth, upr, st.pool, st.ctr};
  }
  // Small batches: one kernel that locates its own work (no worklist buffer).
  int grid = grid_size(dev, pairs, true);
  if (vlca::fused_fits(num_users, max_tiles, n_heads, grid)) {
    if (split.p > 1) grid = grid_size(dev, pairs * kSplitParts, true);
    const int layer_log2 = snake_layer_log2(dev, grid, n_heads, static_cast<int64_t>(num_users) * max_tiles);
    if (vlca::launch_attention_fused(qkv, cu_seqlens, num_users, max_tiles, n_heads, scale * kLog2e, split, out,
                                     lse, grid, layer_log2, stream) != hipSuccess)
      return VLCA_ERR_HIP;
    return VLCA_OK;
  }
  // The worklist holds the whole items, or a split list of at most upr units.
  const int64_t need = required_capacity(num_users, max_seqlen);
  StreamState st;
  rc = get_workspace(dev, stream, split.p > 1 ? std::max<int64_t>(need, upr) : need, &st);
  if (rc != VLCA_OK) return rc;
  return launch_pair(qkv, cu_seqlens, num_users, max_seqlen, n_heads, scale, st.items, workspace_count(&st),
                     workspace_count(&st) + vlca::kQueueStride, split, out, lse, stream, true);
}

}  // namespace

extern "C" {

int varlen_causal_attn_fwd(const void* qkv, const int32_t* cu_seqlens, int num_users, int max_seqlen, int n_heads,
                           int head_dim, float scale, void* out, hipStream_t stream) {
  return fwd_impl(qkv, cu_seqlens, num_users, max_seqlen, n_heads, head_dim, scale, out, nullptr, stream);
}

int varlen_causal_attn_fwd_lse(const void* qkv, const int32_t* cu_seqlens, int num_users, int max_seqlen,
                               int n_heads, int head_dim, float scale, void* out, float* lse, hipStream_t stream) {
  if (num_users > 0 && max_seqlen > 0 && lse == nullptr) return VLCA_ERR_NULL_POINTER;
  if (!aligned(lse, 4)) return VLCA_ERR_ALIGN;
  return fwd_impl(qkv, cu_seqlens, num_users, max_seqlen, n_heads, head_dim, scale, out, lse, stream);
}
int varlen_causal_attn_fwd_masked(const void* qkv, const int32_t* cu_seqlens, int num_users, int max_seqlen,
                                  int n_heads, int head_dim, float scale, const vlca_mask* mask, void* out,
                                  hipStream_t stream) {
  if (mask != nullptr) {
    if (mask->target_group_size < 1 || mask->window_left < -1 || mask->window_right < -1) return VLCA_ERR_MASK;
    if ((mask->num_contexts != nullptr || mask->num_targets != nullptr) && mask->window_right != 0)
      return VLCA_ERR_MASK;
    if (!aligned(mask->num_contexts, 4) || !aligned(mask->num_targets, 4)) return VLCA_ERR_ALIGN;
  }
  const bool plain = mask == nullptr || (mask->num_contexts == nullptr && mask->num_targets == nullptr &&
                                         mask->window_left == -1 && mask->window_right == 0);
  if (plain) return fwd_impl(qkv, cu_seqlens, num_users, max_seqlen, n_heads, head_dim, scale, out, nullptr, stream);
  int rc = check_attention_args(qkv, cu_seqlens, num_users, max_seqlen, n_heads, head_dim, scale, out);
  if (rc != VLCA_OK) return rc;
  if (num_users == 0 || max_seqlen == 0) return VLCA_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return VLCA_ERR_HIP;
  const int max_tiles = static_cast<int>(max_tiles_of(max_seqlen));
  // Small batches (the causal forward's condition): one kernel that locates its
  // own items.  Each item computes the same thing on either plan, so the choice
  // changes no bits.
  {
    const int64_t pairs = item_pairs(num_users, max_seqlen, n_heads);
    int64_t g = static_cast<int64_t>(cu_count(dev)) * vlca::masked_blocks_per_cu(true);
    g = std::min<int64_t>(g, vlca::kMaxGrid);
    g -= g % 8;
    g = std::max<int64_t>(std::min<int64_t>(g, pairs), 1);
    const int grid = static_cast<int>(g);
    if (vlca::fused_fits(num_users, max_tiles, n_heads, grid)) {
      const int layer_log2 = snake_layer_log2(dev, grid, n_heads, static_cast<int64_t>(num_users) * max_tiles);
      if (vlca::launch_masked_attention_fused(qkv, cu_seqlens, num_users, max_tiles, n_heads, scale * kLog2e,
                                              mask->num_contexts, mask->num_targets, mask->target_group_size,
                                              mask->window_left, mask->window_right, out, grid, layer_log2,
                                              stream) != hipSuccess)
        return VLCA_ERR_HIP;
      return VLCA_OK;
    }
  }
  const int64_t need = required_capacity(num_users, max_seqlen);
  StreamState st;
  rc = get_workspace(dev, stream, need, &st);
  if (rc != VLCA_OK) return rc;
  int32_t* count = workspace_count(&st);
  int32_t* queue = count + vlca::kQueueStride;
  if (vlca::launch_schedule(cu_seqlens, num_users, max_tiles, st.items, count, queue,
                            vlca::SplitArgs{0, 0, 0, nullptr, nullptr}, stream) != hipSuccess)
    return VLCA_ERR_HIP;
  int64_t g = static_cast<int64_t>(cu_count(dev)) * vlca::masked_blocks_per_cu(false);
  g = std::min<int64_t>(g, vlca::kMaxGrid);
  g -= g % 8;
  g = std::max<int64_t>(std::min<int64_t>(g, need * n_heads), 1);
  if (vlca::launch_masked_attention(qkv, st.items, count, queue, n_heads, scale * kLog2e, mask->num_contexts,
                                    mask->num_targets, mask->target_group_size, mask->window_left,
                                    mask->window_right, out, static_cast<int>(g), stream) != hipSuccess)
    return VLCA_ERR_HIP;
  return VLCA_OK;
}

int varlen_causal_attn_ln_qkv(const void* x, const void* gamma, const void* beta, float eps, const void* w_qkv,
                              const void* b_qkv, int total_tokens, int d_model, int n_out, void* qkv,
                              hipStream_t stream) {
  if (total_tokens < 0) return VLCA_ERR_NEGATIVE_SIZE;
  if (d_model != 512 || n_out < 128 || n_out % 128 != 0 || n_out > vlca::kMaxProjOut) return VLCA_ERR_SHAPE;
  if (!std::isfinite(eps) || eps < 0.f) return VLCA_ERR_SCALE;
  if (total_tokens == 0) return VLCA_OK;
  if (x == nullptr || gamma == nullptr || beta == nullptr || w_qkv == nullptr || b_qkv == nullptr || qkv == nullptr)
    return VLCA_ERR_NULL_POINTER;
  if (qkv == x) return VLCA_ERR_ALIAS;
  if (!aligned(x, 16) || !aligned(gamma, 16) || !aligned(beta, 16) || !aligned(w_qkv, 16) || !aligned(qkv, 16) ||
      !aligned(b_qkv, 8))
    return VLCA_ERR_ALIGN;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return VLCA_ERR_HIP;
  return vlca::launch_ln_qkv(x, gamma, beta, eps, w_qkv, b_qkv, total_tokens, n_out, qkv, cu_count(dev), stream) ==
                 hipSuccess
             ? VLCA_OK
             : VLCA_ERR_HIP;
}

int varlen_causal_attn_out_residual(const void* attn, const void* w_out, const void* b_out, const void* residual,
                                    int total_tokens, int d_model, int n_out, void* y, hipStream_t stream) {
  if (total_tokens < 0) return VLCA_ERR_NEGATIVE_SIZE;
  if (d_model != 512 || n_out < 128 || n_out % 128 != 0 || n_out > vlca::kMaxProjOut) return VLCA_ERR_SHAPE;
  if (total_tokens == 0) return VLCA_OK;
  if (attn == nullptr || w_out == nullptr || b_out == nullptr || residual == nullptr || y == nullptr)
    return VLCA_ERR_NULL_POINTER;
  if (y == attn) return VLCA_ERR_ALIAS;
  if (!aligned(attn, 16) || !aligned(w_out, 16) || !aligned(residual, 16) || !aligned(y, 16) || !aligned(b_out, 8))
    return VLCA_ERR_ALIGN;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return VLCA_ERR_HIP;
  return vlca::launch_out_residual(attn, w_out, b_out, residual, total_tokens, n_out, y, cu_count(dev), stream) ==
                 hipSuccess
             ? VLCA_OK
             : VLCA_ERR_HIP;
}

int varlen_causal_attn_bwd(const void* qkv, const void* out, const void* dout, const float* lse,
                           const int32_t* cu_seqlens, int num_users, int max_seqlen, int n_heads, int head_dim,
                           float scale, void* dqkv, hipStream_t stream) {
  int rc = check_attention_args(qkv, cu_seqlens, num_users, max_seqlen, n_heads, head_dim, scale, out);
  if (rc != VLCA_OK) return rc;
  if (num_users > 0 && (dout == nullptr || lse == nullptr || dqkv == nullptr)) return VLCA_ERR_NULL_POINTER;
  if (dqkv != nullptr && (dqkv == qkv || dqkv == out || dqkv == dout)) return VLCA_ERR_ALIAS;
  if (!aligned(dout, 16) || !aligned(dqkv, 16) || !aligned(lse, 4)) return VLCA_ERR_ALIGN;
  if (num_users == 0 || max_seqlen == 0) return VLCA_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return VLCA_ERR_HIP;
  const int64_t need = required_capacity(num_users, max_seqlen);
  StreamState st;
  rc = get_workspace(dev, stream, need, &st);
  if (rc != VLCA_OK) return rc;
  const int max_tiles = static_cast<int>(max_tiles_of(max_seqlen));
  int32_t* const count = workspace_count(&st);
  int32_t* const queue = count + vlca::kQueueStride;
  if (vlca::launch_bwd_prepare(out, dout, lse, cu_seqlens, num_users, max_tiles, st.items, count, queue, n_heads, dqkv,
                                cu_count(dev), stream) != hipSuccess)
    return VLCA_ERR_HIP;
  if (vlca::launch_backward(qkv, dout, lse, st.items, count, queue, need, n_heads, scale, dqkv, cu_count(dev),
                            stream) != hipSuccess)
    return VLCA_ERR_HIP;
  return VLCA_OK;
}

int varlen_causal_attn_fwd_noalloc(const void* qkv, const int32_t* cu_seqlens, int num_users, int max_seqlen,
                                   int n_heads, int head_dim, float scale, void* out, hipStream_t stream) {
  int rc = check_attention_args(qkv, cu_seqlens, num_users, max_seqlen, n_heads, head_dim, scale, out);
  if (rc != VLCA_OK) return rc;
  if (num_users == 0 || max_seqlen == 0) return VLCA_OK;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return VLCA_ERR_HIP;
  const int max_tiles = static_cast<int>(max_tiles_of(max_seqlen));
  const int64_t pairs = item_pairs(num_users, max_seqlen, n_heads);
  const int upr = split_units_per_round(dev, n_heads);
  const bool may_split = max_tiles > kSplitMinWidth && upr >= kSplitParts;
  int grid = grid_size(dev, pairs, true);
  const bool fused = vlca::fused_fits(num_users, max_tiles, n_heads, grid);
  // The same plan and split settings as varlen_causal_attn_fwd, over the
  // device's scratch array instead of the stream's state.
  const int64_t need = required_capacity(num_users, max_seqlen);
  if (!fused && (may_split ? std::max<int64_t>(need, upr) : need) > vlca::kNoAllocItems) return VLCA_ERR_SCRATCH;
  char* base = nullptr;
  if (vlca::noalloc_scratch(&base) != hipSuccess) return VLCA_ERR_HIP;
  vlca::SplitArgs split{0, 0, 0, nullptr, nullptr};
  if (may_split)
    split = vlca::SplitArgs{kSplitParts, kSplitMinWidth, upr, reinterpret_cast<float*>(base),
                            reinterpret_cast<int32_t*>(base + vlca::kNoAllocPoolBytes)};
  if (fused) {
    if (split.p > 1) grid = grid_size(dev, pairs * kSplitParts, true);
    const int layer_log2 = snake_layer_log2(dev, grid, n_heads, static_cast<int64_t>(num_users) * max_tiles);
    if (vlca::launch_attention_fused(qkv, cu_seqlens, num_users, max_tiles, n_heads, scale * kLog2e, split, out,
                                     nullptr, grid, layer_log2, stream) != hipSuccess)
      return VLCA_ERR_HIP;
    return VLCA_OK;
  }
  int4* items = reinterpret_cast<int4*>(base + vlca::kNoAllocItemsOffset);
  int32_t* count = reinterpret_cast<int32_t*>(items + vlca::kNoAllocItems);
  return launch_pair(qkv, cu_seqlens, num_users, max_seqlen, n_heads, scale, items, count,
                     count + vlca::kQueueStride, split, out, nullptr, stream, true);
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
  if (!aligned(items, 16) || !aligned(count, 4) || !aligned(cu_seqlens, 4)) return VLCA_ERR_ALIGN;
  const int max_tiles = static_cast<int>(max_tiles_of(max_seqlen));
  if (vlca::launch_schedule(cu_seqlens, num_users, max_tiles, reinterpret_cast<int4*>(items), count, nullptr,
                            vlca::SplitArgs{0, 0, 0, nullptr, nullptr}, stream) != hipSuccess)
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
  if (!aligned(items, 16) || !aligned(count, 4)) return VLCA_ERR_ALIGN;
  if (num_users == 0 || max_seqlen == 0) return VLCA_OK;
  return launch_pair(qkv, cu_seqlens, num_users, max_seqlen, n_heads, scale,
                     reinterpret_cast<int4*>(const_cast<int32_t*>(items)), const_cast<int32_t*>(count), nullptr,
                     vlca::SplitArgs{0, 0, 0, nullptr, nullptr}, out, nullptr, stream, false);
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
    case VLCA_ERR_SCRATCH: return "batch needs more worklist items than the no-allocation scratch holds";
    case VLCA_ERR_BUCKETS: return "bucket sizes must be positive and strictly increasing (at most 64 buckets)";
    case VLCA_ERR_MASK: return "mask out of range (group size >= 1, windows >= -1, contexts/targets need window_right 0)";
    case VLCA_ERR_SHAPE: return "d_model must be 512 and the output width a positive multiple of 128";
    case VLCA_ERR_ALIGN: return "bf16 tensors and worklist items must be 16-byte aligned, biases 8-byte, int32/fp32 arrays 4-byte";
    default: return "unknown error code";
  }
}

}  // extern "C"
