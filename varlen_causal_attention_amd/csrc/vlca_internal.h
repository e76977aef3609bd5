// Internal launch interface between the C ABI (vlca_api.cpp) and the gfx950
// kernels (vlca_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "varlen_causal_attn.h"

namespace vlca {

constexpr int kTileRows = 64;        // query rows per work item == keys per K/V tile
constexpr int kHeadDim = 64;
constexpr int kMaxLevels = 4096;     // q-tiles per user the scheduler can order
constexpr int kMaxGrid = 4096;       // persistent grid cap

// Work counters of the attention kernel's dynamic assignment (one per head, or
// one over all (item, head) pairs when there are more heads), each alone in its
// own 256-byte block: counter q is queue[q * kQueueStride].
constexpr int kQueues = 8;
constexpr int kQueueStride = 64;

// Key-range splitting of long items: an item runs as at most kMaxSplitParts
// parts; each part leaves its softmax state in a pool slot of kPoolSlotFloats
// floats; one arrival counter per split item, kSplitCtrStride int32 apart, is zero
// between calls (the last part resets it).  A split list holds at most upr units
// per head, and upr * n_heads <= kPoolMaxSlots, so every split rank has a slot.
constexpr int kMaxSplitParts = 2;
constexpr int kPoolSlotFloats = 4608;  // O: 64 rows x 64 dims, then (m, l) per thread
constexpr int kSplitCtrStride = 16;
constexpr int kPoolMaxSlots = 1024;

struct SplitArgs {
  int p;          // 2: split long items in two parts; <= 1: no splitting
  int min_width;  // items of at most this many key tiles always run whole
  int upr;        // split only if the list with split items holds at most this many units per head
  float* pool;    // [upr][n_heads] slots
  int32_t* ctr;   // [upr][n_heads] arrival counters
};

// Scheduler: one workgroup builds the (user, q_tile, row_start, length) list and,
// when queue is not null, zeroes the kQueues counters at queue.  split.p == 2:
// the list may hold split units (same rule and decision as the single-kernel
// plan); launch_attention must then get the same split.
hipError_t launch_schedule(const int32_t* cu_seqlens, int num_users, int max_tiles,
                           int4* items, int32_t* count, int32_t* queue, const SplitArgs& split, hipStream_t stream);

// Attention: persistent grid walking the first *count items.  queue null: a fixed
// assignment of items to workgroups; otherwise workgroups claim items from the
// zeroed counters at queue (reset by launch_schedule).  layer_log2: -1, or (when
// the work is known to fit in one round of the fixed assignment) log2 of the
// slots between workgroups that share a CU, so that the assignment balances each
// CU's items.
// lse: null, or [T, n_heads] fp32 receiving each row's log-sum-exp of its scaled
// scores (natural log).
hipError_t launch_attention(const void* qkv, const int4* items, const int32_t* count, int32_t* queue, int n_heads,
                            float scale_log2e, const SplitArgs& split, void* out, float* lse, int grid, int layer_log2,
                            hipStream_t stream);

// Attention alone with the ordering done inside the kernel (no worklist buffer):
// for batches where fused_fits() holds.  split.p == 2 splits long items (needs
// split.pool / split.ctr).
hipError_t launch_attention_fused(const void* qkv, const int32_t* cu_seqlens, int num_users, int max_tiles,
                                  int n_heads, float scale_log2e, const SplitArgs& split, void* out, float* lse,
                                  int grid, int layer_log2, hipStream_t stream);

// Users the single-kernel plan takes at most (one per thread of a workgroup),
// and the rounds of whole items a workgroup can run when it orders the work
// itself.
constexpr int kFusedUsers = 256;
constexpr int kFusedRounds = 16;

// Whether a batch of these sizes runs on the single-kernel plan with this grid.
inline bool fused_fits(int64_t num_users, int64_t max_tiles, int64_t n_heads, int64_t grid) {
  if (num_users > kFusedUsers || grid <= 0) return false;
  // The prologue's scans carry the item count in 15 bits (and up to twice it in 17).
  if (num_users * max_tiles > 32767) return false;
  // rounds = ceil(items * H / grid) when the grid is a multiple of H; items <= users x max q-tiles
  return num_users * max_tiles * n_heads <= static_cast<int64_t>(kFusedRounds) * grid;
}

// The backward's first kernel (vlca_kernels.hip): the worklist of whole items
// (as launch_schedule without splitting) and, alongside it, D = rowsum(dO o O)
// and -lse log2(e) into dqkv's dq columns.  It zeroes two sets of kQueues work
// counters at queue: the dK/dV kernel's (queue[q * kQueueStride]) and the dQ
// kernel's (kBwdDqQueue further).  cus: compute units of the device.
constexpr int kBwdDqQueue = kQueueStride / 2;
hipError_t launch_bwd_prepare(const void* out, const void* dout, const float* lse, const int32_t* cu_seqlens,
                              int num_users, int max_tiles, int4* items, int32_t* count, int32_t* queue, int n_heads,
                              void* dqkv, int cus, hipStream_t stream);

// The rest of the backward over that worklist: the dK/dV kernel, then the dQ
// kernel (see vlca_backward.hip), each claiming items from its zeroed counters
// at queue.
hipError_t launch_backward(const void* qkv, const void* dout, const float* lse, const int4* items,
                           const int32_t* count, int32_t* queue, int64_t max_items, int n_heads, float scale,
                           void* dqkv, int cus, hipStream_t stream);

// The forward with the HSTU-style mask variants (vlca_masked.hip) over the
// scheduler's worklist of whole items, claiming items from the zeroed counters
// at queue.  num_contexts / num_targets: device [num_users] or null.
hipError_t launch_masked_attention(const void* qkv, const int4* items, const int32_t* count, int32_t* queue,
                                   int n_heads, float scale_log2e, const int32_t* num_contexts,
                                   const int32_t* num_targets, int group, int window_left, int window_right,
                                   void* out, int grid, hipStream_t stream);
// The same forward as one kernel for batches where fused_fits() holds: every
// workgroup locates its own items from cu_seqlens (no worklist, no counters).
hipError_t launch_masked_attention_fused(const void* qkv, const int32_t* cu_seqlens, int num_users, int max_tiles,
                                         int n_heads, float scale_log2e, const int32_t* num_contexts,
                                         const int32_t* num_targets, int group, int window_left, int window_right,
                                         void* out, int grid, int layer_log2, hipStream_t stream);
int masked_blocks_per_cu(bool fused);

// The attention's neighbours in the packed layer (vlca_proj.hip), d_in = 512,
// N a multiple of 128 (at most kMaxProjOut): qkv = LayerNorm(x) W_qkv^T + b_qkv,
// and y = residual + attn W_out^T + b_out.  cus: the device's compute units
// (sizes the grid).
constexpr int kMaxProjOut = 65536;
hipError_t launch_ln_qkv(const void* x, const void* gamma, const void* beta, float eps, const void* w_qkv,
                         const void* b_qkv, int T, int N, void* qkv, int cus, hipStream_t stream);
hipError_t launch_out_residual(const void* attn, const void* w_out, const void* b_out, const void* residual, int T,
                               int N, void* y, int cus, hipStream_t stream);

// Fixed-length offsets for a captured graph: out[i] = min(cu_seqlens[min(i,
// num_users)], total) for i = 0 .. max_users (num_users <= max_users).
hipError_t launch_pad_offsets(const int32_t* cu_seqlens, int num_users, int total, int32_t* out, int max_users,
                              hipStream_t stream);

// Scratch memory of the no-allocation entry point: one fixed array per device
// (file-scope in vlca_noalloc.hip), laid out as the split pool, its arrival
// counters, then a worklist of kNoAllocItems items followed by its count and
// work counters.
constexpr int64_t kNoAllocItems = VLCA_NOALLOC_MAX_ITEMS;
constexpr size_t kNoAllocPoolBytes = size_t(kPoolMaxSlots) * kPoolSlotFloats * sizeof(float);
constexpr size_t kNoAllocCtrBytes = size_t(kPoolMaxSlots) * kSplitCtrStride * sizeof(int32_t);
constexpr size_t kNoAllocItemsOffset = kNoAllocPoolBytes + kNoAllocCtrBytes;
constexpr size_t kNoAllocTailBytes = size_t(1 + kQueues) * kQueueStride * sizeof(int32_t);
constexpr size_t kNoAllocScratchBytes = kNoAllocItemsOffset + size_t(kNoAllocItems) * 16 + kNoAllocTailBytes;

// Device address of the current device's scratch array (looked up once per
// device with hipGetSymbolAddress; the array's host-side name is no device
// address).
hipError_t noalloc_scratch(char** ptr);

// Attention workgroups that fit on one CU at once (occupancy of the current device),
// for the kernel over a worklist or the single-kernel variant.
int attention_blocks_per_cu(bool fused);

}  // namespace vlca
