// Internal launch interface between the C ABI (vlca_api.cpp) and the gfx950
// kernels (vlca_kernels.hip).  Not installed, not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// Key-range splitting of long items in the single-kernel plan: an item runs as
// at most kMaxSplitParts parts; each part leaves its softmax state in a pool slot
// of kPoolSlotFloats floats; one arrival counter per split item, kSplitCtrStride
// int32 apart, is zero between calls (the last part resets it).
constexpr int kMaxSplitParts = 2;
constexpr int kPoolSlotFloats = 4608;  // O: 64 rows x 64 dims, then (m, l) per thread
constexpr int kSplitCtrStride = 16;

struct SplitArgs {
  int p;          // 2: split long items in two parts; <= 1: no splitting
  int min_width;  // items of at most this many key tiles always run whole
  int upr;        // split only if the list with split items holds at most this many units
  int cap;        // pool slots per head: items whose parts' split ranks reach it run whole
  float* pool;    // [cap][n_heads] slots
  int32_t* ctr;   // [cap][n_heads] arrival counters
};

// Scheduler: one workgroup builds the (user, q_tile, row_start, length) list and,
// when queue is not null, zeroes the kQueues counters at queue.  split.p == 2:
// batches of at most 1024 users may get a list of split units (same rule as the
// single-kernel plan); launch_attention must then get the same split.
hipError_t launch_schedule(const int32_t* cu_seqlens, int num_users, int max_tiles,
                           int4* items, int32_t* count, int32_t* queue, const SplitArgs& split, hipStream_t stream);

// Attention: persistent grid walking the first *count items.  queue null: a fixed
// assignment of items to workgroups; otherwise workgroups claim items from the
// zeroed counters at queue (reset by launch_schedule).  layer_log2: -1, or (when
// the work is known to fit in one round of the fixed assignment) log2 of the
// slots between workgroups that share a CU, so that the assignment balances each
// CU's items.
hipError_t launch_attention(const void* qkv, const int4* items, const int32_t* count, int32_t* queue, int n_heads,
                            float scale_log2e, const SplitArgs& split, void* out, int grid, int layer_log2,
                            hipStream_t stream);

// Attention alone with the ordering done inside the kernel (no worklist buffer):
// for batches where fused_fits() holds.  split.p == 2 splits long items (needs
// split.pool / split.ctr).
hipError_t launch_attention_fused(const void* qkv, const int32_t* cu_seqlens, int num_users, int max_tiles,
                                  int n_heads, float scale_log2e, const SplitArgs& split, void* out, int grid,
                                  int layer_log2, hipStream_t stream);
bool fused_fits(int64_t num_users, int64_t max_tiles, int64_t n_heads, int64_t grid);

// Users the single-kernel plan takes at most (one per lane of four chunks).
constexpr int kFusedUsers = 256;

// Attention workgroups that fit on one CU at once (occupancy of the current device),
// for the kernel over a worklist or the single-kernel variant.
int attention_blocks_per_cu(bool fused);

}  // namespace vlca
