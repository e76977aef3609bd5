// gfx950 (MI355X / CDNA4) kernels for block-diagonal causal attention over
// packed variable-length users.
//
// What is computed follows the cti2026 README (git.firegun.top/Days-gone/cti2026),
// FlashAttention_Varlen section, "operator design": each program owns one 64-row
// query block of one user and one head, reads the user's row range from
// cu_seqlens (no padding), walks key blocks only up to the diagonal, and keeps a
// running row max m, running denominator l and fp32 accumulator acc that are
// updated block by block, writing bf16 at the end.  The design below is written
// for CDNA4, not taken from the page's Triton kernel:
//
//  * schedule_kernel -- one workgroup turns cu_seqlens into a compact worklist of
//    (user, q_tile) items, longest first, so no workgroup is launched for rows
//    that do not exist (the page's dense grid relied on early exit instead).
//  * attention_kernel -- a persistent grid over (item, head) pairs.  With H = 8
//    and a grid that is a multiple of 8, a workgroup on XCD x (workgroups are
//    dealt to the 8 XCDs round-robin) always runs head x, so each XCD's L2 holds
//    one head's K/V columns and serves the re-reads of later q-tiles of the same
//    user.  After the scheduler kernel, workgroups claim items from one counter
//    per head; in the single-kernel plan (and over a caller's worklist) each
//    workgroup takes a fixed snake over the list, dealt across the workgroups
//    that share a CU when all the work fits one round.
//  * Key-range splitting -- in small batches whose units all fit one round of
//    the grid, the longest items run as two parts over disjoint key ranges on
//    two workgroups; the last part to finish merges the two (m, l, acc) states.
//
// Attention workgroup: 4 waves; wave w owns query rows 16w..16w+15 of the tile.
//  * K and V tiles (64 keys x 64 dims, 8 KB each) are copied from HBM straight
//    into LDS with global_load_lds_dwordx4 (no VGPRs, no VALU), through a
//    two-stage ring, so the next tile is in flight while one is consumed.
//  * Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_bf16
//    (A = K rows from LDS, B = Q held in registers): a lane holds 4 keys of one
//    query per 16x16 block, so the row max is in-lane work plus two cross-lane
//    steps and every per-row factor is a per-lane scalar.
//  * P^T stays in registers and is the B operand of O^T = V^T P^T.  The A operand
//    (V^T) is read from the natural [key][dim] V tile with ds_read_b64_tr_b16:
//    within each 16-lane group, lane i gets element i%4 of source lanes
//    {i/4, 4+i/4, 8+i/4, 12+i/4}; if source lane j points at key row j/4, dims
//    4(j%4)..4(j%4)+3, lane i receives 4 consecutive keys of dim i.  The rows of
//    each S^T block are permuted so that P^T comes out in that key order.
//  * The softmax denominator is one more MFMA per 32 keys: an all-ones A operand
//    times P^T sums the same bf16-rounded weights that multiply V.
//  * The running max is only raised when a tile's max exceeds it by more than
//    2^kRescaleLog2 in exp2 units; weights stay <= 2^8 and the rescale of acc (a
//    wave-uniform branch) is skipped on almost every tile.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "vlca_device.h"
#include "vlca_internal.h"
#include "vlca_order.h"

namespace vlca {
namespace {

constexpr int kSchedThreads = 1024;
constexpr int kSchedCache = 8160;  // cu_seqlens entries cached in LDS by the scheduler (LDS <= 64 KB)

// ----------------------------------------------------------------- scheduler

constexpr int kShortTiles = 16;    // users with more tiles are emitted by a whole wave

// LDS scratch of the ordering pass for a workgroup of kThreads.
template <int kThreads>
struct OrderScratch {
  int tot[kClasses];                  // tiles (units) per class
  int base[kClasses];                 // next free slot of each class
  int wsum[kThreads / 64][kClasses];  // per-wave class sums of the current chunk
  int long_u[kThreads];               // long users of the current chunk ...
  int long_off[kThreads];             // ... and their first slots
  int nlong;
  int count;                          // items (units) in the list
  int n_whole, n_split;               // any split item; units of the split list (saturated)
};

// Worklist order: users grouped by length class floor(log2(tiles)), highest
// class first; inside a class users ascend; each user's q-tiles are adjacent,
// from its last q-tile (the most key tiles) down to q-tile 0.  The first slot of
// user u is then
//   sum of the tiles of all higher classes + sum of the tiles of the users
//   before u in its own class,
// computed in two passes over the users (class totals, then per-class running
// sums in chunks of kThreads users), or, when every user fits one chunk, in one
// pass whose per-class wave scans give both.  emit(slot, user, q_tile, segment) stores
// one item; S.count receives the number of items.  All threads of the
// workgroup must call this (it contains barriers).  The barriers order LDS
// only: the emitted items' global stores are not waited for (a full
// __syncthreads() would wait for their completion at every chunk; they are
// visible to later kernels once this one has ended).
//
// Key-range splitting (sp.p > 1): the same rule and decision as the
// single-kernel plan (split when the list with split items holds at most sp.upr
// units), taken over every user of the batch; zero-length users add nothing to
// either count, so they cannot change it.  The counts are then carried packed
// (whole items in the low 15 bits, units in the high 17: a split list has at most
// sp.upr <= kMaxGrid units) and emit(slot, x, y, segment) gets y = q_tile | kind
// << 16 and x = the user (kind 0, a whole item) or the split rank of the item's
// first part (kind 1, 2: first / second part).  Without splitting, x = user and
// y = q_tile.
template <int kThreads, typename CachePtr, typename Emit>
__device__ void order_items(const int32_t* __restrict__ cu, CachePtr s_cu, bool cached, int nusers, int total,
                            int max_tiles, const SplitArgs& sp, LDS OrderScratch<kThreads>* S, Emit emit) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  if (tid < kClasses) S->tot[tid] = 0;
  if (tid == 0) {
    S->n_whole = 0;
    S->n_split = 0;
  }
  lds_barrier();
  bool split = false;
  if (sp.p > 1) {  // uniform
    // Units of the split list, saturated at sp.upr + 1 (enough to decide), and
    // whether any item would split at all.
    const int sat = sp.upr + 1;
    int x = 0, any = 0;
    for (int u0 = 0; u0 < nusers; u0 += kThreads) {
      const int u = u0 + tid;
      const int t = u < nusers ? segment_of(cu, s_cu, cached, u, total, max_tiles).tiles : 0;
      const int e = split_user(t, 1, sp.min_width).split;
      x = min(x + min(t + e, sat), sat);
      any |= e;
    }
    // Wave sums of the per-thread saturated counts (<= 64 x sat): the total is
    // <= sp.upr exactly when the true count is.
    x = __builtin_amdgcn_readlane(wave_inclusive_sum(x), 63);
    const bool wany = __ballot(any != 0) != 0;
    if (lane == 0) {
      __atomic_fetch_add(&S->n_split, x, __ATOMIC_RELAXED);  // <= 16 waves x 64 sat: no overflow
      if (wany) __atomic_fetch_or(&S->n_whole, 1, __ATOMIC_RELAXED);
    }
    lds_barrier();
    split = S->n_whole != 0 && S->n_split <= sp.upr;
  }
  // The count a user adds to the list: its q-tiles, or both counts packed.
  auto units_of_user = [&](int t) {
    return split ? t | ((t + split_user(t, 1, sp.min_width).split) << 15) : t;
  };
  // The items of user u (segment s) from its first slot `both` (both counts
  // packed when splitting).  Users of more than kShortTiles tiles are left to a
  // whole wave (S->long_u / long_off) after the next barrier.
  auto emit_user = [&](int u, const Seg& s, int both) {
    const int t = s.tiles;
    if (split) {
      const int off = both >> 15;
      const int roff = 2 * ((both >> 15) - (both & 0x7fff));
      const SplitUser spl = split_user(t, 1, sp.min_width);
      for (int i = 0; i < t + spl.split; ++i) {
        int nk, k, p;
        unit_of(t, spl, i, nk, k, p);
        // A split item's parts: kind 1 + k, x = split rank r0 of its first part
        // (ranks r0, r0 + 1 < the list's units <= sp.upr, the pool's slots per head).
        const int kind = p > 1 ? 1 + k : 0;
        const int x = p > 1 ? roff + i - k : u;
        emit(off + i, x, (nk - 1) | (kind << 16), s);
      }
    } else if (t <= kShortTiles) {
      for (int i = 0; i < t; ++i) emit(both + i, u, t - 1 - i, s);
    } else {
      const int k = __atomic_fetch_add(&S->nlong, 1, __ATOMIC_RELAXED);
      S->long_u[k] = u;
      S->long_off[k] = both;
    }
  };
  auto emit_long = [&]() {
    const int nlong = S->nlong;
    for (int i = wid; i < nlong; i += kThreads / 64) {
      const int lu = S->long_u[i];
      const int off = S->long_off[i];
      const Seg ls = segment_of(cu, s_cu, cached, lu, total, max_tiles);
      for (int k = lane; k < ls.tiles; k += 64) emit(off + k, lu, ls.tiles - 1 - k, ls);
    }
  };
  if (nusers <= kThreads) {  // uniform
    // One chunk: a single pass of per-class wave scans gives each user its prefix
    // inside its wave and each wave's class sums; wave 0 turns these into
    // per-wave offsets and class bases.
    const int u = tid;
    Seg s{0, 0, 0};
    if (u < nusers) s = segment_of(cu, s_cu, cached, u, total, max_tiles);
    const int t = s.tiles;
    const int cl = t > 0 ? length_class(t) : -1;
    const int val = units_of_user(t);
    if (lane < kClasses) S->wsum[wid][lane] = 0;
    if (tid == 0) S->nlong = 0;
    int pre = 0;
    unsigned long long pending = __ballot(t > 0);
    while (pending) {
      const int lc = __builtin_amdgcn_readlane(cl, __builtin_ctzll(pending));
      const bool mine = cl == lc;
      const int x = mine ? val : 0;
      const int incl = wave_inclusive_sum(x);
      if (mine) pre = incl - x;
      if (lane == 63) S->wsum[wid][lc] = incl;
      pending &= ~__ballot(mine);
    }
    lds_barrier();
    if (wid == 0) {
      // Lane l handles class 12 - l: the exclusive prefix over the waves in place,
      // then the class bases (tiles of all higher classes).
      int v = 0;
      if (lane < kClasses) {
        const int c = kClasses - 1 - lane;
#pragma unroll
        for (int w = 0; w < kThreads / 64; ++w) {
          const int x = S->wsum[w][c];
          S->wsum[w][c] = v;
          v += x;
        }
      }
      const int incl = wave_inclusive_sum(v);
      if (lane < kClasses) S->base[kClasses - 1 - lane] = incl - v;
      if (lane == kClasses - 1) S->count = split ? incl >> 15 : incl;
    }
    lds_barrier();
    if (t > 0) emit_user(u, s, S->base[cl] + S->wsum[wid][cl] + pre);
    lds_barrier();
    emit_long();
    return;
  }
  // Pass 1: tiles per class (one LDS atomic per class present in a wave).
  for (int u0 = 0; u0 < nusers; u0 += kThreads) {
    const int u = u0 + tid;
    const int t = u < nusers ? segment_of(cu, s_cu, cached, u, total, max_tiles).tiles : 0;
    const int cl = t > 0 ? length_class(t) : -1;
    const int val = units_of_user(t);
    unsigned long long pending = __ballot(t > 0);
    while (pending) {
      const int lc = __builtin_amdgcn_readlane(cl, __builtin_ctzll(pending));
      const bool mine = cl == lc;
      const int sum = __builtin_amdgcn_readlane(wave_inclusive_sum(mine ? val : 0), 63);
      if (lane == 0) __atomic_fetch_add(&S->tot[lc], sum, __ATOMIC_RELAXED);
      pending &= ~__ballot(mine);
    }
  }
  lds_barrier();
  if (wid == 0) {  // first slot of class c = tiles of all higher classes: lane l holds class 12-l
    const int v = lane < kClasses ? S->tot[kClasses - 1 - lane] : 0;
    const int incl = wave_inclusive_sum(v);
    if (lane < kClasses) S->base[kClasses - 1 - lane] = incl - v;
    if (lane == kClasses - 1) S->count = split ? incl >> 15 : incl;
  }
  // Pass 2: slots, chunk by chunk in ascending user order.
  for (int c0 = 0; c0 < nusers; c0 += kThreads) {
    if (tid == 0) S->nlong = 0;
    if (lane < kClasses) S->wsum[wid][lane] = 0;
    const int u = c0 + tid;
    Seg s{0, 0, 0};
    if (u < nusers) s = segment_of(cu, s_cu, cached, u, total, max_tiles);
    const int t = s.tiles;
    const int cl = t > 0 ? length_class(t) : -1;
    const int val = units_of_user(t);
    // Exclusive prefix of the counts of earlier lanes in the same class, one wave
    // scan per class present in the wave.
    int pre = 0;
    unsigned long long pending = __ballot(t > 0);
    while (pending) {
      const int lc = __builtin_amdgcn_readlane(cl, __builtin_ctzll(pending));
      const bool mine = cl == lc;
      const int x = mine ? val : 0;
      const int incl = wave_inclusive_sum(x);
      if (mine) pre = incl - x;
      if (lane == 63) S->wsum[wid][lc] = incl;
      pending &= ~__ballot(mine);
    }
    lds_barrier();
    if (t > 0) {
      int both = S->base[cl] + pre;
      for (int w = 0; w < wid; ++w) both += S->wsum[w][cl];
      emit_user(u, s, both);
    }
    lds_barrier();
    emit_long();
    if (tid < kClasses) {
      int sum = 0;
      for (int w = 0; w < kThreads / 64; ++w) sum += S->wsum[w][tid];
      S->base[tid] += sum;
    }
    lds_barrier();
  }
  lds_barrier();  // S->count is visible to all threads
}

// The worklist in global memory: items[slot] = (user, q_tile, row_start, length),
// or with key-range splitting the units described at order_items.  Run by one
// workgroup of kSchedThreads threads.
__device__ __forceinline__ void schedule_body(const int32_t* __restrict__ cu, int U, int max_tiles,
                                              int4* __restrict__ items, int32_t* __restrict__ count,
                                              int32_t* __restrict__ queue, SplitArgs sp) {
  // The attention kernel's work counters start at zero; so do the split pool's
  // arrival counters (every call also leaves them zero).
  if (queue != nullptr && threadIdx.x < kQueues) queue[threadIdx.x * kQueueStride] = 0;
  if (sp.p > 1)
    for (int i = threadIdx.x; i < kPoolMaxSlots; i += kSchedThreads) sp.ctr[i * kSplitCtrStride] = 0;
  __shared__ int s_cu_lds[kSchedCache + 1];
  __shared__ OrderScratch<kSchedThreads> S_lds;
  LDS int* const s_cu = (LDS int*)s_cu_lds;
  LDS OrderScratch<kSchedThreads>* const S = (LDS OrderScratch<kSchedThreads>*)&S_lds;
  const bool cached = U <= kSchedCache;
  if (U > 0 && max_tiles > 0 && cached) {
    for (int i = threadIdx.x; i <= U; i += kSchedThreads) s_cu[i] = cu[i];
  }
  lds_barrier();
  const int total = (U > 0 && max_tiles > 0) ? (cached ? s_cu[U] : cu[U]) : 0;
  const int nusers = max_tiles > 0 ? U : 0;
  order_items<kSchedThreads>(cu, s_cu, cached, nusers, total, max_tiles, sp, S,
                             [&](int slot, int x, int y, const Seg& sg) {
                               items[slot] = make_int4(x, y, sg.start, sg.len);
                             });
  if (threadIdx.x == 0) *count = S->count;
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(const int32_t* __restrict__ cu, int U,
                                                                 int max_tiles, int4* __restrict__ items,
                                                                 int32_t* __restrict__ count,
                                                                 int32_t* __restrict__ queue, SplitArgs sp) {
  schedule_body(cu, U, max_tiles, items, count, queue, sp);
}

// ------------------------------------------------ backward: the first kernel
// The backward's two independent preliminaries in one launch, so that the
// worklist's latency hides under the row pass: workgroup 0 builds the worklist
// (schedule_body, no split, no work counters); the others form, for every row t
// < T = cu[U] (read on the device) and head h, with eight lanes per (row, head)
// pair and 16 bytes of dO and of O each, a persistent grid over the pairs:
//   D[t, h] = sum_d dO[t, h, d] O[t, h, d] (fp32), and -lse[t, h] log2(e),
// written as fp32 into the first 8 bytes of that row's and head's dq columns of
// dqkv (the dq kernel, which runs last, reads D there before overwriting them).
__global__ __launch_bounds__(kSchedThreads) void bwd_prepare_kernel(
    const int32_t* __restrict__ cu, int U, int max_tiles, int4* __restrict__ items, int32_t* __restrict__ count,
    int32_t* __restrict__ queue, const uint16_t* __restrict__ o, const uint16_t* __restrict__ dout,
    const float* __restrict__ lse, int n_heads, uint16_t* __restrict__ dqkv) {
  if (blockIdx.x == 0) {
    // The two gradient kernels' work counters start at zero.
    if (threadIdx.x < 2 * kQueues)
      queue[(threadIdx.x >> 1) * kQueueStride + (threadIdx.x & 1) * kBwdDqQueue] = 0;
    schedule_body(cu, U, max_tiles, items, count, nullptr, SplitArgs{0, 0, 0, nullptr, nullptr});
    return;
  }
  constexpr float kLog2eF = 1.4426950408889634f;
  const int T = max(cu[U], 0);
  const int64_t pairs = (int64_t)T * n_heads;
  const int part = threadIdx.x & 7;
  const int64_t ldo = (int64_t)n_heads * kHeadDim;
  constexpr int kPairsPerPass = kSchedThreads / 8;
  for (int64_t p0 = (int64_t)(blockIdx.x - 1) * kPairsPerPass; p0 < pairs;
       p0 += (int64_t)(gridDim.x - 1) * kPairsPerPass) {
    const int64_t pair = p0 + (threadIdx.x >> 3);
    const bool live = pair < pairs;
    const int64_t t = live ? pair / n_heads : 0;
    const int h = live ? (int)(pair - t * n_heads) : 0;
    float acc = 0.f;
    if (live) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(o + t * ldo + h * kHeadDim + 8 * part);
      const u32x4 b = *reinterpret_cast<const u32x4*>(dout + t * ldo + h * kHeadDim + 8 * part);
      const bf16x8 av = __builtin_bit_cast(bf16x8, a), bv = __builtin_bit_cast(bf16x8, b);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = __builtin_fmaf((float)av[i], (float)bv[i], acc);
    }
    acc += __shfl_xor(acc, 1);
    acc += __shfl_xor(acc, 2);
    acc += __shfl_xor(acc, 4);
    if (live && part == 0) {
      float* const dst = reinterpret_cast<float*>(dqkv + t * 3 * ldo + h * kHeadDim);
      dst[0] = acc;
      dst[1] = -lse[t * n_heads + h] * kLog2eF;
    }
  }
}

// ----------------------------------------------------------------- attention




// ------------------------------------------------------ key-range splitting
// In the single-kernel plan the longest items bound the kernel: one item walks
// all of its user's key tiles up to the diagonal.  Such an item can instead run
// as parts over disjoint key-tile ranges on different workgroups, each part
// keeping its own (m, l, O) online-softmax state; the state of a softmax over a
// union of key sets is the rescaled sum of the states over the parts, so the
// last part to finish folds the others' states into its own and writes the row.
//
// Each part's state goes to a pool slot in global memory, [wave][d][half][lane]
// float2 for O (4096 floats) then (m, l) per thread (512 floats).  The parts of
// one item run on different workgroups and possibly different XCDs, whose L2
// caches are not coherent with each other.  The slots are therefore written and
// read with agent-scope relaxed atomic accesses, which go through to the
// device-coherent level, and ordered by waiting for the stores' completion
// before the arrival count and by reading only after the count has returned.
// An agent-scope fence would do the same by writing back and invalidating the
// whole L2 of the XCD, which costs far more with many parts in flight.
__device__ __forceinline__ void store_coherent(float* p, f32x2 v) {
  __hip_atomic_store(reinterpret_cast<uint64_t*>(p), __builtin_bit_cast(uint64_t, v), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ f32x2 load_coherent(const float* p) {
  return __builtin_bit_cast(f32x2, __hip_atomic_load(reinterpret_cast<uint64_t*>(const_cast<float*>(p)),
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Float offset of a lane's O registers (dims 16d + 4g + 0..1; + 128 for + 2..3)
// inside a pool slot.
__device__ __forceinline__ int slot_o_offset(const Lanes& L, int d) { return ((L.wid * 4 + d) * 128 + L.lane) * 2; }

// This part's state into its pool slot.
__device__ __forceinline__ void store_partial(float* slot, const Lanes& L, const Acc& A) {
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    float* const o = slot + slot_o_offset(L, d);
    store_coherent(o, f32x2{A.o[d][0], A.o[d][1]});
    store_coherent(o + 128, f32x2{A.o[d][2], A.o[d][3]});
  }
  store_coherent(slot + 4096 + 2 * threadIdx.x, f32x2{A.m, A.l[0]});
}

// Run by the last part to finish (of two): fold the other part's state, read
// from its slot, into this one's.  The fold is written in part order -- part 0's
// state times its factor, plus part 1's -- whichever part runs it, so the result
// does not depend on which part finished last.
__device__ __forceinline__ void merge_parts(const float* other, int part, const Lanes& L, float sl2, Acc& A) {
  const f32x2 ml = load_coherent(other + 4096 + 2 * threadIdx.x);
  const bool first = part == 0;
  const float m0 = first ? A.m : ml[0], m1 = first ? ml[0] : A.m;
  const float l0 = first ? A.l[0] : ml[1], l1 = first ? ml[1] : A.l[0];
  const float mn = fmaxf(m0, m1);
  const float a = __builtin_amdgcn_exp2f((m0 - mn) * sl2);
  const float b = __builtin_amdgcn_exp2f((m1 - mn) * sl2);
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const f32x2 x = load_coherent(other + slot_o_offset(L, d));
    const f32x2 y = load_coherent(other + slot_o_offset(L, d) + 128);
    const f32x4 xo = f32x4{x[0], x[1], y[0], y[1]};
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float o0 = first ? A.o[d][r] : xo[r], o1 = first ? xo[r] : A.o[d][r];
      A.o[d][r] = __builtin_fmaf(o0, a, o1 * b);
    }
  }
  A.l[0] = __builtin_fmaf(l0, a, l1 * b);
  A.m = mn;
}

// kFused = false: walk the first *count items of a worklist built by
// schedule_kernel.  kFused = true: every workgroup first locates its own work
// units in the same order from cu_seqlens (only for batches with at most
// kFusedUsers users and kFusedRounds rounds of whole items) and keeps their
// descriptors; with sp.p > 1 the long items run as key-range parts.
template <bool kFused, bool kSplit, bool kLse>
__device__ __forceinline__ void attention_body(const uint16_t* __restrict__ qkv, const int4* __restrict__ items,
                                               const int32_t* __restrict__ count, int32_t* __restrict__ queue,
                                               const int32_t* __restrict__ cu, int U, int max_tiles, int n_heads,
                                               int layer_log2, float sl2, SplitArgs sp, uint16_t* __restrict__ out,
                                               float* __restrict__ lse) {
  // Two ring stages (K tile then V tile); tile j of an item lives in stage j%2.
  // The key loop is unrolled by two so that every LDS address is a per-lane
  // register plus an immediate.
  __shared__ __attribute__((aligned(1024))) char ring_lds[2 * kStageBytes];
  LDS char* const st0 = (LDS char*)ring_lds;
  LDS char* const st1 = st0 + kStageBytes;

  // Until its first item is known, a workgroup runs at the highest wave priority:
  // co-resident workgroups already inside long items (raised below) must not
  // starve the short work that precedes every item.
  __builtin_amdgcn_s_setprio(3);
  const int64_t ldq = 3 * n_heads * kHeadDim;
  const int64_t ldo = n_heads * kHeadDim;
  const int hd = n_heads * kHeadDim;
  Lanes L;
  make_lanes(L, ldq);
  const float rescale_thr = kRescaleLog2 / sl2;  // in raw score units
  // The all-ones A operand of the denominator MFMA, kept in registers (the empty
  // asm hides the constant, so it is not rebuilt before every use).
  bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
  asm volatile("" : "+v"(ones));
  // M0 (LDS destination) of this wave's first copy slice in the K half of stage 0;
  // the second slice is 1 KB further, the V half 8 KB, stage 1 16 KB.
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(st0 + 2048 * L.wid));

  // Work assignment: the fixed snake over the list (Snake, vlca_order.h).
  const int G = gridDim.x;
  const Snake sn(n_heads, layer_log2);
  const bool by_head = sn.by_head;
  const int slots = sn.slots, slot = sn.slot, head0 = sn.head0;
  auto work_of = [&](int round, int& item, int& h) { sn.unit(round, item, h); };

  // kFused: the workgroup's unit descriptors (q_tile | kind << 16, row_start,
  // length, head | split rank of part 0 << 16), negative past its last round;
  // shared by the waves.
  // kind: 0 the whole item, 1 / 2 its first / second key-range part.
  __shared__ i32x4 s_desc[kFused ? kDescRounds : 1];
  int desc_base = 0;  // the descriptors: s_desc[desc_base + round]
  __shared__ int s_arrived;
  int nitems = 0, qt_max = 0;
  if constexpr (kFused) {
    // The workgroup's own units (own_units, vlca_order.h); a workgroup past the
    // last unit (the grid may exceed the work) leaves now.
    if (!own_units<false>(cu, U, max_tiles, sp, L, st0, (LDS i32x4*)s_desc, work_of, desc_base)) return;
  } else {
    nitems = *count;
    qt_max = nitems > 0 ? items[0].y & 0xffff : 0;  // the first unit is of a longest user's last q-tile
  }
  // Dynamic assignment (worklist path with work counters): after the first two
  // rounds, which follow the snake (the workgroups of the longest first-round
  // items take the shortest second-round ones), a workgroup takes the next
  // unclaimed item from a counter in global memory, so workgroups that drew
  // short items take more of them.  With one head per workgroup (by_head, H <=
  // kQueues) each head has its own counter and items are taken in list order
  // (users kept together, so later q-tiles find the user's K/V in the L2 of the
  // XCD serving that head); otherwise the work units run over all (item, head)
  // pairs, heads fastest, with one counter.  Thread 0 claims the next item while
  // the second-round and later items run; LDS passes it to all waves at the
  // item's last barrier.  No claim precedes the first items: every workgroup
  // claiming at the kernel's start serialises the atomics on each counter's line.
  const bool dyn = !kFused && queue != nullptr;
  const bool per_head = by_head && n_heads <= kQueues;
  int32_t* const qctr = dyn ? queue + (per_head ? head0 : 0) * kQueueStride : nullptr;
  const int nslots = per_head ? slots : G;           // work units per round
  const int wfirst = per_head ? slot : (int)blockIdx.x;  // this workgroup's unit of round 0
  __shared__ int s_next;
  int claimed = 0;
  for (int round = 0;; ++round) {
    int qt, start, len, h;
    // Key tiles [klo, khi) of the item; a split item's part `part` of `parts`,
    // whose state goes to pool slot rank0 + part (split ranks of this head).
    int klo = 0, khi, parts = 1, rank0 = 0, part = 0;
    if constexpr (kFused) {
      if (round >= kDescRounds) break;
      const i32x4 d = s_desc[desc_base + round];
      const int w0 = __builtin_amdgcn_readfirstlane(d[0]);
      if (w0 < 0) break;
      start = __builtin_amdgcn_readfirstlane(d[1]);
      len = __builtin_amdgcn_readfirstlane(d[2]);
      const int w3 = __builtin_amdgcn_readfirstlane(d[3]);
      qt = w0 & 0xffff;
      h = w3 & 0xffff;
      const int kind = w0 >> 16;
      khi = qt + 1;
      if (kind != 0) {  // key tiles [0, nk/2) or [nk/2, nk)
        parts = 2;
        part = kind - 1;
        rank0 = w3 >> 16;
        if (part == 0)
          khi >>= 1;
        else
          klo = khi >> 1;
      }
    } else {
      int item;
      if (dyn) {
        const int w = round == 0   ? wfirst
                      : round == 1 ? 2 * nslots - 1 - wfirst
                                   : __builtin_amdgcn_readfirstlane(s_next);
        if (per_head) {
          item = w;
          h = head0;
        } else {
          item = w / n_heads;
          h = w - item * n_heads;
        }
        if (item >= nitems) break;
        if (round >= 1 && threadIdx.x == 0)
          claimed = 2 * nslots + __hip_atomic_fetch_add(qctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } else {
        work_of(round, item, h);
        if (item >= nitems) break;
      }
      const int4 it = items[item];
      qt = it.y & 0xffff;
      start = it.z;
      len = it.w;
      khi = qt + 1;
      if constexpr (kSplit) {
        const int kind = it.y >> 16;  // 0 in a list without split items
        if (kind != 0) {  // key tiles [0, nk/2) or [nk/2, nk)
          parts = 2;
          part = kind - 1;
          rank0 = it.x;
          if (part == 0)
            khi >>= 1;
          else
            klo = khi >> 1;
        }
      }
    }
    const int q0 = qt * kTileRows;
    const int lim = len - 1 - q0;  // the user's last row, relative to the diagonal tile
    // Scheduler plan: the longest items bound the kernel's critical path, so their
    // waves get issue priority over co-resident shorter items.  Single-kernel plan
    // (one or two rounds): equal priority, or the short items of the
    // last-dispatched workgroups, which also take the second round, fall behind
    // the longest item.
    if (kFused)
      __builtin_amdgcn_s_setprio(0);
    else if (qt >= 1 && 2 * qt >= qt_max)
      __builtin_amdgcn_s_setprio(3);
    else if (qt >= 1 && 4 * qt >= qt_max)
      __builtin_amdgcn_s_setprio(2);
    else if (qt >= 1)
      __builtin_amdgcn_s_setprio(1);
    else
      __builtin_amdgcn_s_setprio(0);
    const uint16_t* kg = qkv + (int64_t)start * ldq + hd + h * kHeadDim;
    const int64_t tstride = (int64_t)kTileRows * ldq;

    // This wave's copies of key tile jj into the stage at M0 offset `so`.  Tiles
    // before the diagonal lie wholly inside the user; the diagonal tile clamps rows
    // past the user's end to its last row (finite data under the causal mask,
    // never another user's rows).
    auto issue_tile = [&](uint32_t so, int jj) {
      const uint16_t* kt = kg + jj * tstride;
      const uint16_t* vt = kt + hd;
      if (jj == qt) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = min(L.crow[i], lim);
          const uint32_t o = (uint32_t)(r * ldq * 2 + 16 * ((L.lane & 7) ^ swz(L.crow[i])));
          copy_to_lds(kt, o, m0 + so + 1024 * i);
          copy_to_lds(vt, o, m0 + so + kTileBytes + 1024 * i);
        }
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          copy_to_lds(kt, L.cofs_g[i], m0 + so + 1024 * i);
          copy_to_lds(vt, L.cofs_g[i], m0 + so + kTileBytes + 1024 * i);
        }
      }
    };

    // The wave's Q rows go into its own rows of the K half of stage 1, which only
    // this wave refills (with tile 1), after its Q reads have completed.
    {
      const uint16_t* qg = qkv + ((int64_t)start + q0) * ldq + h * kHeadDim;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = min(L.crow[i], lim);
        copy_to_lds(qg, (uint32_t)(r * ldq * 2 + 16 * ((L.lane & 7) ^ swz(L.crow[i]))), m0 + kStageBytes + 1024 * i);
      }
    }
    issue_tile(0, klo);
    wait_vmem_lds<4>();  // this wave's Q rows have landed (the first tile's 4 copies may be in flight)
    bf16x8 qf[2];
    qf[0] = lds_b128(st1, L.qr * 128 + ((L.g ^ swz(L.qr)) << 4));
    qf[1] = lds_b128(st1, L.qr * 128 + (((4 + L.g) ^ swz(L.qr)) << 4));

    Acc A;
    A.m = -__builtin_inff();
    A.moff = __builtin_inff();
    A.mthr = -__builtin_inff();
    A.l = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = 0; d < 4; ++d) A.o[d] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Before consuming tile j: wait for this wave's copies of it, then a barrier
    // makes every wave's copies visible and guarantees that the other stage (tile
    // j-1, or the Q rows) has been read by every wave, so tile j+1 may refill it.
    // Tile j of the range sits in stage (j - klo) % 2.  Only the diagonal tile
    // (qt, the last tile of the range when khi == qt + 1) needs a mask; the last
    // tile of a first part takes the unmasked step (a uniform branch: a variable
    // mask limit cost 14 VGPRs).
    //
    // A wave whose 16 rows all lie past the user's end (the user's last q-tile)
    // computes nothing: it only issues its share of the copies and meets the
    // barriers.
    const bool diag_last = !kSplit || khi == qt + 1;
    const bool wave_on = __builtin_amdgcn_readfirstlane(16 * L.wid < len - q0);
    // The diagonal tile, specialised for each wave (blocks above the wave's rows
    // are neither formed nor weighed); it ends an item once, so its stage is a
    // run-time choice.
    auto last_step = [&](const LDS char* base) {
      if (!diag_last) {
        tile_step(base, L, qf, ones, sl2, rescale_thr, A, NoMask{});
        return;
      }
      const int lim = L.lq - 4 * L.g;
      switch (__builtin_amdgcn_readfirstlane(L.wid)) {
        case 0: tile_step(base, L, qf, ones, sl2, rescale_thr, A, DiagWave<0>{lim}); break;
        case 1: tile_step(base, L, qf, ones, sl2, rescale_thr, A, DiagWave<1>{lim}); break;
        case 2: tile_step(base, L, qf, ones, sl2, rescale_thr, A, DiagWave<2>{lim}); break;
        default: tile_step(base, L, qf, ones, sl2, rescale_thr, A, DiagWave<3>{lim}); break;
      }
    };
    // The tile loop, in two copies: with the tile steps (a wave with rows of the
    // user), and with the copies and barriers alone.  (A condition around each
    // step inside one loop left the accumulators in different registers on the
    // two paths, with copies back at every join.)
    auto tiles = [&](auto compute) {
      constexpr bool kOn = decltype(compute)::value;
      int j = klo;
      for (; j + 2 < khi; j += 2) {
        wait_and_barrier<0>();
        issue_tile(kStageBytes, j + 1);
        if constexpr (kOn) tile_step(st0, L, qf, ones, sl2, rescale_thr, A, NoMask{});
        wait_and_barrier<0>();
        issue_tile(0, j + 2);
        if constexpr (kOn) tile_step(st1, L, qf, ones, sl2, rescale_thr, A, NoMask{});
      }
      const bool two_left = j + 1 < khi;  // j in stage 0, the last one goes to stage 1
      if (two_left) {
        wait_and_barrier<0>();
        issue_tile(kStageBytes, j + 1);
        if constexpr (kOn) tile_step(st0, L, qf, ones, sl2, rescale_thr, A, NoMask{});
      }
      wait_and_barrier<0>();
      if constexpr (kOn) last_step(two_left ? st1 : st0);
    };
    if (wave_on)
      tiles(std::true_type{});
    else
      tiles(std::false_type{});
    // The claim made at the item's start is passed on; every wave read s_next
    // before this item's first barrier.
    if (dyn && round >= 1 && threadIdx.x == 0) s_next = claimed;
    wait_and_barrier<0>();  // every wave is done with the ring before the next item refills it

    if (kSplit && parts > 1) {
      // Leave this part's state in its slot; count the arrival once every wave's
      // stores have completed.  The last part to arrive resets the counter for
      // the next call and merges; the others are done with this unit.
      const int64_t slot_stride = (int64_t)n_heads * kPoolSlotFloats;
      float* const slot0 = sp.pool + (int64_t)rank0 * slot_stride + (int64_t)h * kPoolSlotFloats;
      store_partial(slot0 + part * slot_stride, L, A);
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      lds_barrier();
      if (threadIdx.x == 0) {
        int32_t* const c = sp.ctr + ((int64_t)rank0 * n_heads + h) * kSplitCtrStride;
        const int before = __hip_atomic_fetch_add(c, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (before == parts - 1) __hip_atomic_store(c, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_arrived = before;
      }
      lds_barrier();
      if (__builtin_amdgcn_readfirstlane(s_arrived) != parts - 1) continue;
      merge_parts(slot0 + (1 - part) * slot_stride, part, L, sl2, A);
    }

    if (wave_on) {
      // The wave's 16 output rows go through its own rows of stage 0's K half
      // (every wave is past the item's last barrier, and only this wave copies into
      // those rows, after these reads), so that each row leaves as one 128-byte
      // write of 8 lanes instead of four 32-byte pieces from four instructions.
      // 16-byte chunk c of row r sits at chunk c ^ (r % 8): conflict-free both ways.
      // The lane id passes through an empty asm so that the addresses are formed
      // here rather than kept live across the item loop.
      int lane = L.lane;
      asm volatile("" : "+v"(lane));
      const int lq = lane & 15, g = lane >> 4;
      LDS char* const rows = st0 + 2048 * L.wid;
      const float inv = 1.0f / A.l[0];
      // Log-sum-exp of the row's scaled scores (natural log), for the backward pass:
      // sum_j exp(scale q.k_j) = 2^(m sl2) * l.
      if (kLse && g == 0 && L.qr < len - q0)
        lse[((int64_t)start + q0 + L.qr) * n_heads + h] = (A.m * sl2 + __builtin_amdgcn_logf(A.l[0])) * 0.6931471805599453f;
#pragma unroll
      for (int d = 0; d < 4; ++d) {  // dims 16d + 4g .. +3 of row lq: bytes 32d + 8g
        const u32x2 wv = {pack_bf16x2(A.o[d][0] * inv, A.o[d][1] * inv),
                          pack_bf16x2(A.o[d][2] * inv, A.o[d][3] * inv)};
        *(LDS u32x2*)(rows + lq * 128 + (((2 * d + (g >> 1)) ^ swz(lq)) << 4) + 8 * (g & 1)) = wv;
      }
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int i = 0; i < 2; ++i) {  // row r: lanes 8(r%8) .. +7, one 16-byte chunk each
        const int r = 8 * i + (lane >> 3), c = lane & 7;
        const u32x4 v = *(const LDS u32x4*)(rows + r * 128 + ((c ^ swz(r)) << 4));
        // Non-temporal: the kernel never reads the output back, so its lines need
        // not displace K/V in L2.
        if (16 * L.wid + r < len - q0)
          __builtin_nontemporal_store(
              v, reinterpret_cast<u32x4*>(out + ((int64_t)start + q0 + 16 * L.wid + r) * ldo + h * kHeadDim + 8 * c));
      }
    }
  }
}

#define VLCA_ATTENTION_PARAMS                                                                                   \
  const uint16_t *__restrict__ qkv, const int4 *__restrict__ items, const int32_t *__restrict__ count,          \
      int32_t *__restrict__ queue, const int32_t *__restrict__ cu, int U, int max_tiles, int n_heads,             \
      int layer_log2, float sl2, SplitArgs sp, uint16_t *__restrict__ out, float *__restrict__ lse
#define VLCA_ATTENTION_ARGS qkv, items, count, queue, cu, U, max_tiles, n_heads, layer_log2, sl2, sp, out, lse

// Four workgroups per CU (at most 128 VGPRs a lane) is the occupancy the tile
// step is tuned for.  Every instance fits it without an occupancy bound; such a
// bound made the compiler schedule the tile step worse (the 25523-token batch 8%
// slower over a worklist).
// kLse: also write each row's log-sum-exp (the training forward); a template
// flag, so that the plain forward's instances keep their registers.
template <bool kFused, bool kSplit, bool kLse>
__global__ __launch_bounds__(kAttnThreads) void attention_kernel(VLCA_ATTENTION_PARAMS) {
  attention_body<kFused, kSplit, kLse>(VLCA_ATTENTION_ARGS);
}

#undef VLCA_ATTENTION_ARGS
#undef VLCA_ATTENTION_PARAMS

// Offsets padded to a fixed user count: out[i] = min(cu[min(i, U)], total) for
// i = 0 .. U_max, so users U .. U_max-1 have no rows and no offset passes total.
__global__ __launch_bounds__(256) void pad_offsets_kernel(const int32_t* __restrict__ cu, int U, int total,
                                                          int32_t* __restrict__ out, int U_max) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i > U_max) return;
  const int v = U > 0 ? cu[i < U ? i : U] : 0;
  out[i] = v < 0 ? 0 : (v > total ? total : v);
}

}  // namespace

hipError_t launch_pad_offsets(const int32_t* cu_seqlens, int num_users, int total, int32_t* out, int max_users,
                              hipStream_t stream) {
  hipLaunchKernelGGL(pad_offsets_kernel, dim3((max_users + 1 + 255) / 256), dim3(256), 0, stream, cu_seqlens,
                     num_users, total, out, max_users);
  return hipGetLastError();
}

hipError_t launch_schedule(const int32_t* cu_seqlens, int num_users, int max_tiles, int4* items, int32_t* count,
                           int32_t* queue, const SplitArgs& split, hipStream_t stream) {
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, cu_seqlens, num_users, max_tiles,
                     items, count, queue, split);
  return hipGetLastError();
}

hipError_t launch_bwd_prepare(const void* out, const void* dout, const float* lse, const int32_t* cu_seqlens,
                              int num_users, int max_tiles, int4* items, int32_t* count, int32_t* queue, int n_heads,
                              void* dqkv, int cus, hipStream_t stream) {
  // Workgroup 0 and two row-pass workgroups of 1024 threads per CU.
  hipLaunchKernelGGL(bwd_prepare_kernel, dim3(1 + 2 * cus), dim3(kSchedThreads), 0, stream, cu_seqlens, num_users,
                     max_tiles, items, count, queue, static_cast<const uint16_t*>(out),
                     static_cast<const uint16_t*>(dout), lse, n_heads, static_cast<uint16_t*>(dqkv));
  return hipGetLastError();
}

hipError_t launch_attention(const void* qkv, const int4* items, const int32_t* count, int32_t* queue, int n_heads,
                            float scale_log2e, const SplitArgs& split, void* out, float* lse, int grid, int layer_log2,
                            hipStream_t stream) {
  // The split-capable instance runs whole items as well (every unit of a list
  // without split items is kind 0), so the training forward needs only that one.
  auto* k = lse != nullptr     ? attention_kernel<false, true, true>
            : split.p > 1      ? attention_kernel<false, true, false>
                               : attention_kernel<false, false, false>;
  hipLaunchKernelGGL(k, dim3(grid), dim3(kAttnThreads), 0, stream, static_cast<const uint16_t*>(qkv), items, count,
                     queue, nullptr, 0, 0, n_heads, layer_log2, scale_log2e, split, static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

hipError_t launch_attention_fused(const void* qkv, const int32_t* cu_seqlens, int num_users, int max_tiles,
                                  int n_heads, float scale_log2e, const SplitArgs& split, void* out, float* lse,
                                  int grid, int layer_log2, hipStream_t stream) {
  auto* k = lse != nullptr ? attention_kernel<true, true, true> : attention_kernel<true, true, false>;
  hipLaunchKernelGGL(k, dim3(grid), dim3(kAttnThreads), 0, stream, static_cast<const uint16_t*>(qkv), nullptr,
                     nullptr, nullptr, cu_seqlens, num_users, max_tiles, n_heads, layer_log2, scale_log2e, split,
                     static_cast<uint16_t*>(out), lse);
  return hipGetLastError();
}

int attention_blocks_per_cu(bool fused) {
  int n = 0;
  const hipError_t e =
      fused ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attention_kernel<true, true, false>, kAttnThreads, 0)
            : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attention_kernel<false, false, false>, kAttnThreads, 0);
  if (e != hipSuccess || n < 1) n = 1;
  return n;
}

}  // namespace vlca
