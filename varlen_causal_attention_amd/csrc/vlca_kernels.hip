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

#include "vlca_internal.h"

namespace vlca {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
#define LDS __attribute__((address_space(3)))
typedef LDS bf16x4 lds_bf16x4;

constexpr int kSchedThreads = 1024;
constexpr int kSchedCache = 8160;  // cu_seqlens entries cached in LDS by the scheduler (LDS <= 64 KB)
constexpr int kWaves = 4;                              // wave w owns query rows 16w .. 16w+15
constexpr int kAttnThreads = 64 * kWaves;
constexpr int kTileBytes = kTileRows * kHeadDim * 2;  // 8 KB: one 64 x 64 bf16 tile, 128 B rows
constexpr int kStageBytes = 2 * kTileBytes;           // K tile then V tile
constexpr float kRescaleLog2 = 8.0f;

// ----------------------------------------------------------------- scheduler

struct Seg {
  int start, len, tiles;
};

template <typename CachePtr>
__device__ __forceinline__ Seg segment_of(const int32_t* __restrict__ cu, CachePtr s_cu, bool cached, int u, int total,
                                          int max_tiles) {
  const int a = cached ? s_cu[u] : cu[u];
  const int b = cached ? s_cu[u + 1] : cu[u + 1];
  Seg s{a, 0, 0};
  // Rows outside [0, total) are never touched, whatever the offsets hold.
  if (a >= 0 && b > a && b <= total) {
    s.len = b - a;
    const int t = (s.len - 1) / kTileRows + 1;
    s.tiles = t < max_tiles ? t : max_tiles;
  }
  return s;
}

// Length class of a user with t >= 1 tiles: floor(log2(t)).
__device__ __forceinline__ int length_class(int t) { return 31 - __builtin_clz((unsigned)t); }

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and row
// broadcasts (no LDS traffic): sums within each row of 16 lanes, then row 0's
// total is added to row 1 (and row 2's to row 3), then lane 31's to rows 2-3.
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}

// Split width of a user of t q-tiles: c = max(ceil(t / 2), min_width) key tiles
// (0 = no splitting).  Its items with nk > c key tiles (the last t - c q-tiles)
// run as two parts, key tiles [0, nk/2) and [nk/2, nk) (the diagonal tile in the
// second); the rest run whole.  The rule depends on the user's own length only.
// The user's run of work units: the two parts of each split item, q-tiles
// descending, then its whole items, q-tiles descending.
struct SplitUser {
  int c;      // split width (0: no splitting)
  int split;  // split items: max(t - c, 0)
};

__device__ __forceinline__ SplitUser split_user(int t, int on, int min_width) {
  SplitUser r{0, 0};
  if (on && t > 0) {
    const int half = (t + 1) >> 1;
    r.c = half > min_width ? half : min_width;
    r.split = t > r.c ? t - r.c : 0;
  }
  return r;
}

// Unit i of the run of a user of t q-tiles: its item has nk key tiles and it is
// part k of p (p = 1: the whole item).
__device__ __forceinline__ void unit_of(int t, const SplitUser& su, int i, int& nk, int& k, int& p) {
  if (i < 2 * su.split) {
    nk = t - (i >> 1);
    k = i & 1;
    p = 2;
  } else {
    nk = t - su.split - (i - 2 * su.split);
    k = 0;
    p = 1;
  }
}

constexpr int kClasses = 13;       // tile counts up to kMaxLevels = 4096 -> classes 0..12
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
  int n_whole, n_split;               // list sizes without and with key-range splitting
};

// Worklist order: users grouped by length class floor(log2(tiles)), highest
// class first; inside a class users ascend; each user's q-tiles are adjacent,
// from its last q-tile (the most key tiles) down to q-tile 0.  The first slot of
// user u is then
//   sum of the tiles of all higher classes + sum of the tiles of the users
//   before u in its own class,
// computed in two passes over the users (class totals, then per-class running
// sums in chunks of kThreads users).  emit(slot, user, q_tile, segment) stores
// one item; S.count receives the number of items.  All threads of the
// workgroup must call this (it contains barriers).
//
// Key-range splitting (sp.p > 1, batches of at most kThreads users only): the
// same rule and decision as the single-kernel plan (split when the list with
// split items holds at most sp.upr units), so both plans give the same bits.
// The counts are then carried packed (whole items in the low 15 bits, units in
// the high 17) and emit(slot, x, y, segment) gets y = q_tile | kind << 16 and x
// = the user (kind 0, a whole item) or the split rank of the item's first part
// (kind 1, 2: first / second part; kind 3: a first part that runs nothing).
// Without splitting, x = user and y = q_tile.
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
  __syncthreads();
  bool split = false;
  if (sp.p > 1 && nusers <= kThreads) {  // uniform
    const int t = tid < nusers ? segment_of(cu, s_cu, cached, tid, total, max_tiles).tiles : 0;
    int w = t, x = t + split_user(t, 1, sp.min_width).split;
    for (int o = 32; o > 0; o >>= 1) {
      w += __shfl_xor(w, o);
      x += __shfl_xor(x, o);
    }
    if (lane == 0) {
      __atomic_fetch_add(&S->n_whole, w, __ATOMIC_RELAXED);
      __atomic_fetch_add(&S->n_split, x, __ATOMIC_RELAXED);
    }
    __syncthreads();
    split = S->n_split > S->n_whole && S->n_split <= sp.upr;
  }
  // The count a user adds to the list: its q-tiles, or both counts packed.
  auto units_of_user = [&](int t) {
    return split ? t | ((t + split_user(t, 1, sp.min_width).split) << 15) : t;
  };
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
  __syncthreads();
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
    __syncthreads();
    if (t > 0 && split) {  // at most kThreads users: a single chunk
      int both = S->base[cl] + pre;
      for (int w = 0; w < wid; ++w) both += S->wsum[w][cl];
      const int off = both >> 15;
      const int roff = 2 * ((both >> 15) - (both & 0x7fff));
      const SplitUser spl = split_user(t, 1, sp.min_width);
      for (int i = 0; i < t + spl.split; ++i) {
        int nk, k, p;
        unit_of(t, spl, i, nk, k, p);
        int kind = 0, x = u;
        if (p > 1) {
          const int r0 = roff + i - k;  // split ranks r0, r0+1
          if (r0 + 2 <= sp.cap) {
            kind = 1 + k;
            x = r0;
          } else if (k == 0) {
            kind = 3;  // pool full: the second part runs the whole item, the first nothing
          }
        }
        emit(off + i, x, (nk - 1) | (kind << 16), s);
      }
    } else if (t > 0) {
      int off = S->base[cl] + pre;
      for (int w = 0; w < wid; ++w) off += S->wsum[w][cl];
      if (t <= kShortTiles) {
        for (int i = 0; i < t; ++i) emit(off + i, u, t - 1 - i, s);
      } else {
        const int k = __atomic_fetch_add(&S->nlong, 1, __ATOMIC_RELAXED);
        S->long_u[k] = u;
        S->long_off[k] = off;
      }
    }
    __syncthreads();
    const int nlong = S->nlong;
    for (int i = wid; i < nlong; i += kThreads / 64) {
      const int lu = S->long_u[i];
      const int off = S->long_off[i];
      const Seg ls = segment_of(cu, s_cu, cached, lu, total, max_tiles);
      for (int k = lane; k < ls.tiles; k += 64) emit(off + k, lu, ls.tiles - 1 - k, ls);
    }
    if (tid < kClasses) {
      int sum = 0;
      for (int w = 0; w < kThreads / 64; ++w) sum += S->wsum[w][tid];
      S->base[tid] += sum;
    }
    __syncthreads();
  }
  __syncthreads();  // S->count and every emitted item are visible to all threads
}

// The worklist in global memory: items[slot] = (user, q_tile, row_start, length),
// or with key-range splitting the units described at order_items.
__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(const int32_t* __restrict__ cu, int U,
                                                                 int max_tiles, int4* __restrict__ items,
                                                                 int32_t* __restrict__ count,
                                                                 int32_t* __restrict__ queue, SplitArgs sp) {
  // The attention kernel's work counters start at zero.
  if (queue != nullptr && threadIdx.x < kQueues) queue[threadIdx.x * kQueueStride] = 0;
  __shared__ int s_cu_lds[kSchedCache + 1];
  __shared__ OrderScratch<kSchedThreads> S_lds;
  LDS int* const s_cu = (LDS int*)s_cu_lds;
  LDS OrderScratch<kSchedThreads>* const S = (LDS OrderScratch<kSchedThreads>*)&S_lds;
  const bool cached = U <= kSchedCache;
  if (U > 0 && max_tiles > 0 && cached) {
    for (int i = threadIdx.x; i <= U; i += kSchedThreads) s_cu[i] = cu[i];
  }
  __syncthreads();
  const int total = (U > 0 && max_tiles > 0) ? (cached ? s_cu[U] : cu[U]) : 0;
  const int nusers = max_tiles > 0 ? U : 0;
  order_items<kSchedThreads>(cu, s_cu, cached, nusers, total, max_tiles, sp, S,
                             [&](int slot, int x, int y, const Seg& sg) {
                               items[slot] = make_int4(x, y, sg.start, sg.len);
                             });
  if (threadIdx.x == 0) *count = S->count;
}

// ----------------------------------------------------------------- attention

// XOR swizzle of the 16-byte chunk index inside a 128-byte LDS tile row: chunk
// c of row r is stored at chunk c ^ (r % 8).  With the fragment row orders below
// (16 consecutive rows per K read; 4 rows per 16-lane group per V^T read) both
// the K/Q reads (ds_read_b128) and the V^T reads (ds_read_b64_tr_b16) are free of
// bank conflicts on gfx950 (4 and 2 LDS cycles per wave instruction).
__device__ __forceinline__ int swz(int r) { return r & 7; }

__device__ __forceinline__ bf16x8 lds_b128(const LDS char* base, int byte_off) {
  return __builtin_bit_cast(bf16x8, *(const LDS u32x4*)(base + byte_off));
}

__device__ __forceinline__ bf16x4 lds_tr16(const LDS char* base, int byte_off) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(base + byte_off));
}

// Max over lanes l, l^16, l^32, l^48 (the 4 lane groups holding one query's keys),
// with the gfx950 row-swap permutes: each lane ends up holding its own value and
// its partner's, so the max of the pair is the pairwise max.
__device__ __forceinline__ float max_across_lane_groups(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// NaN-propagating maximum (v_maximum3_f32 on gfx950; no canonicalising moves).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));  // RNE
}

// Wait until at most n vector-memory operations of this wave are outstanding and
// all of its LDS operations have completed.  An asm statement with a "memory"
// clobber, so no memory access is moved across it.
template <int n>
__device__ __forceinline__ void wait_vmem_lds() {
  static_assert(n >= 0 && n < 64, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(n) : "memory");
}

// The same wait followed by a workgroup barrier.  __syncthreads() would add a
// release fence that also waits for every LDS copy still in flight; here only
// what the caller names (n copies may stay in flight).
template <int n>
__device__ __forceinline__ void wait_and_barrier() {
  static_assert(n >= 0 && n < 64, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(n) : "memory");
}

// Copy 16 bytes per lane from global memory into LDS (global_load_lds_dwordx4):
// lane l reads base + voff (a wave-uniform 64-bit base, a per-lane 32-bit byte
// offset) and its bytes land at LDS address m + 16*l (m wave-uniform).  Issued
// from inline asm so that the compiler, which would otherwise track these LDS
// writes coarsely and insert waits for every copy in flight before unrelated LDS
// reads, leaves all waits on them to the explicit wait_vmem_lds /
// wait_and_barrier calls.  The instruction has no register result; M0 (the LDS
// base operand) is saved and restored around it.
__device__ __forceinline__ void copy_to_lds(const void* base, uint32_t voff, uint32_t m) {
  // readfirstlane returns int: widen through uint32_t so the low word is not
  // sign-extended into the high word of the 64-bit base.
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)base);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)((uintptr_t)base >> 32));
  const uint64_t sbase = (uint64_t)lo | ((uint64_t)hi << 32);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m), "v"(voff), "s"(sbase)
      : "memory");
}

// Per-lane constants of the attention workgroup.  Wave w owns query rows
// 16w .. 16w+15 of the tile; it also copies those rows of every K, V and Q tile
// into LDS (two 1 KB copies of 8 rows each per tile).
struct Lanes {
  int g, lq, wid, lane;
  int qr;                 // query row of this lane inside the tile
  int crow[2];            // tile row copied by this lane, per copy instruction
  uint32_t cofs_g[2];     // byte offset of the copied 16-byte chunk from the tile's first row
  int kofs[2];            // K fragment byte offsets inside a stage (block 0; block b: + 2048 b)
  int vofs[4];            // V^T fragment byte offsets inside a stage (dim block d; + 4096 hh + 2048 s)
};

__device__ __forceinline__ void make_lanes(Lanes& L, int64_t ldq) {
  const int tid = threadIdx.x;
  L.lane = tid & 63;
  L.wid = tid >> 6;
  L.g = L.lane >> 4;
  L.lq = L.lane & 15;
  L.qr = 16 * L.wid + L.lq;
  // Copy role: instruction i moves tile rows 16w + 8i .. +7; lane l lands at byte
  // 16*l of that 1 KB slice (row l/8, physical chunk l%8, logical chunk
  // (l%8) ^ (row%8)).
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    L.crow[i] = 16 * L.wid + 8 * i + (L.lane >> 3);
    L.cofs_g[i] = (uint32_t)(L.crow[i] * ldq * 2 + 16 * ((L.lane & 7) ^ swz(L.crow[i])));
  }
  // K fragments: S^T block b covers keys 16b .. 16b+15 in order (MFMA row lq <-
  // key 16b + lq), so output reg r in lane group g is key 16b + 4g + r.  The lane
  // reads dims 8g .. 8g+7 (k-step 0) and 32+8g .. (k-step 1) of that row.
  L.kofs[0] = L.lq * 128 + ((L.g ^ swz(L.lq)) << 4);
  L.kofs[1] = L.lq * 128 + (((4 + L.g) ^ swz(L.lq)) << 4);
  // V^T fragments for keys 32hh .. 32hh+31 in the P^T slot order of lane group g:
  // slots 0..3 = keys 32hh + 4g + 0..3 (score block 2hh), slots 4..7 = keys
  // 32hh + 16 + 4g + 0..3 (block 2hh+1).  ds_read_b64_tr_b16 gives lane i of a
  // 16-lane group element i%4 of source lanes {i/4, 4+i/4, 8+i/4, 12+i/4}; with
  // source lane j reading key row 4g + j/4, dims 16d + 4(j%4) .. +3, lane i gets
  // the 4 keys of dim 16d + i.  The second half (slots 4..7) is 16 rows on
  // (+2048 bytes), the second 32 keys 32 rows on (+4096): neither changes row%8.
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const int rho = 4 * L.g + (L.lq >> 2);
    const int chunk = 2 * d + ((L.lq & 3) >> 1);
    L.vofs[d] = kTileBytes + rho * 128 + ((chunk ^ swz(rho)) << 4) + 8 * (L.lq & 1);
  }
}

// Online-softmax state of one lane: the running reference max m (raw score
// units), the O^T accumulator (dims 16d + 4g + r) and the denominator (every
// register of l holds it).
struct Acc {
  float m;
  float moff;  // -m * sl2: the exponent offset of the weights
  float mthr;  // m + rescale threshold: keys above it raise m
  f32x4 o[4];
  f32x4 l;
};

// One key tile of one item: S^T = K Q^T, mask (diagonal tile only), softmax
// update, O^T += V^T P^T and l += 1^T P^T.
// kDiag: keys kk > lim are masked (lim = the lane's query row on the diagonal
// tile; 63 or more masks nothing).
template <bool kDiag>
__device__ __forceinline__ void tile_step(const LDS char* base, const Lanes& L, const bf16x8 (&qf)[2],
                                          const bf16x8& ones, float sl2, float rescale_thr, Acc& A, int lim = 0) {
  f32x4 s[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const bf16x8 k0 = lds_b128(base, L.kofs[0] + 2048 * b);
    const bf16x8 k1 = lds_b128(base, L.kofs[1] + 2048 * b);
    s[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    s[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[1], s[b], 0, 0, 0);
  }
  if (kDiag) {  // key kk visible iff kk <= lim (on the diagonal tile, lim = qr)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (16 * b + 4 * L.g + r > lim) s[b][r] = -__builtin_inff();
  }
  // The tile is taken in two halves of 32 keys (score blocks 2hh, 2hh+1), so the
  // second half's QK^T MFMAs run while the first half's softmax is computed.
  // Lane-local max over this lane's 8 keys of the half.  The reference max m of a
  // query is shared by its 4 lane groups; only when some key exceeds it by more
  // than the threshold (and on the first tile, m = -inf; the first half always
  // holds a visible key of every query) is the true max formed across the lane
  // groups and m raised, with the accumulators rescaled.  The common path needs
  // no cross-lane traffic.
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    const f32x4& s0 = s[2 * hh];
    const f32x4& s1 = s[2 * hh + 1];
    const float lm = vmax(vmax(vmax(vmax(s0[0], s0[1]), s0[2]), vmax(vmax(s0[3], s1[0]), s1[1])), vmax(s1[2], s1[3]));
    if (__any(lm > A.mthr)) {  // wave-uniform
      const float mt = max_across_lane_groups(lm);
      const float mn = fmaxf(A.m, mt);
      const float alpha = __builtin_amdgcn_exp2f((A.m - mn) * sl2);
#pragma unroll
      for (int d = 0; d < 4; ++d) A.o[d] *= alpha;
      A.l *= alpha;
      A.m = mn;
      A.moff = -mn * sl2;
      A.mthr = mn + rescale_thr;
    }
    const float moff = A.moff;
    // P^T slots 0..3 of lane group g = keys 32hh + 4g + 0..3 (block 2hh), slots
    // 4..7 = keys 32hh + 16 + 4g + 0..3 (block 2hh+1)
    uint4 pw;
    pw.x = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(s0[0], sl2, moff)),
                       __builtin_amdgcn_exp2f(__builtin_fmaf(s0[1], sl2, moff)));
    pw.y = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(s0[2], sl2, moff)),
                       __builtin_amdgcn_exp2f(__builtin_fmaf(s0[3], sl2, moff)));
    pw.z = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(s1[0], sl2, moff)),
                       __builtin_amdgcn_exp2f(__builtin_fmaf(s1[1], sl2, moff)));
    pw.w = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(s1[2], sl2, moff)),
                       __builtin_amdgcn_exp2f(__builtin_fmaf(s1[3], sl2, moff)));
    const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const bf16x4 lo = lds_tr16(base, L.vofs[d] + 4096 * hh);
      const bf16x4 hi = lds_tr16(base, L.vofs[d] + 4096 * hh + 2048);
      const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      A.o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, A.o[d], 0, 0, 0);
    }
    A.l = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb, A.l, 0, 0, 0);
  }
}

// Wait for this wave's LDS operations, then a workgroup barrier (no wait on
// copies in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Rounds a workgroup can run when it orders the work itself (kFused), and the
// most users that path takes (one per thread).  The launch condition counts
// whole items (kFusedRounds rounds); key-range splitting (below) turns an item
// into at most kMaxSplitParts work units, so the descriptors hold that many more.
constexpr int kFusedRounds = 16;
static_assert(kFusedUsers == kAttnThreads, "the shared-list prologue takes one user per thread");
constexpr int kDescRounds = kFusedRounds * kMaxSplitParts;

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

// Run by the last part to finish: fold the states of parts 0 .. parts-1 in that
// order (its own from registers, the others from their slots, slot_stride floats
// apart), so the result does not depend on which part finished last.
__device__ __forceinline__ void merge_parts(const float* slot0, int64_t slot_stride, int parts, int part,
                                            const Lanes& L, float sl2, Acc& A) {
  float cm = 0.f, cl = 0.f;
  f32x4 co[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) co[d] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < parts; ++k) {
    float xm, xl;
    f32x4 xo[4];
    if (k == part) {
      xm = A.m;
      xl = A.l[0];
#pragma unroll
      for (int d = 0; d < 4; ++d) xo[d] = A.o[d];
    } else {
      const float* const s = slot0 + k * slot_stride;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const f32x2 a = load_coherent(s + slot_o_offset(L, d));
        const f32x2 b = load_coherent(s + slot_o_offset(L, d) + 128);
        xo[d] = f32x4{a[0], a[1], b[0], b[1]};
      }
      const f32x2 ml = load_coherent(s + 4096 + 2 * threadIdx.x);
      xm = ml[0];
      xl = ml[1];
    }
    if (k == 0) {
      cm = xm;
      cl = xl;
#pragma unroll
      for (int d = 0; d < 4; ++d) co[d] = xo[d];
    } else {
      const float mn = fmaxf(cm, xm);
      const float a = __builtin_amdgcn_exp2f((cm - mn) * sl2);
      const float b = __builtin_amdgcn_exp2f((xm - mn) * sl2);
#pragma unroll
      for (int d = 0; d < 4; ++d) co[d] = co[d] * a + xo[d] * b;
      cl = cl * a + xl * b;
      cm = mn;
    }
  }
  A.m = cm;
  A.l[0] = cl;
#pragma unroll
  for (int d = 0; d < 4; ++d) A.o[d] = co[d];
}

// kFused = false: walk the first *count items of a worklist built by
// schedule_kernel.  kFused = true: every workgroup first locates its own work
// units in the same order from cu_seqlens (only for batches with at most
// kFusedUsers users and kFusedRounds rounds of whole items) and keeps their
// descriptors; with sp.p > 1 the long items run as key-range parts.
template <bool kFused, bool kSplit>
__device__ __forceinline__ void attention_body(const uint16_t* __restrict__ qkv, const int4* __restrict__ items,
                                               const int32_t* __restrict__ count, int32_t* __restrict__ queue,
                                               const int32_t* __restrict__ cu, int U, int max_tiles, int n_heads,
                                               int layer_log2, float sl2, SplitArgs sp, uint16_t* __restrict__ out) {
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

  // Work assignment.  With the grid a multiple of H, workgroup g always runs head
  // g % H (with H = 8 that is the XCD it sits on) and item slot g / H of each
  // round; rounds alternate direction (snake), so the workgroups that drew the
  // longest items of round 0 draw the shortest of round 1.
  const int G = gridDim.x;
  const bool by_head = G % n_heads == 0;
  const int slots = by_head ? G / n_heads : G;
  const int slot = by_head ? blockIdx.x / n_heads : blockIdx.x;
  const int head0 = by_head ? blockIdx.x - slot * n_heads : 0;
  // When all the work fits in one round, the workgroups that share a CU
  // (g, g + CUs, g + 2 CUs, ... in launch order) hold slots `layer` apart, and
  // the snake runs across them instead: odd layers take their ranks in reverse,
  // so the sums of the items on each CU come out even rather than the first CUs
  // drawing the longest item of every layer.  With more rounds the plain snake
  // is kept: it leaves the second round's items to the CUs of the shortest
  // first-round items, away from the longest ones.
  // (Every round after the first is then empty, so the layered rank can stand
  // in for the slot in every round.)  The launch passes layer_log2 >= 0 only
  // when the work fits in one round and `layer` is a power of two.
  int rank = slot;
  if (layer_log2 >= 0) {
    const int layer = 1 << layer_log2;
    const int lyr = slot >> layer_log2, lyr_pos = slot & (layer - 1);
    const int lyr_len = min(layer, slots - (lyr << layer_log2));
    rank = slot - lyr_pos + ((lyr & 1) ? lyr_len - 1 - lyr_pos : lyr_pos);
  }
  auto work_of = [&](int round, int& item, int& h) {
    const int pos = (round & 1) ? slots - 1 - rank : rank;
    if (by_head) {
      item = round * slots + pos;
      h = head0;
    } else {
      const int w = round * slots + pos;
      item = w / n_heads;
      h = w - item * n_heads;
    }
  };

  // kFused: the workgroup's unit descriptors (q_tile | kind << 16, row_start,
  // length, head | split rank of part 0 << 16), negative past its last round;
  // shared by the waves, or one copy per wave when each wave orders the users.
  // kind: 0 the whole item, 1 / 2 its first / second key-range part, 3 nothing
  // (a first part whose item runs whole as the second).
  __shared__ i32x4 s_desc[kFused ? kWaves * kDescRounds : 1];
  int desc_base = 0;  // this wave's descriptors: s_desc[desc_base + round]
  __shared__ int s_arrived;
  int nitems = 0, qt_max = 0;
  if constexpr (kFused) {
    // The unit list: users grouped by length class, classes descending, users
    // ascending inside a class (the same order as the scheduler kernel); a
    // user's units adjacent (the two parts of each split item, then its whole
    // items, q-tiles descending).  A user's first unit is the units of all
    // higher classes plus those of the users before it in its class.  The scans
    // sum whole items (low 15 bits) and the units with split items (high 17 bits)
    // at once; which list runs is decided from the totals, and twice the
    // difference of the two prefixes counts the split parts before a user (the
    // split rank that names a part's pool slot).  The unit of round r is found by
    // the lane whose range holds it.
    const int lane = L.lane;
    const int nusers = max_tiles > 0 ? U : 0;
    const int total = nusers > 0 ? cu[nusers] : 0;
    // At most 64 users: every wave orders them by itself (a user per lane), with
    // no LDS exchange and no barrier, and keeps its own copy of the descriptors.
    // Otherwise one user per thread, per-wave class sums through LDS.
    const bool one_wave = nusers <= 64;
    const int me = one_wave ? lane : threadIdx.x;  // this thread's user
    Seg sg{0, 0, 0};
    if (me < nusers) sg = segment_of(cu, cu, false, me, total, max_tiles);
    const int t = sg.tiles;
    const int cl = t > 0 ? length_class(t) : -1;
    SplitUser spl = split_user(t, sp.p > 1, sp.min_width);
    const int packed = t | ((t + spl.split) << 15);
    int both = 0, n_both = 0;
    if (one_wave) {
      // Classes in descending order: the running total is the next class's base.
      for (int c = kClasses - 1; c >= 0; --c) {
        const bool mine = cl == c;
        if (__ballot(mine) == 0) continue;  // uniform
        const int x = mine ? packed : 0;
        const int incl = wave_inclusive_sum(x);
        if (mine) both = n_both + incl - x;
        n_both += __builtin_amdgcn_readlane(incl, 63);
      }
    } else {
      LDS int* const s_wsum = (LDS int*)st0;  // [kWaves][kClasses]
      const int wid = L.wid;
      if (lane < kClasses) s_wsum[wid * kClasses + lane] = 0;
      int pre = 0;
      unsigned long long pending = __ballot(t > 0);
      while (pending) {
        const int lc = __builtin_amdgcn_readlane(cl, __builtin_ctzll(pending));
        const bool mine = cl == lc;
        const int x = mine ? packed : 0;
        const int incl = wave_inclusive_sum(x);
        if (mine) pre = incl - x;
        if (lane == 63) s_wsum[wid * kClasses + lc] = incl;
        pending &= ~__ballot(mine);
      }
      lds_barrier();
      // Class totals and bases (lane l handles class 12-l), the user's first slot.
      int tot = 0;
      if (lane < kClasses) {
#pragma unroll
        for (int w = 0; w < kWaves; ++w) tot += s_wsum[w * kClasses + kClasses - 1 - lane];
      }
      const int incl = wave_inclusive_sum(tot);
      n_both = __builtin_amdgcn_readlane(incl, kClasses - 1);
      const int base = incl - tot;  // first slot of class 12-lane
      // Every lane takes part in the permute (a lane reads the base of its class
      // from the lane that holds that class).
      const int cbase = __builtin_amdgcn_ds_bpermute(4 * (kClasses - 1 - (t > 0 ? cl : 0)), base);
      if (t > 0) {
        both = cbase + pre;
        for (int w = 0; w < wid; ++w) both += s_wsum[w * kClasses + cl];
      }
    }
    const int n_whole = n_both & 0x7fff, n_split = n_both >> 15;
    // Split only when every unit of the split list gets a workgroup of its own:
    // then all parts start at once and none waits for a second round.
    const bool split = n_split > n_whole && n_split <= sp.upr;
    const int n = split ? n_split : n_whole;
    if (!split) spl = SplitUser{0, 0};
    const int su = t + spl.split;  // work units of this user
    {  // a workgroup past the last item (the grid may exceed the work) leaves now
      int item0, h0;
      work_of(0, item0, h0);
      if (item0 >= n) return;  // uniform across the workgroup
    }
    // The user's first unit, and the split rank of its first split part (two per
    // split item of the users before it).
    const int off = split ? both >> 15 : both & 0x7fff;
    const int roff = 2 * ((both >> 15) - (both & 0x7fff));
    // Units of later rounds lie further down the list, so the first round past
    // the end closes the descriptors.  (The list without split items has its own
    // copy of the loop: it is on every batch's critical path.)
    LDS i32x4* const desc = (LDS i32x4*)s_desc + (one_wave ? L.wid * kDescRounds : 0);
    const bool writer = one_wave ? lane == 0 : threadIdx.x == 0;
    auto fill = [&](auto with_split) {
      for (int r = 0; r < kDescRounds; ++r) {
        int item, h;
        work_of(r, item, h);
        if (item >= n) {
          if (writer) desc[r] = i32x4{-1, 0, 0, 0};
          break;
        }
        if (t > 0 && item >= off && item < off + su) {
          const int i = item - off;
          if constexpr (decltype(with_split)::value) {
            int nk, k, p;
            unit_of(t, spl, i, nk, k, p);
            int kind = 0, rank0 = 0;
            if (p > 1) {
              const int r0 = roff + i - k;  // split ranks r0, r0+1
              if (r0 + 2 <= sp.cap) {
                kind = 1 + k;
                rank0 = r0;
              } else if (k == 0) {
                kind = 3;  // pool full: the second part runs the whole item, the first nothing
              }
            }
            desc[r] = i32x4{(nk - 1) | (kind << 16), sg.start, sg.len, h | (rank0 << 16)};
          } else {
            desc[r] = i32x4{t - 1 - i, sg.start, sg.len, h};
          }
        }
      }
    };
    if (split)
      fill(std::true_type{});
    else
      fill(std::false_type{});
    if (one_wave) {
      // The descriptors came from lanes of this wave: wait for the writes.
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
      __builtin_amdgcn_wave_barrier();
    } else {
      lds_barrier();  // descriptors visible; the ring is free again
    }
    desc_base = one_wave ? L.wid * kDescRounds : 0;
  } else {
    nitems = *count;
    qt_max = nitems > 0 ? items[0].y & 0xffff : 0;  // the first unit is of a longest user's last q-tile
  }
  // Dynamic assignment (worklist path with work counters): instead of the fixed
  // snake, a workgroup takes the next unclaimed item from a counter in global
  // memory, so workgroups that drew short items take more of them.  With one
  // head per workgroup (by_head, H <= kQueues) each head has its own counter and
  // items are taken in list order (users kept together, so later q-tiles find
  // the user's K/V in the L2 of the XCD serving that head); otherwise one counter
  // runs over all (item, head) pairs, heads fastest.  Thread 0 claims the next
  // item while the current one runs; LDS passes it to all waves at the item's
  // last barrier.
  const bool dyn = !kFused && queue != nullptr;
  const bool per_head = by_head && n_heads <= kQueues;
  int32_t* const qctr = dyn ? queue + (per_head ? head0 : 0) * kQueueStride : nullptr;
  __shared__ int s_next;
  int claimed = 0;
  if (dyn) {
    if (threadIdx.x == 0) s_next = __hip_atomic_fetch_add(qctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    lds_barrier();
  }
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
      if (kind == 3) continue;  // its item runs whole as the second part
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
        const int w = __builtin_amdgcn_readfirstlane(s_next);
        if (per_head) {
          item = w;
          h = head0;
        } else {
          item = w / n_heads;
          h = w - item * n_heads;
        }
        if (item >= nitems) break;
        if (threadIdx.x == 0) claimed = __hip_atomic_fetch_add(qctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
        if (kind == 3) {  // its item runs whole as the second part
          if (dyn) {      // pass the claim on once every wave has read s_next
            lds_barrier();
            if (threadIdx.x == 0) s_next = claimed;
            lds_barrier();
          }
          continue;
        }
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
    // tile of a first part goes through the same masked step with nothing masked.
    const int mlim = (!kSplit || khi == qt + 1) ? L.qr : kTileRows - 1;
    int j = klo;
    for (; j + 2 < khi; j += 2) {
      wait_and_barrier<0>();
      issue_tile(kStageBytes, j + 1);
      tile_step<false>(st0, L, qf, ones, sl2, rescale_thr, A);
      wait_and_barrier<0>();
      issue_tile(0, j + 2);
      tile_step<false>(st1, L, qf, ones, sl2, rescale_thr, A);
    }
    if (j + 1 < khi) {  // two tiles left: j in stage 0, the last one goes to stage 1
      wait_and_barrier<0>();
      issue_tile(kStageBytes, j + 1);
      tile_step<false>(st0, L, qf, ones, sl2, rescale_thr, A);
      wait_and_barrier<0>();
      tile_step<true>(st1, L, qf, ones, sl2, rescale_thr, A, mlim);
    } else {  // one tile left, in stage 0
      wait_and_barrier<0>();
      tile_step<true>(st0, L, qf, ones, sl2, rescale_thr, A, mlim);
    }
    // The claim made at the item's start is passed on; every wave read s_next
    // before this item's first barrier.
    if (dyn && threadIdx.x == 0) s_next = claimed;
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
      merge_parts(slot0, slot_stride, parts, part, L, sl2, A);
    }

    {
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
      int layer_log2, float sl2, SplitArgs sp, uint16_t *__restrict__ out
#define VLCA_ATTENTION_ARGS qkv, items, count, queue, cu, U, max_tiles, n_heads, layer_log2, sl2, sp, out

// Four workgroups per CU (128 VGPRs a lane) is the occupancy the tile step is
// tuned for.  The split-capable worklist instance needs the occupancy bound to
// stay there (129 VGPRs without it); on the other instances, which fit anyway,
// the bound made the compiler schedule the tile step worse (the 25523-token
// batch 8% slower), so they do without.
template <bool kFused, bool kSplit>
__global__ __launch_bounds__(kAttnThreads) void attention_kernel(VLCA_ATTENTION_PARAMS) {
  attention_body<kFused, kSplit>(VLCA_ATTENTION_ARGS);
}

template <>
__global__ __launch_bounds__(kAttnThreads, 4) void attention_kernel<false, true>(VLCA_ATTENTION_PARAMS) {
  attention_body<false, true>(VLCA_ATTENTION_ARGS);
}

#undef VLCA_ATTENTION_ARGS
#undef VLCA_ATTENTION_PARAMS

}  // namespace

hipError_t launch_schedule(const int32_t* cu_seqlens, int num_users, int max_tiles, int4* items, int32_t* count,
                           int32_t* queue, const SplitArgs& split, hipStream_t stream) {
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, cu_seqlens, num_users, max_tiles,
                     items, count, queue, split);
  return hipGetLastError();
}

hipError_t launch_attention(const void* qkv, const int4* items, const int32_t* count, int32_t* queue, int n_heads,
                            float scale_log2e, const SplitArgs& split, void* out, int grid, int layer_log2,
                            hipStream_t stream) {
  if (split.p > 1)
    hipLaunchKernelGGL((attention_kernel<false, true>), dim3(grid), dim3(kAttnThreads), 0, stream,
                       static_cast<const uint16_t*>(qkv), items, count, queue, nullptr, 0, 0, n_heads, layer_log2,
                       scale_log2e, split, static_cast<uint16_t*>(out));
  else
    hipLaunchKernelGGL((attention_kernel<false, false>), dim3(grid), dim3(kAttnThreads), 0, stream,
                       static_cast<const uint16_t*>(qkv), items, count, queue, nullptr, 0, 0, n_heads, layer_log2,
                       scale_log2e, split, static_cast<uint16_t*>(out));
  return hipGetLastError();
}

hipError_t launch_attention_fused(const void* qkv, const int32_t* cu_seqlens, int num_users, int max_tiles,
                                  int n_heads, float scale_log2e, const SplitArgs& split, void* out, int grid,
                                  int layer_log2, hipStream_t stream) {
  hipLaunchKernelGGL((attention_kernel<true, true>), dim3(grid), dim3(kAttnThreads), 0, stream,
                     static_cast<const uint16_t*>(qkv), nullptr, nullptr, nullptr, cu_seqlens, num_users, max_tiles,
                     n_heads, layer_log2, scale_log2e, split, static_cast<uint16_t*>(out));
  return hipGetLastError();
}

bool fused_fits(int64_t num_users, int64_t max_tiles, int64_t n_heads, int64_t grid) {
  if (num_users > kFusedUsers || grid <= 0) return false;
  // The prologue's scans carry the item count in 15 bits (and up to twice it in 17).
  if (num_users * max_tiles > 32767) return false;
  // rounds = ceil(items * H / grid) when the grid is a multiple of H; items <= users x max q-tiles
  return num_users * max_tiles * n_heads <= static_cast<int64_t>(kFusedRounds) * grid;
}

int attention_blocks_per_cu(bool fused) {
  int n = 0;
  const hipError_t e =
      fused ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attention_kernel<true, true>, kAttnThreads, 0)
            : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, attention_kernel<false, false>, kAttnThreads, 0);
  if (e != hipSuccess || n < 1) n = 1;
  return n;
}

}  // namespace vlca
