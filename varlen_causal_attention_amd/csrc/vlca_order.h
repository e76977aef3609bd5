// Ordering of (user, q-tile) work in the order every attention plan shares,
// and the fixed assignment of that work to a persistent grid: the helpers of the
// scheduler kernel (vlca_kernels.hip) and the in-kernel ordering with which a
// workgroup of a single-kernel plan (causal forward, masked forward) locates its
// own units from cu_seqlens.  Internal; included by HIP sources only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "vlca_device.h"
#include "vlca_internal.h"

namespace vlca {
namespace {

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

// The launch condition of the single-kernel plan counts whole items
// (kFusedRounds rounds); key-range splitting turns an item into at most
// kMaxSplitParts work units, so the descriptors hold that many more.
static_assert(kFusedUsers == kAttnThreads, "the shared-list ordering takes one user per thread");
constexpr int kDescRounds = kFusedRounds * kMaxSplitParts;

// The fixed assignment of the list's units to a persistent grid.  With the grid
// a multiple of H, workgroup g always runs head g % H (with H = 8 that is the
// XCD it sits on) and item slot g / H of each round; rounds alternate direction
// (snake), so the workgroups that drew the longest items of round 0 draw the
// shortest of round 1.
//
// When all the work fits in one round, the workgroups that share a CU
// (g, g + CUs, g + 2 CUs, ... in launch order) hold slots `layer` apart, and
// the snake runs across them instead: odd layers take their ranks in reverse,
// so the sums of the items on each CU come out even rather than the first CUs
// drawing the longest item of every layer.  With more rounds the plain snake
// is kept: it leaves the second round's items to the CUs of the shortest
// first-round items, away from the longest ones.  (Every round after the first
// is then empty, so the layered rank can stand in for the slot in every round.)
// The launch passes layer_log2 >= 0 only when the work fits in one round and
// `layer` is a power of two.
struct Snake {
  bool by_head;
  int n_heads, slots, slot, head0, rank;
  __device__ Snake(int heads, int layer_log2) : n_heads(heads) {
    const int G = gridDim.x;
    by_head = G % n_heads == 0;
    slots = by_head ? G / n_heads : G;
    slot = by_head ? blockIdx.x / n_heads : blockIdx.x;
    head0 = by_head ? blockIdx.x - slot * n_heads : 0;
    rank = slot;
    if (layer_log2 >= 0) {
      const int layer = 1 << layer_log2;
      const int lyr = slot >> layer_log2, lyr_pos = slot & (layer - 1);
      const int lyr_len = min(layer, slots - (lyr << layer_log2));
      rank = slot - lyr_pos + ((lyr & 1) ? lyr_len - 1 - lyr_pos : lyr_pos);
    }
  }
  // The item and head of this workgroup's unit of round `round`.
  __device__ void unit(int round, int& item, int& h) const {
    const int pos = (round & 1) ? slots - 1 - rank : rank;
    if (by_head) {
      item = round * slots + pos;
      h = head0;
    } else {
      const int w = round * slots + pos;
      item = w / n_heads;
      h = w - item * n_heads;
    }
  }
};

// Single-kernel plan: this workgroup locates its own work units of every round
// (at most kDescRounds) from cu_seqlens and writes their descriptors to LDS:
// (q_tile | kind << 16, row_start, length, head | split rank of part 0 << 16)
// -- with kUser (no splitting) head | user << 16 -- negative past its last
// round; kind 0 is a whole item, 1 / 2 its first / second key-range part.  The
// descriptors (kDescRounds of them) are shared by the waves; desc_base is 0.
// `scratch` (at least kWaves * kClasses ints of LDS) is free again on return.
// Returns false, for every thread of the workgroup, when the workgroup has no
// unit.
template <bool kUser, typename WorkOf>
__device__ __forceinline__ bool own_units(const int32_t* __restrict__ cu, int U, int max_tiles, const SplitArgs& sp,
                                          const Lanes& L, LDS char* scratch, LDS i32x4* s_desc,
                                          const WorkOf& work_of, int& desc_base) {
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
  // At most 64 users: one wave of the workgroup orders them (a user per lane)
  // and writes the shared descriptors; the other waves wait at the one barrier.
  // The ordering wave is 0..3 by the workgroup's layer on its CU (workgroups g,
  // g + 256, ... share a CU on a 256-CU device), so the co-resident workgroups'
  // ordering waves do not all share one SIMD.  Otherwise one user per thread,
  // per-wave class sums through LDS.
  const bool one_wave = nusers <= 64;
  if (one_wave && __builtin_amdgcn_readfirstlane(L.wid) != ((blockIdx.x >> 8) & (kWaves - 1))) {
    lds_barrier();
    desc_base = 0;
    return __builtin_amdgcn_readfirstlane(s_desc[0][0]) >= 0;
  }
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
    LDS int* const s_wsum = (LDS int*)scratch;  // [kWaves][kClasses]
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
    if (item0 >= n && !one_wave) return false;  // uniform (one wave: the descriptors say so)
  }
  // The user's first unit, and the split rank of its first split part (two per
  // split item of the users before it).
  const int off = split ? both >> 15 : both & 0x7fff;
  const int roff = 2 * ((both >> 15) - (both & 0x7fff));
  // Units of later rounds lie further down the list, so the first round past
  // the end closes the descriptors.  (The list without split items has its own
  // copy of the loop: it is on every batch's critical path.)
  LDS i32x4* const desc = s_desc;
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
          const int kind = p > 1 ? 1 + k : 0;
          const int rank0 = p > 1 ? roff + i - k : 0;  // split ranks rank0, rank0 + 1
          desc[r] = i32x4{(nk - 1) | (kind << 16), sg.start, sg.len, h | (rank0 << 16)};
        } else {
          desc[r] = i32x4{t - 1 - i, sg.start, sg.len, kUser ? h | (me << 16) : h};
        }
      }
    }
  };
  if (split)
    fill(std::true_type{});
  else
    fill(std::false_type{});
  lds_barrier();  // descriptors visible to every wave; the ring is free again
  desc_base = 0;
  return !one_wave || __builtin_amdgcn_readfirstlane(s_desc[0][0]) >= 0;
}

}  // namespace
}  // namespace vlca
