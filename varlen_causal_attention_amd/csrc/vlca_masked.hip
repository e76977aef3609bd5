// gfx950 forward of varlen attention with the HSTU-style mask variants.
//
// The recsys README (github.com/cry-daniel/recsys), HSTU section, lists the
// masks its varlen attention takes beside the plain causal one: no mask, a local
// (sliding-window) mask given as window_size = (left, right) with (-1, 0) the
// causal default, and per-user contextual and target tokens, the sequence being
// [contextual tokens][history][candidate tokens] with the contextual part
// attended bidirectionally, the history causally and the candidates in groups
// of target_group_size.  Per user of length L with c context and g candidate
// tokens (nc = L - g), query row i sees key j when
//   causal (right = 0):
//     j < c                                   (context keys: every row)
//     i >= c and max(c, lo(i)) <= j <= min(i, nc - 1)   (history, windowed)
//     i >= nc and gs(i) <= j <= i             (its own candidate group)
//   otherwise (c = g = 0): lo(i) <= j <= hi(i)
// with lo(i) = i - left (left >= 0) else 0, hi(i) = i + right (right >= 0) else
// L - 1, gs(i) = nc + floor((i - nc) / G) G.  Softmax over the visible keys as in
// the causal forward.
//
// Same layout as the causal forward (vlca_kernels.hip): a persistent grid over
// the scheduler's (user, q-tile) items, claimed per head; K/V tiles by LDS DMA
// through a two-stage ring; S^T = K Q^T and O^T += V^T P^T on bf16 MFMA.  An
// item visits the key tiles holding context keys, then the tiles from the
// smallest visible history key of its rows to its last row (or, without causal
// order, the union of its rows' windows).  A tile that every row of the item
// sees whole takes the unmasked step; the others a step that tests each key
// against the row's three intervals.  Rows may see no key of a tile (a window,
// a candidate group), so the online softmax runs in its NaN-safe form.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "vlca_device.h"
#include "vlca_internal.h"
#include "vlca_order.h"

namespace vlca {
namespace {

// The key intervals a lane's query sees, relative to a tile's first key: [0, a)
// (context), [bl, bh] (history or window) and [cl, ch] (own candidate group).
// Each interval test is one unsigned compare of k - lo against hi - lo (an empty
// interval has hi - lo = -1, which no k - lo reaches... as unsigned it would be
// the largest value, so empty intervals are given lo past every key instead).
// kCtx / kCand: whether the context / candidate interval can meet this tile for
// some row of the item (uniform per tile); the history interval always can.
template <bool kCtx, bool kCand>
struct IntervalMask {
  static constexpr bool kAny = true;
  int a, bl, bspan, cl, cspan, g;  // spans: hi - lo as unsigned
  bool full;                       // wave-uniform: every row of the item sees the whole tile
  __device__ bool all() const { return full; }
  __device__ bool operator()(int b, int r) const {
    const int k = 16 * b + 4 * g + r;
    bool v = (uint32_t)(k - bl) <= (uint32_t)bspan;
    if constexpr (kCtx) v = v || k < a;
    if constexpr (kCand) v = v || (uint32_t)(k - cl) <= (uint32_t)cspan;
    return v;
  }
};

// An interval [lo, hi] of a user's keys as (start, span) for IntervalMask: an
// empty interval starts at 1 << 20, past every key of any tile (keys are below
// 2^18), with span 0.
__device__ __forceinline__ void as_span(int lo, int hi, int& start, int& span) {
  const bool empty = lo > hi;
  start = empty ? (1 << 20) : lo;
  span = empty ? 0 : hi - lo;
}

// kFused = false: the items of the scheduler's worklist (items, count), claimed
// per head after two rounds of the snake.  kFused = true (single-kernel plan,
// the causal forward's condition): every workgroup locates its own items of the
// same list from cu_seqlens (own_units, vlca_order.h) and takes them in the
// fixed snake (layered when layer_log2 >= 0).
template <bool kFused>
__global__ __launch_bounds__(kAttnThreads, 4) void masked_attention_kernel(
    const uint16_t* __restrict__ qkv, const int4* __restrict__ items, const int32_t* __restrict__ count,
    int32_t* __restrict__ queue, const int32_t* __restrict__ cu, int U, int max_tiles, int layer_log2, int n_heads,
    float sl2, const int32_t* __restrict__ num_contexts, const int32_t* __restrict__ num_targets, int group, int wl,
    int wr, uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) char ring_lds[2 * kStageBytes];
  LDS char* const st0 = (LDS char*)ring_lds;
  LDS char* const st1 = st0 + kStageBytes;
  const int64_t ldq = 3 * n_heads * kHeadDim;
  const int64_t ldo = n_heads * kHeadDim;
  const int hd = n_heads * kHeadDim;
  Lanes L;
  make_lanes(L, ldq);
  const float rescale_thr = kRescaleLog2 / sl2;
  bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
  asm volatile("" : "+v"(ones));
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(st0 + 2048 * L.wid));
  const bool causal = wr == 0;

  // The workgroup's own items (single-kernel plan): descriptors (q_tile,
  // row_start, length, head | user << 16), negative past its last round; until
  // they are known the workgroup runs at the highest wave priority, so that
  // co-resident workgroups already inside items do not starve the ordering.
  __shared__ i32x4 s_desc[kFused ? kDescRounds : 1];
  int desc_base = 0;
  if constexpr (kFused) {
    __builtin_amdgcn_s_setprio(3);
    const Snake sn(n_heads, layer_log2);
    auto work_of = [&](int round, int& item, int& h) { sn.unit(round, item, h); };
    if (!own_units<true>(cu, U, max_tiles, SplitArgs{0, 0, 0, nullptr, nullptr}, L, st0, (LDS i32x4*)s_desc,
                         work_of, desc_base))
      return;
    __builtin_amdgcn_s_setprio(0);
  }

  // Work units: with the grid a multiple of H (and H <= kQueues), head g % H,
  // units counted per head; else units over (item, head) pairs.  The first two
  // rounds follow the snake over the list; later items are claimed from counter
  // g % H (or the one counter), the claim made while the second-round and later
  // items run.  No claim precedes the first items: every workgroup claiming at
  // the kernel's start serialises the atomics on each counter's line.
  const bool by_head = gridDim.x % n_heads == 0;
  const bool per_head = by_head && n_heads <= kQueues;
  const int head0 = by_head ? blockIdx.x % n_heads : 0;
  int32_t* const qctr = queue + (per_head ? head0 : 0) * kQueueStride;
  const int nslots = per_head ? gridDim.x / n_heads : gridDim.x;
  const int wfirst = per_head ? blockIdx.x / n_heads : blockIdx.x;
  const int nitems = kFused ? 0 : *count;
  __shared__ int s_next;
  for (int round = 0;; ++round) {
    int h, u, qt, start, len;
    int claimed = 0;
    if constexpr (kFused) {
      if (round >= kDescRounds) break;
      const i32x4 d = s_desc[desc_base + round];
      const int w0 = __builtin_amdgcn_readfirstlane(d[0]);
      if (w0 < 0) break;
      qt = w0 & 0xffff;
      start = __builtin_amdgcn_readfirstlane(d[1]);
      len = __builtin_amdgcn_readfirstlane(d[2]);
      const int w3 = __builtin_amdgcn_readfirstlane(d[3]);
      h = w3 & 0xffff;
      u = w3 >> 16;
    } else {
      const int w =
          round == 0 ? wfirst : round == 1 ? 2 * nslots - 1 - wfirst : __builtin_amdgcn_readfirstlane(s_next);
      int item;
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
      const int4 it = items[item];
      u = it.x;
      qt = it.y & 0xffff;
      start = it.z;
      len = it.w;
    }
    const int q0 = qt * kTileRows;
    const int lim = len - 1 - q0;
    // The user's mask geometry (clamped to its length).
    int c = 0, g = 0;
    if (causal) {
      if (num_contexts != nullptr) c = min(max(num_contexts[u], 0), len);
      if (num_targets != nullptr) g = min(max(num_targets[u], 0), len - c);
    }
    c = __builtin_amdgcn_readfirstlane(c);
    g = __builtin_amdgcn_readfirstlane(g);
    const int nc = len - g;
    const int r0 = q0, r1 = min(q0 + kTileRows - 1, len - 1);
    auto lo_of = [&](int i) { return wl >= 0 ? max(0, i - wl) : 0; };
    auto hi_of = [&](int i) { return wr >= 0 ? min(len - 1, i + wr) : len - 1; };
    // Key tiles: [0, n_ctx) then [t_lo, t_hi] (merged when they meet).
    int n_ctx = 0, t_lo, t_hi;
    if (causal) {
      n_ctx = (c + kTileRows - 1) / kTileRows;
      const int first_hist = max(r0, c);  // first row of the item that is not a context row
      if (first_hist <= r1) {
        // Lowest visible non-context key: the window start of the first such row,
        // or the group start of its first candidate row if that lies lower.
        int klo = max(c, lo_of(first_hist));
        if (r1 >= nc) {
          const int fc = max(r0, nc);
          klo = min(klo, nc + ((fc - nc) / group) * group);
        }
        t_lo = klo / kTileRows;
        t_hi = r1 / kTileRows;
      } else {  // context rows only: they see the context keys
        t_lo = n_ctx;
        t_hi = n_ctx - 1;
      }
      if (t_lo <= n_ctx) {  // contiguous: one range from 0
        t_hi = max(t_hi, n_ctx - 1);
        t_lo = 0;
        n_ctx = 0;
      }
    } else {
      t_lo = lo_of(r0) / kTileRows;
      t_hi = hi_of(r1) / kTileRows;
    }
    const int ntiles = n_ctx + max(t_hi - t_lo + 1, 0);
    auto tile_of = [&](int t) { return t < n_ctx ? t : t_lo + (t - n_ctx); };
    // A tile every row of the item sees whole.
    const int full_lo = lo_of(r1);
    const int full_hi = causal ? min(r0, nc - 1) : hi_of(r0);
    auto full_tile = [&](int k) {
      const int kf = k * kTileRows, kl = kf + kTileRows - 1;
      if (causal && kl < c) return true;
      return (!causal || r0 >= c) && kf >= full_lo && kl <= full_hi;
    };
    // This lane's query row (rows past the user's end take its last row) and its intervals.
    const int i = q0 + min(L.qr, lim);
    int a, bl, bh, cl = 1, ch = 0;
    if (causal) {
      a = c;
      if (i < c) {
        bl = 1;
        bh = 0;
      } else {
        bl = max(c, lo_of(i));
        bh = min(i, nc - 1);
      }
      if (i >= nc) {
        cl = nc + ((i - nc) / group) * group;
        ch = i;
      }
    } else {
      a = 0;
      bl = lo_of(i);
      bh = hi_of(i);
    }

    int bstart, bspan, cstart, cspan;
    as_span(bl, bh, bstart, bspan);
    as_span(cl, ch, cstart, cspan);

    const uint16_t* kg = qkv + (int64_t)start * ldq + hd + h * kHeadDim;
    const int64_t tstride = (int64_t)kTileRows * ldq;
    // Copies of key tile jj; rows past the user's end repeat its last row (a
    // tile wholly inside the user takes the precomputed offsets).
    auto issue_tile = [&](uint32_t so, int jj) {
      const uint16_t* kt = kg + jj * tstride;
      const uint16_t* vt = kt + hd;
      const int klim = len - 1 - jj * kTileRows;
      const bool inside = klim >= kTileRows - 1;  // uniform
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        uint32_t o = L.cofs_g[r];
        if (!inside) o = (uint32_t)(min(L.crow[r], klim) * ldq * 2 + 16 * ((L.lane & 7) ^ swz(L.crow[r])));
        copy_to_lds(kt, o, m0 + so + 1024 * r);
        copy_to_lds(vt, o, m0 + so + kTileBytes + 1024 * r);
      }
    };
    // Q rows through the wave's own rows of stage 1 (read back before stage 1 is refilled).
    {
      const uint16_t* qg = qkv + ((int64_t)start + q0) * ldq + h * kHeadDim;
#pragma unroll
      for (int r = 0; r < 2; ++r) {
        const int row = min(L.crow[r], lim);
        copy_to_lds(qg, (uint32_t)(row * ldq * 2 + 16 * ((L.lane & 7) ^ swz(L.crow[r]))),
                    m0 + kStageBytes + 1024 * r);
      }
    }
    issue_tile(0, tile_of(0));
    wait_vmem_lds<4>();
    bf16x8 qf[2];
    qf[0] = lds_b128(st1, L.qr * 128 + ((L.g ^ swz(L.qr)) << 4));
    qf[1] = lds_b128(st1, L.qr * 128 + (((4 + L.g) ^ swz(L.qr)) << 4));
    Acc A;
    A.m = -__builtin_inff();
    A.moff = 0.0f;
    A.mthr = -__builtin_inff();
    A.l = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = 0; d < 4; ++d) A.o[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    // One step for both kinds of tile (the mask is skipped on a tile every row
    // sees whole): two step instances left the accumulators in different
    // registers, copied back at every join.  Tile t sits in stage t % 2; the loop
    // is unrolled by two so that each stage's LDS addresses are fixed.
    auto step = [&](const LDS char* base, int t) {
      const int k = tile_of(t), k0 = k * kTileRows;
      tile_step<true>(base, L, qf, ones, sl2, rescale_thr, A,
                      IntervalMask<true, true>{a - k0, bstart - k0, bspan, cstart - k0, cspan, L.g, full_tile(k)});
    };
    // A wave whose 16 rows all lie past the user's end (the user's last q-tile)
    // computes nothing: it issues its share of the copies and meets the barriers,
    // in a second copy of the loop.
    auto tiles = [&](auto compute) {
      constexpr bool kOn = decltype(compute)::value;
      int t = 0;
      for (; t + 1 < ntiles; t += 2) {
        wait_and_barrier<0>();
        issue_tile(kStageBytes, tile_of(t + 1));
        if constexpr (kOn) step(st0, t);
        wait_and_barrier<0>();
        if (t + 2 < ntiles) issue_tile(0, tile_of(t + 2));
        if constexpr (kOn) step(st1, t + 1);
      }
      if (t < ntiles) {
        wait_and_barrier<0>();
        if constexpr (kOn) step(st0, t);
      }
    };
    if (__builtin_amdgcn_readfirstlane(16 * L.wid < len - q0))
      tiles(std::true_type{});
    else
      tiles(std::false_type{});
    if (!kFused && round >= 1 && threadIdx.x == 0) s_next = claimed;
    wait_and_barrier<0>();  // every wave is done with the ring; s_next is visible
    store_rows(st0 + 2048 * L.wid, A.o, 1.0f / A.l[0],
               out + ((int64_t)start + q0 + 16 * L.wid) * ldo + h * kHeadDim, ldo, len - q0 - 16 * L.wid);
  }
}

}  // namespace

hipError_t launch_masked_attention(const void* qkv, const int4* items, const int32_t* count, int32_t* queue,
                                   int n_heads, float scale_log2e, const int32_t* num_contexts,
                                   const int32_t* num_targets, int group, int window_left, int window_right,
                                   void* out, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(masked_attention_kernel<false>, dim3(grid), dim3(kAttnThreads), 0, stream,
                     static_cast<const uint16_t*>(qkv), items, count, queue, nullptr, 0, 0, -1, n_heads, scale_log2e,
                     num_contexts, num_targets, group, window_left, window_right, static_cast<uint16_t*>(out));
  return hipGetLastError();
}

hipError_t launch_masked_attention_fused(const void* qkv, const int32_t* cu_seqlens, int num_users, int max_tiles,
                                         int n_heads, float scale_log2e, const int32_t* num_contexts,
                                         const int32_t* num_targets, int group, int window_left, int window_right,
                                         void* out, int grid, int layer_log2, hipStream_t stream) {
  hipLaunchKernelGGL(masked_attention_kernel<true>, dim3(grid), dim3(kAttnThreads), 0, stream,
                     static_cast<const uint16_t*>(qkv), nullptr, nullptr, nullptr, cu_seqlens, num_users, max_tiles,
                     layer_log2, n_heads, scale_log2e, num_contexts, num_targets, group, window_left, window_right,
                     static_cast<uint16_t*>(out));
  return hipGetLastError();
}

int masked_blocks_per_cu(bool fused) {
  int n = 0;
  const hipError_t e =
      fused ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, masked_attention_kernel<true>, kAttnThreads, 0)
            : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, masked_attention_kernel<false>, kAttnThreads, 0);
  if (e != hipSuccess || n < 1) n = 1;
  return n;
}

}  // namespace vlca
