// gfx950 kernels of the backward pass of block-diagonal causal attention over
// packed variable-length users: given dO = dL/dout, the gradients dQ, dK, dV
// (the packed dqkv) of the forward's softmax(scale Q K^T + causal mask) V.
//
// With P the forward's softmax weights (recomputed from the row log-sum-exp the
// forward wrote), per user and head:
//   D_i  = sum_d dO_id O_id                 (= sum_j P_ij dP_ij)
//   dP   = dO V^T,  dS = P o (dP - D)
//   dV   = P^T dO,  dK = scale dS^T Q,  dQ = scale dS K.
// This is the FlashAttention-2 backward (recompute P tile by tile from the
// log-sum-exp; the attention backward of the recsys README's FusedHSTULayer
// listing), laid out for CDNA4:
//  * bwd_prepare_kernel (vlca_kernels.hip, run first, with the worklist): D
//    for every (row, head), and the row's -log-sum-exp log2(e), written as
//    fp32 into the first 8 bytes of that row's and head's dq columns of dqkv
//    (the dq kernel, which runs last, reads them there before overwriting
//    those columns), so the backward needs no scratch memory;
//  * bwd_dkdv_kernel: one item per (user, key tile, head); the wave's 16 key
//    rows of K and V stay in registers as MFMA B operands while the user's
//    query tiles from the key tile to the last stream through a two-stage LDS
//    ring (Q tile, dO tile, and the tile's log-sum-exp and D values, all by
//    LDS DMA); S = Q K^T and dP = dO V^T are formed with queries as rows, so P
//    and dS come out of the MFMA in the B-operand layout of dV^T += dO^T P and
//    dK^T += Q^T dS, whose A operands are read transposed from the staged
//    tiles with ds_read_b64_tr_b16 (as the forward reads V^T);
//  * bwd_dq_kernel: one item per (user, query tile, head), shaped like the
//    forward: the wave's 16 query rows of Q and dO in registers, key tiles 0 ..
//    the diagonal streaming through the ring, S^T = K Q^T and dP^T = V dO^T,
//    dQ^T += K^T dS^T.
// No atomic accumulation: every gradient element is produced by one
// workgroup, so the result is deterministic (atomics only hand out items).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "vlca_device.h"
#include "vlca_internal.h"

namespace vlca {
namespace {

constexpr float kLog2eF = 1.4426950408889634f;
// One ring stage of the dK/dV kernel: Q tile, dO tile, then 64 log-sum-exp and
// 64 D values of the query tile.
constexpr int kBwdStatsBytes = 2 * kTileRows * 4;
constexpr int kBwdStageBytes = 2 * kTileBytes + kBwdStatsBytes;

// 4-byte LDS DMA: lane l copies the dword at base + voff to LDS address m + 4 l.
__device__ __forceinline__ void copy_dword_to_lds(const void* base, uint32_t voff, uint32_t m) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)base);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)((uintptr_t)base >> 32));
  const uint64_t sbase = (uint64_t)lo | ((uint64_t)hi << 32);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dword %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m), "v"(voff), "s"(sbase)
      : "memory");
}

// Work assignment, in list order (longest users first, each user's items
// together).  With the grid a multiple of H and H <= kQueues, workgroup g always
// runs head g % H (with H = 8, the XCD it sits on) and takes slot g / H of the
// list's first two rounds of items, in a snake (the workgroups of the longest
// first-round items take the shortest second-round ones); later items are
// claimed from that head's zeroed counter in global memory, so a user's items
// run side by side where its rows are in L2.  Otherwise work unit w runs over all
// (item, head) pairs, heads fastest, with the same two rounds and one counter.
// Thread 0 claims the next item while the second-round and later items run and
// hands it over through LDS at the item's last barrier.  No claim is made at the
// kernel's start: every workgroup claiming at once serialises the atomics on the
// counter's line, and batches of one or two rounds need none.
struct Claim {
  int32_t* ctr;
  int head0, n_heads;
  int w0, w1;  // the workgroup's work units in the first two rounds
  int wbase;   // work unit of claim 0
  bool per_head;
  __device__ void init(int32_t* queue, int nh) {
    n_heads = nh;
    per_head = gridDim.x % nh == 0 && nh <= kQueues;
    const int slots = per_head ? gridDim.x / nh : gridDim.x;
    head0 = per_head ? blockIdx.x % nh : 0;
    w0 = per_head ? blockIdx.x / nh : blockIdx.x;
    w1 = 2 * slots - 1 - w0;
    wbase = 2 * slots;
    ctr = queue + head0 * kQueueStride;
  }
  // The work unit of the next claim.
  __device__ int next() const {
    return wbase + __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __device__ void decode(int w, int& item, int& h) const {
    if (per_head) {
      item = w;
      h = head0;
    } else {
      item = w / n_heads;
      h = w - item * n_heads;
    }
  }
};

// ------------------------------------------------------------- dK, dV

// One query tile of a dK/dV item.  base: the stage (Q tile, dO tile, the query
// rows' -log-sum-exp log2(e), D).  kMask: the diagonal tile (query q sees key k iff
// q >= k) and/or the user's last query tile (rows q >= qvalid do not exist).
template <bool kMask>
__device__ __forceinline__ void dkdv_step(const LDS char* base, const Lanes& L, const bf16x8 (&kf)[2],
                                          const bf16x8 (&vf)[2], float sl2, f32x4 (&dk)[4], f32x4 (&dv)[4],
                                          bool diag = false, int qvalid = kTileRows) {
  // S = Q K^T and dP = dO V^T, queries as rows, one half of 32 queries at a
  // time: block b holds queries 16 b .. 16 b + 15; lane (g, lq) gets queries
  // 16 b + 4 g + r of the wave's key lq.
  const int key = 16 * L.wid + L.lq;  // this lane's key inside the tile
  // Visible queries of this lane's key: qlo <= q < qvalid, with qlo = key on the
  // diagonal tile and 0 elsewhere; tested as one unsigned compare of q - qlo
  // against the span (0 when no query is visible).  The mask is applied only on
  // the tiles that need it (a uniform branch), and only to P: dS = P (dP - D)
  // is then exactly 0 as well, dP - D being finite.
  const bool masked_tile = kMask && (diag || qvalid < kTileRows);
  const int qlo = diag ? key : 0;
  const uint32_t qspan = (uint32_t)max(qvalid - qlo, 0);
  // On the diagonal tile the queries of half hh all precede this wave's keys
  // when 32 hh + 31 < 16 w: the half weighs nothing and is skipped (uniform).
  const int wu = __builtin_amdgcn_readfirstlane(L.wid);
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    if (kMask && diag && 2 * hh + 1 < wu) continue;
    f32x4 s[2], dp[2];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int b = 2 * hh + half;
      const bf16x8 q0 = lds_b128(base, L.kofs[0] + 2048 * b);
      const bf16x8 q1 = lds_b128(base, L.kofs[1] + 2048 * b);
      s[half] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q0, kf[0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      s[half] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(q1, kf[1], s[half], 0, 0, 0);
      const bf16x8 o0 = lds_b128(base, kTileBytes + L.kofs[0] + 2048 * b);
      const bf16x8 o1 = lds_b128(base, kTileBytes + L.kofs[1] + 2048 * b);
      dp[half] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o0, vf[0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      dp[half] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(o1, vf[1], dp[half], 0, 0, 0);
    }
    uint32_t pw[4], dw[4];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int b = 2 * hh + half;
      const int q4 = 16 * b + 4 * L.g;  // first of this lane's four queries in block b
      const f32x4 nl = *(const LDS f32x4*)(base + 2 * kTileBytes + 4 * q4);  // -lse log2(e)
      const f32x4 dd = *(const LDS f32x4*)(base + 2 * kTileBytes + 4 * kTileRows + 4 * q4);
      float p[4], ds[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) p[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[half][r], sl2, nl[r]));
      if (masked_tile) {
        // The query indices are formed here, on the masked tiles only: the lane
        // group passes through an empty asm so that they are not hoisted out of
        // the item loop and held in registers across it.
        int g = L.g;
        asm volatile("" : "+v"(g));
        const int qm = 16 * b + 4 * g - qlo;
#pragma unroll
        for (int r = 0; r < 4; ++r) p[r] = (uint32_t)(qm + r) < qspan ? p[r] : 0.f;
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) ds[r] = p[r] * (dp[half][r] - dd[r]);
      // B-operand slots of this half of 32 queries: 0..3 = block 2hh, 4..7 = block 2hh + 1.
      pw[2 * half] = pack_bf16x2(p[0], p[1]);
      pw[2 * half + 1] = pack_bf16x2(p[2], p[3]);
      dw[2 * half] = pack_bf16x2(ds[0], ds[1]);
      dw[2 * half + 1] = pack_bf16x2(ds[2], ds[3]);
    }
    const bf16x8 pb = __builtin_bit_cast(bf16x8, uint4{pw[0], pw[1], pw[2], pw[3]});
    const bf16x8 db = __builtin_bit_cast(bf16x8, uint4{dw[0], dw[1], dw[2], dw[3]});
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      // dO^T and Q^T fragments for queries 32 hh .. 32 hh + 31 in the slot order.
      const bf16x4 olo = lds_tr16(base, L.vofs[d] + 4096 * hh);
      const bf16x4 ohi = lds_tr16(base, L.vofs[d] + 4096 * hh + 2048);
      dv[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_shufflevector(olo, ohi, 0, 1, 2, 3, 4, 5, 6, 7), pb,
                                                      dv[d], 0, 0, 0);
      const bf16x4 qlo = lds_tr16(base, L.vofs[d] - kTileBytes + 4096 * hh);
      const bf16x4 qhi = lds_tr16(base, L.vofs[d] - kTileBytes + 4096 * hh + 2048);
      dk[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7), db,
                                                      dk[d], 0, 0, 0);
    }
  }
}

// items: the scheduler's (user, q_tile, row_start, length) list; item i stands
// for key tile kt = tiles - 1 - q_tile of its user, which needs q_tile + 1 query
// tiles (the list's longest-first order carries over).
__global__ __launch_bounds__(kAttnThreads) void bwd_dkdv_kernel(const uint16_t* __restrict__ qkv,
                                                                const uint16_t* __restrict__ dout,
                                                                const float* __restrict__ lse,
                                                                const int4* __restrict__ items,
                                                                const int32_t* __restrict__ count,
                                                                int32_t* __restrict__ queue, int n_heads,
                                                                float scale, uint16_t* __restrict__ dqkv) {
  __shared__ __attribute__((aligned(1024))) char ring_lds[2 * kBwdStageBytes];
  __shared__ int s_next;
  LDS char* const st0 = (LDS char*)ring_lds;
  LDS char* const st1 = st0 + kBwdStageBytes;
  const int64_t ldq = 3 * n_heads * kHeadDim;
  const int64_t ldo = n_heads * kHeadDim;
  const int hd = n_heads * kHeadDim;
  const float sl2 = scale * kLog2eF;
  Lanes L;
  make_lanes(L, ldq);
  Claim cl;
  cl.init(queue, n_heads);
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(st0 + 2048 * L.wid));
  const uint32_t m0s = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(st0 + 2 * kTileBytes));
  // Unclamped copy offsets of this lane: dO rows (stride ldo; Q rows use
  // L.cofs_g, stride ldq) and the lane's row of the per-row values (stride ldq).
  uint32_t ocofs[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) ocofs[i] = (uint32_t)(L.crow[i] * ldo * 2 + 16 * ((L.lane & 7) ^ swz(L.crow[i])));
  const uint32_t lane_row_ofs = (uint32_t)(L.lane * ldq * 2);
  const int nitems = *count;
  int claimed = 0;
  for (int round = 0, w = cl.w0;; ++round, w = round == 1 ? cl.w1 : __builtin_amdgcn_readfirstlane(s_next)) {
    int item, h;
    cl.decode(w, item, h);
    if (item >= nitems) break;
    if (round >= 1 && threadIdx.x == 0) claimed = cl.next();
    const int4 it = items[item];
    const int start = it.z, len = it.w;
    const int tiles = (len + kTileRows - 1) / kTileRows;
    const int kt = tiles - 1 - (it.y & 0xffff);
    const int k0 = kt * kTileRows;
    const int last = tiles - 1;
    const int64_t tstride = (int64_t)kTileRows * ldq;
    const uint16_t* qg = qkv + (int64_t)start * ldq + h * kHeadDim;  // Q of the user's row 0, head h
    const uint16_t* og = dout + (int64_t)start * ldo + h * kHeadDim;
    // This wave's copies of query tile jj into the stage at M0 offset so: Q rows,
    // dO rows (rows past the user's end repeat its last row), and, from waves 0
    // and 1, the 64 rows' -log-sum-exp log2(e) and D.  Only the user's last
    // query tile clamps rows; the others take the offsets formed once below.
    auto issue_tile = [&](uint32_t so, int jj) {
      const uint16_t* const qt_g = qg + (int64_t)jj * tstride;
      const uint16_t* const ot_g = og + (int64_t)jj * kTileRows * ldo;
      const int64_t row0 = (int64_t)start + jj * kTileRows;
      uint32_t qo[2], oo[2], so_row;
      if (jj == last) {
        const int qlim = len - 1 - jj * kTileRows;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int r = min(L.crow[i], qlim);
          const uint32_t chunk = 16 * ((L.lane & 7) ^ swz(L.crow[i]));
          qo[i] = (uint32_t)(r * ldq * 2) + chunk;
          oo[i] = (uint32_t)(r * ldo * 2) + chunk;
        }
        so_row = (uint32_t)(min(L.lane, qlim) * ldq * 2);  // this lane's query row inside the tile
      } else {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          qo[i] = L.cofs_g[i];
          oo[i] = ocofs[i];
        }
        so_row = lane_row_ofs;
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        copy_to_lds(qt_g, qo[i], m0 + so + 1024 * i);
        copy_to_lds(ot_g, oo[i], m0 + so + kTileBytes + 1024 * i);
      }
      if (L.wid == 0)  // -lse log2(e), bytes 4..7 of the row's dq columns
        copy_dword_to_lds(dqkv + row0 * ldq + h * kHeadDim + 2, so_row, m0s + so);
      else if (L.wid == 1)
        copy_dword_to_lds(dqkv + row0 * ldq + h * kHeadDim, so_row, m0s + so + 256);
    };
    // K and V rows of the wave (its 16 keys) go into its own rows of stage 1,
    // read back as B-operand fragments before stage 1 is refilled.
    {
      const int klim = len - 1 - k0;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = min(L.crow[i], klim);
        const uint32_t off = (uint32_t)(r * ldq * 2 + 16 * ((L.lane & 7) ^ swz(L.crow[i])));
        copy_to_lds(qkv + ((int64_t)start + k0) * ldq + hd + h * kHeadDim, off, m0 + kBwdStageBytes + 1024 * i);
        copy_to_lds(qkv + ((int64_t)start + k0) * ldq + 2 * hd + h * kHeadDim, off,
                    m0 + kBwdStageBytes + kTileBytes + 1024 * i);
      }
    }
    issue_tile(0, kt);
    // The first tile's copies (4, or 5 on waves 0 and 1) may stay in flight.
    if (L.wid < 2)
      wait_vmem_lds<5>();
    else
      wait_vmem_lds<4>();
    bf16x8 kf[2], vf[2];
    kf[0] = lds_b128(st1, L.qr * 128 + ((L.g ^ swz(L.qr)) << 4));
    kf[1] = lds_b128(st1, L.qr * 128 + (((4 + L.g) ^ swz(L.qr)) << 4));
    vf[0] = lds_b128(st1, kTileBytes + L.qr * 128 + ((L.g ^ swz(L.qr)) << 4));
    vf[1] = lds_b128(st1, kTileBytes + L.qr * 128 + (((4 + L.g) ^ swz(L.qr)) << 4));
    f32x4 dk[4], dv[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      dk[d] = f32x4{0.f, 0.f, 0.f, 0.f};
      dv[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    // Query tile j sits in stage (j - kt) % 2.  One step serves every tile, its
    // mask under a uniform branch (the diagonal masks keys after the query, the
    // last tile rows past the user's end; elsewhere nothing): a second, unmasked
    // copy of the step, or a loop unrolled by two, took the kernel past 128 VGPRs.
    // A wave whose 16 keys all lie past the user's end (on the user's last key
    // tile) computes nothing: it issues its share of the copies and meets the
    // barriers, in a second copy of the loop.
    auto query_tiles = [&](auto compute) {
      for (int j = kt; j <= last; ++j) {
        wait_and_barrier<0>();
        if (j + 1 <= last) issue_tile(((j + 1 - kt) & 1) * kBwdStageBytes, j + 1);
        if constexpr (decltype(compute)::value)
          dkdv_step<true>((j - kt) & 1 ? st1 : st0, L, kf, vf, sl2, dk, dv, j == kt, len - j * kTileRows);
      }
    };
    if (__builtin_amdgcn_readfirstlane(16 * L.wid < len - k0))
      query_tiles(std::true_type{});
    else
      query_tiles(std::false_type{});
    // The claim made at the item's start is passed on; every wave read s_next
    // before this item's first barrier.
    if (round >= 1 && threadIdx.x == 0) s_next = claimed;
    wait_and_barrier<0>();  // every wave is done with the ring
    const int nvalid = len - k0 - 16 * L.wid;
    uint16_t* const drow = dqkv + ((int64_t)start + k0 + 16 * L.wid) * ldq + h * kHeadDim;
    store_rows(st0 + 2048 * L.wid, dk, scale, drow + hd, ldq, nvalid);
    store_rows(st0 + kTileBytes + 2048 * L.wid, dv, 1.0f, drow + 2 * hd, ldq, nvalid);
  }
}

// ------------------------------------------------------------- dQ

// One key tile of a dQ item: S^T = K Q^T, dP^T = V dO^T (keys as rows: lane
// (g, lq) holds keys 16 b + 4 g + r of the wave's query lq), dS^T, then
// dQ^T += K^T dS^T.  nlse: -(log-sum-exp) log2(e) of the lane's query; dd: its
// D.  kDiagW >= 0: the diagonal tile as wave kDiagW sees it -- key blocks below
// the wave's rows are visible whole, block kDiagW up to the lane's own row, and
// the blocks above are neither formed nor weighed (their dS is exactly 0).
template <int kDiagW>
__device__ __forceinline__ void dq_step(const LDS char* base, const Lanes& L, const bf16x8 (&qf)[2],
                                        const bf16x8 (&of)[2], float sl2, float nlse, float dd, f32x4 (&dq)[4]) {
  constexpr int kNB = kDiagW < 0 ? 4 : kDiagW + 1;  // key blocks formed
  f32x4 s[4], dp[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (b >= kNB) break;
    const bf16x8 k0 = lds_b128(base, L.kofs[0] + 2048 * b);
    const bf16x8 k1 = lds_b128(base, L.kofs[1] + 2048 * b);
    s[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    s[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[1], s[b], 0, 0, 0);
    const bf16x8 v0 = lds_b128(base, kTileBytes + L.kofs[0] + 2048 * b);
    const bf16x8 v1 = lds_b128(base, kTileBytes + L.kofs[1] + 2048 * b);
    dp[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v0, of[0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    dp[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(v1, of[1], dp[b], 0, 0, 0);
  }
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    if (2 * hh >= kNB) break;
    const bool two = 2 * hh + 1 < kNB;  // the half's second block is formed
    uint32_t dw[4];
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int b = 2 * hh + half;
      if (b >= kNB) {
        dw[2 * half] = 0u;
        dw[2 * half + 1] = 0u;
        continue;
      }
      float ds[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(s[b][r], sl2, nlse));
        ds[r] = p * (dp[b][r] - dd);
        if (b == kDiagW && 4 * L.g + r > L.lq) ds[r] = 0.f;
      }
      dw[2 * half] = pack_bf16x2(ds[0], ds[1]);
      dw[2 * half + 1] = pack_bf16x2(ds[2], ds[3]);
    }
    const bf16x8 db = __builtin_bit_cast(bf16x8, uint4{dw[0], dw[1], dw[2], dw[3]});
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      // K^T fragments (the K half of the stage) for keys 32 hh .. 32 hh + 31; an
      // unformed second block is taken as 0.
      const bf16x4 lo = lds_tr16(base, L.vofs[d] - kTileBytes + 4096 * hh);
      const bf16x4 hi = two ? lds_tr16(base, L.vofs[d] - kTileBytes + 4096 * hh + 2048) : bf16x4{};
      dq[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7), db,
                                                      dq[d], 0, 0, 0);
    }
  }
}

__global__ __launch_bounds__(kAttnThreads) void bwd_dq_kernel(const uint16_t* __restrict__ qkv,
                                                              const uint16_t* __restrict__ dout,
                                                              const float* __restrict__ lse,
                                                              const int4* __restrict__ items,
                                                              const int32_t* __restrict__ count,
                                                              int32_t* __restrict__ queue, int n_heads,
                                                              float scale, uint16_t* __restrict__ dqkv) {
  __shared__ __attribute__((aligned(1024))) char ring_lds[2 * kStageBytes];
  __shared__ int s_next;
  LDS char* const st0 = (LDS char*)ring_lds;
  LDS char* const st1 = st0 + kStageBytes;
  const int64_t ldq = 3 * n_heads * kHeadDim;
  const int64_t ldo = n_heads * kHeadDim;
  const int hd = n_heads * kHeadDim;
  const float sl2 = scale * kLog2eF;
  Lanes L;
  make_lanes(L, ldq);
  Claim cl;
  cl.init(queue + kBwdDqQueue, n_heads);
  const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(st0 + 2048 * L.wid));
  const int nitems = *count;
  int claimed = 0;
  for (int round = 0, w = cl.w0;; ++round, w = round == 1 ? cl.w1 : __builtin_amdgcn_readfirstlane(s_next)) {
    int item, h;
    cl.decode(w, item, h);
    if (item >= nitems) break;
    if (round >= 1 && threadIdx.x == 0) claimed = cl.next();
    const int4 it = items[item];
    const int qt = it.y & 0xffff, start = it.z, len = it.w;
    const int q0 = qt * kTileRows;
    const int lim = len - 1 - q0;
    const int64_t tstride = (int64_t)kTileRows * ldq;
    const uint16_t* kg = qkv + (int64_t)start * ldq + hd + h * kHeadDim;
    auto issue_tile = [&](uint32_t so, int jj) {
      const uint16_t* kt = kg + jj * tstride;
      const uint16_t* vt = kt + hd;
#pragma unroll
      for (int i = 0; i < 2; ++i) {  // only the diagonal tile clamps rows
        const uint32_t o = jj == qt ? (uint32_t)(min(L.crow[i], lim) * ldq * 2 + 16 * ((L.lane & 7) ^ swz(L.crow[i])))
                                    : L.cofs_g[i];
        copy_to_lds(kt, o, m0 + so + 1024 * i);
        copy_to_lds(vt, o, m0 + so + kTileBytes + 1024 * i);
      }
    };
    // The wave's Q and dO rows go into its own rows of stage 1 (read back as
    // B-operand fragments before stage 1 is refilled); the lane's query's
    // log-sum-exp and D come straight from memory.
    {
      const uint16_t* qg = qkv + ((int64_t)start + q0) * ldq + h * kHeadDim;
      const uint16_t* og = dout + ((int64_t)start + q0) * ldo + h * kHeadDim;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = min(L.crow[i], lim);
        const uint32_t chunk = 16 * ((L.lane & 7) ^ swz(L.crow[i]));
        copy_to_lds(qg, (uint32_t)(r * ldq * 2) + chunk, m0 + kStageBytes + 1024 * i);
        copy_to_lds(og, (uint32_t)(r * ldo * 2) + chunk, m0 + kStageBytes + kTileBytes + 1024 * i);
      }
    }
    const int64_t qrow = (int64_t)start + q0 + min(L.qr, lim);
    const float nlse = -lse[qrow * n_heads + h] * kLog2eF;
    const float dd = *reinterpret_cast<const float*>(dqkv + qrow * ldq + h * kHeadDim);
    issue_tile(0, 0);
    wait_vmem_lds<4>();  // Q and dO rows have landed (the first tile's 4 copies may be in flight)
    bf16x8 qf[2], of[2];
    qf[0] = lds_b128(st1, L.qr * 128 + ((L.g ^ swz(L.qr)) << 4));
    qf[1] = lds_b128(st1, L.qr * 128 + (((4 + L.g) ^ swz(L.qr)) << 4));
    of[0] = lds_b128(st1, kTileBytes + L.qr * 128 + ((L.g ^ swz(L.qr)) << 4));
    of[1] = lds_b128(st1, kTileBytes + L.qr * 128 + (((4 + L.g) ^ swz(L.qr)) << 4));
    f32x4 dq[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) dq[d] = f32x4{0.f, 0.f, 0.f, 0.f};
    // A wave whose 16 query rows all lie past the user's end (the user's last
    // q-tile) computes nothing: it issues its share of the copies and meets the
    // barriers, in a second copy of the loop.
    const int khi = qt + 1;
    // The diagonal tile, specialised for each wave; it ends an item once, so its
    // stage is a run-time choice.
    auto diag_step = [&](const LDS char* base) {
      switch (__builtin_amdgcn_readfirstlane(L.wid)) {
        case 0: dq_step<0>(base, L, qf, of, sl2, nlse, dd, dq); break;
        case 1: dq_step<1>(base, L, qf, of, sl2, nlse, dd, dq); break;
        case 2: dq_step<2>(base, L, qf, of, sl2, nlse, dd, dq); break;
        default: dq_step<3>(base, L, qf, of, sl2, nlse, dd, dq); break;
      }
    };
    auto tiles = [&](auto compute) {
      constexpr bool kOn = decltype(compute)::value;
      int j = 0;
      for (; j + 2 < khi; j += 2) {
        wait_and_barrier<0>();
        issue_tile(kStageBytes, j + 1);
        if constexpr (kOn) dq_step<-1>(st0, L, qf, of, sl2, nlse, dd, dq);
        wait_and_barrier<0>();
        issue_tile(0, j + 2);
        if constexpr (kOn) dq_step<-1>(st1, L, qf, of, sl2, nlse, dd, dq);
      }
      const bool two_left = j + 1 < khi;
      if (two_left) {
        wait_and_barrier<0>();
        issue_tile(kStageBytes, j + 1);
        if constexpr (kOn) dq_step<-1>(st0, L, qf, of, sl2, nlse, dd, dq);
      }
      wait_and_barrier<0>();
      if constexpr (kOn) diag_step(two_left ? st1 : st0);
    };
    if (__builtin_amdgcn_readfirstlane(16 * L.wid < len - q0))
      tiles(std::true_type{});
    else
      tiles(std::false_type{});
    if (round >= 1 && threadIdx.x == 0) s_next = claimed;  // every wave read s_next before this item's first barrier
    wait_and_barrier<0>();  // every wave is done with the ring (and has read its D)
    store_rows(st0 + 2048 * L.wid, dq, scale, dqkv + ((int64_t)start + q0 + 16 * L.wid) * ldq + h * kHeadDim, ldq,
               len - q0 - 16 * L.wid);
  }
}

std::mutex g_occ_mu;

int occupancy(const void* kernel) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kAttnThreads, 0) != hipSuccess || n < 1) n = 1;
  return n;
}

}  // namespace

hipError_t launch_backward(const void* qkv, const void* dout, const float* lse, const int4* items,
                           const int32_t* count, int32_t* queue, int64_t max_items, int n_heads, float scale,
                           void* dqkv, int cus, hipStream_t stream) {
  static int occ_dkdv = 0, occ_dq = 0;
  {
    std::lock_guard<std::mutex> lk(g_occ_mu);
    if (occ_dkdv == 0) {
      occ_dkdv = occupancy(reinterpret_cast<const void*>(bwd_dkdv_kernel));
      occ_dq = occupancy(reinterpret_cast<const void*>(bwd_dq_kernel));
    }
  }
  auto grid_of = [&](int occ) {
    int64_t g = (int64_t)cus * occ;
    if (g > kMaxGrid) g = kMaxGrid;
    g -= g % 8;
    if (g < 8) g = 8;
    const int64_t work = max_items * n_heads;
    if (work < g) g = work;
    return (int)(g < 1 ? 1 : g);
  };
  hipLaunchKernelGGL(bwd_dkdv_kernel, dim3(grid_of(occ_dkdv)), dim3(kAttnThreads), 0, stream,
                     static_cast<const uint16_t*>(qkv), static_cast<const uint16_t*>(dout), lse, items, count, queue,
                     n_heads, scale, static_cast<uint16_t*>(dqkv));
  hipLaunchKernelGGL(bwd_dq_kernel, dim3(grid_of(occ_dq)), dim3(kAttnThreads), 0, stream,
                     static_cast<const uint16_t*>(qkv), static_cast<const uint16_t*>(dout), lse, items, count, queue,
                     n_heads, scale, static_cast<uint16_t*>(dqkv));
  return hipGetLastError();
}

}  // namespace vlca
