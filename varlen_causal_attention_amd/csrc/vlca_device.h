// Device-side building blocks shared by the gfx950 attention kernels (forward
// in vlca_kernels.hip, backward in vlca_backward.hip): vector types, the LDS tile
// layout (64 rows x 128 B, 16-byte chunks XOR-swizzled by row), LDS fragment
// reads for the v_mfma_f32_16x16x32_bf16 operands, waits and barriers, and the
// global -> LDS copy.  Internal; included by HIP sources only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

constexpr int kWaves = 4;                              // wave w owns rows 16w .. 16w+15 of a tile
constexpr int kAttnThreads = 64 * kWaves;
constexpr int kTileBytes = kTileRows * kHeadDim * 2;  // 8 KB: one 64 x 64 bf16 tile, 128 B rows
constexpr int kStageBytes = 2 * kTileBytes;           // two tiles (K then V, or Q then dO)
// The running max of a query is raised only when a key exceeds it by more than
// 2^kRescaleLog2 in exp2 units.
constexpr float kRescaleLog2 = 8.0f;

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

// Wait for this wave's LDS operations, then a workgroup barrier (no wait on
// copies in flight).
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

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

// Masks of a tile step: which of the lane's 16 keys of a tile (key 16 b + 4 g + r
// of lane group g) its query sees.  A mask with kAny also tells, wave-uniformly,
// whether it passes every key of the tile (all()): the step then skips it.
struct NoMask {  // every key
  static constexpr bool kAny = false;
  __device__ bool operator()(int, int) const { return true; }
};
// The diagonal tile as wave W sees it (its rows 16W .. 16W+15 against keys 0..63
// of the same rows): score blocks below W are visible whole, block W up to the
// lane's own row (key 16W + 4g + r for r <= lq - 4g), blocks above W not at all.
// Only blocks 0..W are formed; the weights of the others are exactly 0.
template <int W>
struct DiagWave {
  static constexpr bool kAny = false;
  static constexpr int kBlocks = W + 1;  // score blocks formed
  static constexpr int kPartial = W;     // the block masked per lane
  int lim;                               // lq - 4g
};

// Score blocks a mask lets the step form, and the one it masks per lane (-1:
// none); masks that do not say are taken whole (kAny decides per key).
template <typename M, typename = void>
struct MaskShape {
  static constexpr int kBlocks = 4, kPartial = -1;
};
template <typename M>
struct MaskShape<M, decltype((void)M::kPartial)> {
  static constexpr int kBlocks = M::kBlocks, kPartial = M::kPartial;
};

// One key tile of one item: S^T = K Q^T, mask, softmax update, O^T += V^T P^T
// and l += 1^T P^T.  Masked keys score -inf.  kSafe: a query may see no key of
// the tile's first half (or of the tiles so far) -- its running max is then still
// -inf, and the rescale factor and weight offset are taken as 1 and 0 instead of
// the NaN that -inf - (-inf) gives; without kSafe the caller guarantees that the
// first half of the first tile holds a visible key of every query.  halves = 1
// (wave-uniform): the tile's second 32 keys are masked for every row of the wave
// and are skipped -- their weights would be exactly 0, so the result is the same.
template <bool kSafe = false, typename Mask>
__device__ __forceinline__ void tile_step(const LDS char* base, const Lanes& L, const bf16x8 (&qf)[2],
                                          const bf16x8& ones, float sl2, float rescale_thr, Acc& A,
                                          const Mask& mask, int halves = 2) {
  constexpr int kNB = MaskShape<Mask>::kBlocks;
  constexpr int kPB = MaskShape<Mask>::kPartial;
  f32x4 s[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    if (b >= kNB || (b >= 2 && halves < 2)) break;
    const bf16x8 k0 = lds_b128(base, L.kofs[0] + 2048 * b);
    const bf16x8 k1 = lds_b128(base, L.kofs[1] + 2048 * b);
    s[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    s[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[1], s[b], 0, 0, 0);
  }
  if constexpr (Mask::kAny) {
    if (!mask.all()) {
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (!mask(b, r)) s[b][r] = -__builtin_inff();
    }
  }
  if constexpr (kPB >= 0) {
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (r > mask.lim) s[kPB][r] = -__builtin_inff();
  }
  // The tile is taken in two halves of 32 keys (score blocks 2hh, 2hh+1), so the
  // second half's QK^T MFMAs run while the first half's softmax is computed.
  // Lane-local max over this lane's 8 keys of the half.  The reference max m of a
  // query is shared by its 4 lane groups; only when some key exceeds it by more
  // than the threshold (and on the first tile, m = -inf; the first half always
  // holds a visible key of every query) is the true max formed across the lane
  // groups and m raised, with the accumulators rescaled.  The common path needs
  // no cross-lane traffic.  A block the mask leaves unformed (the half's second
  // block) weighs 0, and its V^T fragments are taken as 0.
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    if (2 * hh >= kNB || hh >= halves) break;
    const bool two = 2 * hh + 1 < kNB;  // the half's second block is formed
    const f32x4& s0 = s[2 * hh];
    float lm = vmax(vmax(s0[0], s0[1]), vmax(s0[2], s0[3]));
    if (two) {
      const f32x4& s1 = s[2 * hh + 1];
      lm = vmax(vmax(vmax(lm, s1[0]), s1[1]), vmax(s1[2], s1[3]));
    }
    if (__any(lm > A.mthr)) {  // wave-uniform
      const float mt = max_across_lane_groups(lm);
      const float mn = fmaxf(A.m, mt);
      const bool none = kSafe && mn == -__builtin_inff();  // no visible key yet
      const float alpha = none ? 1.0f : __builtin_amdgcn_exp2f((A.m - mn) * sl2);
#pragma unroll
      for (int d = 0; d < 4; ++d) A.o[d] *= alpha;
      A.l *= alpha;
      A.m = mn;
      A.moff = none ? 0.0f : -mn * sl2;
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
    if (two) {
      const f32x4& s1 = s[2 * hh + 1];
      pw.z = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(s1[0], sl2, moff)),
                         __builtin_amdgcn_exp2f(__builtin_fmaf(s1[1], sl2, moff)));
      pw.w = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(s1[2], sl2, moff)),
                         __builtin_amdgcn_exp2f(__builtin_fmaf(s1[3], sl2, moff)));
    } else {
      pw.z = 0u;
      pw.w = 0u;
    }
    const bf16x8 pb = __builtin_bit_cast(bf16x8, pw);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const bf16x4 lo = lds_tr16(base, L.vofs[d] + 4096 * hh);
      const bf16x4 hi = two ? lds_tr16(base, L.vofs[d] + 4096 * hh + 2048) : bf16x4{};
      const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      A.o[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb, A.o[d], 0, 0, 0);
    }
    A.l = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb, A.l, 0, 0, 0);
  }
}

// The wave's 16 rows of a 64 x 64 fp32 result held in the MFMA C layout of a
// transposed product (lane (g, lq): dims 16 d + 4 g + r of row lq) times `mul`
// (per lane, i.e. per row),
// rounded to bf16, staged through the wave's own 2 KB of LDS at `rows`, and
// stored as full 128-byte rows: row i goes to dst + i * ld if i < nvalid.
__device__ __forceinline__ void store_rows(LDS char* rows, const f32x4 (&acc)[4], float mul, uint16_t* dst, int64_t ld,
                                           int nvalid) {
  int lane = threadIdx.x & 63;
  asm volatile("" : "+v"(lane));
  const int lq = lane & 15, g = lane >> 4;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    const u32x2 wv = {pack_bf16x2(acc[d][0] * mul, acc[d][1] * mul), pack_bf16x2(acc[d][2] * mul, acc[d][3] * mul)};
    *(LDS u32x2*)(rows + lq * 128 + (((2 * d + (g >> 1)) ^ swz(lq)) << 4) + 8 * (g & 1)) = wv;
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int r = 8 * i + (lane >> 3), c = lane & 7;
    const u32x4 v = *(const LDS u32x4*)(rows + r * 128 + ((c ^ swz(r)) << 4));
    if (r < nvalid) __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(dst + r * ld + 8 * c));
  }
}

}  // namespace
}  // namespace vlca
