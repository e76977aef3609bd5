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

}  // namespace
}  // namespace vlca
