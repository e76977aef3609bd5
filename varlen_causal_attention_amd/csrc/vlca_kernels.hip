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
//  * attention_kernel -- a persistent grid; work index w maps to item w / H and
//    head w % H.  With H = 8 and a grid that is a multiple of 8, a workgroup on
//    XCD x (workgroups are dealt to the 8 XCDs round-robin) always runs head x,
//    so each XCD's L2 holds one head's K/V columns and serves the re-reads of
//    later q-tiles of the same user.
//
// Attention workgroup: 4 waves; wave w owns query rows 16w..16w+15 of the tile.
//  * K and V tiles (64 keys x 64 dims, 8 KB each) are copied from HBM straight
//    into LDS with global_load_lds_dwordx4 (no VGPRs, no VALU), through a ring of
//    kStages buffers, so kStages-1 tiles are in flight while one is consumed.
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

#include "vlca_internal.h"

namespace vlca {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
#define LDS __attribute__((address_space(3)))
typedef LDS bf16x4 lds_bf16x4;

constexpr int kSchedThreads = 1024;
constexpr int kSchedCache = 8160;  // cu_seqlens entries cached in LDS by the scheduler (LDS <= 64 KB)
#ifndef VLCA_QUERY_BLOCKS_PER_WAVE
#define VLCA_QUERY_BLOCKS_PER_WAVE 1
#endif
constexpr int kQB = VLCA_QUERY_BLOCKS_PER_WAVE;        // 16-row query blocks per wave (1, 2 or 4)
constexpr int kRowsPerWave = 16 * kQB;
constexpr int kWaves = kTileRows / kRowsPerWave;       // waves per workgroup
constexpr int kAttnThreads = 64 * kWaves;
constexpr int kCopyInstr = kRowsPerWave / 8;           // 1 KB copy instructions per wave per 8 KB tile
constexpr int kTileBytes = kTileRows * kHeadDim * 2;  // 8 KB: one 64 x 64 bf16 tile, 128 B rows
constexpr int kStageBytes = 2 * kTileBytes;           // K tile then V tile
constexpr float kRescaleLog2 = 8.0f;

// ----------------------------------------------------------------- scheduler

struct Seg {
  int start, len, tiles;
};

__device__ __forceinline__ Seg segment_of(const int32_t* __restrict__ cu, const int* s_cu, bool cached,
                                          int u, int total, int max_tiles) {
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

// out[k] = sum_{j > k} a[j] for k < n (in place, one wave); returns the total.
__device__ int wave_suffix_exclusive(int* a, int n, int lane) {
  const int chunk = (n + 63) / 64;
  const int lo = lane * chunk;
  const int hi = min(lo + chunk, n);
  int local = 0;
  for (int k = lo; k < hi; ++k) local += a[k];
  int incl = local;  // inclusive suffix over lanes >= lane
  for (int off = 1; off < 64; off <<= 1) {
    const int t = __shfl_down(incl, off);
    if (lane + off < 64) incl += t;
  }
  int run = incl - local;
  for (int k = hi - 1; k >= lo; --k) {
    const int v = a[k];
    a[k] = run;
    run += v;
  }
  return __shfl(incl, 0);
}

__global__ __launch_bounds__(kSchedThreads) void schedule_kernel(const int32_t* __restrict__ cu, int U,
                                                                 int max_tiles, int4* __restrict__ items,
                                                                 int32_t* __restrict__ count) {
  __shared__ int s_cu[kSchedCache + 1];
  __shared__ int s_cnt[kMaxLevels + 1];  // histogram of tile counts, then users per level
  __shared__ int s_pos[kMaxLevels + 1];  // first worklist slot of each level
  __shared__ int s_wmax[kSchedThreads / 64];
  __shared__ int s_total;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const bool cached = U <= kSchedCache;
  if (U > 0 && max_tiles > 0 && cached) {
    for (int i = tid; i <= U; i += kSchedThreads) s_cu[i] = cu[i];
  }
  __syncthreads();
  const int total = (U > 0 && max_tiles > 0) ? (cached ? s_cu[U] : cu[U]) : 0;
  const int nusers = max_tiles > 0 ? U : 0;

  // Largest tile count over users.
  int tmax = 0;
  for (int u = tid; u < nusers; u += kSchedThreads)
    tmax = max(tmax, segment_of(cu, s_cu, cached, u, total, max_tiles).tiles);
  for (int off = 32; off > 0; off >>= 1) tmax = max(tmax, __shfl_xor(tmax, off));
  if (lane == 0) s_wmax[wid] = tmax;
  for (int k = tid; k <= kMaxLevels; k += kSchedThreads) s_cnt[k] = 0;
  __syncthreads();
  int levels = 0;
  for (int i = 0; i < kSchedThreads / 64; ++i) levels = max(levels, s_wmax[i]);

  for (int u = tid; u < nusers; u += kSchedThreads) {
    const int t = segment_of(cu, s_cu, cached, u, total, max_tiles).tiles;
    if (t > 0) atomicAdd(&s_cnt[t], 1);
  }
  __syncthreads();
  // users with more than k tiles: c[k] = sum_{t > k} hist[t]
  if (wid == 0) wave_suffix_exclusive(s_cnt, levels + 1, lane);
  __syncthreads();
  for (int k = tid; k < levels; k += kSchedThreads) s_pos[k] = s_cnt[k];
  __syncthreads();
  // first slot of level k: the items of all higher levels come first
  if (wid == 0) {
    const int n = wave_suffix_exclusive(s_pos, levels, lane);
    if (lane == 0) s_total = n;
  }
  __syncthreads();

  // Each wave emits whole levels; inside a level users ascend (ballot compaction).
  for (int k = wid; k < levels; k += kSchedThreads / 64) {
    int slot = s_pos[k];
    const int end = slot + s_cnt[k];
    for (int base = 0; base < nusers && slot < end; base += 64) {
      const int u = base + lane;
      Seg s{0, 0, 0};
      if (u < nusers) s = segment_of(cu, s_cu, cached, u, total, max_tiles);
      const bool take = s.tiles > k;
      const unsigned long long m = __ballot(take);
      if (take) {
        const int rank = __popcll(m & ((1ull << lane) - 1ull));
        items[slot + rank] = make_int4(u, k, s.start, s.len);
      }
      slot += __popcll(m);
    }
  }
  if (tid == 0) *count = s_total;
}

// ----------------------------------------------------------------- attention

// XOR swizzles of the 16-byte chunk index inside a 128-byte LDS tile row, chosen
// so that the fragment reads below touch distinct banks (checked for both 32 and
// 64 four-byte banks).  K rows are read 16 at a time as rows 8a+4e+{0..3}
// (a = 0..3); V rows 4 at a time per 16-lane group as rows 8g+{0..3}.
__device__ __forceinline__ int swz_k(int r) { return ((r & 3) ^ ((r >> 4) & 1)) | (((r >> 3) & 1) << 2); }
__device__ __forceinline__ int swz_v(int r) { return ((r & 3) ^ ((r >> 3) & 1)) << 1; }

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

// LDS reads go through address-space-3 pointers derived from the stage object
// itself, so the compiler can see which copies they may depend on.
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
// release fence that also waits for every LDS copy still in flight, draining the
// tile ring; here only what the caller names (n copies may stay in flight).
template <int n>
__device__ __forceinline__ void wait_and_barrier() {
  static_assert(n >= 0 && n < 64, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(n) : "memory");
}

// Largest number of copies a wave can have in flight behind the one it waits for.
constexpr int kMaxPending = 2 * kCopyInstr * (kStages - 1);

// Wait until at most n tiles' copies (2*kCopyInstr per wave each) are in flight.
__device__ __forceinline__ void wait_tiles_pending(int n) {
  if (n <= 0)
    wait_vmem_lds<0>();
  else if (n == 1)
    wait_vmem_lds<2 * kCopyInstr>();
  else if (n == 2)
    wait_vmem_lds<4 * kCopyInstr>();
  else
    wait_vmem_lds<6 * kCopyInstr>();
}

// The same, then the workgroup barrier.
__device__ __forceinline__ void wait_tiles_pending_barrier(int n) {
  if (n <= 0)
    wait_and_barrier<0>();
  else if (n == 1)
    wait_and_barrier<2 * kCopyInstr>();
  else if (n == 2)
    wait_and_barrier<4 * kCopyInstr>();
  else
    wait_and_barrier<6 * kCopyInstr>();
}

// Copy 16 bytes per lane from global memory into LDS (global_load_lds_dwordx4):
// lane l reads base + voff (a wave-uniform 64-bit base, a per-lane 32-bit byte
// offset) and its bytes land at lds_wave_base + 16*l.  Issued from inline asm so
// that the compiler, which would otherwise track these LDS writes coarsely and
// insert waits for every copy in flight before unrelated LDS reads, leaves all
// waits on them to the explicit wait_vmem_lds / wait_and_barrier calls.  The
// instruction has no register result; M0 (the LDS base operand) is saved and
// restored around it.
__device__ __forceinline__ void copy_to_lds(const void* base, uint32_t voff, const LDS void* lds_wave_base) {
  // readfirstlane returns int: widen through uint32_t so the low word is not
  // sign-extended into the high word of the 64-bit base.
  const uint32_t m = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)lds_wave_base);
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

// One ring stage: the K tile then the V tile.
struct Stage {
  char bytes[kStageBytes];
};

// Per-lane constants of the attention workgroup.  Wave w owns query rows
// kRowsPerWave*w .. kRowsPerWave*(w+1)-1 of the 64-row tile, as kQB blocks of 16;
// it also copies those rows of every K, V and Q tile into LDS.
struct Lanes {
  int g, lq, wid, lane;
  int qr[kQB];                       // query row (inside the tile) of block qb
  int crow[kCopyInstr];              // tile row copied by this lane, per instruction
  int ck[kCopyInstr], cv[kCopyInstr];  // logical 16-byte chunk copied (K/Q and V swizzle)
  uint32_t kofs_g[kCopyInstr], vofs_g[kCopyInstr];  // byte offset of that chunk from the tile's first row
  int kofs[4][2];                    // K fragment byte offsets inside a stage
  int vofs[2][4][2];                 // V^T fragment byte offsets inside a stage
};

__device__ __forceinline__ void make_lanes(Lanes& L, int64_t ldq) {
  const int tid = threadIdx.x;
  L.lane = tid & 63;
  L.wid = tid >> 6;
  L.g = L.lane >> 4;
  L.lq = L.lane & 15;
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) L.qr[qb] = L.wid * kRowsPerWave + 16 * qb + L.lq;
  // Copy role: instruction i moves tile rows kRowsPerWave*wid + 8i .. +7; lane l
  // lands at byte 16*l of that 1 KB slice (row l/8, physical chunk l%8).
  const int cpos = L.lane & 7;
#pragma unroll
  for (int i = 0; i < kCopyInstr; ++i) {
    L.crow[i] = kRowsPerWave * L.wid + 8 * i + (L.lane >> 3);
    L.ck[i] = cpos ^ swz_k(L.crow[i]);
    L.cv[i] = cpos ^ swz_v(L.crow[i]);
    L.kofs_g[i] = (uint32_t)(L.crow[i] * ldq * 2 + 16 * L.ck[i]);
    L.vofs_g[i] = (uint32_t)(L.crow[i] * ldq * 2 + 16 * L.cv[i]);
  }
  // K fragment rows: S^T block b (keys 32h..32h+31 with h = b/2, e = b%2), MFMA row
  // lq <- key 32h + 8(lq/4) + 4e + lq%4; its output reg r in lane group g is then
  // key 32h + 8g + 4e + r, the order ds_read_b64_tr_b16 gives V^T below.
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int rho = 32 * (b >> 1) + 8 * (L.lq >> 2) + 4 * (b & 1) + (L.lq & 3);
    L.kofs[b][0] = rho * 128 + ((L.g ^ swz_k(rho)) << 4);
    L.kofs[b][1] = rho * 128 + (((4 + L.g) ^ swz_k(rho)) << 4);
  }
  // V^T fragment sources: keys 32h + 8g + lq/4 (+4), dims 16d + 4(lq%4) .. +3.
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int d = 0; d < 4; ++d)
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const int rho = 32 * h + 8 * L.g + (L.lq >> 2) + 4 * s;
        const int chunk = 2 * d + ((L.lq & 3) >> 1);
        L.vofs[h][d][s] = kTileBytes + rho * 128 + ((chunk ^ swz_v(rho)) << 4) + 8 * (L.lq & 1);
      }
}

// Issue this wave's copies of key tile j of the current item into stage `dst`.
// Tiles before the diagonal lie wholly inside the user, so their lanes use the
// fixed offsets from the tile's first row; the diagonal tile clamps rows past the
// user's end to its last row (finite data under the causal mask, never another
// user's rows).
__device__ __forceinline__ void issue_tile(LDS char* dst, const Lanes& L, const uint16_t* kg, const uint16_t* vg,
                                           int64_t ldq, int j, int len, bool clamp) {
  LDS char* sk = dst + kRowsPerWave * L.wid * 128;
  const uint16_t* kt = kg + (int64_t)j * kTileRows * ldq;
  const uint16_t* vt = vg + (int64_t)j * kTileRows * ldq;
#pragma unroll
  for (int i = 0; i < kCopyInstr; ++i) {
    uint32_t ko = L.kofs_g[i], vo = L.vofs_g[i];
    if (clamp) {
      const int r = min(L.crow[i], len - 1 - j * kTileRows);
      ko = (uint32_t)(r * ldq * 2 + 16 * L.ck[i]);
      vo = (uint32_t)(r * ldq * 2 + 16 * L.cv[i]);
    }
    copy_to_lds(kt, ko, sk + 1024 * i);
    copy_to_lds(vt, vo, sk + kTileBytes + 1024 * i);
  }
}

// Online-softmax state of one lane for each of its query blocks: the running
// reference max m (raw score units), the O^T accumulator (dims 16d + 4g + r) and
// the denominator (every register of l holds it).
struct Acc {
  float m[kQB];
  f32x4 o[kQB][4];
  f32x4 l[kQB];
};

// One key tile of one item: S^T = K Q^T, mask (diagonal tile only), softmax
// update, O^T += V^T P^T and l += 1^T P^T, for every query block of the wave.
template <bool kDiag>
__device__ __forceinline__ void tile_step(const LDS char* base, const Lanes& L, const bf16x8 (&qf)[kQB][2],
                                          float sl2, float rescale_thr, Acc& A) {
  const float NEG_INF = -__builtin_inff();
  const bf16x8 ones = __builtin_bit_cast(bf16x8, make_uint4(0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u));
  f32x4 s[kQB][4];
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const bf16x8 k0 = lds_b128(base, L.kofs[b][0]);
    const bf16x8 k1 = lds_b128(base, L.kofs[b][1]);
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      s[qb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[qb][0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      s[qb][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[qb][1], s[qb][b], 0, 0, 0);
    }
  }
  if (kDiag) {  // key kk visible to query qr iff kk <= qr
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (32 * (b >> 1) + 8 * L.g + 4 * (b & 1) + r > L.qr[qb]) s[qb][b][r] = NEG_INF;
  }
  // Lane-local max over this lane's 16 keys of each query block.  The reference
  // max m of a query is shared by its 4 lane groups; only when some key exceeds it
  // by more than the threshold (and on the first tile, m = -inf) is the true row
  // max formed across the lane groups and m raised, with the accumulators
  // rescaled.  The common path needs no cross-lane traffic.
  float lm[kQB];
  bool raise = false;
#pragma unroll
  for (int qb = 0; qb < kQB; ++qb) {
    float x = s[qb][0][0];
#pragma unroll
    for (int e = 1; e < 16; ++e) x = fmaxf(x, s[qb][e >> 2][e & 3]);
    lm[qb] = x;
    raise |= x > A.m[qb] + rescale_thr;
  }
  if (__any(raise)) {  // wave-uniform
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const float mt = max_across_lane_groups(lm[qb]);
      const float mn = fmaxf(A.m[qb], mt);
      const float alpha = __builtin_amdgcn_exp2f((A.m[qb] - mn) * sl2);
#pragma unroll
      for (int d = 0; d < 4; ++d) A.o[qb][d] *= alpha;
      A.l[qb] *= alpha;
      A.m[qb] = mn;
    }
  }
#pragma unroll
  for (int hh = 0; hh < 2; ++hh) {
    // P^T slots 0..7 of lane group g = keys 32hh + 8g + 0..7 = blocks 2hh, 2hh+1
    bf16x8 pb[kQB];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const float moff = -A.m[qb] * sl2;
      const f32x4& s0 = s[qb][2 * hh];
      const f32x4& s1 = s[qb][2 * hh + 1];
      uint4 pw;
      pw.x = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(s0[0], sl2, moff)),
                         __builtin_amdgcn_exp2f(__builtin_fmaf(s0[1], sl2, moff)));
      pw.y = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(s0[2], sl2, moff)),
                         __builtin_amdgcn_exp2f(__builtin_fmaf(s0[3], sl2, moff)));
      pw.z = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(s1[0], sl2, moff)),
                         __builtin_amdgcn_exp2f(__builtin_fmaf(s1[1], sl2, moff)));
      pw.w = pack_bf16x2(__builtin_amdgcn_exp2f(__builtin_fmaf(s1[2], sl2, moff)),
                         __builtin_amdgcn_exp2f(__builtin_fmaf(s1[3], sl2, moff)));
      pb[qb] = __builtin_bit_cast(bf16x8, pw);
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const bf16x4 lo = lds_tr16(base, L.vofs[hh][d][0]);
      const bf16x4 hi = lds_tr16(base, L.vofs[hh][d][1]);
      const bf16x8 va = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
      for (int qb = 0; qb < kQB; ++qb)
        A.o[qb][d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pb[qb], A.o[qb][d], 0, 0, 0);
    }
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) A.l[qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pb[qb], A.l[qb], 0, 0, 0);
  }
}

__global__ __launch_bounds__(kAttnThreads) void attention_kernel(const uint16_t* __restrict__ qkv,
                                                                 const int4* __restrict__ items,
                                                                 const int32_t* __restrict__ count,
                                                                 int n_heads, float sl2,
                                                                 uint16_t* __restrict__ out) {
  static_assert(kStages >= 2 && kStages <= 4, "ring depth");
  __shared__ __attribute__((aligned(1024))) Stage ring_lds[kStages];
  LDS char* const ring = (LDS char*)ring_lds[0].bytes;
  auto stage = [&](int j) { return ring + (j % kStages) * kStageBytes; };

  const int64_t ldq = 3 * n_heads * kHeadDim;
  Lanes L;
  make_lanes(L, ldq);
  const int64_t ldo = n_heads * kHeadDim;
  const float rescale_thr = kRescaleLog2 / sl2;  // in raw score units

  // Work assignment.  With the grid a multiple of H, workgroup g always runs head
  // g % H (with H = 8 that is the XCD it sits on) and item slot g / H of each
  // round; rounds alternate direction (snake), so the workgroups that drew the
  // longest items of round 0 draw the shortest of round 1.
  const int nitems = *count;
  const int G = gridDim.x;
  const bool by_head = G % n_heads == 0;
  const int slots = by_head ? G / n_heads : G;
  const int slot = by_head ? blockIdx.x / n_heads : blockIdx.x;
  const int head0 = by_head ? blockIdx.x - slot * n_heads : 0;
  const int qt_max = nitems > 0 ? items[0].y : 0;  // items arrive longest first
  for (int round = 0;; ++round) {
    const int pos = (round & 1) ? slots - 1 - slot : slot;
    int item, h;
    if (by_head) {
      item = round * slots + pos;
      h = head0;
    } else {
      const int w = round * slots + pos;
      item = w / n_heads;
      h = w - item * n_heads;
    }
    if (item >= nitems) break;
    const int4 it = items[item];
    const int qt = it.y;
    const int start = it.z;
    const int len = it.w;
    const int q0 = qt * kTileRows;
    // The longest items bound the kernel's critical path: their waves get issue
    // priority over co-resident shorter items.
    if (qt >= 1 && 2 * qt >= qt_max)
      __builtin_amdgcn_s_setprio(3);
    else if (qt >= 1 && 4 * qt >= qt_max)
      __builtin_amdgcn_s_setprio(2);
    else if (qt >= 1)
      __builtin_amdgcn_s_setprio(1);
    else
      __builtin_amdgcn_s_setprio(0);
    const uint16_t* kg = qkv + (int64_t)start * ldq + n_heads * kHeadDim + h * kHeadDim;
    const uint16_t* vg = kg + n_heads * kHeadDim;

    // The wave's Q rows go through the K half of the last ring stage: each wave
    // copies and reads only its own rows, and tile kStages-1 later overwrites
    // exactly those rows of the same wave, after its Q reads have completed.
    LDS char* const qstage = ring + (kStages - 1) * kStageBytes;
    {
      LDS char* sq = qstage + kRowsPerWave * L.wid * 128;
      const uint16_t* qg = qkv + ((int64_t)start + q0) * ldq + h * kHeadDim;
#pragma unroll
      for (int i = 0; i < kCopyInstr; ++i) {
        const int r = min(L.crow[i], len - 1 - q0);
        copy_to_lds(qg, (uint32_t)(r * ldq * 2 + 16 * L.ck[i]), sq + 1024 * i);
      }
    }
    // Prologue: tiles 0 .. kStages-2 (those that exist) into stages 0 .. kStages-2.
    const int pre = min(qt, kStages - 2);  // index of the last prologue tile
#pragma unroll
    for (int j = 0; j <= kStages - 2; ++j)
      if (j <= pre) issue_tile(ring + j * kStageBytes, L, kg, vg, ldq, j, len, j == qt);
    wait_tiles_pending(pre + 1);  // this wave's Q rows have landed (all prologue tiles may be in flight)
    bf16x8 qf[kQB][2];
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      const int row = L.qr[qb];
      qf[qb][0] = lds_b128(qstage, row * 128 + ((L.g ^ swz_k(row)) << 4));
      qf[qb][1] = lds_b128(qstage, row * 128 + (((4 + L.g) ^ swz_k(row)) << 4));
    }
    wait_vmem_lds<kMaxPending>();  // ... and been read (lgkmcnt) before that stage is refilled

    Acc A;
#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      A.m[qb] = -__builtin_inff();
      A.l[qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int d = 0; d < 4; ++d) A.o[qb][d] = f32x4{0.f, 0.f, 0.f, 0.f};
    }

    // Tile j lives in stage j % kStages.  Before consuming it, only the copies of
    // tiles j+1 .. j+kStages-2 (those that exist) may still be in flight: wait
    // for the rest, then a barrier makes every wave's copies visible and frees
    // stage (j-1) % kStages for tile j+kStages-1.  Off-diagonal tiles (j < qt)
    // need no mask; the diagonal tile runs last.
    for (int j = 0; j < qt; ++j) {
      wait_tiles_pending_barrier(min(qt - j, kStages - 2));
      if (j + kStages - 1 <= qt) issue_tile(stage(j + kStages - 1), L, kg, vg, ldq, j + kStages - 1, len,
                                            j + kStages - 1 == qt);
      tile_step<false>(stage(j), L, qf, sl2, rescale_thr, A);
    }
    wait_and_barrier<0>();
    tile_step<true>(stage(qt), L, qf, sl2, rescale_thr, A);
    wait_and_barrier<0>();  // every wave is done with the ring before the next item refills it

#pragma unroll
    for (int qb = 0; qb < kQB; ++qb) {
      if (q0 + L.qr[qb] < len) {
        const float inv = 1.0f / A.l[qb][0];
        uint16_t* o = out + ((int64_t)start + q0 + L.qr[qb]) * ldo + h * kHeadDim + 4 * L.g;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          uint2 wv;
          wv.x = pack_bf16x2(A.o[qb][d][0] * inv, A.o[qb][d][1] * inv);
          wv.y = pack_bf16x2(A.o[qb][d][2] * inv, A.o[qb][d][3] * inv);
          *reinterpret_cast<uint2*>(o + 16 * d) = wv;
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_schedule(const int32_t* cu_seqlens, int num_users, int max_tiles, int4* items, int32_t* count,
                           hipStream_t stream) {
  hipLaunchKernelGGL(schedule_kernel, dim3(1), dim3(kSchedThreads), 0, stream, cu_seqlens, num_users, max_tiles,
                     items, count);
  return hipGetLastError();
}

hipError_t launch_attention(const void* qkv, const int4* items, const int32_t* count, int n_heads,
                            float scale_log2e, void* out, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(attention_kernel, dim3(grid), dim3(kAttnThreads), 0, stream,
                     static_cast<const uint16_t*>(qkv), items, count, n_heads, scale_log2e,
                     static_cast<uint16_t*>(out));
  return hipGetLastError();
}

}  // namespace vlca
