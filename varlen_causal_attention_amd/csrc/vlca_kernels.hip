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
// Scores are formed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_bf16
// (A = K rows from LDS, B = Q held in registers), so each lane holds 4 keys of a
// single query per 16x16 block: the row max and row sum are in-lane work plus two
// cross-lane steps, and the rescale factor is a per-lane scalar.  P^T stays in
// registers and feeds O^T = V^T P^T directly as the B operand; V is staged in LDS
// transposed ([dim][key]) with keys permuted so that each A fragment is one
// 16-byte LDS read.  K/V tiles are double-buffered in LDS; the next tile's
// global loads are issued before the current tile's MFMAs.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vlca_internal.h"

namespace vlca {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kSchedThreads = 1024;
constexpr int kSchedCache = 8160;  // cu_seqlens entries cached in LDS by the scheduler (LDS <= 64 KB)
constexpr int kAttnThreads = 256;
constexpr int kLdsRow = 72;        // bf16 per LDS tile row: 64 + 8 pad (144 B, 16 B aligned)
constexpr int kTileElems = kTileRows * kLdsRow;

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
  const int n = s_total;
  if (tid == 0) *count = n;
  for (int i = tid; i < kWorklistTail; i += kSchedThreads) items[n + i] = make_int4(-1, -1, 0, 0);
}

// ----------------------------------------------------------------- attention

// Position of tile-local key kk (0..63) inside a V^T LDS row.  Within each
// 32-key half, lane group g (lanes 16g..16g+15) needs keys {4g..4g+3} and
// {16+4g..16+4g+3} as its 8 consecutive MFMA k-slots; storing them contiguously
// makes each V^T fragment a single 16-byte read.
__device__ __forceinline__ int vt_pos(int kk) {
  const int half = kk >> 5, k = kk & 31;
  return (half << 5) | (((k & 15) >> 2) << 3) | ((k >> 4) << 2) | (k & 3);
}

__device__ __forceinline__ uint4 ldg16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ bf16x8 lds_frag(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));  // RNE
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__global__ __launch_bounds__(kAttnThreads) void attention_kernel(const uint16_t* __restrict__ qkv,
                                                                 const int4* __restrict__ items,
                                                                 int n_heads, float sl2,
                                                                 uint16_t* __restrict__ out) {
  __shared__ __attribute__((aligned(16))) uint16_t sK[2][kTileElems];
  __shared__ __attribute__((aligned(16))) uint16_t sV[2][kTileElems];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int g = lane >> 4;   // lane group: k-slot block of the MFMA operands
  const int lq = lane & 15;  // query column of this lane inside the wave's 16
  const int qr = wid * 16 + lq;  // query row inside the 64-row tile
  const int64_t ldq = 3 * n_heads * kHeadDim;
  const int64_t ldo = n_heads * kHeadDim;
  // staging role: 16-byte chunk sc (dims 8sc..8sc+7) of keys 2kp, 2kp+1
  const int sc = tid & 7;
  const int kp = tid >> 3;
  const int vpos = vt_pos(2 * kp);
  const float NEG_INF = -__builtin_inff();

  for (int w = blockIdx.x;; w += gridDim.x) {
    const int item = w / n_heads;
    const int h = w - item * n_heads;
    const int4 it = items[item];
    if (it.x < 0) break;  // sentinel: no more work
    const int qt = it.y;
    const int start = it.z;
    const int len = it.w;
    const int q0 = qt * kTileRows;
    const bool qvalid = q0 + qr < len;
    const int64_t qrow = (int64_t)start + q0 + qr;

    bf16x8 qf0, qf1;
    {
      uint4 a = make_uint4(0, 0, 0, 0), b = make_uint4(0, 0, 0, 0);
      if (qvalid) {
        const uint16_t* p = qkv + qrow * ldq + h * kHeadDim + 8 * g;
        a = ldg16(p);
        b = ldg16(p + 32);
      }
      qf0 = __builtin_bit_cast(bf16x8, a);
      qf1 = __builtin_bit_cast(bf16x8, b);
    }
    const uint16_t* kg = qkv + (int64_t)start * ldq + n_heads * kHeadDim + h * kHeadDim + 8 * sc;
    const uint16_t* vg = kg + n_heads * kHeadDim;

    uint4 rk0, rk1, rv0, rv1;
    auto gload = [&](int j) {
      const int r = j * kTileRows + 2 * kp;
      rk0 = rk1 = rv0 = rv1 = make_uint4(0, 0, 0, 0);
      if (r < len) {
        rk0 = ldg16(kg + r * ldq);
        rv0 = ldg16(vg + r * ldq);
      }
      if (r + 1 < len) {
        rk1 = ldg16(kg + (r + 1) * ldq);
        rv1 = ldg16(vg + (r + 1) * ldq);
      }
    };
    auto sstore = [&](int buf) {
      uint16_t* k = sK[buf];
      *reinterpret_cast<uint4*>(k + (2 * kp) * kLdsRow + 8 * sc) = rk0;
      *reinterpret_cast<uint4*>(k + (2 * kp + 1) * kLdsRow + 8 * sc) = rk1;
      // V^T: row = dim, the two keys of this thread side by side.
      uint32_t* v = reinterpret_cast<uint32_t*>(sV[buf] + (8 * sc) * kLdsRow + vpos);
      constexpr int rs = kLdsRow / 2;
      v[0 * rs] = (rv0.x & 0xffffu) | (rv1.x << 16);
      v[1 * rs] = (rv0.x >> 16) | (rv1.x & 0xffff0000u);
      v[2 * rs] = (rv0.y & 0xffffu) | (rv1.y << 16);
      v[3 * rs] = (rv0.y >> 16) | (rv1.y & 0xffff0000u);
      v[4 * rs] = (rv0.z & 0xffffu) | (rv1.z << 16);
      v[5 * rs] = (rv0.z >> 16) | (rv1.z & 0xffff0000u);
      v[6 * rs] = (rv0.w & 0xffffu) | (rv1.w << 16);
      v[7 * rs] = (rv0.w >> 16) | (rv1.w & 0xffff0000u);
    };

    gload(0);
    sstore(0);
    __syncthreads();

    float m = NEG_INF;  // running max of raw scores (this lane's query)
    float l = 0.f;      // this lane's share of the running denominator
    f32x4 acc[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) acc[d] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int j = 0; j <= qt; ++j) {
      const int buf = j & 1;
      if (j < qt) gload(j + 1);

      // S^T block kb: keys 16kb..16kb+15 of the tile x this wave's 16 queries.
      const uint16_t* kt = sK[buf] + lq * kLdsRow + 8 * g;
      f32x4 s[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        s[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_frag(kt + 16 * kb * kLdsRow), qf0, s[kb], 0, 0, 0);
        s[kb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_frag(kt + 16 * kb * kLdsRow + 32), qf1, s[kb], 0,
                                                        0, 0);
      }
      if (j == qt) {  // diagonal tile: key kk visible to query qr iff kk <= qr
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * kb + 4 * g + r > qr) s[kb][r] = NEG_INF;
      }
      float mt = s[0][0];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mt = fmaxf(mt, s[kb][r]);
      mt = fmaxf(mt, __shfl_xor(mt, 16));
      mt = fmaxf(mt, __shfl_xor(mt, 32));
      const float mn = fmaxf(m, mt);
      const float alpha = __builtin_amdgcn_exp2f((m - mn) * sl2);
      const float moff = -mn * sl2;
      m = mn;

      uint32_t pw[8];  // P^T as bf16 pairs: pw[4*half + 2*blk + i]
      float ls = 0.f;
#pragma unroll
      for (int half = 0; half < 2; ++half)
#pragma unroll
        for (int blk = 0; blk < 2; ++blk)
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const f32x4& sv = s[2 * half + blk];
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i], sl2, moff));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[2 * i + 1], sl2, moff));
            const uint32_t wv = pack_bf16x2(p0, p1);
            pw[4 * half + 2 * blk + i] = wv;
            ls += bf16lo(wv) + bf16hi(wv);  // denominator from the rounded weights
          }
      l = l * alpha + ls;
#pragma unroll
      for (int d = 0; d < 4; ++d) acc[d] *= alpha;

      const uint16_t* vt = sV[buf] + lq * kLdsRow + 8 * g;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const uint4 pv = make_uint4(pw[4 * half], pw[4 * half + 1], pw[4 * half + 2], pw[4 * half + 3]);
        const bf16x8 pb = __builtin_bit_cast(bf16x8, pv);
#pragma unroll
        for (int d = 0; d < 4; ++d)
          acc[d] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lds_frag(vt + 16 * d * kLdsRow + 32 * half), pb, acc[d],
                                                           0, 0, 0);
      }

      if (j < qt) sstore(buf ^ 1);
      __syncthreads();
    }

    float lt = l + __shfl_xor(l, 16);
    lt += __shfl_xor(lt, 32);
    const float inv = 1.0f / lt;
    if (qvalid) {
      uint16_t* o = out + qrow * ldo + h * kHeadDim + 4 * g;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        uint2 wv;
        wv.x = pack_bf16x2(acc[d][0] * inv, acc[d][1] * inv);
        wv.y = pack_bf16x2(acc[d][2] * inv, acc[d][3] * inv);
        *reinterpret_cast<uint2*>(o + 16 * d) = wv;
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

hipError_t launch_attention(const void* qkv, const int4* items, int n_heads, float scale_log2e, void* out, int grid,
                            hipStream_t stream) {
  hipLaunchKernelGGL(attention_kernel, dim3(grid), dim3(kAttnThreads), 0, stream,
                     static_cast<const uint16_t*>(qkv), items, n_heads, scale_log2e, static_cast<uint16_t*>(out));
  return hipGetLastError();
}

}  // namespace vlca
