// gfx950 kernels for the attention's neighbours in the packed Transformer layer
// (cti2026 README, Transformer-layer listing: the residual is kept, x goes
// through LayerNorm and Linear_qkv, the varlen attention runs over the user
// offsets, and the output projection is added back to the residual), with the
// elementwise work fused into the matrix products around the attention:
//  * ln_proj_kernel: qkv = LayerNorm(x) W_qkv^T + b_qkv -- each row is
//    normalised once, in registers, and the normalised bf16 row feeds every
//    output column the workgroup computes; it never touches HBM;
//  * res_proj_kernel: y = residual + attn W_out^T + b_out -- bias and residual
//    are added to the fp32 accumulators before the one rounding to bf16.
// Both are bf16 products with fp32 accumulation on v_mfma_f32_16x16x32_bf16
// over d_in = 512 (the model width), formed transposed (C^T = W A^T) so that a
// lane holds four consecutive output columns of one row.
//
// ln_proj_kernel: the input side is stationary.  A workgroup of eight waves owns
// 128 rows; each pair of waves owns 32 rows and splits k in halves, each wave
// loading its 32 rows x 256 columns straight into registers as MFMA operands
// (64 VGPRs), normalising them there, and keeping them while the workgroup
// sweeps its column chunks.  The weight side streams through a two-slot LDS
// ring by LDS DMA (per step 128 output columns x 64 k of each half, in
// nn.Linear's [out, in] layout); a weight fragment read from LDS feeds two
// MFMAs.  At a chunk's end the pair hands partial sums over through LDS and
// each wave finishes half of the chunk's columns; the finished rows are staged
// row-major in LDS and leave as whole 128-byte lines.  The waves of half 0 issue
// every weight copy and no store; the waves of half 1 issue every store and no
// copy: a barrier only has to wait for the copies of the waves that issued
// them, so the stores' completion never holds the ring up.  The host picks how
// many 128-column chunks a workgroup sweeps, so that the per-row work (loading
// and LayerNorm) is amortised over as many columns as the grid's fill allows.
//
// res_proj_kernel: a workgroup computes a 64-row x 128-column output tile, the
// input's 64 x 64 and the weight's 128 x 64 k-chunks in a two-stage LDS ring,
// both by LDS DMA.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "vlca_device.h"
#include "vlca_internal.h"

namespace vlca {
namespace {

constexpr int kDin = 512;                      // input width (d_model)
constexpr int kHalf = kDin / 2;                // k range of one wave of a pair
constexpr int kThreads = 512;                  // 8 waves: 4 row groups x 2 k halves
constexpr int kWaveRows = 32;                  // rows of a row group
constexpr int kPBM = 4 * kWaveRows;            // rows per workgroup
constexpr int kPBN = 128;                      // output columns per chunk
constexpr int kPBK = 64;                       // k per half-stage
constexpr int kStepsPerChunk = kHalf / kPBK;   // 4
constexpr int kKF = kHalf / 32;                // 32-wide k fragments a wave holds per row: 8
constexpr int kHalfStageBytes = kPBN * kPBK * 2;  // 16 KB: 128 weight rows of 128 B
constexpr int kStepBytes = 2 * kHalfStageBytes;   // both halves of one step
constexpr int kRedBytes = 8 * 4 * 2 * 64 * 16;    // partial sums handed over: 8 waves x 8 KB
constexpr int kMaxChunksPerBlock = 16;            // bounds the block's bias slice in LDS

__device__ __forceinline__ float lo_f32(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float hi_f32(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }

typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));

// a.lo*b.lo + a.hi*b.hi + c, the bf16 products exact, summed in fp32.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v, a), __builtin_bit_cast(bf16x2v, b), c, false);
}

// Sum over the four lanes that hold pieces of one row (lanes lq, lq+16, lq+32, lq+48).
__device__ __forceinline__ float row_sum(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// out = LayerNorm(x) W^T + bias (gamma, beta, eps over the 512 columns of each
// row).  Grid: one workgroup per (128-row block, group of chunks_per_block
// 128-column chunks (at most kMaxChunksPerBlock)), numbered so that the groups
// of one row block share id % 8: workgroups are dealt to the 8 XCDs round-robin,
// so they sit on one XCD and read the block's rows of x through one L2 (with
// the plain (x, y) grid they sat on four).  Ids past the last row block exit.
//
// Wave w: row group rg = w % 4 (rows m0 .. m0 + 31), k half h = w / 4 (columns
// 256 h .. 256 h + 255 of A and W).  The two waves of a row group form partial
// products over their halves; at the end of a chunk each hands the partner the
// half of the columns the partner finishes (h = 0 finishes columns 0..63 of the
// chunk, h = 1 columns 64..127) through LDS, and half 0 hands its finished bf16
// values to half 1, which stores both.  A step stages, for both halves, 128
// weight rows x 64 k; four steps make a chunk.
__global__ __launch_bounds__(kThreads) void ln_proj_kernel(const uint16_t* __restrict__ x,
                                                           const uint16_t* __restrict__ gamma,
                                                           const uint16_t* __restrict__ beta, float eps,
                                                           const uint16_t* __restrict__ w,
                                                           const uint16_t* __restrict__ bias, uint16_t* __restrict__ out,
                                                           int T, int N, int chunks_per_block, int groups) {
  // id = (rb / 8) * 8 groups + 8 cg + rb % 8
  const int bid = blockIdx.x, q = bid >> 3;
  const int row_block = (q / groups) * 8 + (bid & 7), group = q - (q / groups) * groups;
  if (row_block * kPBM >= T) return;  // uniform: a padding workgroup
  __shared__ __attribute__((aligned(1024))) char ring[2 * kStepBytes];
  __shared__ __attribute__((aligned(16))) char red[kRedBytes];
  __shared__ __attribute__((aligned(16))) uint16_t s_bias[kMaxChunksPerBlock * kPBN];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (LDS DMA bases are scalars)
  const int rg = wid & 3, h = wid >> 2;
  const int lq = lane & 15, g = lane >> 4;
  const int m0 = row_block * kPBM + kWaveRows * rg;  // this wave's first row
  const int c_begin = group * chunks_per_block;
  const int c_end = min(c_begin + chunks_per_block, N / kPBN);
  const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)ring);

  // Step (chunk c, step j) into ring slot `slot`, issued by the waves of half 0
  // only: wave (rg, 0) copies weight rows 32 rg .. 32 rg + 31 of both halves, 1
  // KB (8 rows x 128 B) per instruction.  Chunk q (16 B) of staged row r lives at
  // chunk q ^ (r % 8).
  auto issue_step = [&](int slot, int c, int j) {
    if (h != 0) return;
#pragma unroll
    for (int hh = 0; hh < 2; ++hh)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 32 * rg + 8 * i + (lane >> 3);
        const uint32_t off =
            (uint32_t)(((c * kPBN + r) * kDin + kHalf * hh + kPBK * j) * 2 + 16 * ((lane & 7) ^ (r & 7)));
        copy_to_lds(w, off, lds0 + slot * kStepBytes + hh * kHalfStageBytes + 1024 * (4 * rg + i));
      }
  };
  // A barrier after which every copy issued so far has landed: the waves that
  // issue copies wait for their own, the others (which issue the stores) wait
  // for nothing but their LDS operations.
  auto step_barrier = [&]() {
    if (h == 0)
      wait_and_barrier<0>();
    else
      lds_barrier();
  };
  issue_step(0, c_begin, 0);  // lands while the rows load
  for (int i = tid; i < (c_end - c_begin) * kPBN; i += kThreads) s_bias[i] = bias[c_begin * kPBN + i];

  // The wave's half rows as MFMA operands: fragment kf of row block rb holds, in
  // lane (g, lq), row m0 + 16 rb + lq, columns 256 h + 32 kf + 8 g .. + 7.  Rows
  // past T repeat row T - 1 (computed, never stored).
  u32x4 a[2][kKF];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = min(m0 + 16 * rb + lq, T - 1);
    const uint16_t* xr = x + (int64_t)row * kDin + kHalf * h + 8 * g;
#pragma unroll
    for (int kf = 0; kf < kKF; ++kf) a[rb][kf] = *reinterpret_cast<const u32x4*>(xr + 32 * kf);
  }

  {
    // Row statistics: each wave sums its half of every row (sum and sum of
    // squares of the bf16 values, one dot2 per pair), the halves meet in LDS.
    // Where the mean dominates the spread of some row of the workgroup
    // (mean^2 > 16 var) the variance is taken again, for every row, as the mean
    // square deviation, which has no cancellation.
    float2* const st = reinterpret_cast<float2*>(red);  // [h][rg][rb][lq]
    const uint32_t ones = 0x3F803F80u;
    float part_s[2], part_q[2];
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float s0 = 0.f, s1 = 0.f, q0 = 0.f, q1 = 0.f;
#pragma unroll
      for (int kf = 0; kf < kKF; ++kf) {
        const u32x4 v = a[rb][kf];
        s0 = dot2(v[0], ones, s0);
        s1 = dot2(v[1], ones, s1);
        s0 = dot2(v[2], ones, s0);
        s1 = dot2(v[3], ones, s1);
        q0 = dot2(v[0], v[0], q0);
        q1 = dot2(v[1], v[1], q1);
        q0 = dot2(v[2], v[2], q0);
        q1 = dot2(v[3], v[3], q1);
      }
      part_s[rb] = row_sum(s0 + s1);
      part_q[rb] = row_sum(q0 + q1);
      if (g == 0) st[((h * 4 + rg) * 2 + rb) * 16 + lq] = make_float2(part_s[rb], part_q[rb]);
    }
    lds_barrier();
    float mean[2], var[2];
    int need = 0;
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      const float2 o = st[(((1 - h) * 4 + rg) * 2 + rb) * 16 + lq];
      // The same order of addition in both waves of the pair: half 0 first.
      const float s = h == 0 ? part_s[rb] + o.x : o.x + part_s[rb];
      const float q = h == 0 ? part_q[rb] + o.y : o.y + part_q[rb];
      mean[rb] = s * (1.0f / kDin);
      var[rb] = fmaxf(q * (1.0f / kDin) - mean[rb] * mean[rb], 0.f);
      need |= mean[rb] * mean[rb] > 16.f * var[rb];
    }
    if (__syncthreads_or(need)) {
      float part_d[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int kf = 0; kf < kKF; ++kf) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float u = lo_f32(a[rb][kf][e]) - mean[rb], t = hi_f32(a[rb][kf][e]) - mean[rb];
            d0 = __builtin_fmaf(u, u, d0);
            d1 = __builtin_fmaf(t, t, d1);
          }
        }
        part_d[rb] = row_sum(d0 + d1);
        if (g == 0) st[256 + ((h * 4 + rg) * 2 + rb) * 16 + lq] = make_float2(part_d[rb], 0.f);
      }
      lds_barrier();
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const float o = st[256 + (((1 - h) * 4 + rg) * 2 + rb) * 16 + lq].x;
        var[rb] = (h == 0 ? part_d[rb] + o : o + part_d[rb]) * (1.0f / kDin);
      }
    }
    // y = ((x - mean) rstd) gamma + beta, rounded to bf16 in place.
#pragma unroll
    for (int kf = 0; kf < kKF; ++kf) {
      const int k = kHalf * h + 32 * kf + 8 * g;
      const bf16x8 gb = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(gamma + k));
      const bf16x8 bb = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(beta + k));
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const float rstd = __builtin_amdgcn_rsqf(var[rb] + eps);
        const float nm = -mean[rb] * rstd;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t v = a[rb][kf][e];
          const float y0 = __builtin_fmaf(__builtin_fmaf(lo_f32(v), rstd, nm), (float)gb[2 * e], (float)bb[2 * e]);
          const float y1 =
              __builtin_fmaf(__builtin_fmaf(hi_f32(v), rstd, nm), (float)gb[2 * e + 1], (float)bb[2 * e + 1]);
          a[rb][kf][e] = pack_bf16x2(y0, y1);
        }
      }
    }
  }

  // Partial sums handed over at a chunk's end: wave (rg, h) writes the four
  // column blocks its partner finishes, the partner reads them at the next
  // barrier.  [rg][h][cb 0..3][rb][lane] of f32x4.
  f32x4* const red_out = reinterpret_cast<f32x4*>(red) + (rg * 2 + h) * 512;
  const f32x4* const red_in = reinterpret_cast<const f32x4*>(red) + (rg * 2 + (1 - h)) * 512;
  // The finished bf16 rows of the row group, staged row-major in its first 8 KB
  // of the partial-sum buffer once both waves have read their partials: 32 rows
  // x 256 bytes, 16-byte chunk q of row r at chunk q ^ (r % 16) (conflict-free
  // both ways), so that half 1 writes them out as whole 128-byte lines.
  char* const stage = red + rg * 16384;
  // This wave finishes column blocks 4 h .. 4 h + 3 of a chunk: lane (g, lq) of
  // block (cb, rb) holds row m0 + 16 rb + lq, columns 128 c + 16 (4 h + cb) + 4 g.
  f32x4 acc[8][2];
  u32x2 pend[4][2];  // finished bf16 values, until they are staged
  int pend_chunk = -1, staged_chunk = -1;
  auto finish = [&](int c) {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const u32x2 bw = *(const LDS u32x2*)(s_bias + (c - c_begin) * kPBN + 16 * (4 * h + cb) + 4 * g);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const f32x4 o = red_in[(cb * 2 + rb) * 64 + lane];
        const f32x4 mine = h == 0 ? acc[cb][rb] : acc[4 + cb][rb];  // no runtime index into acc
        // Half 0's partial first in both waves: the sum does not depend on which wave finishes.
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = h == 0 ? mine[e] + o[e] : o[e] + mine[e];
        pend[cb][rb] = u32x2{pack_bf16x2(v[0] + lo_f32(bw[0]), v[1] + hi_f32(bw[0])),
                             pack_bf16x2(v[2] + lo_f32(bw[1]), v[3] + hi_f32(bw[1]))};
      }
    }
    pend_chunk = c;
  };
  // Both waves of the row group stage their finished columns (after the barrier
  // that follows the partial-sum reads).
  auto stage_pending = [&]() {
#pragma unroll
    for (int cb = 0; cb < 4; ++cb)
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int r = 16 * rb + lq;
        const int byte = 128 * h + 32 * cb + 8 * g;  // inside the row's 256 bytes
        *(LDS u32x2*)(stage + r * 256 + ((((byte >> 4) ^ (r & 15)) << 4) | (byte & 15))) = pend[cb][rb];
      }
    staged_chunk = pend_chunk;
    pend_chunk = -1;
  };
  // Half 1 writes the staged rows out: per instruction four rows of 256 bytes,
  // 16 bytes a lane.  Plain stores: the attention that follows in the layer reads
  // qkv, and finds it in the caches (non-temporal stores made the sub-block 5%
  // slower, though this kernel alone 2-6% faster).
  auto store_staged = [&]() {
    if (h != 0) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 4 * i + (lane >> 4), q = lane & 15;
        const u32x4 v = *(const LDS u32x4*)(stage + r * 256 + ((q ^ (r & 15)) << 4));
        const int row = m0 + r;
        if (row < T) *reinterpret_cast<u32x4*>(out + (int64_t)row * N + staged_chunk * kPBN + 8 * q) = v;
      }
    }
    staged_chunk = -1;
  };

  int slot = 0;
#pragma unroll 1
  for (int c = c_begin; c < c_end; ++c) {
#pragma unroll
    for (int j = 0; j < kStepsPerChunk; ++j) {
      // Step (c, j) landed for every wave; the other slot is free; the previous
      // chunk's partial sums (j == 0) or staged rows (j == 2) are in LDS, and
      // at j == 1 every wave is past its partial-sum reads.
      step_barrier();
      if (j == 0 && c > c_begin) finish(c - 1);
      if (j == 1 && pend_chunk >= 0) stage_pending();
      if (j == 2 && staged_chunk >= 0) store_staged();
      if (j + 1 < kStepsPerChunk)
        issue_step(slot ^ 1, c, j + 1);
      else if (c + 1 < c_end)
        issue_step(slot ^ 1, c + 1, 0);
      if (j == 0) {
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) acc[cb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      // All sixteen weight fragments of the step are requested before the first
      // product: the eight waves leave the barrier together, and LDS latency is
      // only hidden if each wave has its whole step's reads in flight.
      const LDS char* w_st = (const LDS char*)ring + slot * kStepBytes + h * kHalfStageBytes;
      bf16x8 wf[2][8];
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int cb = 0; cb < 8; ++cb) {
          const int r = 16 * cb + lq;
          wf[ks][cb] = lds_b128(w_st, r * 128 + (((4 * ks + g) ^ (r & 7)) << 4));
        }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
#pragma unroll
        for (int cb = 0; cb < 8; ++cb)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb)
            acc[cb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                wf[ks][cb], __builtin_bit_cast(bf16x8, a[rb][2 * j + ks]), acc[cb][rb], 0, 0, 0);
      if (j == kStepsPerChunk - 1) {  // hand the partner its column blocks
#pragma unroll
        for (int cb = 0; cb < 4; ++cb)
#pragma unroll
          for (int rb = 0; rb < 2; ++rb) red_out[(cb * 2 + rb) * 64 + lane] = h == 0 ? acc[4 + cb][rb] : acc[cb][rb];
      }
      slot ^= 1;
    }
  }
  step_barrier();
  if (staged_chunk >= 0) store_staged();  // a one-chunk run has none; a longer run stored its last but one at j == 2
  finish(c_end - 1);
  lds_barrier();  // every partial-sum read is done
  stage_pending();
  lds_barrier();  // the staged rows are visible
  store_staged();
}

// Chunks per workgroup: the fewest workgroup-rounds x (row work + chunks), one
// workgroup per CU, the row work (loading and LayerNorm) counted as `row_cost`
// chunks.
int chunks_per_block(int T, int N, int cus, float row_cost) {
  const int nchunks = N / kPBN;
  const int64_t row_blocks = (static_cast<int64_t>(T) + kPBM - 1) / kPBM;
  int best = 1;
  double best_t = 1e300;
  for (int cpb = 1; cpb <= std::min(nchunks, kMaxChunksPerBlock); ++cpb) {
    const int groups = (nchunks + cpb - 1) / cpb;
    if (cpb > 1 && (nchunks + cpb - 2) / (cpb - 1) == groups) continue;  // same grid as a smaller cpb
    const int64_t blocks = row_blocks * groups;
    const int64_t rounds = (blocks + std::max(cus, 1) - 1) / std::max(cus, 1);
    const double t = static_cast<double>(rounds) * (row_cost + cpb);
    if (t <= best_t) {
      best_t = t;
      best = cpb;
    }
  }
  return best;
}

constexpr int kTBM = 64;                          // res_proj_kernel: output rows per workgroup
constexpr int kTBN = 128;                         // output columns per workgroup
constexpr int kTBK = 64;                          // k-chunk
constexpr int kTAChunkBytes = kTBM * kTBK * 2;    // 8 KB: 64 input rows of 128 B
constexpr int kTWChunkBytes = kTBN * kTBK * 2;    // 16 KB: 128 weight rows of 128 B
constexpr int kTStageBytes = kTAChunkBytes + kTWChunkBytes;

// y = residual + A W^T + bias over one 64 x 128 output tile.
__global__ __launch_bounds__(256) void res_proj_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ w,
                                                       const uint16_t* __restrict__ bias,
                                                       const uint16_t* __restrict__ residual,
                                                       uint16_t* __restrict__ out, int T, int N) {
  __shared__ __attribute__((aligned(1024))) char ring_lds[2 * kTStageBytes];
  LDS char* const st0 = (LDS char*)ring_lds;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (LDS DMA bases are scalars)
  const int lq = lane & 15, g = lane >> 4;
  const int m0 = blockIdx.x * kTBM;  // first row
  const int n0 = blockIdx.y * kTBN;  // first output column
  const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)st0);

  // k-chunk kc into the stage at byte offset so, both operands by LDS DMA: W
  // 128 rows x 128 B (4 wave instructions per wave), A 64 rows x 128 B (2 per
  // wave).  Chunk c (16 B) of tile row r lives at chunk c ^ (r % 8).
  auto issue = [&](uint32_t so, int kc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 32 * wid + 8 * i + (lane >> 3);
      const uint32_t off = (uint32_t)(((int64_t)(n0 + r) * kDin + kc * kTBK) * 2 + 16 * ((lane & 7) ^ (r & 7)));
      copy_to_lds(w, off, lds0 + so + kTAChunkBytes + 1024 * (4 * wid + i));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 16 * wid + 8 * i + (lane >> 3);
      const int row = min(m0 + r, T - 1);
      const uint32_t off = (uint32_t)(((int64_t)(row - m0) * kDin + kc * kTBK) * 2 + 16 * ((lane & 7) ^ (r & 7)));
      copy_to_lds(x + (int64_t)m0 * kDin, off, lds0 + so + 1024 * (2 * wid + i));
    }
  };

  // Waves 2 x 2: rows 32 wr .. +31, columns 64 wc .. +63.  C^T block (cb, rb):
  // lane (g, lq) holds output row 32 wr + 16 rb + lq, columns 64 wc + 16 cb + 4 g + 0..3.
  const int wr = wid >> 1, wc = wid & 1;
  f32x4 acc[4][2];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) acc[cb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  issue(0, 0);
  constexpr int kChunks = kDin / kTBK;
#pragma unroll 1
  for (int kc = 0; kc < kChunks; ++kc) {
    wait_and_barrier<0>();  // chunk kc landed everywhere; the other stage is free
    if (kc + 1 < kChunks) issue(((kc + 1) & 1) * kTStageBytes, kc + 1);
    const LDS char* a_st = st0 + (kc & 1) * kTStageBytes;
    const LDS char* w_st = a_st + kTAChunkBytes;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {  // 32 k per MFMA
      bf16x8 bfr[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int r = 32 * wr + 16 * rb + lq;
        bfr[rb] = lds_b128(a_st, r * 128 + (((4 * ks + g) ^ (r & 7)) << 4));
      }
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) {
        const int r = 64 * wc + 16 * cb + lq;
        const bf16x8 afr = lds_b128(w_st, r * 128 + (((4 * ks + g) ^ (r & 7)) << 4));
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          acc[cb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afr, bfr[rb], acc[cb][rb], 0, 0, 0);
      }
    }
  }

  // Epilogue: + bias + residual, one rounding to bf16, staged row-major in the
  // ring (64 rows x 256 bytes, 16-byte chunk q of row r at chunk q ^ (r % 16))
  // and written out as whole 128-byte lines.  The workgroup reads its tile's
  // residual before the barrier and writes the tile after it, so y may alias
  // the residual.
  lds_barrier();  // every wave is done with the ring
  LDS char* const stage = st0;
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int r = 32 * wr + 16 * rb + lq;
    const int row = min(m0 + r, T - 1);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int cl = 64 * wc + 16 * cb + 4 * g;  // column inside the tile
      const u32x2 bw = *reinterpret_cast<const u32x2*>(bias + n0 + cl);
      const u32x2 rw = *reinterpret_cast<const u32x2*>(residual + (int64_t)row * N + n0 + cl);
      const float v0 = acc[cb][rb][0] + lo_f32(bw[0]) + lo_f32(rw[0]);
      const float v1 = acc[cb][rb][1] + hi_f32(bw[0]) + hi_f32(rw[0]);
      const float v2 = acc[cb][rb][2] + lo_f32(bw[1]) + lo_f32(rw[1]);
      const float v3 = acc[cb][rb][3] + hi_f32(bw[1]) + hi_f32(rw[1]);
      const int byte = 2 * cl;
      *(LDS u32x2*)(stage + r * 256 + ((((byte >> 4) ^ (r & 15)) << 4) | (byte & 15))) =
          u32x2{pack_bf16x2(v0, v1), pack_bf16x2(v2, v3)};
    }
  }
  lds_barrier();  // the staged tile is visible; every residual read is done
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // four rows of 256 bytes per wave instruction
    const int r = 16 * i + (tid >> 4), q = tid & 15;
    const u32x4 v = *(const LDS u32x4*)(stage + r * 256 + ((q ^ (r & 15)) << 4));
    if (m0 + r < T)
      __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(out + (int64_t)(m0 + r) * N + n0 + 8 * q));
  }
}

}  // namespace

hipError_t launch_ln_qkv(const void* x, const void* gamma, const void* beta, float eps, const void* w_qkv,
                         const void* b_qkv, int T, int N, void* qkv, int cus, hipStream_t stream) {
  const int cpb = chunks_per_block(T, N, cus, 0.75f);
  const int groups = (N / kPBN + cpb - 1) / cpb;
  const int64_t row_blocks = (static_cast<int64_t>(T) + kPBM - 1) / kPBM;
  const int64_t grid = (row_blocks + 7) / 8 * 8 * groups;  // row blocks padded to a multiple of 8
  hipLaunchKernelGGL(ln_proj_kernel, dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, stream,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(gamma),
                     static_cast<const uint16_t*>(beta), eps, static_cast<const uint16_t*>(w_qkv),
                     static_cast<const uint16_t*>(b_qkv), static_cast<uint16_t*>(qkv), T, N, cpb, groups);
  return hipGetLastError();
}

hipError_t launch_out_residual(const void* attn, const void* w_out, const void* b_out, const void* residual, int T,
                               int N, void* y, int, hipStream_t stream) {
  hipLaunchKernelGGL(res_proj_kernel, dim3((T + kTBM - 1) / kTBM, N / kTBN), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(attn), static_cast<const uint16_t*>(w_out),
                     static_cast<const uint16_t*>(b_out), static_cast<const uint16_t*>(residual),
                     static_cast<uint16_t*>(y), T, N);
  return hipGetLastError();
}

}  // namespace vlca
