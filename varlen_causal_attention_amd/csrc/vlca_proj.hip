// gfx950 kernels for the attention's neighbours in the packed Transformer layer
// (cti2026 README, Transformer-layer listing: residual = x; x = LayerNorm(x);
// qkv = Linear_qkv(x); attn_out = FlashAttention_Varlen(qkv, user_offsets);
// x = residual + Linear_out(attn_out)), with the elementwise work fused into the
// matrix products that surround it:
//  * proj_kernel<true, false>: qkv = LayerNorm(x) W_qkv^T + b_qkv -- the
//    LayerNorm (row mean and variance over d_in, then gamma, beta) is applied
//    while x is staged into LDS for the product, so the normalised rows never
//    touch HBM;
//  * proj_kernel<false, true>: y = residual + attn W_out^T + b_out -- bias and
//    residual are added to the accumulators before the one rounding to bf16.
// Both are bf16 products with fp32 accumulation on v_mfma_f32_16x16x32_bf16,
// d_in = 512 (the model's width): a workgroup computes a 64-row x 128-column
// output tile, with the weight's 128 x 64 and the input's 64 x 64 k-chunks in a
// two-stage LDS ring (weights by LDS DMA, in nn.Linear's [out, in] layout).  The
// product is formed transposed (C^T = W A^T), so a lane holds four consecutive
// output columns of one row and stores them as one 8-byte write.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vlca_device.h"
#include "vlca_internal.h"

namespace vlca {
namespace {

constexpr int kDin = 512;          // input width (d_model)
constexpr int kPBM = 64;           // output rows per workgroup
constexpr int kPBN = 128;          // output columns per workgroup
constexpr int kPBK = 64;           // k-chunk
constexpr int kAChunkBytes = kPBM * kPBK * 2;  // 8 KB: 64 rows of 128 B
constexpr int kWChunkBytes = kPBN * kPBK * 2;  // 16 KB: 128 rows of 128 B
constexpr int kPStageBytes = kAChunkBytes + kWChunkBytes;

__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// kLN: A = LayerNorm(x) (gamma, beta, eps over the 512 columns of each row);
// kRes: out = residual + A W^T + bias, else A W^T + bias.
template <bool kLN, bool kRes>
__global__ __launch_bounds__(256) void proj_kernel(const uint16_t* __restrict__ x, const uint16_t* __restrict__ gamma,
                                                   const uint16_t* __restrict__ beta, float eps,
                                                   const uint16_t* __restrict__ w, const uint16_t* __restrict__ bias,
                                                   const uint16_t* __restrict__ residual, uint16_t* __restrict__ out,
                                                   int T, int N) {
  __shared__ __attribute__((aligned(1024))) char ring_lds[2 * kPStageBytes];
  __shared__ float s_stats[2 * kPBM];  // mean, rstd per row
  LDS char* const st0 = (LDS char*)ring_lds;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (LDS DMA bases are scalars)
  const int lq = lane & 15, g = lane >> 4;
  const int m0 = blockIdx.x * kPBM;  // first row
  const int n0 = blockIdx.y * kPBN;  // first output column
  const uint32_t lds0 = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)st0);

  // Row statistics (LayerNorm): 4 threads per row, 128 columns each, kept in
  // registers for the two passes (mean, then the mean square deviation).
  if constexpr (kLN) {
    const int r = tid >> 2, q = tid & 3;
    const int row = min(m0 + r, T - 1);
    const uint16_t* xr = x + (int64_t)row * kDin + 128 * q;
    u32x4 v[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = *reinterpret_cast<const u32x4*>(xr + 8 * i);
    float sum = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bf16x8 b = __builtin_bit_cast(bf16x8, v[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) sum += (float)b[e];
    }
    sum += __shfl_xor(sum, 1);
    sum += __shfl_xor(sum, 2);
    const float mean = sum * (1.0f / kDin);
    float ss = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bf16x8 b = __builtin_bit_cast(bf16x8, v[i]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float d = (float)b[e] - mean;
        ss = __builtin_fmaf(d, d, ss);
      }
    }
    ss += __shfl_xor(ss, 1);
    ss += __shfl_xor(ss, 2);
    if (q == 0) {
      s_stats[2 * r] = mean;
      s_stats[2 * r + 1] = __builtin_amdgcn_rsqf(ss * (1.0f / kDin) + eps);
    }
    __syncthreads();
  }

  // Staging of k-chunk kc into the stage at byte offset so.  W: 128 rows x 128 B
  // by LDS DMA, 1 KB (8 rows) per wave instruction, 4 per wave.  A: with
  // LayerNorm, 16 elements per thread through registers (normalised, rounded to
  // bf16, written swizzled); without, by LDS DMA (2 per wave).
  // Chunk c (16 B) of tile row r lives at chunk c ^ (r % 8).
  auto issue_w = [&](uint32_t so, int kc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 32 * wid + 8 * i + (lane >> 3);  // weight row inside the 128-row block
      const int n = min(n0 + r, N - 1);
      const uint32_t off = (uint32_t)(((int64_t)n * kDin + kc * kPBK) * 2 + 16 * ((lane & 7) ^ (r & 7)));
      copy_to_lds(w, off, lds0 + so + kAChunkBytes + 1024 * (4 * wid + i));
    }
  };
  auto issue_a_dma = [&](uint32_t so, int kc) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = 16 * wid + 8 * i + (lane >> 3);
      const int row = min(m0 + r, T - 1);
      const uint32_t off = (uint32_t)(((int64_t)(row - m0) * kDin + kc * kPBK) * 2 + 16 * ((lane & 7) ^ (r & 7)));
      copy_to_lds(x + (int64_t)m0 * kDin, off, lds0 + so + 1024 * (2 * wid + i));
    }
  };
  // LayerNorm path: thread t loads row t/4, chunks 2(t%4), 2(t%4)+1 of the k-chunk.
  const int ar = tid >> 2, ac = 2 * (tid & 3);
  const int arow = min(m0 + ar, T - 1);
  auto load_a = [&](int kc, u32x4 (&v)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
      v[i] = *reinterpret_cast<const u32x4*>(x + (int64_t)arow * kDin + kc * kPBK + 8 * (ac + i));
  };
  auto store_a = [&](uint32_t so, int kc, const u32x4 (&v)[2]) {
    const float mean = s_stats[2 * ar], rstd = s_stats[2 * ar + 1];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int k = kc * kPBK + 8 * (ac + i);
      const bf16x8 xb = __builtin_bit_cast(bf16x8, v[i]);
      const bf16x8 gb = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(gamma + k));
      const bf16x8 bb = __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(beta + k));
      uint32_t p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float y0 = __builtin_fmaf(((float)xb[2 * e] - mean) * rstd, (float)gb[2 * e], (float)bb[2 * e]);
        const float y1 = __builtin_fmaf(((float)xb[2 * e + 1] - mean) * rstd, (float)gb[2 * e + 1],
                                        (float)bb[2 * e + 1]);
        p[e] = pack_bf16x2(y0, y1);
      }
      *(LDS u32x4*)(st0 + so + ar * 128 + (((ac + i) ^ (ar & 7)) << 4)) = u32x4{p[0], p[1], p[2], p[3]};
    }
  };

  // Waves 2 x 2: rows 32 wr .. +31 (row blocks 2 wr, 2 wr + 1), columns 64 wc ..
  // +63 (column blocks 4 wc .. 4 wc + 3).  C^T block (cb, rb): lane (g, lq) holds
  // output row 16 rb + lq, columns 16 cb + 4 g + 0..3.
  const int wr = wid >> 1, wc = wid & 1;
  f32x4 acc[4][2];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb)
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) acc[cb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};

  u32x4 av[2];
  issue_w(0, 0);
  if constexpr (kLN) {
    load_a(0, av);
    store_a(0, 0, av);
  } else {
    issue_a_dma(0, 0);
  }
  constexpr int kChunks = kDin / kPBK;
#pragma unroll 1
  for (int kc = 0; kc < kChunks; ++kc) {
    const uint32_t so = (kc & 1) * kPStageBytes;
    const uint32_t sn = ((kc + 1) & 1) * kPStageBytes;
    wait_and_barrier<0>();  // chunk kc landed everywhere; stage sn is free
    const bool more = kc + 1 < kChunks;
    if (more) {
      issue_w(sn, kc + 1);
      if constexpr (kLN)
        load_a(kc + 1, av);
      else
        issue_a_dma(sn, kc + 1);
    }
    const LDS char* a_st = st0 + so;
    const LDS char* w_st = st0 + so + kAChunkBytes;
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
    if constexpr (kLN) {
      if (more) store_a(sn, kc + 1, av);
    }
  }

  // Epilogue: + bias (+ residual), one rounding to bf16, 8-byte stores.
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int row = m0 + 32 * wr + 16 * rb + lq;
    if (row >= T) continue;
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) {
      const int col = n0 + 64 * wc + 16 * cb + 4 * g;
      if (col >= N) continue;
      const u32x2 bw = *reinterpret_cast<const u32x2*>(bias + col);
      float v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        v[e] = acc[cb][rb][e] + bf16_to_f32((uint16_t)(bw[e >> 1] >> (16 * (e & 1))));
      if constexpr (kRes) {
        const u32x2 rw = *reinterpret_cast<const u32x2*>(residual + (int64_t)row * N + col);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += bf16_to_f32((uint16_t)(rw[e >> 1] >> (16 * (e & 1))));
      }
      *reinterpret_cast<u32x2*>(out + (int64_t)row * N + col) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
    }
  }
}

}  // namespace

hipError_t launch_ln_qkv(const void* x, const void* gamma, const void* beta, float eps, const void* w_qkv,
                         const void* b_qkv, int T, int N, void* qkv, hipStream_t stream) {
  hipLaunchKernelGGL((proj_kernel<true, false>), dim3((T + kPBM - 1) / kPBM, N / kPBN), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(gamma),
                     static_cast<const uint16_t*>(beta), eps, static_cast<const uint16_t*>(w_qkv),
                     static_cast<const uint16_t*>(b_qkv), nullptr, static_cast<uint16_t*>(qkv), T, N);
  return hipGetLastError();
}

hipError_t launch_out_residual(const void* attn, const void* w_out, const void* b_out, const void* residual, int T,
                               int N, void* y, hipStream_t stream) {
  hipLaunchKernelGGL((proj_kernel<false, true>), dim3((T + kPBM - 1) / kPBM, N / kPBN), dim3(256), 0, stream,
                     static_cast<const uint16_t*>(attn), nullptr, nullptr, 0.f, static_cast<const uint16_t*>(w_out),
                     static_cast<const uint16_t*>(b_out), static_cast<const uint16_t*>(residual),
                     static_cast<uint16_t*>(y), T, N);
  return hipGetLastError();
}

}  // namespace vlca
